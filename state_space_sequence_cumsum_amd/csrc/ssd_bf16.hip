// ssd_bf16.hip -- gfx950 state-pass and chunk-output kernels for bf16 inputs
// (bf16 MFMA operands, fp32 accumulation, fp32 running state).
//
// Method: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核",
// sections "Kernel 2: fwd_pass_state" (decayed chunk jump) and
// "Kernel 3：compute_out" (decayed chunk output).
//
// Both kernels contract over tokens, which are the strided dimension of every
// input tensor, and an MFMA operand packs 8 consecutive values of the
// contraction index per lane.  The state pass copies its tiles into LDS in their
// natural token-major layout with 16-byte writes and reads the token-packed
// operands back with the gfx950 LDS transpose read (ds_read_b64_tr_b16); the
// head-blocked chunk output transposes its x tile with byte permutes while
// staging it, so that the many later reads of that tile are plain 16-byte reads.
#include <algorithm>
#include <type_traits>
#include <utility>
#include <vector>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

__device__ __forceinline__ bf16x8 ld16(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

__device__ __forceinline__ bf16x8 zero8()
{
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
    return z;
}

// WG index -> (major, minor) with all minors of one major on the same XCD when
// `xcd` is set (workgroups are dealt to the 8 XCDs round-robin by index).
__device__ __forceinline__ void xcd_split(int id, int n_minor, bool xcd, int &major, int &minor)
{
    if (xcd) {
        const int x = id & 7, slot = id >> 3;
        major = x + 8 * (slot / n_minor);
        minor = slot % n_minor;
    } else {
        major = id / n_minor;
        minor = id % n_minor;
    }
}

// ===========================================================================
// State pass.  Workgroup = one (batch*head, range of NR state columns, group
// of up to K consecutive chunks), NR the largest of 256, 128, 64 dividing N; it
// keeps h^T [NR x 64] in fp32 MFMA accumulators, wave w owning RTW 32-row tiles
// of n and CTW 32-column tiles of p.
//
// The chunk jump h <- a_c h + sum_t w_t x_t (outer) B_t (a_c = exp2(G2_last),
// w_t = dt_t exp2(G2_last - G2_t) from stage 1) is evaluated with the weight on
// the x side: the contraction operand is x~ = round_bf16(w_t x_t), 64 wide, so
// the N-wide B tile is used exactly as loaded.
//
// Both inputs are token-major and the MFMA operands hold 8 consecutive tokens per
// lane.  Each chunk is processed in sub-steps of TS = 64 tokens:
//   * B reaches LDS by 16-byte global->LDS loads (each lane of a load instruction
//     writes its 16 bytes at base + 16 lane, so a wave fills 1 KB of consecutive
//     rows), two sub-steps ahead into three unpadded buffers.  Unit u of row r is
//     stored at unit u ^ swz(r), chosen on the global-address side, so that the
//     operand's transpose reads (ds_read_b64_tr_b16, 4 rows x 64 bytes per 32
//     lanes) touch 16 distinct bank groups.  No registers, no LDS writes by the
//     waves, no wait before a copy.
//   * x~: each thread loads its tokens of two columns of x as 4-byte words
//     (buffer loads; rows past L read as zero), scales them by the tokens' weights
//     and writes the two k-packed rows straight into a double-buffered LDS tile,
//     which the waves read with 16-byte reads.
//   * at a chunk start the state goes to an LDS staging tile (bf16), which is
//     stored to HBM as whole 16-byte-per-lane rows, and then decays.
// One barrier per sub-step; each waits (vmcnt) only for the B tile used next, the
// count of memory instructions issued after it being a compile-time constant of the
// unrolled step.  Rows past L are clamped out of the loads (zeros) and indices past
// the group's end to its last sub-step, so the loop has no branches around memory
// operations.
//
// Groups.  The jump is linear, so a run of chunks can start from a zero state
// and be corrected afterwards: group g (chunks [gK, gK+K)) starts from h0 if
// g == 0 and from 0 otherwise, stores its local chunk-start states, its final
// local state U_g, the decay products beta_c = prod_{gK <= c' < c} a_c' and
// gamma_g = prod_{c' in g} a_c'.  A scan over groups (group_scan_kernel) then
// gives the true state at each group start, H_g, and the true chunk-start state
// is S_local[c] + beta_c H_g.  With one group (K >= nc) the kernel is the plain
// serial state pass and writes true states and hT directly.
// ===========================================================================
constexpr int gcd_(int a, int b) { return b == 0 ? a : gcd_(b, a % b); }
constexpr int lcm3(int a, int b, int c)
{
    const int ab = a / gcd_(a, b) * b;
    return ab / gcd_(ab, c) * c;
}

template <int Q, int N>   // N = NR, the columns of one workgroup
struct SpCfg {
    static constexpr int P = 64;
    static constexpr int TS = 64;                                // tokens per sub-step
    static constexpr int NSUB = Q / TS;                          // sub-steps per chunk
    static constexpr int NWAVE = (N == 64) ? 4 : 8;
    static constexpr int NTHR = 64 * NWAVE;
    static constexpr int RTW = 1;                                // n tiles per wave
    static constexpr int CTW = (N == 256) ? 2 : 1;               // p tiles per wave
    static constexpr int SSP = N + 8;                            // chunk-start state staging rows
    static constexpr int SPT = P * N / 8 / NTHR;                 // 16-byte state pieces per thread
    static_assert((N / 32 / RTW) * (2 / CTW) == NWAVE, "wave tiling");
    static_assert(Q % TS == 0, "sub-steps per chunk");
};

typedef __attribute__((address_space(3))) void lds_void;

// LDS stores written as inline assembly.  The compiler cannot tell which LDS bytes a
// global-to-LDS load writes, so before an ordinary LDS store it waits for every such
// load still in flight, including the B tile just requested for two sub-steps later;
// these stores carry no such wait.  The state pass uses them only for buffers no
// global-to-LDS load in flight writes (the k-packed x~ tiles and the chunk-start
// staging tile), and waits for them itself (lgkmcnt(0) before each barrier).
__device__ __forceinline__ void lds_st64(void *p, u32x2 v)
{
    asm volatile("ds_write_b64 %0, %1" ::"v"((uint32_t)(uintptr_t)(lds_void *)p), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_st128(void *p, u32x4 v)
{
    asm volatile("ds_write_b128 %0, %1" ::"v"((uint32_t)(uintptr_t)(lds_void *)p), "v"(v) : "memory");
}

// WT: the weights w_t come precomputed (wt = wT of stage 1); otherwise wt is dtT and the
// kernel forms w_t = dtT_t exp2(G2_last - G2_t) from it and the cumsum
template <int Q, int NR, bool WT>
__global__ __launch_bounds__((SpCfg<Q, NR>::NTHR)) void state_pass_dma_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const float *__restrict__ G2,
    const float *__restrict__ wt, const float *__restrict__ h0, bf16 *__restrict__ S,
    float *__restrict__ hT, float *__restrict__ Ug, float *__restrict__ gam,
    float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng, int xcd)
{
    using Cf = SpCfg<Q, NR>;
    constexpr int P = 64, TS = 64, NSUB = Q / TS, NTHR = Cf::NTHR, NWAVE = Cf::NWAVE;
    constexpr int RTW = Cf::RTW, CTW = Cf::CTW, SSP = Cf::SSP, SPT = Cf::SPT;
    constexpr int XKP = 72;                 // k-packed x~ row pitch: 144 bytes
    constexpr int UPR = NR / 8;             // 16-byte units per B row
    constexpr int RPI = 64 / UPR;           // B rows per DMA instruction (one wave, 1 KB)
    constexpr int IPW = TS / RPI / NWAVE;   // DMA instructions per wave per sub-step
    constexpr int TPP = 2048 / NTHR;        // tokens per x piece (two columns)
    static_assert(IPW >= 1 && TS % (RPI * NWAVE) == 0, "B DMA cover");
    static_assert(TPP == 4 || TPP == 8, "x piece");
    __shared__ __attribute__((aligned(16))) bf16 Bs0[TS * NR];
    __shared__ __attribute__((aligned(16))) bf16 Bs1[TS * NR];
    __shared__ __attribute__((aligned(16))) bf16 Bs2[TS * NR];
    __shared__ __attribute__((aligned(16))) bf16 Xk[2][P * XKP];
    __shared__ __attribute__((aligned(16))) bf16 Ss[P * SSP];
    auto bsel = [&](int k) -> bf16 * { return k == 0 ? Bs0 : (k == 1 ? Bs1 : Bs2); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int grp, minor;
    xcd_split(blockIdx.x, (int)(gridDim.x / ng), xcd != 0, grp, minor);
    const int ntiles = N / NR, bh = minor / ntiles, n0 = (minor % ntiles) * NR;
    const int c0 = grp * K, c1 = min(c0 + K, nc);
    const int U = (c1 - c0) * NSUB;                               // sub-steps of this group
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int rt0 = (wave / (2 / CTW)) * RTW, ct0 = (wave % (2 / CTW)) * CTW;
    const int64_t st_off = (int64_t)bh * P * N;
    const float *Gh = G2 + (int64_t)bh * Lp;
    const float *wh = wt + (int64_t)bh * Lp;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const char *xbytes = reinterpret_cast<const char *>(x + (int64_t)b * L * xstride + (int64_t)h * P);
    const char *Bbytes = reinterpret_cast<const char *>(Bm + (int64_t)b * L * bstride + (int64_t)g * N + n0);
    const int xrow = (int)xstride * 2, brow = (int)bstride * 2;
    float gend0;
    {
        int gi = min(c0 + lane, c1 - 1) * Q + Q - 1;
        asm volatile("" : "+v"(gi));
        gend0 = G2[(int64_t)bh * Lp + gi];
    }

    f32x16 acc[RTW][CTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int j = 0; j < CTW; ++j) acc[i][j] = zero_acc();
    if (h0 != nullptr && grp == 0) {
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int j = 0; j < CTW; ++j) {
                const int p = 32 * (ct0 + j) + (lane & 31), n = n0 + 32 * (rt0 + i) + 4 * (lane >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(h0 + st_off + (int64_t)p * N + n + 8 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] = v[r];
                }
            }
    }

    // B tile unit swizzle: XOR of bits 2-3 of the unit index with the row, so the four
    // rows of a 32-lane transpose read land in four different 64-byte bank ranges
    auto swz = [](int r) { return (NR >= 128) ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
    // DMA instruction k of this wave covers rows R0 .. R0 + RPI - 1; lane: row R0 + lane / UPR,
    // physical unit lane % UPR, which holds logical unit (lane % UPR) ^ swz(row)
    uint32_t bdoff[IPW];
#pragma unroll
    for (int k = 0; k < IPW; ++k) {
        const int row = (wave * IPW + k) * RPI + lane / UPR;
        bdoff[k] = (uint32_t)(row * brow + 16 * ((lane % UPR) ^ swz(row)));
    }
    // x piece: columns 2 pp, 2 pp + 1 of tokens TPP tq .. TPP tq + TPP - 1
    const int pp = tid & 31, tq = tid >> 5;
    const uint32_t xoff = (uint32_t)(TPP * tq * xrow + 4 * pp);
    struct Regs {
        uint32_t xv[TPP];
        f32x4 w[TPP / 4];              // the tokens' weights (WT) or their dt
        f32x4 g[WT ? 1 : TPP / 4];     // (without WT) their cumsum values
        float gl;                      // cumsum at the end of the sub-step's chunk
    };
    const int last_sub = U - 1;
    auto tok0 = [&](int u) { return (c0 + u / NSUB) * Q + (u % NSUB) * TS; };
    auto dma_b = [&](int kb, int u) {
        u = min(u, last_sub);
        const int t0 = tok0(u);
        const rsrc_t br = make_rsrc(Bbytes + (int64_t)t0 * brow, (L - t0) * brow);
        bf16 *dst = bsel(kb);
#pragma unroll
        for (int k = 0; k < IPW; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)(dst + (wave * IPW + k) * RPI * NR),
                                                     16, (int)bdoff[k], 0, 0, 0);
    };
    // the chunk-end cumsum value (with WT only where sub-step u starts a chunk, the one
    // place that uses it then), the weights (or dt and cumsum) of this thread's tokens and
    // x of sub-step u; `with_gl` is a compile-time constant, so the number of memory
    // instructions a call issues (NLD_GL with it, NLD_NOGL without) is known
    constexpr int NLD_GL = WT ? 1 + TPP / 4 + TPP : 1 + 2 * (TPP / 4) + TPP;
    constexpr int NLD_NOGL = WT ? TPP / 4 + TPP : NLD_GL;
    auto load = [&](Regs &R, int u, auto with_gl) {
        u = min(u, last_sub);
        const int t0 = tok0(u);
        if constexpr (!WT || decltype(with_gl)::value) {
            int gi = (c0 + u / NSUB) * Q + Q - 1;
            asm volatile("" : "+v"(gi));   // per-lane load: a scalar one would share the LDS wait counter
            R.gl = Gh[gi];
        }
        const float *wb = wh + t0 + TPP * tq;
#pragma unroll
        for (int k = 0; k < TPP / 4; ++k) R.w[k] = *reinterpret_cast<const f32x4 *>(wb + 4 * k);
        if constexpr (!WT) {
            const float *gb = Gh + t0 + TPP * tq;
#pragma unroll
            for (int k = 0; k < TPP / 4; ++k) R.g[k] = *reinterpret_cast<const f32x4 *>(gb + 4 * k);
        }
        const rsrc_t xr = make_rsrc(xbytes + (int64_t)t0 * xrow, (L - t0) * xrow);
#pragma unroll
        for (int k = 0; k < TPP; ++k) R.xv[k] = buf_load_b32(xr, xoff + k * xrow);
    };
    // the state-pass weight of token e of a sub-step: its dt times its decay to the chunk's end
    auto weight = [](const Regs &R, int e) {
        if constexpr (WT)
            return R.w[e >> 2][e & 3];
        else
            return R.w[e >> 2][e & 3] * fast_exp2(R.gl - R.g[e >> 2][e & 3]);
    };
    // k-packed x~ row p: 16-byte unit u (8 tokens) stored at unit u ^ ((p >> 4) & 1)
    auto xk_off = [](int p, int u) { return p * XKP + 8 * (u ^ ((p >> 4) & 1)); };
    auto stageX = [&](const Regs &R, int kx) {
        uint32_t f0[TPP / 2], f1[TPP / 2];
#pragma unroll
        for (int k2 = 0; k2 < TPP / 2; ++k2) {
            const float w0 = weight(R, 2 * k2), w1 = weight(R, 2 * k2 + 1);
            const uint32_t a = R.xv[2 * k2], c = R.xv[2 * k2 + 1];
            f0[k2] = pack_bf16(bf_lo(a) * w0, bf_lo(c) * w1);
            f1[k2] = pack_bf16(bf_hi(a) * w0, bf_hi(c) * w1);
        }
        if constexpr (TPP == 8) {
            lds_st128(&Xk[kx][xk_off(2 * pp, tq)], u32x4{f0[0], f0[1], f0[2], f0[3]});
            lds_st128(&Xk[kx][xk_off(2 * pp + 1, tq)], u32x4{f1[0], f1[1], f1[2], f1[3]});
        } else {
            lds_st64(&Xk[kx][xk_off(2 * pp, tq >> 1) + 4 * (tq & 1)], u32x2{f0[0], f0[1]});
            lds_st64(&Xk[kx][xk_off(2 * pp + 1, tq >> 1) + 4 * (tq & 1)], u32x2{f1[0], f1[1]});
        }
    };

    // chunk start: the chunk-start state to the staging tile (bf16, row p, columns n), then
    // the state decays
    auto chunk_start = [&](float gl) {
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int j = 0; j < CTW; ++j) {
                const int p = 32 * (ct0 + j) + (lane & 31), n = 32 * (rt0 + i) + 4 * (lane >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = (bf16)acc[i][j][4 * q + r];
                    lds_st64(&Ss[p * SSP + n + 8 * q], __builtin_bit_cast(u32x2, o));
                }
            }
        const float a = fast_exp2(gl);
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int j = 0; j < CTW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] *= a;
    };
    // The first chunk of every group after the first starts from the zero state: it is not
    // stored (the chunk output reads it as zero).  Its stores still issue, into an empty
    // buffer range, so the wait counts below stay exact.
    auto state_out = [&](int c) {
        const bool empty = grp > 0 && c == c0;
        const rsrc_t sr = make_rsrc(S + ((int64_t)bh * nc + c) * P * N + n0, empty ? 0 : (P * N - n0) * 2);
#pragma unroll
        for (int r = 0; r < SPT; ++r) {
            const int id = tid + NTHR * r, p = id / (NR / 8), c8 = id % (NR / 8);
            const u32x4 v = *reinterpret_cast<const u32x4 *>(&Ss[p * SSP + 8 * c8]);
            buf_store_b128(sr, (uint32_t)((p * N + 8 * c8) * 2), v);
        }
    };
    // transpose-read operand: lane l reads 4 tokens (rows) of 4 columns; rows
    // 8 (l / 32) + (l % 16) / 4 (+ 4 for the second read), columns 32 tile + 16 ((l / 16) & 1) + 4 (l % 4)
    const int arow = 8 * (lane >> 5) + ((lane & 15) >> 2);
    int aoff[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int u = 4 * (rt0 + i) + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        aoff[i] = arow * NR + 8 * (u ^ swz(arow)) + 4 * (lane & 1);
    }
    const int l32 = lane & 31, half = lane >> 5;
    auto mma_sub = [&](int kb, int kx) {
        const bf16 *bt = bsel(kb);
#pragma unroll
        for (int ks = 0; ks < TS / 16; ++ks) {
            bf16x8 bfr[CTW];
#pragma unroll
            for (int j = 0; j < CTW; ++j) bfr[j] = ld16(&Xk[kx][xk_off(32 * (ct0 + j) + l32, 2 * ks + half)]);
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const bf16 *a0 = bt + 16 * ks * NR + aoff[i];
                const bf16x8 af = cat8(tr_read4(a0), tr_read4(a0 + 4 * NR));
#pragma unroll
                for (int j = 0; j < CTW; ++j) mma(acc[i][j], af, bfr[j]);
            }
        }
    };
    // memory instructions issued after the B DMA of step j - 1 and before the barrier of step j
    // (a lower bound, so the wait never falls short): step j - 1's loads and late state
    // stores, step j's DMA, loads and late state stores
    // (nx: the loads a step issues, with the chunk-end value when sub-step s + 2 starts a
    // chunk; the step before position 0 is the prologue or the previous block's last step,
    // which issue the same loads)
    constexpr auto wait_n = [](int j) {
        const auto so_late = [](int i) { return (NSUB > 1 && i % NSUB == 1) ? SPT : 0; };
        const auto nx = [](int i) { return ((i + 2) % NSUB == 0) ? NLD_GL : NLD_NOGL; };
        return nx(j > 0 ? j - 1 : lcm3(NSUB, 3, 2) - 1) + (j > 0 ? so_late(j - 1) : 0) + IPW + nx(j) +
               so_late(j);
    };
// (sched_barrier keeps the scheduler from moving any instruction across: otherwise it
// pulls the next step's register work up, and its wait for this step's x loads drains
// the B loads in flight with them)
#define SP_BARRIER(n)                                                                           \
    do {                                                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        asm volatile("" ::: "memory");                                                          \
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(n));                                               \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                         \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)
#define LDS_BARRIER()                                                                           \
    do {                                                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                         \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)

    Regs R[2];
    // step s: B of sub-step s + 2 and x of sub-step s + 2 go out, products of sub-step s,
    // x~ of sub-step s + 1 into LDS, then wait for B of sub-step s + 1 and synchronise
    auto step = [&](int s, auto jc) {
        constexpr int j = decltype(jc)::value;
        if (j % NSUB == 0) {
            if constexpr (NSUB == 1) {   // the previous chunk's staged state leaves first
                if (s > 0) state_out(c0 + s - 1);
                LDS_BARRIER();
            }
            chunk_start(R[j & 1].gl);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        dma_b((j + 2) % 3, s + 2);
        asm volatile("" ::: "memory");
        load(R[j & 1], s + 2, std::integral_constant<bool, (j + 2) % NSUB == 0>{});
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);   // the loads go out before anything waits
        mma_sub(j % 3, j & 1);
        stageX(R[(j + 1) & 1], (j + 1) & 1);
        if (NSUB > 1 && j % NSUB == 1) state_out(c0 + s / NSUB);
        constexpr int nwait = wait_n(j);
        SP_BARRIER(nwait);
    };

    dma_b(0, 0);
    asm volatile("" ::: "memory");
    load(R[0], 0, std::true_type{});
    asm volatile("" ::: "memory");
    dma_b(1, 1);
    asm volatile("" ::: "memory");
    load(R[1], 1, std::integral_constant<bool, NSUB == 1>{});
    asm volatile("" ::: "memory");
    stageX(R[0], 0);
    constexpr int nwait0 = NLD_GL + IPW + (NSUB == 1 ? NLD_GL : NLD_NOGL);
    SP_BARRIER(nwait0);   // B of sub-step 0
    constexpr int UNR = lcm3(NSUB, 3, 2);
    int s = 0;
    for (; s + UNR <= U; s += UNR) static_for<UNR>([&](auto jc) { step(s + decltype(jc)::value, jc); });
    static_for<UNR>([&](auto jc) {
        if (s + decltype(jc)::value < U) step(s + decltype(jc)::value, jc);
    });
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no LDS load still in flight past this point
    if constexpr (NSUB == 1) state_out(c1 - 1);
#undef SP_BARRIER
#undef LDS_BARRIER

    // decay products of the group (beta_c before each chunk, gamma for the group): lane k of
    // wave 0 holds chunk c0 + k0 + k's decay (the first 64 from the prologue's loads, so no
    // memory wait here) and the running product is taken in chunk order, as a sequential
    // loop over the chunks would
    if (n0 == 0 && wave == 0 && (beta != nullptr || gam != nullptr)) {
        float run = 1.0f;
        auto products = [&](float gv, int k0) {   // chunks c0 + k0 .. c0 + k0 + 63
            const float e = fast_exp2(gv);
            const int cnt = min(64, c1 - c0 - k0);
            float mine = 0.0f;
            for (int k = 0; k < cnt; ++k) {
                if (lane == k) mine = run;
                run *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), k));
            }
            if (beta != nullptr && lane < cnt) beta[(int64_t)bh * nc + c0 + k0 + lane] = mine;
        };
        products(gend0, 0);
        for (int k0 = 64; k0 < c1 - c0; k0 += 64) {   // groups of more than 64 chunks
            int gi = min(c0 + k0 + lane, c1 - 1) * Q + Q - 1;
            asm volatile("" : "+v"(gi));
            products(Gh[gi], k0);
        }
        if (gam != nullptr && lane == 0) gam[(int64_t)bh * ng + grp] = run;
    }

    // the state after the group's last chunk
    float *dst = (Ug != nullptr) ? Ug + ((int64_t)bh * ng + grp) * P * N : (hT ? hT + st_off : nullptr);
    if (dst != nullptr) {
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int j = 0; j < CTW; ++j) {
                const int p = 32 * (ct0 + j) + (lane & 31), n = n0 + 32 * (rt0 + i) + 4 * (lane >> 5);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = acc[i][j][4 * q + r];
                    *reinterpret_cast<f32x4 *>(dst + (int64_t)p * N + n + 8 * q) = o;
                }
            }
    }
}

// ===========================================================================
// State pass, register-transposed operands.  Workgroup = one (batch*head, range
// of NR state columns, group of up to K consecutive chunks), NR/64 waves; wave w
// keeps h[p][n] for all 64 p and its 64 columns n0 + 64 w .. + 64 in four fp32
// MFMA accumulators (v_mfma_f32_32x32x16_bf16, row = p, column = n).
//
// The jump h <- a_c h + sum_t w_t x_t (outer) B_t contracts over tokens, the
// strided dimension of both inputs, and an MFMA operand lane holds 8 consecutive
// values of the contraction index.  So:
//   * B (the N-wide operand, read once per workgroup): every lane loads its own
//     two columns for 8 tokens as 4-byte words (lanes 0-31 tokens 0-7, lanes 32-63
//     tokens 8-15 of a 16-token step; one 128-byte row segment per 32 lanes) and
//     byte-permutes them into two k-packed operands, columns 2l and 2l + 1 of the
//     wave's range.  B never goes through LDS.
//   * x~ = round_bf16(w_t x_t) (64 wide, shared by all waves): each thread loads 8
//     tokens x 2 columns of x, scales them by the tokens' weights and writes the two
//     k-packed rows straight into a double-buffered LDS tile, which the waves read
//     with 16-byte reads.  One barrier per 64-token sub-step.
// The chunk-start state goes to HBM straight from the accumulators: lane l holds
// columns 2l and 2l + 1 of a row, so a 4-byte store per lane writes 128 contiguous
// bytes per 32 lanes.  Loads run D sub-steps ahead in a register ring; rows past
// L are clamped to row L-1 (their weight is 0) and indices past the group's end
// to its last sub-step, so the loop has no branches around memory operations.
// Groups and the decay products for the group scan as in the LDS-transposed kernel.
// ===========================================================================
// WT as for the kernel above
template <int Q, int NR, int D, bool WT>
__global__ __launch_bounds__(NR) void state_pass_rt_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const float *__restrict__ G2,
    const float *__restrict__ wt, const float *__restrict__ h0, bf16 *__restrict__ S,
    float *__restrict__ hT, float *__restrict__ Ug, float *__restrict__ gam,
    float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng, int xcd)
{
    constexpr int P = 64, TS = 64, NSUB = Q / TS, NTHR = NR, KS = TS / 16;
    constexpr int XPT = 256 / NTHR;   // x pieces (8 tokens x 2 columns) per thread per sub-step
    constexpr int XKP = 72;           // k-packed x~ row pitch: 144 bytes (16 more than 128)
    static_assert(NR % 64 == 0 && NR <= 256 && Q % TS == 0, "state-pass tiling");
    __shared__ __attribute__((aligned(16))) bf16 Xk[2][P * XKP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, half = lane >> 5;
    int grp, minor;
    xcd_split(blockIdx.x, (int)(gridDim.x / ng), xcd != 0, grp, minor);
    const int ntiles = N / NR, bh = minor / ntiles, n0 = (minor % ntiles) * NR;
    const int c0 = grp * K, c1 = min(c0 + K, nc);
    const int U = (c1 - c0) * NSUB;                               // sub-steps of this group
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int64_t st_off = (int64_t)bh * P * N;
    const float *Gh = G2 + (int64_t)bh * Lp;
    const float *wh = wt + (int64_t)bh * Lp;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    // x and B are read through buffer resources based at the first row of each tile and
    // ending at row L, so rows past the sequence read as zero (their weight is 0 too);
    // per-lane offsets are 32-bit (the host checks that one batch of x and of B spans
    // less than 2^31 bytes)
    const char *xbytes = reinterpret_cast<const char *>(x + (int64_t)b * L * xstride + (int64_t)h * P);
    const char *Bbytes = reinterpret_cast<const char *>(Bm + (int64_t)b * L * bstride + (int64_t)g * N +
                                                        n0 + 64 * wave);
    const int xrow = (int)xstride * 2, brow = (int)bstride * 2;
    const int ncol = n0 + 64 * wave + 2 * l32;                   // this lane's two columns
    // the chunk-end cumsum value of chunk c0 + lane (clamped to the group), for the decay
    // products written at the end; a per-lane load issued now, hidden by the chunk loop
    float gend0;
    {
        int gi = min(c0 + lane, c1 - 1) * Q + Q - 1;
        asm volatile("" : "+v"(gi));
        gend0 = G2[(int64_t)bh * Lp + gi];
    }

    // acc[pt][e] element v: p = 32 pt + acc_row(v, lane), n = ncol + e
    f32x16 acc[2][2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int e = 0; e < 2; ++e) acc[pt][e] = zero_acc();
    if (h0 != nullptr && grp == 0) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int p = 32 * pt + acc_row(v, lane);
                const f32x2 hv = *reinterpret_cast<const f32x2 *>(h0 + st_off + (int64_t)p * N + ncol);
                acc[pt][0][v] = hv[0];
                acc[pt][1][v] = hv[1];
            }
    }

    // x piece r of a sub-step: columns 2 pp, 2 pp + 1 of tokens 8 to .. 8 to + 7, read at
    // byte offsets xoff[r] + k * xrow from the sub-step's first row; B word k of a 16-token
    // step at boffk + k * brow from that step's first row
    int ppv[XPT], tov[XPT];
    uint32_t xoff[XPT];
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
        const int id = tid + NTHR * r;
        ppv[r] = id & 31;
        tov[r] = id >> 5;
        xoff[r] = (uint32_t)(8 * tov[r] * xrow + 4 * ppv[r]);
    }
    const uint32_t boff = (uint32_t)(8 * half * brow + 4 * l32);
    struct Regs {
        uint32_t b[KS][8];      // B words of k-step ks: token 16 ks + 8 half + k, columns ncol, ncol + 1
        uint32_t xv[XPT][8];    // x words of piece r: token 8 to + k, columns 2 pp, 2 pp + 1
        f32x4 w[XPT][2];        // the weights (WT) or dt of those 8 tokens
        f32x4 g[WT ? 1 : XPT][2];   // (without WT) their cumsum values
        float gl;               // cumsum value at the end of the sub-step's chunk
    };
    auto tok0 = [&](int u) { return (c0 + u / NSUB) * Q + (u % NSUB) * TS; };
    // x, weights and the chunk-end value first (used a step earlier), then B
    auto load = [&](Regs &R, int u) {
        u = min(u, U - 1);
        const int t0 = tok0(u);
        int gi = (c0 + u / NSUB) * Q + Q - 1;
        asm volatile("" : "+v"(gi));   // per-lane load: a scalar one would share the LDS wait counter
        R.gl = Gh[gi];
        const rsrc_t xr = make_rsrc(xbytes + (int64_t)t0 * xrow, (L - t0) * xrow);
#pragma unroll
        for (int r = 0; r < XPT; ++r) {
            const float *wb = wh + t0 + 8 * tov[r];
            R.w[r][0] = *reinterpret_cast<const f32x4 *>(wb);
            R.w[r][1] = *reinterpret_cast<const f32x4 *>(wb + 4);
            if constexpr (!WT) {
                const float *gb = Gh + t0 + 8 * tov[r];
                R.g[r][0] = *reinterpret_cast<const f32x4 *>(gb);
                R.g[r][1] = *reinterpret_cast<const f32x4 *>(gb + 4);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) R.xv[r][k] = buf_load_b32(xr, xoff[r] + k * xrow);
        }
        __builtin_amdgcn_sched_barrier(0);   // keeps this issue order
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int tk = t0 + 16 * ks;
            const rsrc_t br = make_rsrc(Bbytes + (int64_t)tk * brow, (L - tk) * brow);
#pragma unroll
            for (int k = 0; k < 8; ++k) R.b[ks][k] = buf_load_b32(br, boff + k * brow);
        }
    };
    // k-packed x~ row p at 16-byte unit u is stored at unit u ^ ((p >> 4) & 1): with the
    // 144-byte pitch both the staging writes (16 rows of one parity) and the operand reads
    // (16 consecutive rows) touch 16 distinct 16-byte bank groups
    auto xk_off = [](int p, int u) { return p * XKP + 8 * (u ^ ((p >> 4) & 1)); };
    auto stageX = [&](const Regs &R, int kb) {
#pragma unroll
        for (int r = 0; r < XPT; ++r) {
            u32x4 f0, f1;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                // the state-pass weight: dt times the decay to the end of the token's chunk
                const int e0 = 2 * k2, e1 = 2 * k2 + 1;
                float w0 = R.w[r][e0 >> 2][e0 & 3], w1 = R.w[r][e1 >> 2][e1 & 3];
                if constexpr (!WT) {
                    w0 *= fast_exp2(R.gl - R.g[WT ? 0 : r][e0 >> 2][e0 & 3]);
                    w1 *= fast_exp2(R.gl - R.g[WT ? 0 : r][e1 >> 2][e1 & 3]);
                }
                const uint32_t a = R.xv[r][2 * k2], c = R.xv[r][2 * k2 + 1];
                f0[k2] = pack_bf16(bf_lo(a) * w0, bf_lo(c) * w1);
                f1[k2] = pack_bf16(bf_hi(a) * w0, bf_hi(c) * w1);
            }
            const int p = 2 * ppv[r];
            *reinterpret_cast<u32x4 *>(&Xk[kb][xk_off(p, tov[r])]) = f0;
            *reinterpret_cast<u32x4 *>(&Xk[kb][xk_off(p + 1, tov[r])]) = f1;
        }
    };
    auto mma_sub = [&](const Regs &R, int kb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 bf[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                u32x4 q;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) q[k2] = pack_halves(R.b[ks][2 * k2], R.b[ks][2 * k2 + 1], e);
                bf[e] = __builtin_bit_cast(bf16x8, q);
            }
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const bf16x8 af = ld16(&Xk[kb][xk_off(32 * pt + l32, 2 * ks + half)]);
#pragma unroll
                for (int e = 0; e < 2; ++e) mma(acc[pt][e], af, bf[e]);
            }
        }
    };
    // chunk start: the state goes to S[c] (bf16, straight from the accumulators), then
    // decays.  As in the kernel above, the zero first state of a group after the first is
    // not stored (its stores go to an empty range).
    const uint32_t srow_off = (uint32_t)((4 * half * N + ncol) * 2);   // lane part of the S offsets
    auto chunk_start = [&](float gl, int c) {
        const bool empty = grp > 0 && c == c0;
        const rsrc_t sr = make_rsrc(S + ((int64_t)bh * nc + c) * P * N, empty ? 0 : P * N * 2);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int prow = 32 * pt + 8 * (v >> 2) + (v & 3);   // acc_row without the lane part
                buf_store_b32(sr, (uint32_t)(prow * N * 2) + srow_off, pack_bf16(acc[pt][0][v], acc[pt][1][v]));
            }
        const float a = fast_exp2(gl);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[pt][e][v] *= a;
    };

    // Register ring of D sub-steps: slot u % D holds sub-step u from its load (step u - D)
    // until its B operands are used (step u); its x~ is staged one step earlier.
    static_assert(D >= 2, "a slot holds one sub-step from the x~ staging to its products");
    Regs R[D];
    auto step = [&](int s, int j) {
        if (j % NSUB == 0) chunk_start(R[j % D].gl, c0 + s / NSUB);
        mma_sub(R[j % D], j & 1);
        stageX(R[(j + 1) % D], (j + 1) & 1);
        load(R[j % D], s + D);
        __syncthreads();
    };
#pragma unroll
    for (int u = 0; u < D; ++u) load(R[u], u);
    stageX(R[0], 0);
    __syncthreads();
    // the body covers UNR = lcm(NSUB, D, 2) sub-steps so that ring slots, LDS buffers and
    // chunk-start positions are compile-time constants
    constexpr int UNR = lcm3(NSUB, D, 2);
    int s = 0;
    for (; s + UNR <= U; s += UNR) {
#pragma unroll
        for (int j = 0; j < UNR; ++j) step(s + j, j);
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j)
        if (s + j < U) step(s + j, j);

    // decay products of the group (beta_c before each chunk, gamma for the group), as in
    // the kernel above
    if (n0 == 0 && wave == 0 && (beta != nullptr || gam != nullptr)) {
        float run = 1.0f;
        auto products = [&](float gv, int k0) {   // chunks c0 + k0 .. c0 + k0 + 63
            const float e = fast_exp2(gv);
            const int cnt = min(64, c1 - c0 - k0);
            float mine = 0.0f;
            for (int k = 0; k < cnt; ++k) {
                if (lane == k) mine = run;
                run *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), k));
            }
            if (beta != nullptr && lane < cnt) beta[(int64_t)bh * nc + c0 + k0 + lane] = mine;
        };
        products(gend0, 0);
        for (int k0 = 64; k0 < c1 - c0; k0 += 64) {   // groups of more than 64 chunks
            int gi = min(c0 + k0 + lane, c1 - 1) * Q + Q - 1;
            asm volatile("" : "+v"(gi));
            products(Gh[gi], k0);
        }
        if (gam != nullptr && lane == 0) gam[(int64_t)bh * ng + grp] = run;
    }

    // the state after the group's last chunk (fp32): 8 bytes per lane, 256 contiguous bytes
    // per 32 lanes
    float *dst = (Ug != nullptr) ? Ug + ((int64_t)bh * ng + grp) * P * N : (hT ? hT + st_off : nullptr);
    if (dst != nullptr) {
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int p = 32 * pt + acc_row(v, lane);
                f32x2 o;
                o[0] = acc[pt][0][v];
                o[1] = acc[pt][1][v];
                *reinterpret_cast<f32x2 *>(dst + (int64_t)p * N + ncol) = o;
            }
    }
}

// ===========================================================================
// Group scan.  For each (batch*head, state element): walk the groups in order,
// H_1 = U_0 and H_{g+1} = gamma_g H_g + U_g; H_g (the true state at group g's
// start) replaces U_g in place for the groups g >= g_f32 (the chunk outputs that
// read fp32 states), a bf16 copy goes to Hb (zeros for group 0, which needs no
// correction), and the state after the last group is hT.
// ===========================================================================
template <int NGMAX>
__global__ __launch_bounds__(256) void group_scan_kernel(float *__restrict__ Ug,
                                                         const float *__restrict__ gam,
                                                         float *__restrict__ hT,
                                                         bf16 *__restrict__ Hb, int PN, int ng,
                                                         int g_f32)
{
    const int bh = blockIdx.y;
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    f32x4 hcar = {0.0f, 0.0f, 0.0f, 0.0f};
    // groups in batches of NGMAX: all loads of a batch are issued before its
    // in-place stores, so their latencies overlap
    for (int g0 = 0; g0 < ng; g0 += NGMAX) {
        f32x4 v[NGMAX];
        float gm[NGMAX];
#pragma unroll
        for (int k = 0; k < NGMAX; ++k) {
            const int g = min(g0 + k, ng - 1);
            v[k] = *reinterpret_cast<const f32x4 *>(Ug + ((int64_t)bh * ng + g) * PN + e);
            // per-lane load, in flight with the state loads (a scalar load is issued and
            // waited for on its own)
            int gi = bh * ng + g;
            asm volatile("" : "+v"(gi));
            gm[k] = gam[gi];
        }
#pragma unroll
        for (int k = 0; k < NGMAX; ++k) {
            const int g = g0 + k;
            if (g < ng) {
                const int64_t off = ((int64_t)bh * ng + g) * PN + e;
                if (g > 0 && g >= g_f32) *reinterpret_cast<f32x4 *>(Ug + off) = hcar;
                if (Hb != nullptr) {
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = (bf16)hcar[r];   // zero for g == 0
                    *reinterpret_cast<bf16x4 *>(Hb + off) = o;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) hcar[r] = gm[k] * hcar[r] + v[k][r];
            }
        }
    }
    if (hT != nullptr) *reinterpret_cast<f32x4 *>(hT + (int64_t)bh * PN + e) = hcar;
}

// ===========================================================================
// Chunk output.  Workgroup = one (chunk, batch*head) with Q/32 waves; wave w
// owns one 32-token row tile I = rowtile(w).  Waves w and w + Q/64 (which the
// hardware places on the same SIMD) get tiles that add up to Q/32 - 1, so every
// SIMD does the same number, Q/32 + 1, of causal tile pairs (J, I), J <= I.
// The output is built transposed, Y^T [64 p x 32 tokens] per row tile.
//
// Prologue: the (dt x)^T tile, the chunk's decays and the chunk-start state
// S_eff [64 x N] (bf16, whole width) go to LDS; these per-item loads are all
// issued together so their latencies overlap.
// Phase 1 streams N in slices of 64: the slice of B (all chunk rows) is staged
// in LDS, the wave's C rows come from global memory, and the next slice is
// loaded while the current one is multiplied (B and C are shared by all heads
// of the chunk, so these loads mostly hit L2):
//   * CB_J = (B C^T)[tile J, tile I] for J <= I (accumulators indexed by J);
//   * Y^T += S_eff C^T (the inter-chunk term).
// Phase 2, per J <= I: the C B^T tile becomes the decay matrix
//   M[j, i] = (i >= j) ? CB[j, i] * exp2(G_i - G_j) : 0      (selection, never a product with a mask)
// rounded to bf16 and fed to MFMA straight from registers against (dt x)^T.
// Off the diagonal (J < I) the decay factors exactly into
// exp2(G_i - G_e) * exp2(G_e - G_j), e the last token of tile J; both factors are
// <= 1, the second a per-token table, so such a tile costs one exp2 per lane.
// The Y^T accumulator is scaled by exp2(G_i) between the two phases.
//
// Chunk-start state handed over by a grouped state pass (CORR): S holds the
// state relative to the start of the chunk's group and S_eff = S + beta_c H_g
// (group 0 already started from the true initial state; beta is 0 there, so it
// reads its group's slot and adds nothing).
//
// Rows past L are not zeroed: they are clamped to row L-1.  Their dt is 0 (stage
// 1 writes zeros there), so their (dt x) rows vanish and the outputs of such
// rows are never stored.  With no per-lane predicates and no branches around
// the slice loads, the wait counts keep the next slice in flight while the
// current one is multiplied.
// ===========================================================================
// NMX: the largest N this instance serves (128, 256 or 512); it sizes the S_eff
// tile, so small states leave LDS for more workgroups per CU.
template <int Q, bool CORR, int NMX>
__global__ __launch_bounds__(2 * Q) void chunk_out_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const float *__restrict__ G2, const float *__restrict__ dtT, const bf16 *__restrict__ S,
    const float *__restrict__ D, bf16 *__restrict__ y, const float *__restrict__ Hg,
    const float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng,
    int c_first, int nc_grid, int xcd)
{
    constexpr int P = 64, NI = Q / 32, NW = Q / 32, NTHR = 2 * Q, NS = 64;
    constexpr int XP = Q + 8, BP = frag_pitch(NS);
    constexpr int BPC = Q * (NS / 8) / NTHR;   // 16-byte B pieces per thread per slice
    constexpr int SPC = P * (NS / 8) / NTHR;   // 16-byte S pieces per thread per 64 columns
    // S_eff columns staged per round: the pieces of a round (S in bf16, H_g in fp32)
    // are in flight together, so with 64-token chunks (four pieces per thread per 64
    // columns) and the correction a round is halved to stay within the registers
    constexpr int SPART = (CORR && SPC >= 4) ? 128 : 256;
    static_assert(BPC >= 1 && SPC >= 1, "slice staging cover");
    // (dt x)^T [p][position]: within each 16-token group the token at offset o is
    // kept at position o with its middle two 4-token blocks swapped, so the
    // accumulator token order 4(l/32)+{0..3}, 8+4(l/32)+{0..3} of lane l becomes 8
    // consecutive positions.
    __shared__ __attribute__((aligned(16))) bf16 Xd[P * XP];
    __shared__ __attribute__((aligned(16))) bf16 Bs[Q * BP];
    // S_eff rows of N + 8 elements: an odd number of 16-byte units, so 16
    // consecutive rows read at the same column hit 16 distinct bank groups
    __shared__ __attribute__((aligned(16))) bf16 Sf[P * (NMX + 8)];
    __shared__ __attribute__((aligned(16))) float Gs[Q];
    __shared__ __attribute__((aligned(16))) float We[Q];   // exp2(G_e - G_j), e = end of j's tile

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int I = (w < NW / 2) ? w : NW - 1 - (w - NW / 2);
    const int SFP = N + 8;

    // Workgroup -> (chunk c_first + k, batch*head), k < nc_grid, heads innermost.
    // With `xcd` set (nc_grid a multiple of 8) XCD x gets the contiguous chunk
    // range [x nc_grid/8, (x+1) nc_grid/8): a chunk's B and C rows are shared by
    // all its heads and a state-pass group's carried state by its consecutive
    // chunks, and both then stay in one L2.
    const int bH = gridDim.x / nc_grid;
    int c, bh;
    if (xcd) {
        const int xx = blockIdx.x & 7, slot = blockIdx.x >> 3;
        c = xx * (nc_grid / 8) + slot / bH;
        bh = slot % bH;
    } else {
        c = blockIdx.x / bH;
        bh = blockIdx.x % bH;
    }
    c += c_first;
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int t0 = c * Q;
    const int nvalid = min(Q, L - t0);          // rows of this chunk inside the sequence
    const int64_t xstride = (int64_t)H * P, cstride = (int64_t)G * N;
    const bf16 *xb = x + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
    const char *Bb = reinterpret_cast<const char *>(Bm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N);
    const char *Cb = reinterpret_cast<const char *>(Cm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N);
    const float *Gh = G2 + (int64_t)bh * Lp + t0;
    const float *dh = dtT + (int64_t)bh * Lp + t0;
    const int kq = 8 * (lane >> 5);
    const int cgrp = CORR ? c / K : 0;
    // the first chunk of a group after the first starts from zero (the state pass stores
    // nothing for it): its S loads read an empty range, which returns zeros
    const rsrc_t sr = make_rsrc(S + ((int64_t)bh * nc + c) * P * N,
                                (CORR && cgrp > 0 && c % K == 0) ? 0 : P * N * 2);
    const char *Hc = reinterpret_cast<const char *>(CORR ? Hg + ((int64_t)bh * ng + cgrp) * P * N : nullptr);
    const float bc = (CORR && cgrp > 0) ? beta[(int64_t)bh * nc + c] : 0.0f;

    const int i_loc = I * 32 + (lane & 31);
    const bool iv = i_loc < nvalid;
    const int crow_off = min(i_loc, nvalid - 1) * (int)cstride * 2 + kq * 2;   // bytes
    const int brow = (int)cstride * 2;

    // ---- slice registers: the next B / C slice while the current one is multiplied
    bf16x8 bq[BPC], cn[NS / 16];
    int bo[BPC];
#pragma unroll
    for (int r = 0; r < BPC; ++r) {
        const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
        bo[r] = min(t, nvalid - 1) * brow + oct * 16;
    }
    auto load_slice = [&](int n0) {
#pragma unroll
        for (int r = 0; r < BPC; ++r) bq[r] = *reinterpret_cast<const bf16x8 *>(Bb + (uint32_t)(bo[r] + n0 * 2));
#pragma unroll
        for (int ks = 0; ks < NS / 16; ++ks)
            cn[ks] = *reinterpret_cast<const bf16x8 *>(Cb + (uint32_t)(crow_off + (n0 + ks * 16) * 2));
    };

    // ---- S_eff staging: piece r of 64-column block q is row p, 8 columns
    auto s_piece = [&](int r) { return tid + NTHR * r; };
    auto stage_state = [&](int nb) {   // columns [nb, nb + SPART) (those below N)
        bf16x8 sq[SPART / 64][SPC];
        f32x4 hq[SPART / 64][SPC][2];
#pragma unroll
        for (int q = 0; q < SPART / 64; ++q) {
            if (nb + 64 * q < N) {
#pragma unroll
                for (int r = 0; r < SPC; ++r) {
                    const int id = s_piece(r), p = id >> 3, col = nb + 64 * q + (id & 7) * 8;
                    sq[q][r] = __builtin_bit_cast(bf16x8, buf_load_b128(sr, (uint32_t)((p * N + col) * 2)));
                    if constexpr (CORR) {
                        hq[q][r][0] = *reinterpret_cast<const f32x4 *>(Hc + (uint32_t)((p * N + col) * 4));
                        hq[q][r][1] = *reinterpret_cast<const f32x4 *>(Hc + (uint32_t)((p * N + col) * 4 + 16));
                    }
                }
            }
        }
        return [&, nb, sq, hq]() {
            (void)hq;   // read only with the correction
#pragma unroll
            for (int q = 0; q < SPART / 64; ++q) {
                if (nb + 64 * q < N) {
#pragma unroll
                    for (int r = 0; r < SPC; ++r) {
                        const int id = s_piece(r), p = id >> 3, col = nb + 64 * q + (id & 7) * 8;
                        bf16x8 sv = sq[q][r];
                        if constexpr (CORR) {
#pragma unroll
                            for (int e2 = 0; e2 < 8; ++e2)
                                sv[e2] = (bf16)((float)sv[e2] + bc * hq[q][r][e2 >> 2][e2 & 3]);
                        }
                        *reinterpret_cast<bf16x8 *>(&Sf[p * SFP + col]) = sv;
                    }
                }
            }
        };
    };

    // (dt x)^T tile and the chunk's decays; the chunk-start state and the first
    // N slice are requested right behind the x tile so all latencies overlap.
    // Thread = one 8-token x 4-p block: rows loaded token-major, scaled by dt,
    // packed per p column.  A wave covers 8 token groups (lane % 8) x 8 column
    // groups (lane / 8).
    {
        // lanes l and l + 32 take the two 4-column halves of one 8-column block: each
        // loads four tokens of the block as 16-byte rows (lane l tokens 0..3, lane l + 32
        // tokens 4..7) and a swap of the upper and lower 32 lanes leaves each with its
        // 4 columns of all 8 tokens
        const int tg = (w >> 1) * 8 + (lane & 7), cg = (w & 1) * 8 + 2 * ((lane >> 3) & 3) + (lane >> 5);
        const char *xbb = reinterpret_cast<const char *>(xb);
        u32x2 xv[8];
        const int c8 = (cg & ~1) * 4, tsel = 4 * (lane >> 5);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                xbb + (uint32_t)((min(tg * 8 + tsel + r, nvalid - 1) * (int)xstride + c8) * 2));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(v[e], v[2 + e], false, false);
                xv[r][e] = sw[0];
                xv[4 + r][e] = sw[1];
            }
        }
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dh + tg * 8);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dh + tg * 8 + 4);
        const int tq = tid & (Q - 1);
        const float gt = Gh[tq], ge = Gh[tq | 31];
        auto commit0 = stage_state(0);
        load_slice(0);
        const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        // positions of this block's tokens: 8 tokens at offset 0 or 8 of a 16-group
        // -> two runs of 4 positions, 8 apart
        const int pos0 = (tg >> 1) * 16 + ((tg & 1) ? 4 : 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 lo, hi;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t a0 = xv[2 * k][j >> 1], a1 = xv[2 * k + 1][j >> 1];
                lo[k] = pack_bf16(((j & 1) ? bf_hi(a0) : bf_lo(a0)) * d[2 * k],
                                  ((j & 1) ? bf_hi(a1) : bf_lo(a1)) * d[2 * k + 1]);
                const uint32_t b0 = xv[4 + 2 * k][j >> 1], b1 = xv[5 + 2 * k][j >> 1];
                hi[k] = pack_bf16(((j & 1) ? bf_hi(b0) : bf_lo(b0)) * d[4 + 2 * k],
                                  ((j & 1) ? bf_hi(b1) : bf_lo(b1)) * d[5 + 2 * k]);
            }
            bf16 *row = Xd + (cg * 4 + j) * XP + pos0;
            *reinterpret_cast<u32x2 *>(row) = lo;
            *reinterpret_cast<u32x2 *>(row + 8) = hi;
        }
        if (tid < Q) {
            Gs[tid] = gt;
            We[tid] = fast_exp2(ge - gt);
        }
        commit0();
        for (int nb = SPART; nb < N; nb += SPART) stage_state(nb)();
    }

    f32x16 cb[NI];
#pragma unroll
    for (int J = 0; J < NI; ++J) cb[J] = zero_acc();
    f32x16 ya[2] = {zero_acc(), zero_acc()};
    const bf16 *sfrow = Sf + (lane & 31) * SFP + kq;

    // ---------------- phase 1: C B^T tiles and S_eff C^T over N slices ----------------
    for (int n0 = 0; n0 < N; n0 += NS) {
        __syncthreads();   // previous slice consumed; first time: Xd, Gs, We, Sf written
#pragma unroll
        for (int r = 0; r < BPC; ++r) {
            const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
            *reinterpret_cast<bf16x8 *>(&Bs[t * BP + oct * 8]) = bq[r];
        }
        bf16x8 cf[NS / 16];
#pragma unroll
        for (int ks = 0; ks < NS / 16; ++ks) cf[ks] = cn[ks];
        // next slice (the last iteration re-requests the last slice; never used)
        load_slice(min(n0 + NS, N - NS));
        __syncthreads();

#pragma unroll
        for (int J = 0; J < NI; ++J) {
            if (J <= I) {
                const bf16 *brow = Bs + (J * 32 + (lane & 31)) * BP + kq;
#pragma unroll
                for (int ks = 0; ks < NS / 16; ++ks)
                    mma(cb[J], *reinterpret_cast<const bf16x8 *>(brow + ks * 16), cf[ks]);
            }
        }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const bf16 *srow = sfrow + pp * 32 * SFP + n0;
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks)
                mma(ya[pp], *reinterpret_cast<const bf16x8 *>(srow + ks * 16), cf[ks]);
        }
    }

    // ---------------- phase 2: Y^T = exp2(G_i) Y^T + M (dt x) ----------------
    const float gi = Gs[i_loc];
    const float si = fast_exp2(gi);
#pragma unroll
    for (int v = 0; v < 16; ++v) { ya[0][v] *= si; ya[1][v] *= si; }
    const int offX = (lane & 31) * XP + 8 * (lane >> 5);
#pragma unroll
    for (int J = 0; J < NI; ++J) {
        if (J > I) continue;
        const int jrow = J * 32 + 4 * (lane >> 5);   // + 8q + r for element 4q + r
        bf16x8 m[2];
        if (J < I) {
            const float ci = fast_exp2(gi - Gs[J * 32 + 31]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 we = *reinterpret_cast<const f32x4 *>(&We[jrow + 8 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) m[q >> 1][4 * (q & 1) + r] = (bf16)(cb[J][4 * q + r] * we[r] * ci);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 gj = *reinterpret_cast<const f32x4 *>(&Gs[jrow + 8 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float val = cb[J][4 * q + r] * fast_exp2(gi - gj[r]);
                    m[q >> 1][4 * (q & 1) + r] = (bf16)((i_loc >= jrow + 8 * q + r) ? val : 0.0f);
                }
            }
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const bf16 *xt = Xd + offX + J * 32 + 16 * sub;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) mma(ya[pp], ld16(xt + pp * 32 * XP), m[sub]);
        }
    }

    // ---------------- y = Y + D x ----------------
    // Lanes l and l + 32 hold the same token (so both or neither pass the row check);
    // the swap of their halves gives each lane 8 whole columns to store as 16 bytes
    if (iv) {
        const float Dh = D[h];
        const int yo = i_loc * (int)xstride;
        bf16 *yb = y + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            u32x2 w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = pp * 32 + 8 * q + 4 * (lane >> 5);
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xb + yo + p);
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = (bf16)(ya[pp][4 * q + r] + Dh * (float)xv[r]);
                w[q] = __builtin_bit_cast(u32x2, o);
            }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(w[2 * pr][d], w[2 * pr + 1][d], false, false);
                    o[d] = sw[0];
                    o[2 + d] = sw[1];
                }
                const int p = pp * 32 + 16 * pr + 8 * (lane >> 5);
                *reinterpret_cast<u32x4 *>(yb + yo + p) = o;
            }
        }
    }
}

// ===========================================================================
// Chunk output, head-blocked.  C B^T depends only on the chunk and the group,
// so a workgroup takes one (chunk, batch, group) and a block of HB heads of that
// group.  It computes the causal C B^T tiles once (fp32 MFMA accumulation),
// rounds them to bf16 into LDS, keeps the wave's C rows in registers, and then
// runs the per-head work head after head:
//   * Y^T = S_eff C^T (inter-chunk term, S_eff = S + beta_c H_g when grouped);
//   * Y^T = exp2(G_i) Y^T + sum_{j <= i} M'[j, i] x_j with the decay matrix
//     M'[j, i] = CB[j, i] exp2(G_i - G_j) dt_j, selected on i >= j; the raw x
//     tile is the MFMA operand and dt_j rides in M' (a per-token table off the
//     diagonal, one extra product on it);
//   * y = Y + D x, the raw x read back from the same LDS tile.
// The next head's x, dt and decays are loaded a whole head ahead and its
// chunk-start state right after the S C^T products.
//
// Waves own 32-token row tiles I(w), SIMD-balanced as in the single-head
// kernel; the output is built transposed, Y^T [64 p x 32 tokens].
// SPL = 2 (N = 512, where one wave cannot hold its C rows for every column in
// registers): two waves share each row tile, on the same SIMD.  Wave half hf
// holds C for columns [hf N/2, (hf+1) N/2), computes C B^T and S_eff C^T over
// those columns and the decay tiles J with J % 2 == hf; the halves then swap
// their partial Y^T through LDS, half hf finishing the 32 p rows pp = hf.  The decay
// matrix tiles J < I use the exact factorization exp2(G_i - G_e) exp2(G_e - G_j),
// e the last token of tile J (both factors <= 1).
// Rounding: C B^T is rounded to bf16 once after its fp32 accumulation and the
// decay matrix again as the MFMA operand; H_g arrives in bf16.
// Chunks are full (a ragged last chunk is left to the single-head kernel).
// ===========================================================================
template <int Q, int NN, bool CORR, int SPL>
__global__ __launch_bounds__(2 * Q * SPL) void chunk_out_hb_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const float *__restrict__ G2, const float *__restrict__ dtT, const bf16 *__restrict__ S,
    const float *__restrict__ D, bf16 *__restrict__ y, const bf16 *__restrict__ Hb,
    const float *__restrict__ beta, int L, int H, int G, int nc, int Lp, int K, int ng, int HB,
    int nc_full, int xcd)
{
    constexpr int P = 64, NI = Q / 32, NW = Q / 32, NTHR = 2 * Q * SPL, NS = 64;
    constexpr int NSL = (NN + NS - 1) / NS;     // B slices
    constexpr int NSW = NN < NS ? NN : NS;      // slice width
    constexpr int NIT = NSL / SPL;              // slice steps (SPL slices staged per step)
    constexpr int NF = NN / 16 / SPL;           // C fragments per lane (its column half)
    constexpr int XP = Q + 8, SFP = NN + 8;
    constexpr int SPT = P * (NN / 8) / NTHR;    // 16-byte S pieces per thread
    // the next head's S (and H_g) pieces are requested before the decay products when
    // they take at most 32 registers per thread, else after them
    constexpr bool EARLY_S = SPL == 1 && SPT * (CORR ? 2 : 1) <= 8;
    static_assert(SPT >= 1 && NN % 16 == 0 && NSL % SPL == 0 && NSW == 64, "staging cover");
    static_assert(SPL == 1 || SPL == 2, "one or two column halves");
    constexpr int NTILE = NI * (NI + 1) / 2;    // causal tiles
    constexpr int CB_EL = NTILE * 32 * 32;      // bf16 C B^T tiles
    constexpr int XC_EL = SPL == 2 ? NW * 2 * 1024 * 2 : 0;   // fp32 partial-Y swap area
    constexpr int U_EL = CB_EL + XC_EL;
    static_assert(SPL == 1 || 4 * CB_EL <= 2 * P * SFP, "partial C B^T fits the S area");
    // raw x^T [p][position] (token order permuted within 16-token groups: the
    // middle two 4-token blocks swapped, so the accumulator token order of a lane
    // becomes 8 consecutive positions); Un holds the bf16 C B^T tiles: tile (I, J) at
    // (I(I+1)/2 + J) * 1024 elements, lane l's elements 0..7 at 8 l and 8..15 at
    // 512 + 8 l, followed (SPL = 2) by the partial-Y swap area.  During the C B^T
    // products Un, Sf and Xd hold the B slices instead.
    __shared__ __attribute__((aligned(16))) bf16 Xd[P * XP];
    __shared__ __attribute__((aligned(16))) bf16 Un[U_EL];
    __shared__ __attribute__((aligned(16))) bf16 Sf[P * SFP];
    __shared__ __attribute__((aligned(16))) float Gs[Q];
    __shared__ __attribute__((aligned(16))) float Wd[Q];   // exp2(G_e - G_j) dt_j
    __shared__ __attribute__((aligned(16))) float Dt[Q];   // dt_j

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar tile loops
    const int hf = SPL == 1 ? 0 : w / NW;      // column half
    const int wi = SPL == 1 ? w : w % NW;      // wave within the half
    const int I = (wi < NW / 2) ? wi : NW - 1 - (wi - NW / 2);

    // workgroup -> (chunk, (batch, group, head block)); with `xcd` (nc_full a
    // multiple of 8) XCD x gets the contiguous chunk range [x nc/8, (x+1) nc/8)
    const int HPG = H / G, nhb = HPG / HB;
    const int minors = gridDim.x / nc_full;
    int c, minor;
    if (xcd) {
        const int xx = blockIdx.x & 7, slot = blockIdx.x >> 3;
        c = xx * (nc_full / 8) + slot / minors;
        minor = slot % minors;
    } else {
        c = blockIdx.x / minors;
        minor = blockIdx.x % minors;
    }
    const int bg = minor / nhb, hblk = minor % nhb;
    const int b = bg / G, g = bg % G;
    const int h_first = g * HPG + hblk * HB;
    const int t0 = c * Q;
    const int N = NN;
    const int64_t xstride = (int64_t)H * P, cstride = (int64_t)G * N;
    const char *Bb = reinterpret_cast<const char *>(Bm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N);
    const char *Cb = reinterpret_cast<const char *>(Cm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N);
    const int kq = 8 * (lane >> 5);
    const int i_loc = I * 32 + (lane & 31);
    const int brow = (int)cstride * 2;
    bf16 *cbl = Un + (I * (I + 1) / 2) * 1024 + 8 * lane;   // this wave's C B^T tiles

    // ================= C B^T, once per workgroup =================
    bf16x8 cfa[NF];                // this wave's C rows, all N: fragment f = columns 16 f ..
    {
        const int crow_off = i_loc * brow + kq * 2 + hf * NF * 32;
#pragma unroll
        for (int f = 0; f < NF; ++f)
            cfa[f] = *reinterpret_cast<const bf16x8 *>(Cb + (uint32_t)(crow_off + f * 32));
        // Every B slice [Q tokens][64 columns] goes to LDS by 16-byte global-to-LDS loads
        // before the first product: the slices fill Un, then Sf, then Xd (both free until
        // the first head is staged), unpadded, with 16-byte unit u of row r stored at unit
        // u ^ ((r >> 1) & 7), so that the 16 rows of a quarter-wave operand read fall in
        // 16 different bank groups.  One load instruction covers 8 rows (1 KB).
        constexpr int SL_EL = Q * NSW;
        constexpr int IN_UN = U_EL / SL_EL, IN_SF = P * SFP / SL_EL, IN_XD = P * XP / SL_EL;
        static_assert(IN_UN + IN_SF + IN_XD >= NSL, "every B slice fits the LDS free before the heads");
        constexpr int IPS = Q / 8, NWV = NTHR / 64;
        static_assert((NSL * IPS) % NWV == 0, "B load cover");
        auto slice_base = [&](int sl) -> bf16 * {
            return sl < IN_UN ? Un + sl * SL_EL
                              : (sl < IN_UN + IN_SF ? Sf + (sl - IN_UN) * SL_EL
                                                    : Xd + (sl - IN_UN - IN_SF) * SL_EL);
        };
        {
            const rsrc_t br = make_rsrc(Bb, Q * brow);
            const int rl = lane >> 3, ul = lane & 7;
#pragma unroll
            for (int kk = 0; kk < NSL * IPS / NWV; ++kk) {
                const int k = kk * NWV + w, sl = k / IPS, ki = k % IPS;
                const int row = ki * 8 + rl;
                const int u = ul ^ ((row >> 1) & 7);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    br, (lds_void *)(slice_base(sl) + ki * 8 * NSW), 16,
                    row * brow + (sl * NSW + 8 * u) * 2, 0, 0, 0);
            }
        }
        f32x16 cb[NI];
#pragma unroll
        for (int J = 0; J < NI; ++J) cb[J] = zero_acc();
        __syncthreads();   // every slice has landed (the barrier waits for this wave's loads)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const bf16 *sb = slice_base(hf * NIT + it);
#pragma unroll
            for (int J = 0; J < NI; ++J) {
                if (J <= I) {
                    const int row = J * 32 + (lane & 31);
                    const bf16 *rp = sb + row * NSW;
#pragma unroll
                    for (int ks = 0; ks < NSW / 16; ++ks) {
                        const int u = ((lane >> 5) + 2 * ks) ^ ((row >> 1) & 7);
                        mma(cb[J], *reinterpret_cast<const bf16x8 *>(rp + 8 * u), cfa[it * (NSW / 16) + ks]);
                    }
                }
            }
        }
        __syncthreads();   // slices consumed: Un becomes the C B^T store, Sf and Xd free
        if constexpr (SPL == 2) {
            // half 1 hands its partial C B^T (fp32) to half 0 through the S area
            float *pcb = reinterpret_cast<float *>(Sf) + (I * (I + 1) / 2) * 1024 + 4 * lane;
            if (hf == 1) {
#pragma unroll
                for (int J = 0; J < NI; ++J)
                    if (J <= I)
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            f32x4 v;
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = cb[J][4 * k + e];
                            *reinterpret_cast<f32x4 *>(pcb + J * 1024 + k * 256) = v;
                        }
            }
            __syncthreads();
            if (hf == 0) {
#pragma unroll
                for (int J = 0; J < NI; ++J)
                    if (J <= I)
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const f32x4 v = *reinterpret_cast<const f32x4 *>(pcb + J * 1024 + k * 256);
#pragma unroll
                            for (int e = 0; e < 4; ++e) cb[J][4 * k + e] += v[e];
                        }
            }
        }
        if (hf == 0) {
#pragma unroll
        for (int J = 0; J < NI; ++J) {
            if (J <= I) {
                u32x4 lo, hi;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    lo[k2] = pack_bf16(cb[J][2 * k2], cb[J][2 * k2 + 1]);
                    hi[k2] = pack_bf16(cb[J][8 + 2 * k2], cb[J][9 + 2 * k2]);
                }
                *reinterpret_cast<u32x4 *>(cbl + J * 1024) = lo;
                *reinterpret_cast<u32x4 *>(cbl + J * 1024 + 512) = hi;
            }
        }
        }
    }

    // ================= per-head work =================
    // thread = 8 tokens (group tg) x 4 columns (group cg); lanes l and l + 32 take the
    // two 4-column halves of one 8-column block
    const int tg = (wi >> 1) * 8 + (lane & 7), cg = (wi & 1) * 8 + 2 * ((lane >> 3) & 3) + (lane >> 5);
    struct XRegs {
        u32x4 raw[4];   // the four 16-byte x loads as they arrive (lanes swapped at staging)
        float gt, ge, dt;
    };
    struct SRegs {
        bf16x8 sq[SPT];
        bf16x8 hq[CORR ? SPT : 1];
        float bc;
    };
    const int tq = tid & (Q - 1);
    auto load_x = [&](XRegs &R, int hl) {
        hl = min(hl, HB - 1);
        const int h = h_first + hl, bh = b * H + h;
        const char *xbb = reinterpret_cast<const char *>(x + ((int64_t)b * L + t0) * xstride + (int64_t)h * P);
        // 16-byte loads: lane l reads tokens 0..3 of the group, lane l + 32 tokens 4..7, both
        // the whole 8-column block (rearranged by stage_head, so that nothing here waits
        // for them)
        const int c8 = (cg & ~1) * 4, tsel = 4 * (lane >> 5);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            R.raw[r] = *reinterpret_cast<const u32x4 *>(
                xbb + (uint32_t)(((tg * 8 + tsel + r) * (int)xstride + c8) * 2));
        const float *Gh = G2 + (int64_t)bh * Lp + t0;
        R.gt = Gh[tq];
        R.ge = Gh[tq | 31];
        R.dt = dtT[(int64_t)bh * Lp + t0 + tq];
    };
    // the first chunk of a group after the first starts from zero (the state pass stores
    // nothing for it): its S loads read an empty range, which returns zeros
    const bool s_zero = CORR && c >= K && c % K == 0;
    auto load_s = [&](SRegs &R, int hl) {
        hl = min(hl, HB - 1);
        const int h = h_first + hl, bh = b * H + h;
        const rsrc_t sr = make_rsrc(S + ((int64_t)bh * nc + c) * P * N, s_zero ? 0 : P * N * 2);
#pragma unroll
        for (int r = 0; r < SPT; ++r) {
            const int id = tid + NTHR * r, pp = id / (NN / 8), oc = id % (NN / 8);
            R.sq[r] = __builtin_bit_cast(bf16x8, buf_load_b128(sr, (uint32_t)((pp * N + oc * 8) * 2)));
        }
        if constexpr (CORR) {
            const int cgrp = c / K;
            const char *Hc = reinterpret_cast<const char *>(Hb + ((int64_t)bh * ng + cgrp) * P * N);
#pragma unroll
            for (int r = 0; r < SPT; ++r) {
                const int id = tid + NTHR * r, pp = id / (NN / 8), oc = id % (NN / 8);
                R.hq[r] = *reinterpret_cast<const bf16x8 *>(Hc + (uint32_t)((pp * N + oc * 8) * 2));
            }
            int bi = bh * nc + c;
            asm volatile("" : "+v"(bi));   // per-lane load: keeps it off the scalar path
            R.bc = beta[bi] * (cgrp > 0 ? 1.0f : 0.0f);
        } else {
            R.bc = 0.0f;
        }
    };
    // head registers -> LDS: raw x^T (permuted positions), decay tables, S_eff
    auto stage_head = [&](const XRegs &R, const SRegs &T) {
        // swapping the upper and lower 32 lanes leaves lane l with columns 0..3 and lane
        // l + 32 with columns 4..7 of all 8 tokens
        u32x2 xv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto sw = __builtin_amdgcn_permlane32_swap(R.raw[r][d], R.raw[r][2 + d], false, false);
                xv[r][d] = sw[0];
                xv[4 + r][d] = sw[1];
            }
        const int pos0 = (tg >> 1) * 16 + ((tg & 1) ? 4 : 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (hf != 0) break;   // half 1 holds a copy of the same x pieces
            u32x2 lo, hi;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                lo[k] = pack_halves(xv[2 * k][j >> 1], xv[2 * k + 1][j >> 1], j & 1);
                hi[k] = pack_halves(xv[4 + 2 * k][j >> 1], xv[5 + 2 * k][j >> 1], j & 1);
            }
            bf16 *row = Xd + (cg * 4 + j) * XP + pos0;
            *reinterpret_cast<u32x2 *>(row) = lo;
            *reinterpret_cast<u32x2 *>(row + 8) = hi;
        }
        if (tid < Q) {
            Gs[tid] = R.gt;
            Wd[tid] = fast_exp2(R.ge - R.gt) * R.dt;
            Dt[tid] = R.dt;
        }
#pragma unroll
        for (int r = 0; r < SPT; ++r) {
            const int id = tid + NTHR * r, pp = id / (NN / 8), oc = id % (NN / 8);
            bf16x8 sv = T.sq[r];
            if constexpr (CORR) {
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) sv[e2] = (bf16)((float)sv[e2] + T.bc * (float)T.hq[r][e2]);
            }
            *reinterpret_cast<bf16x8 *>(&Sf[pp * SFP + oc * 8]) = sv;
        }
    };

    const int offX = (lane & 31) * XP + 8 * (lane >> 5);
    const bf16 *sfrow = Sf + (lane & 31) * SFP + kq;
    // skip-term transpose reads: the addressing lane 4e + k of a 16-lane group
    // points at row p0 + e and the 4-token block of tokens 4k .. 4k+3 of this
    // group's 16 tokens, so lane i receives x at its own token for rows p0 .. p0+3
    const int m16 = lane & 15;
    const int tok16 = I * 32 + 16 * ((lane >> 4) & 1);           // first token of the group
    const int blk = m16 & 3;                                       // 4-token block k
    const int blkpos = (blk == 1) ? 2 : (blk == 2) ? 1 : blk;      // its position block
    const int skip_off = (m16 >> 2) * XP + tok16 + 4 * blkpos + 4 * (lane >> 5) * XP;
    XRegs RX;
    SRegs RS;
    load_x(RX, 0);
    load_s(RS, 0);
    for (int hl = 0; hl < HB; ++hl) {
        const int h = h_first + hl;
        __syncthreads();   // the previous head's tiles are consumed (first time: C B^T stored)
        stage_head(RX, RS);
        load_x(RX, hl + 1);   // next head (the last one re-requests itself; never used)
        __syncthreads();

        // inter-chunk term: Y^T = S_eff C^T
        f32x16 ya[2] = {zero_acc(), zero_acc()};
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                mma(ya[pp], *reinterpret_cast<const bf16x8 *>(sfrow + pp * 32 * SFP + (hf * NF + f) * 16), cfa[f]);

        // next head's chunk-start state: when its pieces fit in 32 registers per
        // thread its latency hides behind the decay-matrix products; otherwise (two
        // column halves, or a 256-column state over 256 threads) it is issued after
        // them, which keeps the kernel within 256 registers (two waves per SIMD)
        if constexpr (EARLY_S) load_s(RS, hl + 1);
        // Y^T = exp2(G_i) Y^T + M' x
        const float gi = Gs[i_loc];
        const float si = fast_exp2(gi);
#pragma unroll
        for (int v = 0; v < 16; ++v) { ya[0][v] *= si; ya[1][v] *= si; }
        auto mfma_tile = [&](int J, const bf16x8 (&m)[2]) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const bf16 *xt = Xd + offX + J * 32 + 16 * sub;
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) mma(ya[pp], ld16(xt + pp * 32 * XP), m[sub]);
            }
        };
        for (int J = hf; J < I; J += SPL) {   // off the diagonal (this half's tiles)
            const int jrow = J * 32 + 4 * (lane >> 5);   // + 8q + r for element 4q + r
            const float ci = fast_exp2(gi - Gs[J * 32 + 31]);
            const u32x4 c0 = *reinterpret_cast<const u32x4 *>(cbl + J * 1024);
            const u32x4 c1 = *reinterpret_cast<const u32x4 *>(cbl + J * 1024 + 512);
            bf16x8 m[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 wd = *reinterpret_cast<const f32x4 *>(&Wd[jrow + 8 * q]);
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const int v = 4 * q + r;
                    const uint32_t pr = (v < 8) ? c0[v >> 1] : c1[(v - 8) >> 1];
                    m[q >> 1][4 * (q & 1) + r] = (bf16)(bf_lo(pr) * wd[r] * ci);
                    m[q >> 1][4 * (q & 1) + r + 1] = (bf16)(bf_hi(pr) * wd[r + 1] * ci);
                }
            }
            mfma_tile(J, m);
        }
        if (SPL == 1 || (I & 1) == hf) {   // the diagonal tile, selected on i >= j
            const int jrow = I * 32 + 4 * (lane >> 5);
            const u32x4 c0 = *reinterpret_cast<const u32x4 *>(cbl + I * 1024);
            const u32x4 c1 = *reinterpret_cast<const u32x4 *>(cbl + I * 1024 + 512);
            bf16x8 m[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 gj = *reinterpret_cast<const f32x4 *>(&Gs[jrow + 8 * q]);
                const f32x4 dj = *reinterpret_cast<const f32x4 *>(&Dt[jrow + 8 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int v = 4 * q + r;
                    const uint32_t pr = (v < 8) ? c0[v >> 1] : c1[(v - 8) >> 1];
                    const float cbv = (r & 1) ? bf_hi(pr) : bf_lo(pr);
                    const float val = cbv * fast_exp2(gi - gj[r]) * dj[r];
                    m[q >> 1][4 * (q & 1) + r] = (bf16)((i_loc >= jrow + 8 * q + r) ? val : 0.0f);
                }
            }
            mfma_tile(I, m);
        }

        if constexpr (!EARLY_S) load_s(RS, hl + 1);
        if constexpr (SPL == 2) {
            // swap partial Y^T with the other half of the row tile: this wave keeps
            // rows pp = hf and sends rows 1 - hf
            float *xc = reinterpret_cast<float *>(Un + CB_EL) + I * 2048 + 4 * lane;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = hf ? ya[0][4 * k + e] : ya[1][4 * k + e];
                *reinterpret_cast<f32x4 *>(xc + (1 - hf) * 1024 + k * 256) = v;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) ya[0][e] = hf ? ya[1][e] : ya[0][e];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(xc + hf * 1024 + k * 256);
#pragma unroll
                for (int e = 0; e < 4; ++e) ya[0][4 * k + e] += v[e];
            }
        }

        // y = Y + D x.  Lanes l and l + 32 hold the same token; lane l has columns
        // 8q .. 8q+3 of each 32-column half and lane l + 32 columns 8q+4 .. 8q+7.  One
        // swap of the upper and lower 32 lanes per pair (q, q+1) gives lane l the 8
        // columns of q and lane l + 32 those of q+1, so each store writes 16 bytes per lane
        // and 32 contiguous bytes per token row (half as many store instructions)
        const float Dh = D[h];
        bf16 *yb = y + ((int64_t)b * L + t0 + i_loc) * xstride + (int64_t)h * P;
#pragma unroll
        for (int pq = 0; pq < 2 / SPL; ++pq) {
            const int pp = SPL == 1 ? pq : hf;
            u32x2 w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x4 xv = tr_read4(Xd + skip_off + (pp * 32 + 8 * q) * XP);
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = (bf16)(ya[pq][4 * q + r] + Dh * (float)xv[r]);
                w[q] = __builtin_bit_cast(u32x2, o);
            }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(w[2 * pr][d], w[2 * pr + 1][d], false, false);
                    o[d] = sw[0];
                    o[2 + d] = sw[1];
                }
                const int p = pp * 32 + 16 * pr + 8 * (lane >> 5);
                *reinterpret_cast<u32x4 *>(yb + p) = o;
            }
        }
    }
}

// ===========================================================================
// Launchers
// ===========================================================================
// Head-blocked kernel: chunks of 128 or 256 tokens with N of 64, 128 or 256, and
// 128-token chunks with N = 512 (column halves split over wave pairs); the
// single-head kernel covers the rest.
static bool head_blocked(const Shape &s)
{
    return ((s.Q == 128 || s.Q == 256) && (s.N == 64 || s.N == 128 || s.N == 256)) ||
           (s.Q == 128 && s.N == 512);
}

// register ring depth of the register-transposed state pass (sub-steps in flight)
constexpr int kSpRtDepth = 2;

// Which state pass runs: the register-transposed kernel for N a multiple of 256 from
// 512 up (256-column workgroups of 4 waves, two per CU), the LDS-transposed kernel
// with DMA staging otherwise.  Measured on MI355X (bf16, one box, µs per state pass): b1 L65536 H32 N512
// Q128 486 -> 433; at N = 256 (b1 L16384 H32 Q256) 38.7 -> 37.5 with one workgroup per
// CU and 35.0 with two (then 16 groups, whose scan costs 4 µs more); at N = 128
// 28.8 -> 30.3-38.0 (b4 L16384 H8 Q128) and 9.9 -> 10.3-11.5 (b2 L2048 H24 Q256).
// Its 4-byte loads (two columns per lane for the in-register transpose) take four
// times the address-unit issue of 16-byte loads per byte.
static bool sp_register_transposed(const Shape &s) { return s.N >= 512 && s.N % 256 == 0; }

// wt: the stage-1 weights wT when wpre, else dtT (the kernel forms the weights)
template <int Q, int NR, bool WPRE>
static hipError_t sp_launch_w(const Shape &s, bool rt, const void *x, const void *B, const float *G2,
                              const float *wt, const float *h0, void *S, float *hT, float *Ug,
                              float *gam, float *beta, int K, int ng, hipStream_t st)
{
    const int units = (int)(s.b * s.H * (s.N / NR));
    const int xcd = (ng % 8 == 0) ? 1 : 0;
    if constexpr (NR == 256) {
        if (rt) {
            hipLaunchKernelGGL((state_pass_rt_kernel<Q, 256, kSpRtDepth, WPRE>), dim3((unsigned)(units * ng)),
                               dim3(256), 0, st, (const bf16 *)x, (const bf16 *)B, G2, wt, h0,
                               (bf16 *)S, hT, Ug, gam, beta, (int)s.L, (int)s.H, (int)s.G, (int)s.N,
                               (int)s.nc, (int)s.Lp, K, ng, xcd);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((state_pass_dma_kernel<Q, NR, WPRE>), dim3((unsigned)(units * ng)),
                       dim3(SpCfg<Q, NR>::NTHR), 0, st, (const bf16 *)x, (const bf16 *)B, G2, wt,
                       h0, (bf16 *)S, hT, Ug, gam, beta, (int)s.L, (int)s.H, (int)s.G, (int)s.N,
                       (int)s.nc, (int)s.Lp, K, ng, xcd);
    return hipGetLastError();
}

template <int Q, int NR>
static hipError_t sp_launch(const Shape &s, bool rt, bool wpre, const void *x, const void *B,
                            const float *G2, const float *wt, const float *h0, void *S, float *hT,
                            float *Ug, float *gam, float *beta, int K, int ng, hipStream_t st)
{
    return wpre ? sp_launch_w<Q, NR, true>(s, rt, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st)
                : sp_launch_w<Q, NR, false>(s, rt, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
}

// columns per state-pass workgroup: the largest of 256, 128, 64 dividing N
static int sp_cols(const Shape &s) { return (s.N % 256 == 0) ? 256 : (s.N % 128 == 0) ? 128 : 64; }

template <int Q>
static hipError_t sp_dispatch_q(const Shape &s, int cols, bool rt, bool wpre, const void *x,
                                const void *B, const float *G2, const float *wt, const float *h0,
                                void *S, float *hT, float *Ug, float *gam, float *beta, int K,
                                int ng, hipStream_t st)
{
    switch (cols) {
    case 256: return sp_launch<Q, 256>(s, rt, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    case 128: return sp_launch<Q, 128>(s, rt, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    default: return sp_launch<Q, 64>(s, rt, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    }
}

// bf16 state pass with `cols` state columns per workgroup (B transposed in registers
// when rt, cols = 256) over ng groups of K chunks per chain; wt is the stage-1 weights
// wT when wpre, else dtT
static hipError_t sp_dispatch(const Shape &s, int cols, bool rt, bool wpre, const void *x,
                              const void *B, const float *G2, const float *wt, const float *h0,
                              void *S, float *hT, float *Ug, float *gam, float *beta, int K,
                              int ng, hipStream_t st)
{
    switch (s.Q) {
    case 64: return sp_dispatch_q<64>(s, cols, rt, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    case 128: return sp_dispatch_q<128>(s, cols, rt, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    default: return sp_dispatch_q<256>(s, cols, rt, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    }
}

hipError_t launch_state_pass_bf16(const Shape &s, const void *x, const void *B, const float *G2,
                                  const float *dtT, const float *h0, void *S, float *hT,
                                  hipStream_t st)
{
    return sp_dispatch(s, sp_cols(s), sp_register_transposed(s), false, x, B, G2, dtT, h0, S, hT,
                       nullptr, nullptr, nullptr, (int)s.nc, 1, st);
}

// Chunks per group and groups per chain for the state pass with `cols` columns per
// workgroup (B transposed in registers when rt): the cost model of the default plan.
struct Grouping {
    int K, ng;
};
static Grouping state_pass_groups(const Shape &s, int cols, bool rt)
{
    Grouping gp;
    const int64_t units = s.b * s.H * (s.N / cols);
    if (!s.bf16) {
        // fp32 (64 columns per workgroup): as many workgroups as the LDS of its Q
        // lets the CUs hold at once
        const int64_t target = 256 * (s.Q == 64 ? 4 : s.Q == 128 ? 2 : 1);
        int64_t ng = (target + units - 1) / units;
        ng = std::max<int64_t>(1, std::min<int64_t>(ng, s.nc));
        const int64_t K = (s.nc + ng - 1) / ng;
        gp.K = (int)K;
        gp.ng = (int)((s.nc + K - 1) / K);
        return gp;
    }
    // bf16: an LDS-transposed workgroup takes most of a CU's LDS (two fit at 64 columns, but
    // they share the CU's issue: measured, two 64-column workgroups per CU take about as long
    // per chunk as one of twice the chains), a register-transposed one half of a CU's
    // registers, so `slots` run at once and units * ng workgroups take
    // ceil(units * ng / slots) rounds of K chunks each.  The count minimises that makespan plus a fixed cost per
    // workgroup (~0.6 chunk: prologue, last state store) and the group scan, in
    // units of one chunk's time (~1.2 us per 64 tokens); ties keep fewer groups.
    // The scan reads and writes every group's state (~6 bytes per element at
    // ~5 TB/s) and walks the groups in order, eight loads in flight (~1.5 us per
    // eight groups): whichever is longer.
    const int64_t slots = rt ? 512 : 256;
    const double tchunk = (double)s.Q / 64 * 1.2e-6;
    const int64_t ng_max = std::min<int64_t>(s.nc, 8 * slots / units + 1);
    double best = 1e300;
    int64_t best_ng = 1, best_K = s.nc;
    for (int64_t ng = 1; ng <= ng_max; ++ng) {
        const int64_t K = (s.nc + ng - 1) / ng, g = (s.nc + K - 1) / K;
        if (g != ng) continue;   // same K as a smaller count
        const double rounds = (double)((units * g + slots - 1) / slots);
        const double scan_bw = (double)(s.b * s.H) * g * s.P * s.N * 6.0 / 5e12;
        const double scan_serial = (double)((g + 7) / 8) * 1.5e-6;
        const double scan = g > 1 ? std::max(scan_bw, scan_serial) / tchunk : 0.0;
        const double cost = rounds * (K + 0.6) + scan;
        if (cost < best - 1e-9) {
            best = cost;
            best_ng = g;
            best_K = K;
        }
    }
    gp.K = (int)best_K;
    gp.ng = (int)best_ng;
    return gp;
}

hipError_t launch_state_pass_grouped(const Shape &s, const LaunchPlan &lp, const void *x,
                                     const void *B, const float *G2, const float *wT,
                                     const float *h0, void *S, float *hT, float *Ug, float *gam,
                                     float *beta, hipStream_t st)
{
    const int K = lp.sp_group_chunks, ng = lp.sp_groups;
    if (!s.bf16)
        return launch_state_pass_f32_grouped(s, x, B, G2, wT, h0, S, ng <= 1 ? hT : nullptr,
                                             ng <= 1 ? nullptr : Ug, gam, beta, K, ng, st);
    const bool rt = lp.sp_register_transposed != 0;
    if (ng <= 1)
        return sp_dispatch(s, lp.sp_columns, rt, true, x, B, G2, wT, h0, S, hT, nullptr, nullptr,
                           nullptr, (int)s.nc, 1, st);
    return sp_dispatch(s, lp.sp_columns, rt, true, x, B, G2, wT, h0, S, nullptr, Ug, gam, beta, K,
                       ng, st);
}

hipError_t launch_group_scan(const Shape &s, const LaunchPlan &lp, float *hT, float *Ug, void *Hb,
                             const float *gam, hipStream_t st)
{
    const int K = lp.sp_group_chunks, ng = lp.sp_groups;
    if (ng <= 1) return hipSuccess;   // one serial chain: the state pass wrote hT itself
    const int PN = (int)(s.P * s.N);
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)(s.b * s.H));
    // fp32 group-start states are read only by one-head chunk-output launches: with the
    // head-blocked kernel, only the ragged last chunk's group (none when L % Q == 0)
    int g_f32 = 1;
    if (s.bf16 && lp.co_head_blocked) g_f32 = (s.L % s.Q != 0) ? (int)((s.nc - 1) / K) : ng;
    hipLaunchKernelGGL(group_scan_kernel<8>, grid, dim3(256), 0, st, Ug, gam, hT,
                       s.bf16 ? (bf16 *)Hb : (bf16 *)nullptr, PN, ng, g_f32);
    return hipGetLastError();
}

template <int Q, int NMX>
static hipError_t co_launch_n(const Shape &s, const void *x, const void *B, const void *C,
                              const float *G2, const float *dtT, const void *S, const float *D,
                              void *y, const float *Hg, const float *beta, int K, int ng,
                              int c_first, int nc_grid, hipStream_t st)
{
    const int xcd = (nc_grid % 8 == 0) ? 1 : 0;
    const dim3 grid((unsigned)(nc_grid * s.b * s.H)), block(2 * Q);
    if (Hg != nullptr)
        hipLaunchKernelGGL((chunk_out_bf16_kernel<Q, true, NMX>), grid, block, 0, st,
                           (const bf16 *)x, (const bf16 *)B, (const bf16 *)C, G2, dtT,
                           (const bf16 *)S, D, (bf16 *)y, Hg, beta, (int)s.L, (int)s.H, (int)s.G,
                           (int)s.N, (int)s.nc, (int)s.Lp, K, ng, c_first, nc_grid, xcd);
    else
        hipLaunchKernelGGL((chunk_out_bf16_kernel<Q, false, NMX>), grid, block, 0, st,
                           (const bf16 *)x, (const bf16 *)B, (const bf16 *)C, G2, dtT,
                           (const bf16 *)S, D, (bf16 *)y, Hg, beta, (int)s.L, (int)s.H, (int)s.G,
                           (int)s.N, (int)s.nc, (int)s.Lp, K, ng, c_first, nc_grid, xcd);
    return hipGetLastError();
}

template <int Q>
static hipError_t co_launch(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, const float *Hg, const float *beta, int K, int ng,
                            int c_first, int nc_grid, hipStream_t st)
{
    if (s.N <= 128)
        return co_launch_n<Q, 128>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, c_first, nc_grid, st);
    if (s.N <= 256)
        return co_launch_n<Q, 256>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, c_first, nc_grid, st);
    return co_launch_n<Q, 512>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, c_first, nc_grid, st);
}

// heads per workgroup of the head-blocked chunk output: the divisor HB of the heads
// per group that minimises the makespan ceil(workgroups / slots) * (HB + c), c the
// per-workgroup cost in units of one head's work (the C B^T phase, ~0.9 N / 256,
// plus ~0.5 for the prologue and launch); ties keep fewer heads per workgroup.  slots:
// workgroups resident at once: two per CU for 128-token chunks with N up to 128 (47-55 KB
// of LDS, 4 waves of at most 208 registers; measured, the N = 256 instance gains nothing
// from a second workgroup), else one
static int heads_per_block(const Shape &s)
{
    const int hpg = (int)(s.H / s.G);
    const int64_t units = s.nc * s.b * s.G;
    const double c = 0.9 * (double)s.N / 256 + 0.5;
    const int64_t slots = (s.Q == 128 && s.N <= 128) ? 512 : 256;
    double best_cost = 1e300;
    int best = 1;
    for (int hb = 1; hb <= hpg; ++hb) {
        if (hpg % hb) continue;
        const double cost = (double)((units * (hpg / hb) + slots - 1) / slots) * (hb + c);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = hb;
        }
    }
    return best;
}

// The plan of the given choices with its derived fields; false when a workgroup count
// or a grid's work-item count (32 bits in the dispatch packet) does not fit.
static bool plan_from(const Shape &s, int K, int ng, int cols, int rt, int co_hb, int hb,
                      LaunchPlan &lp)
{
    const int64_t sp_wg = s.b * s.H * (s.N / cols) * ng;
    const int sp_threads = !s.bf16 ? 256 : rt ? 256 : (cols == 64 ? 256 : 512);
    int64_t co_wg, co_threads;
    int split = 1;
    if (co_hb) {
        const int64_t nc_full = s.L / s.Q;
        split = s.N > 256 ? 2 : 1;
        co_wg = nc_full * s.b * s.G * (s.H / s.G / hb) + (nc_full < s.nc ? s.b * s.H : 0);
        co_threads = 2 * s.Q * split;
    } else {
        hb = 1;
        co_wg = s.nc * s.b * s.H;
        co_threads = s.bf16 ? 2 * s.Q : chunk_out_f32_threads(s);
    }
    const int64_t lim = int64_t(1) << 32;
    if (sp_wg * sp_threads >= lim || co_wg * co_threads >= lim) return false;
    lp.sp_group_chunks = K;
    lp.sp_groups = ng;
    lp.sp_columns = cols;
    lp.sp_workgroups = (int)sp_wg;
    lp.scan = ng > 1 ? 1 : 0;
    lp.co_head_blocked = co_hb;
    lp.co_heads_per_block = hb;
    lp.co_column_split = split;
    lp.co_workgroups = (int)co_wg;
    lp.co_threads = (int)co_threads;
    lp.sp_register_transposed = rt;
    lp.sp_threads = sp_threads;
    lp.fused = 0;
    return true;
}

// The one-launch plan (forward_small): workgroups of 256 threads, two per (batch, head, chunk)
// and two more per (batch, head) for the final state
static LaunchPlan plan_fused(const Shape &s)
{
    LaunchPlan lp;
    lp.sp_group_chunks = (int)s.nc;
    lp.sp_groups = 1;
    lp.sp_columns = (int)s.N;
    lp.sp_workgroups = 0;
    lp.scan = 0;
    lp.co_head_blocked = 0;
    lp.co_heads_per_block = 1;
    lp.co_column_split = 1;
    lp.co_workgroups = (int)forward_small_workgroups(s);
    lp.co_threads = 256;
    lp.sp_register_transposed = 0;
    lp.sp_threads = 0;
    lp.fused = 1;
    return lp;
}

static bool plan_same(const LaunchPlan &a, const LaunchPlan &b)
{
    return a.sp_group_chunks == b.sp_group_chunks && a.sp_groups == b.sp_groups &&
           a.sp_columns == b.sp_columns && a.sp_workgroups == b.sp_workgroups &&
           a.scan == b.scan && a.co_head_blocked == b.co_head_blocked &&
           a.co_heads_per_block == b.co_heads_per_block &&
           a.co_column_split == b.co_column_split && a.co_workgroups == b.co_workgroups &&
           a.co_threads == b.co_threads && a.sp_register_transposed == b.sp_register_transposed &&
           a.sp_threads == b.sp_threads && a.fused == b.fused;
}

LaunchPlan plan_one_chain(const Shape &s)
{
    const int cols = s.bf16 ? sp_cols(s) : 64;
    const bool rt = s.bf16 && sp_register_transposed(s);
    const bool hbk = s.bf16 && head_blocked(s);
    LaunchPlan lp;
    plan_from(s, (int)s.nc, 1, cols, rt ? 1 : 0, hbk ? 1 : 0, hbk ? heads_per_block(s) : 1, lp);
    return lp;
}

LaunchPlan plan_of(const Shape &s)
{
    // a few chunks: the one-launch forward (its repeated state work is bounded by the chunk
    // count; the launches and round trips of the general path cost more)
    if (forward_small_eligible(s)) return plan_fused(s);
    const int cols = s.bf16 ? sp_cols(s) : 64;
    const bool rt = s.bf16 && sp_register_transposed(s);
    const Grouping gp = state_pass_groups(s, cols, rt);
    const bool hbk = s.bf16 && head_blocked(s);
    // fits for every shape the C ABI accepts: its checks bound the one-head output grid,
    // the largest of these launches, to 2^32 work-items
    LaunchPlan lp;
    plan_from(s, gp.K, gp.ng, cols, rt ? 1 : 0, hbk ? 1 : 0, hbk ? heads_per_block(s) : 1, lp);
    return lp;
}

bool plan_valid(const Shape &s, const LaunchPlan &lp)
{
    if (lp.fused != 0) return lp.fused == 1 && forward_small_eligible(s) && plan_same(lp, plan_fused(s));
    const int64_t K = lp.sp_group_chunks;
    if (K < 1 || K > s.nc || lp.sp_groups != (s.nc + K - 1) / K) return false;
    if (s.bf16) {
        if (lp.sp_columns != 64 && lp.sp_columns != 128 && lp.sp_columns != 256) return false;
        if (s.N % lp.sp_columns != 0) return false;
        if (lp.sp_register_transposed != 0 && (lp.sp_register_transposed != 1 || lp.sp_columns != 256))
            return false;
        if (lp.co_head_blocked != 0) {
            if (lp.co_head_blocked != 1 || !head_blocked(s)) return false;
            if (lp.co_heads_per_block < 1 || (s.H / s.G) % lp.co_heads_per_block != 0) return false;
        }
    } else if (lp.sp_columns != 64 || lp.sp_register_transposed != 0 || lp.co_head_blocked != 0) {
        return false;
    }
    LaunchPlan ref;
    return plan_from(s, (int)K, lp.sp_groups, lp.sp_columns, lp.sp_register_transposed,
                     lp.co_head_blocked, lp.co_heads_per_block, ref) &&
           plan_same(ref, lp);
}

int plan_candidates(const Shape &s, LaunchPlan *out, int cap)
{
    std::vector<LaunchPlan> all;
    auto push = [&](const LaunchPlan &lp) {
        for (const LaunchPlan &q : all)
            if (plan_same(q, lp)) return;
        all.push_back(lp);
    };
    push(plan_of(s));
    if (forward_small_eligible(s)) push(plan_fused(s));
    // state-pass kernels: (columns per workgroup, B transposed in registers)
    std::vector<std::pair<int, int>> kernels;
    if (s.bf16) {
        for (int cols : {256, 128, 64}) {
            if (s.N % cols != 0) continue;
            kernels.push_back({cols, 0});
            if (cols == 256) kernels.push_back({cols, 1});
        }
    } else {
        kernels.push_back({64, 0});
    }
    // chunk-output kernels: (head-blocked, heads per workgroup)
    std::vector<std::pair<int, int>> outs;
    if (s.bf16 && head_blocked(s)) {
        const int64_t hpg = s.H / s.G;
        for (int64_t hb = 1; hb <= std::min<int64_t>(hpg, 64); ++hb)
            if (hpg % hb == 0) outs.push_back({1, (int)hb});
    }
    outs.push_back({0, 1});
    for (const auto &kr : kernels) {
        // group counts: the cost model's for this kernel, then 1, 2, 3, 4, 6, 8, ... chunks
        // apart as far as the chain has chunks
        std::vector<Grouping> groups;
        groups.push_back(state_pass_groups(s, kr.first, kr.second != 0));
        for (int64_t g : {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128}) {
            if (g > s.nc) break;
            const int64_t K = (s.nc + g - 1) / g;
            groups.push_back({(int)K, (int)((s.nc + K - 1) / K)});
        }
        for (const Grouping &gp : groups)
            for (const auto &co : outs) {
                LaunchPlan lp;
                if (plan_from(s, gp.K, gp.ng, kr.first, kr.second, co.first, co.second, lp))
                    push(lp);
            }
    }
    const int n = (int)all.size();
    for (int i = 0; i < std::min(n, cap); ++i) out[i] = all[i];
    return n;
}

template <int Q, int NN>
static hipError_t hb_launch(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, const void *Hb, const float *beta, int K, int ng, int nc_full,
                            int HB, hipStream_t st)
{
    constexpr int SPL = NN > 256 ? 2 : 1;
    const int xcd = (nc_full % 8 == 0) ? 1 : 0;
    const dim3 grid((unsigned)(nc_full * s.b * s.G * (s.H / s.G / HB))), block(2 * Q * SPL);
    if (Hb != nullptr)
        hipLaunchKernelGGL((chunk_out_hb_kernel<Q, NN, true, SPL>), grid, block, 0, st, (const bf16 *)x,
                           (const bf16 *)B, (const bf16 *)C, G2, dtT, (const bf16 *)S, D, (bf16 *)y,
                           (const bf16 *)Hb, beta, (int)s.L, (int)s.H, (int)s.G, (int)s.nc,
                           (int)s.Lp, K, ng, HB, nc_full, xcd);
    else
        hipLaunchKernelGGL((chunk_out_hb_kernel<Q, NN, false, SPL>), grid, block, 0, st, (const bf16 *)x,
                           (const bf16 *)B, (const bf16 *)C, G2, dtT, (const bf16 *)S, D, (bf16 *)y,
                           (const bf16 *)nullptr, beta, (int)s.L, (int)s.H, (int)s.G, (int)s.nc,
                           (int)s.Lp, K, ng, HB, nc_full, xcd);
    return hipGetLastError();
}

template <int Q>
static hipError_t hb_dispatch_q(const Shape &s, const void *x, const void *B, const void *C,
                                const float *G2, const float *dtT, const void *S, const float *D,
                                void *y, const void *Hb, const float *beta, int K, int ng, int HB,
                                hipStream_t st)
{
    const int nc_full = (int)(s.L / s.Q);
    switch (s.N) {
    case 64: return hb_launch<Q, 64>(s, x, B, C, G2, dtT, S, D, y, Hb, beta, K, ng, nc_full, HB, st);
    case 128: return hb_launch<Q, 128>(s, x, B, C, G2, dtT, S, D, y, Hb, beta, K, ng, nc_full, HB, st);
    case 256: return hb_launch<Q, 256>(s, x, B, C, G2, dtT, S, D, y, Hb, beta, K, ng, nc_full, HB, st);
    default:
        if constexpr (Q == 128)
            return hb_launch<Q, 512>(s, x, B, C, G2, dtT, S, D, y, Hb, beta, K, ng, nc_full, HB, st);
        return hipErrorInvalidValue;   // not head-blocked: never dispatched here
    }
}


hipError_t launch_chunk_out_bf16(const Shape &s, const void *x, const void *B, const void *C,
                                 const float *G2, const float *dtT, const void *S, const float *D,
                                 void *y, const float *Hg, const void *Hb, const float *beta, int K,
                                 int ng, int hb, hipStream_t st)
{
    auto single = [&](int c_first, int nc_grid) {
        switch (s.Q) {
        case 64: return co_launch<64>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, c_first, nc_grid, st);
        case 128: return co_launch<128>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, c_first, nc_grid, st);
        default: return co_launch<256>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, c_first, nc_grid, st);
        }
    };
    if (hb <= 0 || !head_blocked(s)) return single(0, (int)s.nc);
    // full chunks head-blocked, a ragged last chunk on the one-head kernel
    const int nc_full = (int)(s.L / s.Q);
    hipError_t e = hipSuccess;
    if (nc_full > 0) {
        e = (s.Q == 128) ? hb_dispatch_q<128>(s, x, B, C, G2, dtT, S, D, y, Hb, beta, K, ng, hb, st)
                         : hb_dispatch_q<256>(s, x, B, C, G2, dtT, S, D, y, Hb, beta, K, ng, hb, st);
        if (e != hipSuccess) return e;
    }
    if (nc_full < s.nc) e = single(nc_full, 1);
    return e;
}

}  // namespace ssd
