// ssd_bf16.hip -- gfx950 state-pass and chunk-output kernels for bf16 inputs
// (bf16 MFMA operands, fp32 accumulation, fp32 running state).
//
// Method: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核",
// sections "Kernel 2: fwd_pass_state" (decayed chunk jump) and
// "Kernel 3：compute_out" (decayed chunk output).
//
// Both kernels contract over tokens, which are the strided dimension of every
// input tensor.  Tiles are copied into LDS in their natural token-major layout
// with 16-byte writes and the token-packed MFMA operands are read back with
// the gfx950 LDS transpose read (ds_read_b64_tr_b16), so no element-wise
// transposition happens on the way in.
#include <algorithm>

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
// Each chunk is processed in sub-steps of TS tokens.  Step s of the loop:
//   * copies B of sub-step s+1 into LDS token-major (16-byte rows) and x~ of
//     sub-step s+2 (scaled on the way), both from registers loaded D sub-steps
//     earlier, then reloads the freed registers;
//   * k-packs x~ of s+1, Xk[p][t], by transpose-reading its token-major tile
//     (4 consecutive tokens of one p per lane) and writing 8 bytes;
//   * at a chunk start, writes the chunk-start state (bf16) into an LDS tile,
//     which the next step stores to HBM as whole 16-byte-per-lane rows, and
//     decays the state;
//   * MFMA over sub-step s: A = B^T rows n, transpose-read from the token-major
//     B tile (each B element is read once), B operand = Xk rows p (16-byte
//     reads; every wave reads all of x~, the cheap operand);
//   * one barrier.
// Every LDS buffer is written one step before it is read and rewritten only
// after the barrier that follows its last read, so two copies of each suffice.
// Indices past the group's last sub-step are clamped (the extra copies are
// never read) and rows past L are clamped to row L-1 (their weight is 0), so
// the loop body has no branches around memory operations and the wait counts
// leave later sub-steps in flight.
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
    static constexpr int BP = tr_pitch(N);                       // token-major B rows
    static constexpr int XRP = tr_pitch(P);                      // token-major x rows
    static constexpr int XKP = TS + 8;                           // k-packed x~ rows
    static constexpr int SSP = N + 8;                            // chunk-start state staging rows
    static constexpr int SPT = P * N / 8 / NTHR;                 // 16-byte state pieces per thread
    static constexpr int BPT = TS * N / 8 / NTHR;                // 16-byte B pieces per thread
    static constexpr int XPIECES = TS * P / 8;                   // 16-byte x pieces per sub-step
    static constexpr int XPT = (XPIECES + NTHR - 1) / NTHR;      // per thread (last may idle)
    static constexpr int TRG = TS * P / (4 * 16);                // 16-lane transpose reads per sub-step
    static constexpr int TRL = TRG / (4 * NWAVE);                // ... per lane
    static_assert(BPT >= 1 && TS * N / 8 % NTHR == 0, "B staging cover");
    static_assert(TRL >= 1 && TRG % (4 * NWAVE) == 0, "x~ build cover");
    static_assert((N / 32 / RTW) * (2 / CTW) == NWAVE, "wave tiling");
    static_assert(Q % TS == 0, "sub-steps per chunk");
};

template <int Q, int NR, int D>
__global__ __launch_bounds__((SpCfg<Q, NR>::NTHR)) void state_pass_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const float *__restrict__ G2,
    const float *__restrict__ wT, const float *__restrict__ h0, bf16 *__restrict__ S,
    float *__restrict__ hT, float *__restrict__ Ug, float *__restrict__ gam,
    float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng, int xcd)
{
    using C = SpCfg<Q, NR>;
    constexpr int P = C::P, TS = C::TS, NSUB = C::NSUB, NTHR = C::NTHR, RTW = C::RTW,
                  CTW = C::CTW, BP = C::BP, XRP = C::XRP, XKP = C::XKP, BPT = C::BPT,
                  XPT = C::XPT, XPIECES = C::XPIECES, TRL = C::TRL;
    constexpr int SSP = C::SSP, SPT = C::SPT;
    __shared__ __attribute__((aligned(16))) bf16 Bs[2][TS * BP];
    __shared__ __attribute__((aligned(16))) bf16 Xr[2][TS * XRP];
    __shared__ __attribute__((aligned(16))) bf16 Xk[2][P * XKP];
    __shared__ __attribute__((aligned(16))) bf16 Ss[P * SSP];
    __shared__ float Al[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // workgroup -> (group, batch*head, column range); with `xcd` all heads of one
    // group share an XCD, so the group's B tiles are fetched into one L2
    int grp, minor;
    xcd_split(blockIdx.x, (int)(gridDim.x / ng), xcd != 0, grp, minor);
    const int ntiles = N / NR, bh = minor / ntiles, n0 = (minor % ntiles) * NR;
    const int c0 = grp * K, c1 = min(c0 + K, nc);
    const int U = (c1 - c0) * NSUB;                               // sub-steps of this group
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int rt0 = (wave / (2 / CTW)) * RTW, ct0 = (wave % (2 / CTW)) * CTW;
    const int64_t st_off = (int64_t)bh * P * N;
    const float *Gh = G2 + (int64_t)bh * Lp;
    const float *wh = wT + (int64_t)bh * Lp;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16 *xb = x + (int64_t)b * L * xstride + (int64_t)h * P;
    const bf16 *Bb = Bm + (int64_t)b * L * bstride + (int64_t)g * N + n0;
    const bool keeper = tid == 0 && n0 == 0;   // writes beta / gamma of this group

    // accumulator element v of tile (i, j): row n = 32 (rt0 + i) + acc_row(v, lane),
    // column p = 32 (ct0 + j) + lane % 32
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

    // ---- staging: sub-step u covers tokens t0(u) .. t0(u) + TS of chunk c0 + u / NSUB.
    // Rows past L are clamped to row L-1 instead of zeroed: their weight w is 0 (stage
    // 1 writes zeros there), so their x~ rows are 0 and they add nothing.  Every
    // load is issued unconditionally, which keeps the loop body free of branches
    // around memory operations and lets the wait counts leave later sub-steps in
    // flight.
    // Global offsets are 32-bit byte offsets from the batch's base pointer (the
    // host checks that one batch of x and of B spans less than 2^31 bytes), so
    // the loads use a scalar base plus one vector register.
    int bo[BPT], blo[BPT], bt_[BPT], xo[XPT], xlo[XPT], xt_[XPT];
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
        const int id = tid + NTHR * r, t = id / (NR / 8), c8 = id % (NR / 8);
        bo[r] = c8 * 16;
        bt_[r] = t;
        blo[r] = t * BP + c8 * 8;
    }
#pragma unroll
    for (int r = 0; r < XPT; ++r) {
        const int id = min(tid + NTHR * r, XPIECES - 1), t = id >> 3, c8 = id & 7;
        xo[r] = c8 * 16;
        xt_[r] = t;
        xlo[r] = t * XRP + c8 * 8;
    }
    const char *Bbytes = reinterpret_cast<const char *>(Bb);
    const char *xbytes = reinterpret_cast<const char *>(xb);
    const int brow = (int)bstride * 2, xrow = (int)xstride * 2;
    // x~ k-packing: 16-lane group j transpose-reads tokens 4 tb .. 4 tb + 3 of p
    // block pb (16 p) of the scaled token-major tile; lane m of the group gets
    // those 4 tokens of p = 16 pb + m and writes them k-packed.  The groups of one
    // wave take consecutive token blocks so their 8-byte writes land in distinct
    // banks.
    const int m16 = lane & 15;
    int tbv[TRL], pbv[TRL];
#pragma unroll
    for (int r = 0; r < TRL; ++r) {
        const int gr = (lane >> 4) + 4 * wave + 4 * C::NWAVE * r;
        tbv[r] = gr % (TS / 4);
        pbv[r] = gr / (TS / 4);
    }
    struct Regs {
        bf16x8 b[BPT];
        bf16x8 x[XPT];
        float w[XPT];   // weight of the token of x piece r
        float gl;
    };
    const int last_row = L - 1;
    auto tok0 = [&](int u) { return (c0 + u / NSUB) * Q + (u % NSUB) * TS; };
    auto load = [&](Regs &R, int u) {
        u = min(u, U - 1);
        const int t0 = tok0(u);
#pragma unroll
        for (int r = 0; r < BPT; ++r) {
            const uint32_t off = (uint32_t)(min(t0 + bt_[r], last_row) * brow + bo[r]);
            R.b[r] = *reinterpret_cast<const bf16x8 *>(Bbytes + off);
        }
#pragma unroll
        for (int r = 0; r < XPT; ++r) {
            const uint32_t off = (uint32_t)(min(t0 + xt_[r], last_row) * xrow + xo[r]);
            R.x[r] = *reinterpret_cast<const bf16x8 *>(xbytes + off);
        }
#pragma unroll
        for (int r = 0; r < XPT; ++r) R.w[r] = wh[t0 + xt_[r]];
        // the chunk's last cumsum value, as a per-lane load (a scalar load would
        // share the LDS wait counter and stall every LDS wait behind it)
        int gi = (c0 + u / NSUB) * Q + Q - 1;
        asm volatile("" : "+v"(gi));
        R.gl = Gh[gi];
    };
    // LDS buffer indices are passed in as compile-time constants
    auto storeB = [&](const Regs &R, int kb) {
#pragma unroll
        for (int r = 0; r < BPT; ++r) *reinterpret_cast<bf16x8 *>(&Bs[kb][blo[r]]) = R.b[r];
    };
    auto storeX = [&](const Regs &R, int kx, int ka) {
        // x~ = round(w_t x_t), token-major
#pragma unroll
        for (int r = 0; r < XPT; ++r) {
            const u32x4 xv = __builtin_bit_cast(u32x4, R.x[r]);
            u32x4 o;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) o[k2] = pack_bf16(bf_lo(xv[k2]) * R.w[r], bf_hi(xv[k2]) * R.w[r]);
            if (XPT * NTHR == XPIECES || tid + NTHR * r < XPIECES)
                *reinterpret_cast<u32x4 *>(&Xr[kx][xlo[r]]) = o;
        }
        Al[ka] = fast_exp2(R.gl);   // same value from every thread
    };
    auto build = [&](int k, int kx) {
#pragma unroll
        for (int r = 0; r < TRL; ++r) {
            const int tb = tbv[r], pb = pbv[r];
            const bf16x4 v = tr_read4(&Xr[k][(4 * tb + (m16 >> 2)) * XRP + 16 * pb + 4 * (m16 & 3)]);
            *reinterpret_cast<bf16x4 *>(&Xk[kx][(16 * pb + m16) * XKP + 4 * tb]) = v;
        }
    };

    const int offA = tr_off_natural(lane, BP);
    const int offB = (lane & 31) * XKP + 8 * (lane >> 5);

    // chunk start (sub-step u, u % NSUB == 0): store the chunk-start state, decay
    // chunk start (sub-step u, u % NSUB == 0): the chunk-start state goes to the
    // LDS staging tile as bf16 (row p, columns n), then the state decays
    auto chunk_start = [&](int ka) {
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
                    *reinterpret_cast<bf16x4 *>(&Ss[p * SSP + n + 8 * q]) = o;
                }
            }
        const float a = Al[ka];
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
            for (int j = 0; j < CTW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] *= a;
    };
    // the staged state of chunk c to HBM: thread piece r is row p, 8 columns;
    // consecutive lanes cover consecutive 16 bytes of a row
    auto state_out = [&](int c) {
        char *Sc = reinterpret_cast<char *>(S + ((int64_t)bh * nc + c) * P * N + n0);
#pragma unroll
        for (int r = 0; r < SPT; ++r) {
            const int id = tid + NTHR * r, p = id / (NR / 8), c8 = id % (NR / 8);
            const bf16x8 v = *reinterpret_cast<const bf16x8 *>(&Ss[p * SSP + 8 * c8]);
            *reinterpret_cast<bf16x8 *>(Sc + (uint32_t)((p * N + 8 * c8) * 2)) = v;
        }
    };
    auto mma_sub = [&](int kb, int kx) {
        const bf16 *bt = &Bs[kb][offA];
        const bf16 *xt = &Xk[kx][offB];
#pragma unroll
        for (int ks = 0; ks < TS / 16; ++ks) {
            bf16x8 bfr[CTW];
#pragma unroll
            for (int j = 0; j < CTW; ++j) bfr[j] = ld16(xt + 32 * (ct0 + j) * XKP + 16 * ks);
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const bf16 *a0 = bt + 16 * ks * BP + 32 * (rt0 + i);
                const bf16x8 af = cat8(tr_read4(a0), tr_read4(a0 + 4 * BP));
#pragma unroll
                for (int j = 0; j < CTW; ++j) mma(acc[i][j], af, bfr[j]);
            }
        }
    };

    // Register ring of D sub-steps: sub-step u sits in R[u % D] from its load
    // (step u - 1 - D) until its B tile is copied (step u - 1); its x~ is copied
    // one step earlier (step u - 2).
    static_assert(D >= 2, "a ring slot holds one sub-step from x~ copy to B copy");
    Regs R[D];
    // step s, with j = s mod UNR a compile-time constant
    // The products of sub-step s come first so that the copies for later
    // sub-steps (independent buffers) can issue while the MFMAs run.
    auto step = [&](int s, int j) {
        if (j % NSUB == 0) {
            if constexpr (NSUB == 1) {   // the previous chunk's staged state leaves first
                if (s > 0) state_out(c0 + s - 1);
                __syncthreads();
            }
            chunk_start(j & 3);
        }
        mma_sub(j & 1, j & 1);
        storeB(R[(j + 1) % D], (j + 1) & 1);
        storeX(R[(j + 2) % D], (j + 2) & 1, (j + 2) & 3);
        load(R[(j + 1) % D], s + 1 + D);
        if (NSUB > 1 && j % NSUB == 1) state_out(c0 + s / NSUB);
        build((j + 1) & 1, (j + 1) & 1);
        __syncthreads();
    };

#pragma unroll
    for (int u = 0; u < D; ++u) load(R[u], u);
    storeX(R[0], 0, 0);
    storeB(R[0], 0);
    load(R[0], D);
    storeX(R[1 % D], 1, 1);
    __syncthreads();
    build(0, 0);
    __syncthreads();
    // The body covers UNR = lcm(NSUB, D, 4) sub-steps so that ring slots, LDS
    // buffers and chunk-start positions are compile-time constants.
    constexpr int UNR = lcm3(NSUB, D, 4);
    int s = 0;
    for (; s + UNR <= U; s += UNR) {
#pragma unroll
        for (int j = 0; j < UNR; ++j) step(s + j, j);
    }
#pragma unroll
    for (int j = 0; j < UNR; ++j)
        if (s + j < U) step(s + j, j);
    // with one sub-step per chunk the last chunk's staged state is still in LDS
    if constexpr (NSUB == 1) state_out(c1 - 1);

    // decay products of the group (beta_c before each chunk, gamma for the group)
    if (keeper) {
        float run = 1.0f;
        for (int c = c0; c < c1; ++c) {
            if (beta != nullptr) beta[(int64_t)bh * nc + c] = run;
            run *= fast_exp2(Gh[c * Q + Q - 1]);
        }
        if (gam != nullptr) gam[(int64_t)bh * ng + grp] = run;
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
// Group scan.  For each (batch*head, state element): walk the groups in order,
// H_1 = U_0 and H_{g+1} = gamma_g H_g + U_g; H_g (the true state at group g's
// start) replaces U_g in place, and the state after the last group is hT.
// ===========================================================================
__global__ __launch_bounds__(256) void group_scan_kernel(float *__restrict__ Ug,
                                                         const float *__restrict__ gam,
                                                         float *__restrict__ hT, int PN, int ng)
{
    const int bh = blockIdx.y;
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    f32x4 hcar = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int g = 0; g < ng; ++g) {
        f32x4 *u = reinterpret_cast<f32x4 *>(Ug + ((int64_t)bh * ng + g) * PN + e);
        const f32x4 v = *u;
        if (g > 0) *u = hcar;
        const float gm = gam[(int64_t)bh * ng + g];
#pragma unroll
        for (int r = 0; r < 4; ++r) hcar[r] = gm * hcar[r] + v[r];
    }
    if (hT != nullptr) *reinterpret_cast<f32x4 *>(hT + (int64_t)bh * PN + e) = hcar;
}

// ===========================================================================
// Chunk output.  Workgroup = one (chunk, batch*head) with Q/32 waves; wave w
// owns one 32-token row tile I = rowtile(w).  Waves w and w + Q/64 (which the
// hardware places on the same SIMD) get tiles that add up to Q/32 - 1, so every
// SIMD does the same number, Q/32 + 1, of causal tile pairs (J, I), J <= I.
// Two waves per SIMD let one wave's loads, barriers and exponentials overlap
// the other's matrix products.  The output is built transposed, Y^T [64 p x 32
// tokens] per row tile.
//
// Phase 1 streams N in slices of 64: the slice of B (all chunk rows) and of S
// (all p) is staged in LDS, the wave's C rows come from global memory, and the
// next slice is loaded into registers while the current one is multiplied:
//   * CB_J = (B C^T)[tile J, tile I] for J <= I (accumulators indexed by J);
//   * Y^T += S C^T (the inter-chunk term).
// Phase 2, per J <= I: the C B^T tile becomes the decay matrix
//   M[j, i] = (i >= j) ? CB[j, i] * exp2(G_i - G_j) : 0      (selection, never a product with a mask)
// rounded to bf16 and fed to MFMA straight from registers against (dt x)^T.
// Off the diagonal (J < I) the decay factors exactly into
// exp2(G_i - G_e) * exp2(G_e - G_j), e the last token of tile J; both factors are
// <= 1, the second a per-token table, so such a tile costs one exp2 per lane.
// The Y^T accumulator is scaled by exp2(G_i) between the two phases.
//
// Chunk-start state handed over by a grouped state pass (Hg != NULL): S holds
// the state relative to the start of the chunk's group, to which beta_c H_g is
// added while staging (group 0 already started from the true initial state).
// ===========================================================================
template <int Q>
__global__ __launch_bounds__(2 * Q) void chunk_out_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const float *__restrict__ G2, const float *__restrict__ dtT, const bf16 *__restrict__ S,
    const float *__restrict__ D, bf16 *__restrict__ y, const float *__restrict__ Hg,
    const float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng,
    int xcd)
{
    constexpr int P = 64, NI = Q / 32, NW = Q / 32, NTHR = 2 * Q, NS = 64;
    constexpr int XP = Q + 8, BP = frag_pitch(NS), SP = frag_pitch(NS);
    constexpr int BPC = Q * (NS / 8) / NTHR;   // 16-byte B pieces per thread per slice
    constexpr int SPC = P * (NS / 8) / NTHR;   // 16-byte S pieces per thread per slice
    static_assert(BPC >= 1 && SPC >= 1, "slice staging cover");
    // (dt x)^T [p][position]: within each 16-token group the token at offset o is
    // kept at position o with its middle two 4-token blocks swapped, so the
    // accumulator token order 4(l/32)+{0..3}, 8+4(l/32)+{0..3} of lane l becomes 8
    // consecutive positions.
    __shared__ __attribute__((aligned(16))) bf16 Xd[P * XP];
    __shared__ __attribute__((aligned(16))) bf16 Bs[Q * BP];
    __shared__ __attribute__((aligned(16))) bf16 Ss[P * SP];
    __shared__ __attribute__((aligned(16))) float Gs[Q];
    __shared__ __attribute__((aligned(16))) float We[Q];   // exp2(G_e - G_j), e = end of j's tile

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int I = (w < NW / 2) ? w : NW - 1 - (w - NW / 2);

    // Workgroup -> (chunk, batch*head), heads innermost.  With `xcd` set (nc a
    // multiple of 8) XCD x gets the contiguous chunk range [x nc/8, (x+1) nc/8):
    // a chunk's B and C rows are shared by all its heads and a state-pass group's
    // carried state by its consecutive chunks, and both then stay in one L2.
    const int bH = gridDim.x / nc;
    int c, bh;
    if (xcd) {
        const int xx = blockIdx.x & 7, slot = blockIdx.x >> 3;
        c = xx * (nc / 8) + slot / bH;
        bh = slot % bH;
    } else {
        c = blockIdx.x / bH;
        bh = blockIdx.x % bH;
    }
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int t0 = c * Q;
    const bool full = t0 + Q <= L;
    const int64_t xstride = (int64_t)H * P, cstride = (int64_t)G * N;
    const bf16 *xb = x + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
    const bf16 *Bb = Bm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N;
    const bf16 *Cb = Cm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N;
    const bf16 *Sb = S + ((int64_t)bh * nc + c) * P * N;
    const float *Gh = G2 + (int64_t)bh * Lp + t0;
    const float *dh = dtT + (int64_t)bh * Lp + t0;
    const int kq = 8 * (lane >> 5);
    const int cgrp = (Hg != nullptr) ? c / K : 0;
    const float *Hc = (cgrp > 0) ? Hg + ((int64_t)bh * ng + cgrp) * P * N : nullptr;
    const float bc = (cgrp > 0) ? beta[(int64_t)bh * nc + c] : 0.0f;

    const int i_loc = I * 32 + (lane & 31);
    const bool iv = full || t0 + i_loc < L;
    const bf16 *crow = Cb + i_loc * (int)cstride + kq;

    // registers holding the next N slice while the current one is multiplied
    bf16x8 bq[BPC], sq[SPC], cn[NS / 16];
    f32x4 hq[SPC][2];
    auto load_slice = [&](int n0) {
        if (full) {   // uniform: no per-lane predication
#pragma unroll
            for (int r = 0; r < BPC; ++r) {
                const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
                bq[r] = ld16(Bb + t * (int)cstride + n0 + oct * 8);
            }
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks) cn[ks] = ld16(crow + n0 + ks * 16);
        } else {
#pragma unroll
            for (int r = 0; r < BPC; ++r) {
                const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
                bq[r] = (t0 + t < L) ? ld16(Bb + t * (int)cstride + n0 + oct * 8) : zero8();
            }
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks) cn[ks] = iv ? ld16(crow + n0 + ks * 16) : zero8();
        }
#pragma unroll
        for (int r = 0; r < SPC; ++r) {
            const int id = tid + NTHR * r, p = id >> 3, oct = id & 7;
            sq[r] = ld16(Sb + p * N + n0 + oct * 8);
            if (Hc != nullptr) {
                hq[r][0] = *reinterpret_cast<const f32x4 *>(Hc + p * N + n0 + oct * 8);
                hq[r][1] = *reinterpret_cast<const f32x4 *>(Hc + p * N + n0 + oct * 8 + 4);
            }
        }
    };

    // (dt x)^T tile and the chunk's decays; the first N slice is requested right
    // behind the x tile so both latencies overlap.  Thread = one 8-token x 4-p
    // block: rows loaded token-major, scaled by dt, packed per p column.  A wave
    // covers 8 token groups (lane % 8) x 8 column groups (lane / 8).
    {
        const int tg = (w >> 1) * 8 + (lane & 7), cg = (w & 1) * 8 + (lane >> 3);
        u32x2 xv[8];
        if (full) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                xv[r] = *reinterpret_cast<const u32x2 *>(xb + (tg * 8 + r) * (int)xstride + cg * 4);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                xv[r] = (t0 + tg * 8 + r < L)
                            ? *reinterpret_cast<const u32x2 *>(xb + (tg * 8 + r) * (int)xstride + cg * 4)
                            : u32x2{0u, 0u};
        }
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dh + tg * 8);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dh + tg * 8 + 4);
        float gt = 0.0f, ge = 0.0f;
        if (tid < Q) {
            gt = Gh[tid];
            ge = Gh[tid | 31];
        }
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
    }

    f32x16 cb[NI];
#pragma unroll
    for (int J = 0; J < NI; ++J) cb[J] = zero_acc();
    f32x16 ya[2] = {zero_acc(), zero_acc()};

    // ---------------- phase 1: C B^T tiles and S C^T over N slices ----------------
    for (int n0 = 0; n0 < N; n0 += NS) {
        __syncthreads();   // previous slice consumed; first time: Xd, Gs, We written
#pragma unroll
        for (int r = 0; r < BPC; ++r) {
            const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
            *reinterpret_cast<bf16x8 *>(&Bs[t * BP + oct * 8]) = bq[r];
        }
#pragma unroll
        for (int r = 0; r < SPC; ++r) {
            const int id = tid + NTHR * r, p = id >> 3, oct = id & 7;
            bf16x8 sv = sq[r];
            if (Hc != nullptr) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sv[e] = (bf16)((float)sv[e] + bc * hq[r][e >> 2][e & 3]);
            }
            *reinterpret_cast<bf16x8 *>(&Ss[p * SP + oct * 8]) = sv;
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
            const bf16 *srow = Ss + (pp * 32 + (lane & 31)) * SP + kq;
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
    if (iv) {
        const float Dh = D[h];
        const int yo = i_loc * (int)xstride;
        bf16 *yb = y + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = pp * 32 + 8 * q + 4 * (lane >> 5);
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xb + yo + p);
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = (bf16)(ya[pp][4 * q + r] + Dh * (float)xv[r]);
                *reinterpret_cast<bf16x4 *>(yb + yo + p) = o;
            }
        }
    }
}

// ===========================================================================
// Launchers
// ===========================================================================
// register ring depth of the state pass (sub-steps in flight)
constexpr int kSpDepth = 2;

template <int Q, int NR>
static hipError_t sp_launch(const Shape &s, const void *x, const void *B, const float *G2,
                            const float *wT, const float *h0, void *S, float *hT, float *Ug,
                            float *gam, float *beta, int K, int ng, hipStream_t st)
{
    const int units = (int)(s.b * s.H * (s.N / NR));
    const int xcd = (ng % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((state_pass_bf16_kernel<Q, NR, kSpDepth>), dim3((unsigned)(units * ng)),
                       dim3(SpCfg<Q, NR>::NTHR), 0, st, (const bf16 *)x, (const bf16 *)B, G2, wT,
                       h0, (bf16 *)S, hT, Ug, gam, beta, (int)s.L, (int)s.H, (int)s.G, (int)s.N,
                       (int)s.nc, (int)s.Lp, K, ng, xcd);
    return hipGetLastError();
}

// columns per state-pass workgroup: the largest of 256, 128, 64 dividing N
static int sp_cols(const Shape &s) { return (s.N % 256 == 0) ? 256 : (s.N % 128 == 0) ? 128 : 64; }

template <int Q>
static hipError_t sp_dispatch_q(const Shape &s, const void *x, const void *B, const float *G2,
                                const float *wT, const float *h0, void *S, float *hT, float *Ug,
                                float *gam, float *beta, int K, int ng, hipStream_t st)
{
    switch (sp_cols(s)) {
    case 256: return sp_launch<Q, 256>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    case 128: return sp_launch<Q, 128>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    default: return sp_launch<Q, 64>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    }
}

static hipError_t sp_dispatch(const Shape &s, const void *x, const void *B, const float *G2,
                              const float *wT, const float *h0, void *S, float *hT, float *Ug,
                              float *gam, float *beta, int K, int ng, hipStream_t st)
{
    switch (s.Q) {
    case 64: return sp_dispatch_q<64>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    case 128: return sp_dispatch_q<128>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    default: return sp_dispatch_q<256>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    }
}

hipError_t launch_state_pass_bf16(const Shape &s, const void *x, const void *B, const float *G2,
                                  const float *wT, const float *h0, void *S, float *hT,
                                  hipStream_t st)
{
    return sp_dispatch(s, x, B, G2, wT, h0, S, hT, nullptr, nullptr, nullptr, (int)s.nc, 1, st);
}

Grouping state_pass_groups(const Shape &s)
{
    Grouping gp;
    if (!s.bf16) {
        gp.K = (int)s.nc;
        gp.ng = 1;
        return gp;
    }
    // about one state-pass workgroup per CU (each takes most of a CU's LDS)
    const int64_t units = s.b * s.H * (s.N / sp_cols(s));
    int64_t ng = (256 + units - 1) / units;
    ng = std::max<int64_t>(1, std::min<int64_t>(ng, s.nc));
    const int64_t K = (s.nc + ng - 1) / ng;
    gp.K = (int)K;
    gp.ng = (int)((s.nc + K - 1) / K);
    return gp;
}

hipError_t launch_state_pass_grouped(const Shape &s, const Grouping &gp, const void *x,
                                     const void *B, const float *G2, const float *wT,
                                     const float *h0, void *S, float *hT, float *Ug, float *gam,
                                     float *beta, hipStream_t st)
{
    if (!s.bf16 || gp.ng <= 1) return launch_state_pass(s, x, B, G2, wT, h0, S, hT, st);
    hipError_t e = sp_dispatch(s, x, B, G2, wT, h0, S, nullptr, Ug, gam, beta, gp.K, gp.ng, st);
    if (e != hipSuccess) return e;
    const int PN = (int)(s.P * s.N);
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)(s.b * s.H));
    hipLaunchKernelGGL(group_scan_kernel, grid, dim3(256), 0, st, Ug, gam, hT, PN, gp.ng);
    return hipGetLastError();
}

template <int Q>
static hipError_t co_launch(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, const float *Hg, const float *beta, int K, int ng,
                            hipStream_t st)
{
    const int xcd = (s.nc % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_out_bf16_kernel<Q>), dim3((unsigned)(s.nc * s.b * s.H)), dim3(2 * Q), 0,
                       st, (const bf16 *)x, (const bf16 *)B, (const bf16 *)C, G2, dtT,
                       (const bf16 *)S, D, (bf16 *)y, Hg, beta, (int)s.L, (int)s.H, (int)s.G,
                       (int)s.N, (int)s.nc, (int)s.Lp, K, ng, xcd);
    return hipGetLastError();
}

hipError_t launch_chunk_out_bf16(const Shape &s, const void *x, const void *B, const void *C,
                                 const float *G2, const float *dtT, const void *S, const float *D,
                                 void *y, const float *Hg, const float *beta, int K, int ng,
                                 hipStream_t st)
{
    switch (s.Q) {
    case 64: return co_launch<64>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    case 128: return co_launch<128>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    default: return co_launch<256>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    }
}

}  // namespace ssd
