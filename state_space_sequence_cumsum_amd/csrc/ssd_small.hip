// ssd_small.hip -- the whole forward pass in one launch, for fp32 problems of a few chunks.
//
// Method: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核": the chunked form
// of section "Mamba-2 架构", with the chunk-local cumsum of section "Kernel 1：计算累积和",
// the decayed jump of section "Kernel 2: fwd_pass_state" and the decayed chunk output of
// section "Kernel 3：compute_out".
//
// With a few chunks per sequence the four launches of the general path (cumsum, state
// pass, group scan, chunk output) and their memory round trips take longer than the
// arithmetic.  Here the state rows are split in two halves (headdim 64 = 2 x 32 rows p;
// the rows of the state and of y do not depend on one another), and one workgroup per
// (batch, head, chunk c, half) does all of it for its 32 rows:
//   * the cumsum of chunks 0 .. c (the general path's arithmetic, so G2 and dt equal the
//     stage-1 kernel's bit for bit; they go to the workspace from chunk c's workgroups);
//   * the intra-chunk term of chunk c's output, x^T M with M[j][i] = (i >= j) C_i.B_j
//     exp2(G_i - G_j) dt_j, while the tiles of the chain are still arriving;
//   * the jump h <- exp2(G_last) h + X^T (w B) over chunks 0 .. c-1 from the zero state (or
//     h0), every workgroup repeating the state work of the chunks before its own (bounded by
//     allowing this kernel for short chains only);
//   * the inter-chunk term exp2(G_i) h C^T, then y = both terms + D x.
// One more workgroup per (batch, head, half) walks the jump over all chunks and writes the
// final state.  Products run on fp32 MFMA (v_mfma_f32_32x32x2f32).  Every tile of x and B
// the chain needs is requested at the start with 16-byte global-to-LDS loads into a ring of
// four chunk slots, so their latency is paid about once.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

namespace {

typedef __attribute__((address_space(3))) void lds_ptr_t;

// LDS stores as inline assembly: before an ordinary store the compiler waits for every
// global-to-LDS load in flight, since it cannot tell which LDS bytes those write.  These
// stores go only to buffers no such load writes; the barrier below waits for them.
__device__ __forceinline__ void st_lds32(float *p, float v)
{
    asm volatile("ds_write_b32 %0, %1" ::"v"((uint32_t)(uintptr_t)(lds_ptr_t *)p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_lds128(float *p, f32x4 v)
{
    asm volatile("ds_write_b128 %0, %1" ::"v"((uint32_t)(uintptr_t)(lds_ptr_t *)p), "v"(v) : "memory");
}

}  // namespace

// A workgroup barrier that waits for this wave's LDS operations (lgkmcnt) only, not for its
// global loads in flight, as __syncthreads() would.
#define FS_BARRIER()                                                                            \
    do {                                                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                         \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)

// Chunks of 64 tokens, headdim 64 in two halves of 32 rows, dstate 64; 256 threads (four
// waves).  Wave w:
//   chain:  state columns n in 32 (w & 1) + [0, 32), tokens 32 (w >> 1) + [0, 32) of each
//           chunk (the two token halves keep partial states, summed where read);
//   output: token tile I = w >> 1 of Y^T[p][i], contraction half w & 1 (the partials are
//           summed in LDS before the store); waves 0, 1, 2 compute the C B^T tiles
//           (J, I) = (0, 0), (0, 1), (1, 1).
__global__ __launch_bounds__(256) void forward_small_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const float *__restrict__ Bm, const float *__restrict__ Cm, const float *__restrict__ D,
    const float *__restrict__ h0, float *__restrict__ y, float *__restrict__ hT,
    float *__restrict__ G2, float *__restrict__ dtT, int L, int H, int G, int nc, int Lp)
{
    constexpr int Q = 64, P = 64, PW = 32, N = 64, NF = N / 16;
    constexpr int R = 4;                          // ring slots
    constexpr int XI = 2, BI = 4, CI = XI + BI;   // 1 KB loads per wave: x half-rows, B rows, a chunk
    constexpr int MP = Q + 4, SSP = N + 4, YP = PW + 4;
    // ring slot: x half-rows of a chunk [token][p], then its B rows [token][n] (one array per
    // slot, so the compiler tells the slots apart when it places waits for loads into LDS)
    constexpr int SLOT = Q * PW + Q * N;
    __shared__ __attribute__((aligned(16))) float R0[SLOT], R1[SLOT], R2[SLOT], R3[SLOT];
    __shared__ __attribute__((aligned(16))) float XC[Q * PW];         // x half-rows of chunk c [j][p]
    __shared__ __attribute__((aligned(16))) float MT[Q * MP];         // M^T [i][j]; later y partials
    __shared__ __attribute__((aligned(16))) float MT2[32 * YP];       // wave 3's part of tile (0, 1)
    __shared__ __attribute__((aligned(16))) float Ss[2 * PW * SSP];   // state partials [p][n]
    __shared__ __attribute__((aligned(16))) float Gs[kSmallMaxChunks * Q];   // cumsum, log2 e scaled
    __shared__ __attribute__((aligned(16))) float Ws[kSmallMaxChunks * Q];   // jump weights
    __shared__ __attribute__((aligned(16))) float Ds[Q];                     // dt of chunk c
    __shared__ float Al[kSmallMaxChunks];                                    // exp2(chunk-end cumsum)
    auto xsl = [&](auto k) -> float * {
        constexpr int j = decltype(k)::value;
        return j == 0 ? R0 : (j == 1 ? R1 : (j == 2 ? R2 : R3));
    };
    auto bsl = [&](auto k) -> float * { return xsl(k) + Q * PW; };

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5, kq = 8 * hl;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ncw = nc + 1;
    const int pw = blockIdx.x & 1, rest = blockIdx.x >> 1;
    const int c = rest % ncw, bh = rest / ncw;
    const bool out = c < nc;                 // chunk c's output (else the final state)
    if (!out && hT == nullptr) return;
    const int nchain = out ? c : nc;         // chunks the jump walks
    const int ncs = out ? c + 1 : nc;        // chunks whose cumsum is needed
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
    const float *xb = x + (int64_t)b * L * xrow + (int64_t)h * P + PW * pw;
    const float *Bb = Bm + (int64_t)b * L * brow + (int64_t)g * N;
    const float *Cb = Cm + (int64_t)b * L * brow + (int64_t)g * N;
    float *yb = y + (int64_t)b * L * xrow + (int64_t)h * P + PW * pw;
    const float a = A[h];
    const int tn = w & 1, kt = w >> 1;       // chain: column tile, token half
    const int I = w >> 1, kh = w & 1;        // output: token tile, contraction half
    const int t0c = c * Q, lastc = min(L - t0c, Q) - 1;   // chunk c (output workgroups)

    // -- loads, in the order the waits below count them: dt, C and B rows and h0 into
    //    registers, then x of chunk c and the first R chunks of the chain into LDS.  The
    //    loads into LDS are the same for every wave whatever the workgroup's role (an unused
    //    one reads an empty buffer range), so every register load is followed by at least
    //    (R - 1) CI of them on every path: after the wait below the compiler knows all the
    //    register loads complete, and places no waits of its own for them.
    float dv[2];
    {
        // dt of token t at byte t H 4 from (b, 0, h): tokens at or past L are out of range (0)
        const rsrc_t dr = make_rsrc(dt + (int64_t)b * L * H + h, (int)((L * (int64_t)H - h) * 4));
#pragma unroll
        for (int r = 0; r < 2; ++r)
            dv[r] = __uint_as_float(buf_load_b32(dr, (uint32_t)(((w + 4 * r) * Q + lane) * H * 4)));
    }
    // C rows for h C^T; B and C rows for the C B^T tile: (J, I) = (0, 0) on wave 0, (1, 1) on
    // wave 1, both over all n; (0, 1) on waves 2 and 3, over n in [0, 32) and [32, 64)
    f32x8 cs[NF / 2], bf[NF], cf[NF];
    const int cbJ = (w == 1) ? 1 : 0, cbI = (w == 0) ? 0 : 1;
    const int cbF0 = (w == 3) ? NF / 2 : 0, cbNF = (w < 2) ? NF : NF / 2;   // fragments of n
    if (out) {
        const float *cr = Cb + (int64_t)(t0c + min(I * 32 + l32, lastc)) * brow + (N / 2) * kh + kq;
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) cs[f] = load_frag<float>(cr + 16 * f);
        const float *br = Bb + (int64_t)(t0c + min(cbJ * 32 + l32, lastc)) * brow + 16 * cbF0 + kq;
        const float *cr2 = Cb + (int64_t)(t0c + min(cbI * 32 + l32, lastc)) * brow + 16 * cbF0 + kq;
#pragma unroll
        for (int f = 0; f < NF; ++f) {   // (waves 2, 3 use the first NF / 2; a load under a
                                          // branch would be waited for at the branch's end)
            const int fl = min(f, NF - 1 - cbF0);
            bf[f] = load_frag<float>(br + 16 * fl);
            cf[f] = load_frag<float>(cr2 + 16 * fl);
        }
    }
    // the initial state (h0's rows of this half, or zero) in the first token half's partial
    f32x16 acc = zero_acc();
    if (h0 != nullptr && kt == 0) {
        const float *hr = h0 + ((int64_t)bh * P + PW * pw) * N + 32 * tn + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = hr[acc_row(v, lane) * N];
    }
    // 1 KB loads: x half-rows (8 rows of 32 floats each), B rows (4 rows of 64 floats each);
    // rows past the end of the sequence fall outside the buffer range and read as zero
    uint32_t xoff[XI], boff[BI];
#pragma unroll
    for (int k = 0; k < XI; ++k)
        xoff[k] = (uint32_t)(((w * XI + k) * 8 + lane / 8) * xrow * 4 + 16 * (lane % 8));
#pragma unroll
    for (int k = 0; k < BI; ++k)
        boff[k] = (uint32_t)(((w * BI + k) * 4 + lane / 16) * brow * 4 + 16 * (lane % 16));
    auto dma_x = [&](float *dst, int ck) {
        const int t0 = ck * Q;
        const rsrc_t r = make_rsrc(xb + t0 * xrow, (int)((L - t0) * xrow * 4));
#pragma unroll
        for (int k = 0; k < XI; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t *)(dst + (w * XI + k) * 256), 16,
                                                     (int)xoff[k], 0, 0, 0);
    };
    auto dma_b = [&](float *dst, int ck) {
        const int t0 = ck * Q;
        const rsrc_t r = make_rsrc(Bb + t0 * brow, (int)((L - t0) * brow * 4));
#pragma unroll
        for (int k = 0; k < BI; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t *)(dst + (w * BI + k) * 256), 16,
                                                     (int)boff[k], 0, 0, 0);
    };
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);   // the register loads go out first
    // (chunk c past the end for the final-state workgroup, and ring chunks at or past
    // nchain, read empty ranges: their slots are never read)
    auto ring_chunk = [&](int ck) { return ck < nchain ? ck : nc; };
    dma_x(XC, c);
    static_for<R>([&](auto jc) {
        dma_x(xsl(jc), ring_chunk(decltype(jc)::value));
        dma_b(bsl(jc), ring_chunk(decltype(jc)::value));
    });
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // at most k chunks of the ring still in flight for this wave
    auto wait_chunks = [](int k) {
        if (k <= 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        else if (k == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(CI));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * CI));
    };
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((R - 1) * CI));   // everything above but ring chunks 1 .. R-1

    // -- cumsum of chunks 0 .. ncs-1, chunk ck on wave ck % 4: the stage-1 kernel's
    //    arithmetic for 64-token chunks (the 64-lane DPP scan; padded tokens get dt = 0 and
    //    repeat the last valid cumsum value)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int ck = w + 4 * r;
        const bool used = ck < ncs;   // (the scan runs either way: a use of dv under a branch
                                      // would pull its load into the branch)
        const int t0 = min(ck, nc - 1) * Q;
        const float d = dv[r];
        float part = a * d;
        asm volatile("" : "+v"(part));   // the rounded product, as the stage-1 kernel sums it
        const float excl = wave_shift_up1(wave_inclusive_sum(part));
        const int last = min(L - t0, Q) - 1;
        const float tail = wave_read((excl + part) * kLog2e, last);
        float glast = wave_read((excl + part) * kLog2e, 63);
        if (last < Q - 1) glast = tail;
        const float gt = (lane <= last) ? (excl + part) * kLog2e : tail;
        if (!used) continue;
        st_lds32(&Gs[t0 + lane], gt);
        st_lds32(&Ws[t0 + lane], d * fast_exp2(glast - gt));
        if (lane == 0) st_lds32(&Al[ck], fast_exp2(glast));
        if (out && ck == c) {
            st_lds32(&Ds[lane], d);
            if (pw == 0) {
                G2[(int64_t)bh * Lp + t0 + lane] = gt;
                dtT[(int64_t)bh * Lp + t0 + lane] = d;
            }
        }
    }
    FS_BARRIER();

    // -- chunk c's intra-chunk term: Y^T[p][i] = sum_j x^T[p][j] M[j][i]
    f32x16 ya = zero_acc();
    if (out) {
        {   // C B^T tile (J, I) on MFMA (rows j, column i), then the decayed, masked M^T into LDS
            f32x16 cb = zero_acc();
#pragma unroll
            for (int f = 0; f < NF; ++f)
                if (f < cbNF) mma(cb, bf[f], cf[f]);
            const int i = cbI * 32 + l32;
            const float gi = Gs[t0c + i];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 m;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = cbJ * 32 + acc_row(4 * q + e, lane);
                    const float val = cb[4 * q + e] * fast_exp2(gi - Gs[t0c + j]) * Ds[j];
                    m[e] = (i >= j) ? val : 0.0f;
                }
                if (w == 3) st_lds128(&MT2[l32 * YP + 8 * q + 4 * hl], m);
                else st_lds128(&MT[i * MP + cbJ * 32 + 8 * q + 4 * hl], m);
            }
        }
        FS_BARRIER();
        // tokens j of this wave's contraction half: I = 0: 16 kh + [0, 16); I = 1: 32 kh + [0, 32)
        // (tile (0, 1), on wave 2, is the sum of its two parts)
        const float *mrow = MT + (I * 32 + l32) * MP;
        auto xm = [&](int j0) {
            f32x8 xa;
#pragma unroll
            for (int e = 0; e < 8; ++e) xa[e] = XC[(j0 + kq + e) * PW + l32];
            f32x8 mf = load_frag<float>(mrow + j0 + kq);
            if (w == 2) mf += load_frag<float>(MT2 + l32 * YP + j0 + kq);
            mma(ya, xa, mf);
        };
        if (I == 0) {
            xm(16 * kh);
        } else {
            xm(32 * kh);
            xm(32 * kh + 16);
        }
    }

    // -- the chain: h <- exp2(G_last) h + X^T (w B) over chunks 0 .. nchain-1
    auto jump = [&](const float *Xk, const float *Bk, int ck) {
        const float al = Al[ck];
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] *= al;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int tb = 32 * kt + 16 * f + kq;
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&Ws[ck * Q + tb]);
            const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&Ws[ck * Q + tb + 4]);
            f32x8 xa, ba;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xa[e] = Xk[(tb + e) * PW + l32] * (e < 4 ? w0[e] : w1[e - 4]);
                ba[e] = Bk[(tb + e) * N + 32 * tn + l32];
            }
            mma(acc, xa, ba);
        }
    };
    for (int ck0 = 0; ck0 < nchain; ck0 += R)
        static_for<R>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int ck = ck0 + j;
            if (ck < nchain) {
                if (ck >= 1) {
                    // issued so far: ring chunks 0 .. max(R - 1, min(ck - 2 + R, nchain - 1))
                    wait_chunks(max(R - 1, min(ck - 2 + R, nchain - 1)) - ck);
                    FS_BARRIER();   // chunk ck is in; every wave is done with slot (ck - 1) % R
                    const int nx = ck - 1 + R;
                    if (nx < nchain) {
                        const std::integral_constant<int, (j + R - 1) % R> js{};
                        dma_x(xsl(js), nx);
                        dma_b(bsl(js), nx);
                    }
                }
                jump(xsl(jc), bsl(jc), ck);
            }
        });

    // -- the state after the chain (one partial per token half) into LDS; no load into LDS
    //    stays in flight past this point (ring slot 0 is reused below)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    {
        float *sp = Ss + kt * PW * SSP + 32 * tn + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) st_lds32(sp + acc_row(v, lane) * SSP, acc[v]);
    }
    FS_BARRIER();

    if (!out) {   // the final state: the two partials summed
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int pc = tid + 256 * r, p = pc >> 4, n4 = 4 * (pc & 15);
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&Ss[p * SSP + n4]);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(&Ss[(PW + p) * SSP + n4]);
            *reinterpret_cast<f32x4 *>(hT + ((int64_t)bh * P + PW * pw + p) * N + n4) = s0 + s1;
        }
        return;
    }

    // -- chunk c's inter-chunk term: Y^T += exp2(G_i) h C^T (contraction half kh of n)
    {
        f32x16 sc = zero_acc();
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
            const int n0 = (N / 2) * kh + 16 * f + kq;
            const f32x8 s0 = load_frag<float>(Ss + l32 * SSP + n0);
            const f32x8 s1 = load_frag<float>(Ss + (PW + l32) * SSP + n0);
            mma(sc, s0 + s1, cs[f]);
        }
        const float si = fast_exp2(Gs[t0c + I * 32 + l32]);
#pragma unroll
        for (int v = 0; v < 16; ++v) ya[v] += si * sc[v];
    }
    // the partials to LDS as [i][p] (half kh = 0 over M^T, half 1 over ring slot 0), then
    // y_i = both + D x_i, one 16-byte store per 4 columns
    {
        float *yp = (kh == 0 ? MT : R0) + (I * 32 + l32) * YP;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            st_lds128(yp + 8 * q + 4 * hl, f32x4{ya[4 * q], ya[4 * q + 1], ya[4 * q + 2], ya[4 * q + 3]});
    }
    FS_BARRIER();
    const float Dh = D[h];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int pc = tid + 256 * r, i = pc >> 3, p4 = 4 * (pc & 7);
        if (i > lastc) continue;
        const f32x4 y0 = *reinterpret_cast<const f32x4 *>(&MT[i * YP + p4]);
        const f32x4 y1 = *reinterpret_cast<const f32x4 *>(&R0[i * YP + p4]);
        const f32x4 xv = *reinterpret_cast<const f32x4 *>(&XC[i * PW + p4]);
        *reinterpret_cast<f32x4 *>(yb + (int64_t)(t0c + i) * xrow + p4) = y0 + y1 + Dh * xv;
    }
}
#undef FS_BARRIER

bool forward_small_eligible(const Shape &s)
{
    return !s.bf16 && s.Q == 64 && s.P == 64 && s.N == 64 && s.nc <= kSmallMaxChunks && s.H <= 65536 &&
           s.b * s.H * (s.nc + 1) * 2 * 256 < (int64_t(1) << 31) &&
           s.L * s.H * s.P * 4 < (int64_t(1) << 31) && s.L * s.G * s.N * 4 < (int64_t(1) << 31);
}

int64_t forward_small_workgroups(const Shape &s) { return 2 * s.b * s.H * (s.nc + 1); }

hipError_t launch_forward_small(const Shape &s, const void *x, const void *dt, const float *A,
                                const void *B, const void *C, const float *D, const float *h0,
                                void *y, float *hT, float *G2, float *dtT, hipStream_t st)
{
    hipLaunchKernelGGL(forward_small_f32_kernel, dim3((unsigned)forward_small_workgroups(s)), dim3(256),
                       0, st, (const float *)x, (const float *)dt, A, (const float *)B,
                       (const float *)C, D, h0, (float *)y, hT, G2, dtT, (int)s.L, (int)s.H,
                       (int)s.G, (int)s.nc, (int)s.Lp);
    return hipGetLastError();
}

}  // namespace ssd
