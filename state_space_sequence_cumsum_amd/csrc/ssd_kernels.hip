// ssd_kernels.hip -- the three gfx950 kernels of the Mamba-2 SSD chunked forward pass.
//
// Method: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核".
//   chunk_cumsum_kernel  section "Kernel 1：计算累积和"
//   state_pass_kernel    section "Kernel 2: fwd_pass_state" (the decayed chunk jump)
//   chunk_out_kernel     section "Kernel 3：compute_out"   (the decayed chunk output)
//
// All products run on MFMA: bf16 operands with fp32 accumulation for bf16 inputs,
// fp32 operands for fp32 inputs.  Decays use base-2 exponentials of the
// log2(e)-scaled cumsum (same page, section "Kernel 1").
#include <type_traits>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ===========================================================================
// Stage 1: chunk-local cumsum of A*dt, times log2(e), transposed to [b, H, Lp].
// One workgroup per (chunk, block of 4 heads, batch), one wave per head.  The
// [Q x 4] dt tile is read row by row (heads contiguous) into LDS, then each wave
// scans its head's Q tokens: every lane sums Q/64 consecutive tokens, a 64-lane
// scan on DPP lane moves adds the lane prefixes, and the results are written
// token-contiguous.  Padded tokens (last chunk) get dt = 0 and repeat the last
// valid cumsum value exactly, so G2 at a chunk's last position is the value at its
// last valid token.  With wT the same pass also writes each token's state-pass weight
// w_t = dt_t exp2(G_last - G_t) (its decay to the end of its chunk), which the
// forward's state pass then reads instead of forming it per state tile.
// ===========================================================================
template <typename T, int Q, bool WOUT>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(const T *__restrict__ dt,
                                                           const float *__restrict__ A,
                                                           float *__restrict__ G2,
                                                           float *__restrict__ dtT,
                                                           float *__restrict__ wT, int L, int H,
                                                           int Lp)
{
    constexpr int HB = 4, PER = Q / 64;
    __shared__ float tile[Q][HB + 1];
    const int c = blockIdx.x, hb = blockIdx.y * HB, b = blockIdx.z;
    const int nh = min(HB, H - hb);
    const int t0 = c * Q;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // every load is issued before the first is used (positions clamped into the
    // problem, values outside it zeroed afterwards): a load under a branch would be
    // waited for before the next one is issued
    constexpr int NLD = Q * HB / 256;   // dt elements per thread
    const float a = A[hb + min(wave, nh - 1)];
    float v[NLD];
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
        const int idx = tid + 256 * r, t = idx / HB, hh = idx % HB;
        v[r] = (float)dt[((int64_t)b * L + min(t0 + t, L - 1)) * H + hb + min(hh, nh - 1)];
    }
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
        const int idx = tid + 256 * r, t = idx / HB, hh = idx % HB;
        tile[t][hh] = (hh < nh && t0 + t < L) ? v[r] : 0.0f;
    }
    asm volatile("" ::"v"(a));   // keeps A's load ahead of the barrier, in flight with dt's
    __syncthreads();
    if (wave >= nh) return;

    const int hh = wave;
    float part[PER], run = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        run += a * tile[lane * PER + j][hh];
        part[j] = run;
    }
    const float excl = wave_shift_up1(wave_inclusive_sum(run));
    const int last = min(L - t0, Q) - 1;
    float tail = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (j == last % PER) tail = (excl + part[j]) * kLog2e;
    tail = wave_read(tail, last / PER);
    // value at the chunk's last position (the last valid token's on a ragged chunk)
    float glast = wave_read((excl + part[PER - 1]) * kLog2e, 63);
    if (last < Q - 1) glast = tail;
    const int64_t base = ((int64_t)b * H + hb + hh) * Lp + t0 + lane * PER;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int t = lane * PER + j;
        const float gt = (t <= last) ? (excl + part[j]) * kLog2e : tail;
        const float d = tile[t][hh];
        G2[base + j] = gt;
        dtT[base + j] = d;
        if constexpr (WOUT) wT[base + j] = d * fast_exp2(glast - gt);
    }
}

// ===========================================================================
// Stage 2, fp32 inputs: chunk-start states.  One workgroup per (N tile of 64,
// batch*head, group of K consecutive chunks), four waves, each owning a 32x32
// (P x N) quarter of the fp32 state in MFMA accumulators.  Serially over the
// group's chunks: stage X_c^T and W_c^T = (w * B_c)^T into LDS (token-contiguous
// rows, so MFMA fragments are 8 consecutive tokens), store the chunk-start
// state, scale it by exp2(G_last) and accumulate X^T W.
// Groups (the jump is linear, so a run of chunks can start from zero and be
// corrected later): group g starts from h0 if g == 0 and from 0 otherwise; with
// Ug it stores its final local state U_g there and, from one thread, the decays
// beta_c (group start to chunk c) and gamma_g (the whole group) for the group
// scan; without Ug (one group) the final state goes to hT.
// ===========================================================================
// WPRE: wt holds the stage-1 weights wT; otherwise it holds dtT and the kernel forms the
// weights from it and the cumsum
template <typename T, int Q, bool WPRE>
__global__ __launch_bounds__(256) void state_pass_kernel(
    const T *__restrict__ x, const T *__restrict__ Bm, const float *__restrict__ G2,
    const float *__restrict__ wt, const float *__restrict__ h0, T *__restrict__ S,
    float *__restrict__ hT, float *__restrict__ Ug, float *__restrict__ gam,
    float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng)
{
    constexpr int P = 64, NT = 64;
    constexpr int PITCH = Q + 16 / (int)sizeof(T);  // row pitch in elements; rows 16 B aligned
    __shared__ __attribute__((aligned(16))) T XT[P * PITCH];
    __shared__ __attribute__((aligned(16))) T WT[NT * PITCH];
    __shared__ float wsh[Q];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ph = wave & 1, nh = wave >> 1;
    const int n_base = blockIdx.x * NT;
    const int bh = blockIdx.y, b = bh / H, h = bh % H, g = h / (H / G);
    const int col = n_base + nh * 32 + (lane & 31);
    const int grp = blockIdx.z, c0 = grp * K, c1 = min(c0 + K, nc);

    const int64_t st_off = (int64_t)bh * P * N;
    f32x16 acc = zero_acc();
    if (h0 != nullptr && grp == 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = h0[st_off + (int64_t)(ph * 32 + acc_row(v, lane)) * N + col];
    }

    const float *Gh = G2 + (int64_t)bh * Lp;
    const float *wh = wt + (int64_t)bh * Lp;
    const int64_t xrow = (int64_t)H * P;   // x token stride
    const int64_t brow = (int64_t)G * N;   // B token stride
    // the chunk-end cumsum value of chunk c0 + lane (clamped to the group), for the decay
    // products written at the end; a per-lane load issued now, without a branch around it
    float gend0;
    {
        int gi = min(c0 + lane, c1 - 1) * Q + Q - 1;
        asm volatile("" : "+v"(gi));
        gend0 = Gh[gi];
    }

    // Rows past L are clamped to row L-1 (no load under a per-lane branch, which is waited
    // for before the next is issued): their weight w is 0, so their W rows vanish.
    for (int c = c0; c < c1; ++c) {
        const int t0 = c * Q;
        const float glast = Gh[t0 + Q - 1];
        // the state-pass weight of token t: dt times the decay to the end of its chunk
        for (int t = tid; t < Q; t += 256)
            wsh[t] = WPRE ? wh[t0 + t] : wh[t0 + t] * fast_exp2(glast - Gh[t0 + t]);
        __syncthreads();

        // X_c [Q x 64] -> XT[p][t]
        {
            typename Elem<T>::frag f[Q / 32];
#pragma unroll
            for (int r = 0; r < Q / 32; ++r) {
                const int idx = tid + 256 * r, t = idx >> 3, oct = idx & 7;
                f[r] = load_frag<T>(x + ((int64_t)b * L + min(t0 + t, L - 1)) * xrow + (int64_t)h * P + oct * 8);
            }
#pragma unroll
            for (int r = 0; r < Q / 32; ++r) {
                const int idx = tid + 256 * r, t = idx >> 3, oct = idx & 7;
#pragma unroll
                for (int e = 0; e < 8; ++e) XT[(oct * 8 + e) * PITCH + t] = f[r][e];
            }
        }
        // W_c = round(w * B_c) [Q x 64] -> WT[n][t]
        {
            typename Elem<T>::frag f[Q / 32];
#pragma unroll
            for (int r = 0; r < Q / 32; ++r) {
                const int idx = tid + 256 * r, t = idx >> 3, oct = idx & 7;
                f[r] = load_frag<T>(Bm + ((int64_t)b * L + min(t0 + t, L - 1)) * brow + (int64_t)g * N + n_base + oct * 8);
            }
#pragma unroll
            for (int r = 0; r < Q / 32; ++r) {
                const int idx = tid + 256 * r, t = idx >> 3, oct = idx & 7;
                const float w = wsh[t];
#pragma unroll
                for (int e = 0; e < 8; ++e) WT[(oct * 8 + e) * PITCH + t] = Elem<T>::from_f32((float)f[r][e] * w);
            }
        }
        __syncthreads();

        // chunk-start state, then h <- exp2(G_last) h + X^T W
        T *Sc = S + ((int64_t)bh * nc + c) * P * N;
#pragma unroll
        for (int v = 0; v < 16; ++v) Sc[(int64_t)(ph * 32 + acc_row(v, lane)) * N + col] = Elem<T>::from_f32(acc[v]);
        const float alpha = fast_exp2(glast);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] *= alpha;

        const T *arow = XT + (ph * 32 + (lane & 31)) * PITCH + 8 * (lane >> 5);
        const T *brw = WT + (nh * 32 + (lane & 31)) * PITCH + 8 * (lane >> 5);
#pragma unroll 4
        for (int ks = 0; ks < Q / 16; ++ks) mma(acc, load_frag<T>(arow + ks * 16), load_frag<T>(brw + ks * 16));
        __syncthreads();
    }

    // decay products of the group (beta_c before each chunk, gamma for the group): lane k of
    // wave 0 holds chunk c0 + k0 + k's decay and the running product is taken in chunk order,
    // as a sequential loop over the chunks would
    if (Ug != nullptr && wave == 0 && blockIdx.x == 0) {
        float run = 1.0f;
        auto products = [&](float gend, int k0) {   // chunks c0 + k0 .. c0 + k0 + 63
            const float e = fast_exp2(gend);
            const int cnt = min(64, c1 - c0 - k0);
            float mine = 0.0f;
            for (int k = 0; k < cnt; ++k) {
                if (lane == k) mine = run;
                run *= __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), k));
            }
            if (lane < cnt) beta[(int64_t)bh * nc + c0 + k0 + lane] = mine;
        };
        products(gend0, 0);
        for (int k0 = 64; k0 < c1 - c0; k0 += 64) {   // groups of more than 64 chunks
            int gi = min(c0 + k0 + lane, c1 - 1) * Q + Q - 1;
            asm volatile("" : "+v"(gi));
            products(Gh[gi], k0);
        }
        if (lane == 0) gam[(int64_t)bh * ng + grp] = run;
    }
    float *dst = (Ug != nullptr) ? Ug + ((int64_t)bh * ng + grp) * P * N : (hT ? hT + st_off : nullptr);
    if (dst != nullptr) {
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[(int64_t)(ph * 32 + acc_row(v, lane)) * N + col] = acc[v];
    }
}

// ===========================================================================
// Stage 3, fp32 inputs: chunk output.  One workgroup per (chunk, batch*head) with Q/64 waves.
// The chunk has Q/32 row tiles of 32 tokens; wave w takes tiles w and Q/32-1-w so
// every wave does the same number of causal tile pairs (at Q = 64 with a small grid,
// two waves take one tile each, so the chunk's two tiles run side by side).  The output is built
// transposed, Y^T [P x 32 tokens], so that
//   * C S^T:   A = S rows (p, n), B = C rows (i, n) -- both n-contiguous in HBM;
//   * C B^T:   computed as (B C^T) with A = B rows (j, n), B = C rows (i, n); its
//              accumulator holds column i and rows j, which is exactly the lane
//              layout the next product wants for its B operand;
//   * M (dt X): A = (dt X)^T from LDS (p rows, token-contiguous), B = M straight
//              from registers after the decay, causal select and rounding.
// CORR: S holds chunk-start states relative to the start of the chunk's state-pass
// group, and the state used is S + beta_c H_g (H_g the true state at the group
// start, fp32, from the group scan; beta is 0 in group 0, which adds nothing).
// ===========================================================================
// NTH: threads per workgroup, Q/64 waves taking two row tiles each (NTH = Q) or, for a small
// grid at Q = 64, two waves taking one each (NTH = 128: the chunk's two tiles side by side)
template <typename T, int Q, bool CORR, int NTH>
__global__ __launch_bounds__(NTH) void chunk_out_kernel(
    const T *__restrict__ x, const T *__restrict__ Bm, const T *__restrict__ Cm,
    const float *__restrict__ G2, const float *__restrict__ dtT, const T *__restrict__ S,
    const float *__restrict__ D, T *__restrict__ y, const float *__restrict__ Hg,
    const float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng)
{
    constexpr int P = 64, NI = Q / 32, NTHR = NTH;
    constexpr int NPASS = 2 * Q / NTHR;   // row tiles per wave
    static_assert(NPASS == 1 || NPASS == 2, "one or two row tiles per wave");
    constexpr int PITCH = Q + 16 / (int)sizeof(T);
    __shared__ __attribute__((aligned(16))) T XdT[P * PITCH];
    __shared__ float Gs[Q];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, g = h / (H / G);
    const int t0 = c * Q;
    const int64_t xrow = (int64_t)H * P, crow = (int64_t)G * N;
    const float *Gh = G2 + (int64_t)bh * Lp + t0;
    const float *dh = dtT + (int64_t)bh * Lp + t0;

    // Q <= 128: rows past L are clamped to row L-1 instead of zeroed, so no load sits
    // under a per-lane branch (such a load is waited for before the next is issued):
    // their dt is 0, so their (dt x) rows vanish, and their outputs are never stored.
    // Q = 256 keeps the zero-filled loads, which measured faster there.
    for (int t = tid; t < Q; t += NTHR) Gs[t] = Gh[t];
    const int last = L - 1 - t0;   // last row of the chunk inside the problem
    auto stage_x = [&](int idx, bool clamp) {
        const int t = idx >> 3, oct = idx & 7;
        const T *xr = x + ((int64_t)b * L + t0 + min(t, last)) * xrow + (int64_t)h * P + oct * 8;
        const typename Elem<T>::frag f = (clamp || t <= last) ? load_frag<T>(xr) : zero_frag<T>();
        const float d = dh[t];
#pragma unroll
        for (int e = 0; e < 8; ++e) XdT[(oct * 8 + e) * PITCH + t] = Elem<T>::from_f32((float)f[e] * d);
    };
    if constexpr (Q <= 128) {
#pragma unroll
        for (int r = 0; r < Q * 8 / NTHR; ++r) stage_x(tid + NTHR * r, true);
    } else {
        for (int idx = tid; idx < Q * 8; idx += NTHR) stage_x(idx, false);
    }
    __syncthreads();

    const float Dh = D[h];
    const T *Cc = Cm + ((int64_t)b * L + t0) * crow + (int64_t)g * N;
    const T *Bc = Bm + ((int64_t)b * L + t0) * crow + (int64_t)g * N;
    const T *Sc = S + ((int64_t)bh * nc + c) * P * N;
    const int kq = 8 * (lane >> 5);
    const int cgrp = CORR ? c / K : 0;
    const float bc = (CORR && cgrp > 0) ? beta[(int64_t)bh * nc + c] : 0.0f;
    const float *Hc = CORR ? Hg + ((int64_t)bh * ng + cgrp) * P * N : nullptr;
    // state fragment of row r, columns k + kq .. k + kq + 7 (corrected when grouped)
    auto state_frag = [&](int r, int k) {
        typename Elem<T>::frag f = load_frag<T>(Sc + (int64_t)r * N + kq + k);
        if constexpr (CORR) {
            const f32x8 hv = load_frag<float>(Hc + (int64_t)r * N + kq + k);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = Elem<T>::from_f32((float)f[e] + bc * hv[e]);
        }
        return f;
    };

    for (int pass = 0; pass < NPASS; ++pass) {
        const int I = pass == 0 ? wave : NI - 1 - wave;
        const int i_loc = I * 32 + (lane & 31);
        const bool ivalid = t0 + i_loc < L;
        const T *crow_i = Cc + (int64_t)min(i_loc, last) * crow + kq;

        // inter-chunk term: Y^T = S C^T, then scale column i by exp2(G_i)
        // Q <= 128: N is a multiple of 64, and the fragments of four 16-wide steps
        // are loaded before their products so that their latencies overlap; at
        // Q = 256 the registers this takes cost more occupancy than the overlap gains
        f32x16 acc0 = zero_acc(), acc1 = zero_acc();
        if constexpr (Q <= 128) {
            for (int k0 = 0; k0 < N; k0 += 64) {
                typename Elem<T>::frag cf[4], s0[4], s1[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    cf[u] = load_frag<T>(crow_i + k0 + 16 * u);
                    s0[u] = state_frag(lane & 31, k0 + 16 * u);
                    s1[u] = state_frag(32 + (lane & 31), k0 + 16 * u);
                }
                __builtin_amdgcn_sched_barrier(0);   // keeps the loads ahead of the products
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    mma(acc0, s0[u], cf[u]);
                    mma(acc1, s1[u], cf[u]);
                }
            }
        } else {
            for (int k = 0; k < N; k += 16) {
                const typename Elem<T>::frag cf = ivalid ? load_frag<T>(crow_i + k) : zero_frag<T>();
                mma(acc0, state_frag(lane & 31, k), cf);
                mma(acc1, state_frag(32 + (lane & 31), k), cf);
            }
        }
        const float gi = Gs[i_loc];
        const float si = fast_exp2(gi);
#pragma unroll
        for (int v = 0; v < 16; ++v) { acc0[v] *= si; acc1[v] *= si; }

        // intra-chunk term over causal tiles J <= I
        for (int J = 0; J <= I; ++J) {
            const int j_loc = J * 32 + (lane & 31);
            const T *brow_j = Bc + (int64_t)min(j_loc, last) * crow + kq;
            f32x16 cb = zero_acc();
            if constexpr (Q <= 128) {
                for (int k0 = 0; k0 < N; k0 += 64) {
                    typename Elem<T>::frag bf[4], cf[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        bf[u] = load_frag<T>(brow_j + k0 + 16 * u);
                        cf[u] = load_frag<T>(crow_i + k0 + 16 * u);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < 4; ++u) mma(cb, bf[u], cf[u]);
                }
            } else {
                const bool jvalid = t0 + j_loc < L;
                for (int k = 0; k < N; k += 16) {
                    const typename Elem<T>::frag bf = jvalid ? load_frag<T>(brow_j + k) : zero_frag<T>();
                    const typename Elem<T>::frag cf = ivalid ? load_frag<T>(crow_i + k) : zero_frag<T>();
                    mma(cb, bf, cf);
                }
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                typename Elem<T>::frag m;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int v = 8 * s + e;
                    const int jj = J * 32 + acc_row(v, lane);
                    const float val = (i_loc >= jj) ? cb[v] * fast_exp2(gi - Gs[jj]) : 0.0f;
                    m[e] = Elem<T>::from_f32(val);
                }
                // (dt x)^T fragment with the same token order as m: 4 tokens at
                // J*32 + 16 s + 4*(lane/32), then 4 more 8 tokens further on.
                const int jb = J * 32 + 16 * s + 4 * (lane >> 5);
#pragma unroll
                for (int ph = 0; ph < 2; ++ph) {
                    const T *ar = XdT + (ph * 32 + (lane & 31)) * PITCH + jb;
                    const typename Elem<T>::half lo = *reinterpret_cast<const typename Elem<T>::half *>(ar);
                    const typename Elem<T>::half hi = *reinterpret_cast<const typename Elem<T>::half *>(ar + 8);
                    typename Elem<T>::frag a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[4 + e] = hi[e]; }
                    if (ph == 0) mma(acc0, a, m); else mma(acc1, a, m);
                }
            }
        }

        // y_i = Y_i + D x_i
        if (ivalid) {
            const int64_t yo = ((int64_t)b * L + t0 + i_loc) * xrow + (int64_t)h * P;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int p = acc_row(v, lane);
                y[yo + p] = Elem<T>::from_f32(acc0[v] + Dh * (float)x[yo + p]);
                y[yo + 32 + p] = Elem<T>::from_f32(acc1[v] + Dh * (float)x[yo + 32 + p]);
            }
        }
    }
}

// ===========================================================================
// Launchers
// ===========================================================================
template <typename T, int Q>
static hipError_t cumsum_tq(const Shape &s, const void *dt, const float *A, float *G2, float *dtT,
                            float *wT, hipStream_t st)
{
    dim3 grid((unsigned)s.nc, (unsigned)((s.H + 3) / 4), (unsigned)s.b);
    if (wT != nullptr)
        hipLaunchKernelGGL((chunk_cumsum_kernel<T, Q, true>), grid, dim3(256), 0, st, (const T *)dt,
                           A, G2, dtT, wT, (int)s.L, (int)s.H, (int)s.Lp);
    else
        hipLaunchKernelGGL((chunk_cumsum_kernel<T, Q, false>), grid, dim3(256), 0, st, (const T *)dt,
                           A, G2, dtT, wT, (int)s.L, (int)s.H, (int)s.Lp);
    return hipGetLastError();
}

template <typename T>
static hipError_t cumsum_t(const Shape &s, const void *dt, const float *A, float *G2, float *dtT,
                           float *wT, hipStream_t st)
{
    switch (s.Q) {
    case 64: return cumsum_tq<T, 64>(s, dt, A, G2, dtT, wT, st);
    case 128: return cumsum_tq<T, 128>(s, dt, A, G2, dtT, wT, st);
    default: return cumsum_tq<T, 256>(s, dt, A, G2, dtT, wT, st);
    }
}

hipError_t launch_chunk_cumsum(const Shape &s, const void *dt, const float *A, float *G2,
                               float *dtT, float *wT, hipStream_t st)
{
    return s.bf16 ? cumsum_t<bf16>(s, dt, A, G2, dtT, wT, st)
                  : cumsum_t<float>(s, dt, A, G2, dtT, wT, st);
}

template <typename T, int Q>
static hipError_t state_pass_tq(const Shape &s, bool wpre, const void *x, const void *B,
                                const float *G2, const float *wt, const float *h0, void *S,
                                float *hT, float *Ug, float *gam, float *beta, int K, int ng,
                                hipStream_t st)
{
    dim3 grid((unsigned)(s.N / 64), (unsigned)(s.b * s.H), (unsigned)ng);
    auto launch = [&](auto wc) {
        hipLaunchKernelGGL((state_pass_kernel<T, Q, decltype(wc)::value>), grid, dim3(256), 0, st,
                           (const T *)x, (const T *)B, G2, wt, h0, (T *)S, hT, Ug, gam, beta,
                           (int)s.L, (int)s.H, (int)s.G, (int)s.N, (int)s.nc, (int)s.Lp, K, ng);
    };
    if (wpre)
        launch(std::true_type{});
    else
        launch(std::false_type{});
    return hipGetLastError();
}

// wt: the stage-1 weights wT when wpre, else dtT (the kernel forms the weights)
template <typename T>
static hipError_t state_pass_t(const Shape &s, bool wpre, const void *x, const void *B,
                               const float *G2, const float *wt, const float *h0, void *S,
                               float *hT, float *Ug, float *gam, float *beta, int K, int ng,
                               hipStream_t st)
{
    switch (s.Q) {
    case 64: return state_pass_tq<T, 64>(s, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    case 128: return state_pass_tq<T, 128>(s, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    default: return state_pass_tq<T, 256>(s, wpre, x, B, G2, wt, h0, S, hT, Ug, gam, beta, K, ng, st);
    }
}

hipError_t launch_state_pass(const Shape &s, const void *x, const void *B, const float *G2,
                             const float *dtT, const float *h0, void *S, float *hT,
                             hipStream_t st)
{
    return s.bf16 ? launch_state_pass_bf16(s, x, B, G2, dtT, h0, S, hT, st)
                  : state_pass_t<float>(s, false, x, B, G2, dtT, h0, S, hT, nullptr, nullptr,
                                        nullptr, (int)s.nc, 1, st);
}

hipError_t launch_state_pass_f32_grouped(const Shape &s, const void *x, const void *B,
                                         const float *G2, const float *wT, const float *h0,
                                         void *S, float *hT, float *Ug, float *gam, float *beta,
                                         int K, int ng, hipStream_t st)
{
    return state_pass_t<float>(s, true, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
}

int chunk_out_f32_threads(const Shape &s)
{
    return (s.Q == 64 && s.nc * s.b * s.H < 1024) ? 128 : (int)s.Q;
}

template <typename T, int Q>
static hipError_t chunk_out_tq(const Shape &s, const void *x, const void *B, const void *C,
                               const float *G2, const float *dtT, const void *S, const float *D,
                               void *y, const float *Hg, const float *beta, int K, int ng,
                               hipStream_t st)
{
    dim3 grid((unsigned)s.nc, (unsigned)(s.b * s.H));
    auto launch = [&](auto nth) {
        constexpr int NTH = decltype(nth)::value;
        if (Hg != nullptr)
            hipLaunchKernelGGL((chunk_out_kernel<T, Q, true, NTH>), grid, dim3(NTH), 0, st, (const T *)x,
                               (const T *)B, (const T *)C, G2, dtT, (const T *)S, D, (T *)y, Hg, beta,
                               (int)s.L, (int)s.H, (int)s.G, (int)s.N, (int)s.nc, (int)s.Lp, K, ng);
        else
            hipLaunchKernelGGL((chunk_out_kernel<T, Q, false, NTH>), grid, dim3(NTH), 0, st, (const T *)x,
                               (const T *)B, (const T *)C, G2, dtT, (const T *)S, D, (T *)y,
                               (const float *)nullptr, (const float *)nullptr, (int)s.L, (int)s.H,
                               (int)s.G, (int)s.N, (int)s.nc, (int)s.Lp, (int)s.nc, 1);
    };
    if constexpr (Q == 64) {
        if (chunk_out_f32_threads(s) == 128) {
            launch(std::integral_constant<int, 128>{});
            return hipGetLastError();
        }
    }
    launch(std::integral_constant<int, Q>{});
    return hipGetLastError();
}

template <typename T>
static hipError_t chunk_out_t(const Shape &s, const void *x, const void *B, const void *C,
                              const float *G2, const float *dtT, const void *S, const float *D,
                              void *y, const float *Hg, const float *beta, int K, int ng,
                              hipStream_t st)
{
    switch (s.Q) {
    case 64: return chunk_out_tq<T, 64>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    case 128: return chunk_out_tq<T, 128>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    default: return chunk_out_tq<T, 256>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    }
}

hipError_t launch_chunk_out(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, hipStream_t st)
{
    if (!s.bf16)
        return chunk_out_t<float>(s, x, B, C, G2, dtT, S, D, y, nullptr, nullptr, (int)s.nc, 1, st);
    const LaunchPlan lp = plan_of(s);
    return launch_chunk_out_bf16(s, x, B, C, G2, dtT, S, D, y, nullptr, nullptr, nullptr,
                                 (int)s.nc, 1, lp.co_head_blocked ? lp.co_heads_per_block : 0, st);
}

hipError_t launch_chunk_out_corrected(const Shape &s, const LaunchPlan &lp, const void *x,
                                      const void *B, const void *C, const float *G2,
                                      const float *dtT, const void *S, const float *D, void *y,
                                      const float *Hg, const void *Hb, const float *beta,
                                      hipStream_t st)
{
    const int K = lp.sp_group_chunks, ng = lp.sp_groups;
    const int hb = lp.co_head_blocked ? lp.co_heads_per_block : 0;
    if (ng <= 1) {
        Hg = nullptr;
        Hb = nullptr;
        beta = nullptr;
    }
    if (!s.bf16)
        return ng <= 1 ? chunk_out_t<float>(s, x, B, C, G2, dtT, S, D, y, nullptr, nullptr,
                                            (int)s.nc, 1, st)
                       : chunk_out_t<float>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    return ng <= 1 ? launch_chunk_out_bf16(s, x, B, C, G2, dtT, S, D, y, nullptr, nullptr, nullptr,
                                           (int)s.nc, 1, hb, st)
                   : launch_chunk_out_bf16(s, x, B, C, G2, dtT, S, D, y, Hg, Hb, beta, K, ng, hb,
                                           st);
}

}  // namespace ssd
