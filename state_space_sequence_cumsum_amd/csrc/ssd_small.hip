// ssd_small.hip -- the whole forward pass in one launch, for fp32 problems of a few chunks.
//
// Method: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核": the chunked form
// of section "Mamba-2 架构", with the chunk-local cumsum of section "Kernel 1：计算累积和",
// the decayed jump of section "Kernel 2: fwd_pass_state" and the decayed chunk output of
// section "Kernel 3：compute_out".
//
// With a few chunks per sequence the four launches of the general path (cumsum, state
// pass, group scan, chunk output) and their memory round trips take longer than the
// arithmetic.  Here one workgroup per (batch, head, chunk c) does all of it: it walks the
// jump over chunks 0 .. c-1 itself (every workgroup repeats the state work of the chunks
// before its own, which the planner bounds by allowing this kernel for short chains
// only), keeps the chunk-start state in LDS and computes chunk c's output from it.  Only
// y, the final state (from the last chunk's workgroup) and chunk c's cumsum and dt (the
// stage-1 values the forward leaves in its workspace) go to memory.  The arithmetic of
// every step is the general path's: the same cumsum and weights bit for bit, the same
// products on fp32 MFMA (v_mfma_f32_32x32x2f32), the state stored in fp32.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// Chunks of 64 tokens, headdim 64, dstate 64 * NT; 256 threads (four waves).
//   jump:   wave w keeps h[p][n] (fp32 MFMA accumulators, row p, column n) for the 32 rows
//           p of half w % 2 and, in each 64-column tile of n, the 32 columns of half w / 2;
//   output: wave w computes Y^T[p][i] for the rows p of half w % 2 and the 32 tokens i of
//           row tile I = w / 2.
template <int NT>
__global__ __launch_bounds__(256) void forward_small_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const float *__restrict__ Bm, const float *__restrict__ Cm, const float *__restrict__ D,
    const float *__restrict__ h0, float *__restrict__ y, float *__restrict__ hT,
    float *__restrict__ G2, float *__restrict__ dtT, int L, int H, int G, int nc, int Lp)
{
    constexpr int Q = 64, P = 64, N = 64 * NT, XP = Q + 4, SSP = N + 4, NF = N / 16;
    __shared__ __attribute__((aligned(16))) float XT[P * XP];     // x^T [p][token]
    __shared__ __attribute__((aligned(16))) float WT[N * XP];     // (w B)^T [n][token]
    __shared__ __attribute__((aligned(16))) float Ss[P * SSP];    // chunk-start state [p][n]
    __shared__ float Gs[Q], Ds[Q], Ws[Q];   // cumsum (log2 e scaled), dt, jump weight
    __shared__ float alpha_s;               // exp2(cumsum at the chunk's end)

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x % nc, bh = blockIdx.x / nc;
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int64_t xrow = (int64_t)H * P, brow = (int64_t)G * N;
    const float *xb = x + (int64_t)b * L * xrow + (int64_t)h * P;
    const float *Bb = Bm + (int64_t)b * L * brow + (int64_t)g * N;
    const float *Cb = Cm + (int64_t)b * L * brow + (int64_t)g * N;
    const float a = A[h];
    const int ph = w & 1, nh = w >> 1;
    const int kq = 8 * (lane >> 5);

    // wave 0: chunk ck's cumsum, dt and weights into LDS, the arithmetic of the stage-1
    // kernel for 64-token chunks (one token per lane, a 64-lane shuffle scan; padded
    // tokens get dt = 0 and repeat the last valid cumsum value)
    auto cumsum = [&](int ck, bool write_out) {
        if (w != 0) return;
        const int t0 = ck * Q, t = t0 + lane;
        const float d = t < L ? dt[((int64_t)b * L + t) * H + h] : 0.0f;
        float part = a * d;
        asm volatile("" : "+v"(part));   // the rounded product, as the stage-1 kernel sums it
        float incl = part;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(incl, off, 64);
            if (lane >= off) incl += up;
        }
        float excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.0f;
        const int last = min(L - t0, Q) - 1;
        const float tail = __shfl((excl + part) * kLog2e, last, 64);
        float glast = __shfl((excl + part) * kLog2e, 63, 64);
        if (last < Q - 1) glast = tail;
        const float gt = (lane <= last) ? (excl + part) * kLog2e : tail;
        Gs[lane] = gt;
        Ds[lane] = d;
        Ws[lane] = d * fast_exp2(glast - gt);
        if (lane == 0) alpha_s = fast_exp2(glast);
        if (write_out) {
            G2[(int64_t)bh * Lp + t] = gt;
            dtT[(int64_t)bh * Lp + t] = d;
        }
    };
    // chunk ck's x^T into XT and, with `jump`, (w B)^T into WT (rows past L are clamped to
    // row L-1; their weight is 0 and their outputs are not stored)
    const int st = tid >> 2, sq = tid & 3;   // staging: token, quarter of the row
    auto stage = [&](int ck, bool jump) {
        const int64_t tr = min(ck * Q + st, L - 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int p0 = sq * 16 + 4 * r;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(xb + tr * xrow + p0);
#pragma unroll
            for (int e = 0; e < 4; ++e) XT[(p0 + e) * XP + st] = v[e];
        }
        if (jump) {
            const float wt = Ws[st];
#pragma unroll
            for (int r = 0; r < 4 * NT; ++r) {
                const int n0 = sq * 16 * NT + 4 * r;
                const f32x4 v = *reinterpret_cast<const f32x4 *>(Bb + tr * brow + n0);
#pragma unroll
                for (int e = 0; e < 4; ++e) WT[(n0 + e) * XP + st] = wt * v[e];
            }
        }
    };

    // the state, zero or h0
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero_acc();
    if (h0 != nullptr) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[t][v] = h0[((int64_t)bh * P + ph * 32 + acc_row(v, lane)) * N + 64 * t + 32 * nh + (lane & 31)];
    }
    // h <- exp2(G_last) h + X^T (w B) over the staged chunk
    auto jump = [&]() {
        const float al = alpha_s;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[t][v] *= al;
        const float *arow = XT + (ph * 32 + (lane & 31)) * XP + kq;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float *brw = WT + (64 * t + 32 * nh + (lane & 31)) * XP + kq;
#pragma unroll
            for (int ks = 0; ks < Q / 16; ++ks)
                mma(acc[t], load_frag<float>(arow + 16 * ks), load_frag<float>(brw + 16 * ks));
        }
    };

    // the chunks before this one
    for (int ck = 0; ck < c; ++ck) {
        cumsum(ck, false);
        __syncthreads();
        stage(ck, true);
        __syncthreads();
        jump();
        __syncthreads();
    }

    // this chunk: its start state to LDS; the last chunk's workgroup also takes the jump
    // over it for the final state
    const bool fin = (c == nc - 1) && hT != nullptr;
    cumsum(c, true);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            Ss[(ph * 32 + acc_row(v, lane)) * SSP + 64 * t + 32 * nh + (lane & 31)] = acc[t][v];
    __syncthreads();
    stage(c, fin);
    __syncthreads();
    if (fin) {
        jump();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                hT[((int64_t)bh * P + ph * 32 + acc_row(v, lane)) * N + 64 * t + 32 * nh + (lane & 31)] = acc[t][v];
    }

    // chunk output: Y^T = exp2(G_i) S C^T + (dt x)^T M, M[j, i] = (i >= j) C_i.B_j exp2(G_i - G_j)
    const int I = w >> 1, i_loc = I * 32 + (lane & 31);
    const int t0 = c * Q, last = min(L - t0, Q) - 1;
    f32x8 cf[NF];   // C row i_loc (clamped), all N
#pragma unroll
    for (int f = 0; f < NF; ++f)
        cf[f] = load_frag<float>(Cb + (int64_t)(t0 + min(i_loc, last)) * brow + 16 * f + kq);
    f32x16 ya = zero_acc();
    const float *srow = Ss + (ph * 32 + (lane & 31)) * SSP + kq;
#pragma unroll
    for (int f = 0; f < NF; ++f) mma(ya, load_frag<float>(srow + 16 * f), cf[f]);
    const float gi = Gs[i_loc];
    const float si = fast_exp2(gi);
#pragma unroll
    for (int v = 0; v < 16; ++v) ya[v] *= si;
    for (int J = 0; J <= I; ++J) {
        // C B^T tile (rows j of tile J, column i) on MFMA: A = B rows, B = C rows
        f32x16 cb = zero_acc();
        const float *brw = Bb + (int64_t)(t0 + min(J * 32 + (lane & 31), last)) * brow + kq;
#pragma unroll
        for (int f = 0; f < NF; ++f) mma(cb, load_frag<float>(brw + 16 * f), cf[f]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            f32x8 m;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jj = J * 32 + acc_row(8 * s + e, lane);
                const float val = cb[8 * s + e] * fast_exp2(gi - Gs[jj]) * Ds[jj];
                m[e] = (i_loc >= jj) ? val : 0.0f;
            }
            // x^T fragment in m's token order: 4 tokens at J*32 + 16 s + 4 (lane / 32), then
            // 4 more 8 tokens further on
            const float *ar = XT + (ph * 32 + (lane & 31)) * XP + J * 32 + 16 * s + 4 * (lane >> 5);
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(ar);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(ar + 8);
            f32x8 xa;
#pragma unroll
            for (int e = 0; e < 4; ++e) { xa[e] = lo[e]; xa[4 + e] = hi[e]; }
            mma(ya, xa, m);
        }
    }
    // y_i = Y_i + D x_i
    if (i_loc <= last) {
        const float Dh = D[h];
        float *yr = y + ((int64_t)b * L + t0 + i_loc) * xrow + (int64_t)h * P;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int p = ph * 32 + acc_row(v, lane);
            yr[p] = ya[v] + Dh * XT[p * XP + i_loc];
        }
    }
}

bool forward_small_eligible(const Shape &s)
{
    return !s.bf16 && s.Q == 64 && s.P == 64 && (s.N == 64 || s.N == 128) && s.nc <= kSmallMaxChunks &&
           s.b * s.H * s.nc * 256 < (int64_t(1) << 31);
}

hipError_t launch_forward_small(const Shape &s, const void *x, const void *dt, const float *A,
                                const void *B, const void *C, const float *D, const float *h0,
                                void *y, float *hT, float *G2, float *dtT, hipStream_t st)
{
    const dim3 grid((unsigned)(s.b * s.H * s.nc)), block(256);
    if (s.N == 64)
        hipLaunchKernelGGL((forward_small_f32_kernel<1>), grid, block, 0, st, (const float *)x,
                           (const float *)dt, A, (const float *)B, (const float *)C, D, h0,
                           (float *)y, hT, G2, dtT, (int)s.L, (int)s.H, (int)s.G, (int)s.nc,
                           (int)s.Lp);
    else
        hipLaunchKernelGGL((forward_small_f32_kernel<2>), grid, block, 0, st, (const float *)x,
                           (const float *)dt, A, (const float *)B, (const float *)C, D, h0,
                           (float *)y, hT, G2, dtT, (int)s.L, (int)s.H, (int)s.G, (int)s.nc,
                           (int)s.Lp);
    return hipGetLastError();
}

}  // namespace ssd
