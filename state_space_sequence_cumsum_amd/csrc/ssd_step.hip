// ssd_step.hip -- the single-token decode step: one step of the recurrence of
// section "Mamba-2 架构" (dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核")
// per (batch, head), applied in place to the fp32 state that the forward pass
// returns as its final state (section "Kernel 2: fwd_pass_state": the final state
// is the next call's initial state at inference time).
//
//     h    <- exp(A dt) h + dt x (outer) B
//     y[p]  = sum_n h[p, n] C[n] + D x[p]
//
// The step reads and writes the whole P x N fp32 state once and does 4 flops per
// state element, so it is bound by HBM bandwidth (or by launch latency at small
// batch).  One wave owns RW consecutive state rows of one (batch, head): it keeps
// the head's B and C rows in registers, streams its rows with 16-, 8- or 4-byte
// loads (consecutive lanes on consecutive columns), and reduces the row dot
// products across the wave.
#include <hip/hip_runtime.h>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kStepRows = 4;        // state rows per wave
constexpr int kStepWaves = 4;       // waves per workgroup

template <int V> struct VecF;
template <> struct VecF<1> { typedef float t; };
template <> struct VecF<2> { typedef float t __attribute__((ext_vector_type(2))); };
template <> struct VecF<4> { typedef float t __attribute__((ext_vector_type(4))); };

// V consecutive input elements as fp32.
template <typename T, int V> __device__ __forceinline__ void load_in(const T *p, float *o);

template <> __device__ __forceinline__ void load_in<float, 1>(const float *p, float *o) { o[0] = *p; }
template <> __device__ __forceinline__ void load_in<float, 2>(const float *p, float *o)
{
    const VecF<2>::t v = *reinterpret_cast<const VecF<2>::t *>(p);
    o[0] = v[0]; o[1] = v[1];
}
template <> __device__ __forceinline__ void load_in<float, 4>(const float *p, float *o)
{
    const VecF<4>::t v = *reinterpret_cast<const VecF<4>::t *>(p);
    o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
}
template <> __device__ __forceinline__ void load_in<bf16, 1>(const bf16 *p, float *o) { o[0] = (float)*p; }
template <> __device__ __forceinline__ void load_in<bf16, 2>(const bf16 *p, float *o)
{
    const bf16x2_t v = *reinterpret_cast<const bf16x2_t *>(p);
    o[0] = (float)v[0]; o[1] = (float)v[1];
}
template <> __device__ __forceinline__ void load_in<bf16, 4>(const bf16 *p, float *o)
{
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}

template <int V> __device__ __forceinline__ void load_state(const float *p, float *o)
{
    load_in<float, V>(p, o);
}

template <int V> __device__ __forceinline__ void store_state(float *p, const float *v)
{
    if constexpr (V == 1) {
        *p = v[0];
    } else {
        typename VecF<V>::t t;
#pragma unroll
        for (int i = 0; i < V; ++i) t[i] = v[i];
        *reinterpret_cast<typename VecF<V>::t *>(p) = t;
    }
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Lane l of a wave holds columns n = 64 V e + V l + i (e < E, i < V) of every row,
// so N = 64 V E exactly and each load instruction covers 64 V consecutive columns.
template <typename T, int V, int E>
__global__ __launch_bounds__(64 * kStepWaves) void decode_step_kernel(
    const T *__restrict__ x, const T *__restrict__ dt, const float *__restrict__ A,
    const T *__restrict__ Bm, const T *__restrict__ Cm, const float *__restrict__ D,
    float *__restrict__ h, T *__restrict__ y, int H, int G, int P, int64_t nwaves)
{
    constexpr int N = 64 * V * E;
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * kStepWaves + (threadIdx.x >> 6);
    if (wv >= nwaves) return;   // the whole wave leaves; there are no barriers
    const int nrb = (P + kStepRows - 1) / kStepRows;
    const int64_t bh = wv / nrb;
    const int p0 = (int)(wv % nrb) * kStepRows;
    const int64_t b = bh / H;
    const int head = (int)(bh % H);
    const int grp = head / (H / G);

    const T *Bp = Bm + (b * G + grp) * N + V * lane;
    const T *Cp = Cm + (b * G + grp) * N + V * lane;
    float bv[E][V], cv[E][V];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        load_in<T, V>(Bp + 64 * V * e, bv[e]);
        load_in<T, V>(Cp + 64 * V * e, cv[e]);
    }
    float dtv;
    load_in<T, 1>(dt + bh, &dtv);
    const float decay = fast_exp2(A[head] * dtv * kLog2e);
    const float Dh = D[head];

    float hv[kStepRows][E][V];
    float xv[kStepRows];
    float *hp = h + (bh * P + p0) * N + V * lane;
#pragma unroll
    for (int r = 0; r < kStepRows; ++r) {
        if (p0 + r < P) {
            load_in<T, 1>(x + bh * P + p0 + r, &xv[r]);
#pragma unroll
            for (int e = 0; e < E; ++e) load_state<V>(hp + (int64_t)r * N + 64 * V * e, hv[r][e]);
        }
    }
#pragma unroll
    for (int r = 0; r < kStepRows; ++r) {
        if (p0 + r < P) {
            const float u = dtv * xv[r];
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const float hn = decay * hv[r][e][i] + u * bv[e][i];
                    hv[r][e][i] = hn;
                    part += hn * cv[e][i];
                }
                store_state<V>(hp + (int64_t)r * N + 64 * V * e, hv[r][e]);
            }
            const float yr = wave_sum(part) + Dh * xv[r];
            if (lane == 0) y[bh * P + p0 + r] = Elem<T>::from_f32(yr);
        }
    }
}

template <typename T, int V, int E>
hipError_t step_launch(const Shape &s, const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, float *h, void *y, hipStream_t st)
{
    const int64_t nwaves = s.b * s.H * ((s.P + kStepRows - 1) / kStepRows);
    const int64_t blocks = (nwaves + kStepWaves - 1) / kStepWaves;
    hipLaunchKernelGGL((decode_step_kernel<T, V, E>), dim3((unsigned)blocks), dim3(64 * kStepWaves),
                       0, st, (const T *)x, (const T *)dt, A, (const T *)B, (const T *)C, D, h,
                       (T *)y, (int)s.H, (int)s.G, (int)s.P, nwaves);
    return hipGetLastError();
}

template <typename T>
hipError_t step_dispatch(const Shape &s, const void *x, const void *dt, const float *A,
                         const void *B, const void *C, const float *D, float *h, void *y,
                         hipStream_t st)
{
    switch (s.N) {   // N = 64 V E with the widest vector that divides it
    case 64: return step_launch<T, 1, 1>(s, x, dt, A, B, C, D, h, y, st);
    case 128: return step_launch<T, 2, 1>(s, x, dt, A, B, C, D, h, y, st);
    case 192: return step_launch<T, 1, 3>(s, x, dt, A, B, C, D, h, y, st);
    case 256: return step_launch<T, 4, 1>(s, x, dt, A, B, C, D, h, y, st);
    case 320: return step_launch<T, 1, 5>(s, x, dt, A, B, C, D, h, y, st);
    case 384: return step_launch<T, 2, 3>(s, x, dt, A, B, C, D, h, y, st);
    case 448: return step_launch<T, 1, 7>(s, x, dt, A, B, C, D, h, y, st);
    case 512: return step_launch<T, 4, 2>(s, x, dt, A, B, C, D, h, y, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_step(const Shape &s, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D, float *h, void *y,
                              hipStream_t st)
{
    return s.bf16 ? step_dispatch<bf16>(s, x, dt, A, B, C, D, h, y, st)
                  : step_dispatch<float>(s, x, dt, A, B, C, D, h, y, st);
}

}  // namespace ssd
