// ssd_launch.h -- internal interface between the C ABI (ssd_api.cpp) and the
// kernel launchers (ssd_kernels.hip).  Shapes are already validated here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct Shape {
    int64_t b, L, H, G, P, N, Q, nc, Lp;
    bool bf16;
};

hipError_t launch_chunk_cumsum(const Shape &s, const void *dt, const float *A, float *G2,
                               float *dtT, float *wT, hipStream_t st);

hipError_t launch_state_pass(const Shape &s, const void *x, const void *B, const float *G2,
                             const float *wT, const float *h0, void *S, float *hT,
                             hipStream_t st);

hipError_t launch_chunk_out(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, hipStream_t st);

// bf16 kernels (ssd_bf16.hip)
hipError_t launch_state_pass_bf16(const Shape &s, const void *x, const void *B, const float *G2,
                                  const float *wT, const float *h0, void *S, float *hT,
                                  hipStream_t st);
hipError_t launch_chunk_out_bf16(const Shape &s, const void *x, const void *B, const void *C,
                                 const float *G2, const float *dtT, const void *S, const float *D,
                                 void *y, hipStream_t st);

}  // namespace ssd
