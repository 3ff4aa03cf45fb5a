// ssd_noalloc.hip -- ssd_forward_noalloc: the forward pass with its intermediates in
// a static device array instead of a caller-provided workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// `scratch` is an ordinary file-scope device array: every GPU the library runs on
// holds its own copy, from the moment the code object is loaded until the process
// ends.  Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current, and only
// that pointer is handed to the kernels.
#include "../../include/ssd.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_launch.h"

namespace {

static_assert(SSD_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[SSD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The device address of `dev`'s copy of the array, looked up on the first call for
// that device (with `dev` made current for the lookup, the caller's device restored).
hipError_t scratch_of(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&] {
        int cur = -1;
        d.err = hipGetDevice(&cur);
        if (d.err != hipSuccess) return;
        if (cur != dev && (d.err = hipSetDevice(dev)) != hipSuccess) return;
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess) d.ptr = p;
        if (cur != dev) {
            const hipError_t e = hipSetDevice(cur);
            if (d.err == hipSuccess) d.err = e;
        }
    });
    *out = d.ptr;
    return d.err;
}

}  // namespace

extern "C" ssd_status ssd_forward_noalloc(const ssd_problem *problem, const void *x,
                                          const void *dt, const float *A, const void *B,
                                          const void *C, const float *D, const float *h0,
                                          void *y, float *hT, void *stream)
{
    const ssd_status st = ssd_validate(problem);
    if (st != SSD_OK) return st;
    if (ssd_workspace_bytes(problem) > (size_t)SSD_SCRATCH_BYTES) return SSD_ERR_SCRATCH;
    // the GPU the work runs on is the stream's (the current device for the null stream)
    int dev = -1;
    hipError_t e = hipStreamGetDevice((hipStream_t)stream, &dev);
    void *ws = nullptr;
    if (e == hipSuccess) e = scratch_of(dev, &ws);
    if (e != hipSuccess) return (ssd_status)ssd::hip_status(e);
    return ssd_forward(problem, x, dt, A, B, C, D, h0, y, hT, ws, (size_t)SSD_SCRATCH_BYTES,
                       stream);
}
