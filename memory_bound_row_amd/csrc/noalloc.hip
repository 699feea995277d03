// noalloc.hip -- the library's one static device buffer, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): ln_bwd_noalloc keeps the backward's
// column partials here instead of in a caller workspace.
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side stand-in, so the device address is
// looked up once per device (with that device current) and kept; kernels
// only ever receive that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mbrow_ln.h"

namespace {

static __device__ __align__(256) float scratch[LN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;

}  // namespace

namespace mbrow {

// Device address of the current device's `scratch` (nullptr and an error on
// failure).  The first call on a device looks the address up; later calls
// return the kept value.
hipError_t noalloc_scratch(float** out) {
    static std::mutex mu;
    static float* ptr[kMaxDevices] = {};
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptr[dev] = static_cast<float*>(p);
    }
    *out = ptr[dev];
    return hipSuccess;
}

}  // namespace mbrow
