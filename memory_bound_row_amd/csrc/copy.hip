// A plain device-to-device copy in 16-byte vectors: the attainable-bandwidth
// reference that the row kernels' measured rates are compared against (the
// same bytes moved once each way, with no arithmetic and no reduction).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mbrow_ln.h"

namespace {

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;   // 16-byte vectors per thread, all loads issued first

// Workgroup b copies vectors [b*1024, (b+1)*1024): four coalesced passes of
// 256 lanes.  Loads and stores are nontemporal (each byte is touched once).
__global__ __launch_bounds__(kCopyThreads) void hbm_copy_kernel(const v4u32* __restrict__ src,
                                                               v4u32* __restrict__ dst,
                                                               int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
    v4u32 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

}  // namespace

extern "C" ln_status_t hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return LN_OK;
    if (!src || !dst) return LN_ERR_NULL;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if ((bytes & 15u) || (s & 15u) || (d & 15u)) return LN_ERR_PARAM;
    if (s < d + bytes && d < s + bytes) return LN_ERR_PARAM;   // overlapping ranges
    const int64_t n = (int64_t)(bytes / 16);
    const int64_t per = kCopyThreads * kCopyUnroll;
    const int64_t blocks = (n + per - 1) / per;
    if (blocks > INT32_MAX) return LN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(hbm_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                       static_cast<const v4u32*>(src), static_cast<v4u32*>(dst), n);
    return hipGetLastError() == hipSuccess ? LN_OK : LN_ERR_HIP;
}
