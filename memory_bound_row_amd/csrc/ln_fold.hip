// ln_fold.hip -- stage 2 of the dgamma/dbeta column reduction for gfx950:
// add the P per-partition partials [P][2][m] in a fixed order
// ("Accelerating Transformer on GPU (II)" §2.4: a second small kernel adds
// the P partial sums).
//
// A workgroup of 256 threads covers 16 columns of the [2m] concatenation
// (dgamma columns, then dbeta columns) with 16 slices of the partitions:
// slice k adds partitions [k*P/16, (k+1)*P/16) one after another, then slice
// sums are added in slice order through LDS.  The order depends only on P,
// so the result does not depend on timing; 16-way slicing keeps enough loads
// in flight that this small pass is not latency bound.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ln_launch.hpp"

#pragma clang fp contract(off)

namespace mbrow {

constexpr int FOLD_COLS = 16;
constexpr int FOLD_SLICES = 16;

__global__ __launch_bounds__(FOLD_COLS* FOLD_SLICES) void ln_fold_kernel(
    const float* __restrict__ ws, int64_t parts, int64_t m, float* __restrict__ dgamma,
    float* __restrict__ dbeta) {
    __shared__ float part_sum[FOLD_SLICES][FOLD_COLS];
    const int t = threadIdx.x;
    const int cl = t % FOLD_COLS;
    const int slice = t / FOLD_COLS;
    const int64_t c = (int64_t)blockIdx.x * FOLD_COLS + cl;   // in [0, 2m)
    const bool ok = c < 2 * m;
    const int64_t kind = ok ? c / m : 0;                       // 0: dgamma, 1: dbeta
    const int64_t j = ok ? c - kind * m : 0;
    const int64_t p0 = slice * parts / FOLD_SLICES;
    const int64_t p1 = (slice + 1) * parts / FOLD_SLICES;
    float acc = 0.0f;
    if (ok) {
        const float* src = ws + kind * m + j;
        for (int64_t p = p0; p < p1; ++p) acc = acc + src[p * 2 * m];
    }
    part_sum[slice][cl] = acc;
    __syncthreads();
    if (slice == 0 && ok) {
        float tot = part_sum[0][cl];
#pragma unroll
        for (int k = 1; k < FOLD_SLICES; ++k) tot = tot + part_sum[k][cl];
        if (kind == 0) dgamma[j] = tot;
        else dbeta[j] = tot;
    }
}

hipError_t launch_fold(const float* ws, int64_t parts, int64_t m, float* dgamma, float* dbeta,
                       hipStream_t s) {
    const int64_t blocks = (2 * m + FOLD_COLS - 1) / FOLD_COLS;
    hipLaunchKernelGGL(ln_fold_kernel, dim3((unsigned)blocks), dim3(FOLD_COLS * FOLD_SLICES), 0,
                       s, ws, parts, m, dgamma, dbeta);
    return hipGetLastError();
}

}  // namespace mbrow
