// ln_fold.hip -- stage 2 of the dgamma/dbeta(/dbias) column reduction for
// gfx950: add the P per-partition partials [P][K][m] (K = 1, 2 or 3) in a
// fixed order
// ("Accelerating Transformer on GPU (II)" §2.4: a second small kernel adds
// the P partial sums).
//
// A workgroup of 256 threads covers a block of columns of the [K*m]
// concatenation (dgamma columns, then dbeta, then dbias) with 16 slices of the
// partitions: slice k adds partitions [k*P/16, (k+1)*P/16) one after another,
// then the 16 slice sums are added in slice order through LDS.  Every load of
// a thread is issued before its first add, so the pass is one memory latency
// long.  The order depends only on P, so the result does not depend on
// timing or on the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ln_launch.hpp"

#pragma clang fp contract(off)

namespace mbrow {

constexpr int FOLD_SLICES = 16;
constexpr int FOLD_MAX_PER_SLICE = 16;   // P <= 256 partitions
constexpr int FOLD_COLS = 16;            // column units per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Vector path (m % 4 == 0): a column unit is 4 adjacent columns.
__global__ __launch_bounds__(FOLD_COLS* FOLD_SLICES) void ln_fold4_kernel(
    const float* __restrict__ ws, int64_t parts, int64_t m, int kinds, FoldOut out) {
    __shared__ f32x4 part_sum[FOLD_SLICES][FOLD_COLS];
    const int t = threadIdx.x;
    const int cl = t % FOLD_COLS;
    const int slice = t / FOLD_COLS;
    const int64_t c = ((int64_t)blockIdx.x * FOLD_COLS + cl) * 4;   // first column in [0, K*m)
    const bool ok = c < kinds * m;
    const int64_t kind = ok ? c / m : 0;                              // 0: dgamma, 1: dbeta, 2: dbias
    const int64_t j = ok ? c - kind * m : 0;
    const int64_t p0 = slice * parts / FOLD_SLICES;
    const int64_t p1 = (slice + 1) * parts / FOLD_SLICES;
    const f32x4* src = reinterpret_cast<const f32x4*>(ws + kind * m + j);
    const int64_t stride = kinds * m / 4;
    f32x4 v[FOLD_MAX_PER_SLICE];
#pragma unroll
    for (int k = 0; k < FOLD_MAX_PER_SLICE; ++k) {
        const int64_t p = p0 + k;
        v[k] = (ok && p < p1) ? src[p * stride] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    f32x4 acc = v[0];
#pragma unroll
    for (int k = 1; k < FOLD_MAX_PER_SLICE; ++k) acc = acc + v[k];
    part_sum[slice][cl] = acc;
    __syncthreads();
    if (slice == 0 && ok) {
        f32x4 tot = part_sum[0][cl];
#pragma unroll
        for (int k = 1; k < FOLD_SLICES; ++k) tot = tot + part_sum[k][cl];
        float* dst = out.p[kind] + j;
        dst[0] = tot[0];
        dst[1] = tot[1];
        dst[2] = tot[2];
        dst[3] = tot[3];
    }
}

// Scalar path: a column unit is one column.
__global__ __launch_bounds__(FOLD_COLS* FOLD_SLICES) void ln_fold1_kernel(
    const float* __restrict__ ws, int64_t parts, int64_t m, int kinds, FoldOut out) {
    __shared__ float part_sum[FOLD_SLICES][FOLD_COLS];
    const int t = threadIdx.x;
    const int cl = t % FOLD_COLS;
    const int slice = t / FOLD_COLS;
    const int64_t c = (int64_t)blockIdx.x * FOLD_COLS + cl;
    const bool ok = c < kinds * m;
    const int64_t kind = ok ? c / m : 0;
    const int64_t j = ok ? c - kind * m : 0;
    const int64_t p0 = slice * parts / FOLD_SLICES;
    const int64_t p1 = (slice + 1) * parts / FOLD_SLICES;
    const float* src = ws + kind * m + j;
    float v[FOLD_MAX_PER_SLICE];
#pragma unroll
    for (int k = 0; k < FOLD_MAX_PER_SLICE; ++k) {
        const int64_t p = p0 + k;
        v[k] = (ok && p < p1) ? src[p * kinds * m] : 0.0f;
    }
    float acc = v[0];
#pragma unroll
    for (int k = 1; k < FOLD_MAX_PER_SLICE; ++k) acc = acc + v[k];
    part_sum[slice][cl] = acc;
    __syncthreads();
    if (slice == 0 && ok) {
        float tot = part_sum[0][cl];
#pragma unroll
        for (int k = 1; k < FOLD_SLICES; ++k) tot = tot + part_sum[k][cl];
        out.p[kind][j] = tot;
    }
}

hipError_t launch_fold(const float* ws, int64_t parts, int64_t m, int kinds, FoldOut out,
                       hipStream_t s) {
    if (parts > (int64_t)FOLD_SLICES * FOLD_MAX_PER_SLICE || kinds < 1 || kinds > 3)
        return hipErrorInvalidValue;
    const bool vec = (m % 4) == 0 && (reinterpret_cast<uintptr_t>(ws) & 15u) == 0;
    if (vec) {
        const int64_t units = kinds * m / 4;
        const int64_t blocks = (units + FOLD_COLS - 1) / FOLD_COLS;
        hipLaunchKernelGGL(ln_fold4_kernel, dim3((unsigned)blocks),
                           dim3(FOLD_COLS * FOLD_SLICES), 0, s, ws, parts, m, kinds, out);
    } else {
        const int64_t blocks = (kinds * m + FOLD_COLS - 1) / FOLD_COLS;
        hipLaunchKernelGGL(ln_fold1_kernel, dim3((unsigned)blocks),
                           dim3(FOLD_COLS * FOLD_SLICES), 0, s, ws, parts, m, kinds, out);
    }
    return hipGetLastError();
}

}  // namespace mbrow
