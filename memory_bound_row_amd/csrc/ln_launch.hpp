// ln_launch.hpp -- host-side launch interface between the C ABI (ln_api.cpp)
// and the kernel files.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbrow {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

// Lanes per row and 16-byte slots per lane chosen for one call, plus the
// access width.  g <= 64: a row is owned by g lanes of one wave (64/g rows
// per wave); g > 64: by g/64 waves of one workgroup.
struct Path {
    int g = 64;
    int v = 1;
    bool vec = true;
};

struct FwdArgs {
    const void* x;
    const void* bias;
    const void* residual;
    const void* gamma;
    const void* beta;
    void* residual_out;
    void* y;
    float* mean;
    float* rstd;
    uint8_t* mask_out;
    int64_t rows;
    int64_t m;
    int64_t nslots;   // ceil(m / E)
    float eps;
    float scale;      // 1 / (1 - p)
    uint32_t thr;     // keep iff 16-bit uniform >= thr
    uint32_t seed_lo;
    uint32_t seed_hi;
};

struct BwdArgs {
    const void* dy;
    const void* x;
    const void* gamma;
    const float* mean;
    const float* rstd;
    void* dx;
    float* ws;        // [P][2][m] partials
    int64_t rows;
    int64_t m;
    int64_t nslots;
    int64_t parts;    // P
    float inv_m;
};

enum class BwdMode : int { DX = 0, DX_PARTIALS = 1, PARTIALS = 2 };

// Row partitions of the dgamma/dbeta stage-1 pass: a pure function of
// (rows, cols).  Every partition owns at least one row.
int64_t bwd_partitions(int64_t rows, int64_t cols);

// Path selection from (dtype, cols, alignment); honours the test-only
// override set through ln_debug_force_path.
Path pick_path(Dt dt, int64_t cols, bool vec);
int elems_per_slot(Dt dt);

// Kernel launches; return hipSuccess or the launch error.
hipError_t launch_fwd(Dt dt, const Path& p, bool fused, const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd(Dt dt, const Path& p, BwdMode mode, const BwdArgs& a, hipStream_t s);
hipError_t launch_fold(const float* ws, int64_t parts, int64_t m, float* dgamma,
                       float* dbeta, hipStream_t s);

}  // namespace mbrow
