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

// Row layouts compiled into the library, per storage size: (lanes per row,
// 16-byte slots per lane).  Each list holds only layouts whose kernels fit in
// registers without spilling (the build checks this); the widest covers
// 16384 columns.
#define MBROW_LAYOUTS_F32(X)                                                \
    X(16, 1) X(16, 2) X(16, 4) X(16, 8)                                     \
    X(32, 1) X(32, 2) X(32, 3) X(32, 4) X(32, 5) X(32, 6) X(32, 7) X(32, 8) \
    X(64, 1) X(64, 2) X(64, 3) X(64, 4) X(64, 5) X(64, 6) X(64, 7) X(64, 8) \
    X(128, 4) X(256, 4) X(512, 4) X(1024, 4)
#define MBROW_LAYOUTS_16(X)                                                 \
    X(16, 1) X(16, 2) X(16, 4)                                              \
    X(32, 1) X(32, 2) X(32, 3) X(32, 4) X(32, 5)                            \
    X(64, 1) X(64, 2) X(64, 3) X(64, 4) X(64, 5)                            \
    X(128, 4) X(256, 4) X(512, 4)

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
    uint8_t* mask_out;  // only read by the mask kernel
    int64_t rows;
    int64_t m;
    int64_t nslots;   // ceil(m / E)
    float eps;
    float inv_m;      // 1 / m
    float scale;      // 1 / (1 - p)
    uint32_t thr;     // keep iff 16-bit uniform >= thr
    uint32_t seed_lo;
    uint32_t seed_hi;
};

struct BwdArgs {
    const void* dy;
    const void* x;          // the LayerNorm input (z of the fused forward)
    const void* gamma;
    const float* mean;
    const float* rstd;
    void* dx;               // LayerNorm dx; with the prologue: dresidual = dz
    const void* dz_extra;   // prologue mode: gradient reaching z from its other uses, or NULL
    void* dx_in;            // prologue mode: gradient of the prologue's x
    float* ws;              // [P][K][m] partials (K = 2, or 3 with dbias)
    int ws_vec;             // ws 16-byte aligned (16-byte partial stores on the vector path)
    int64_t rows;
    int64_t m;
    int64_t nslots;
    int64_t parts;    // P
    float inv_m;
    float scale;      // prologue mode: 1 / (1 - p)
    uint32_t thr;     // prologue mode: keep iff 16-bit uniform >= thr
    uint32_t seed_lo;
    uint32_t seed_hi;
};

// DROPOUT: dx of the LayerNorm plus the backward of the bias + dropout +
// residual prologue, with partials of dgamma, dbeta and dbias.  RMS: dx of
// RMSNorm (mean not read), plus dz_extra, with partials of dgamma.
enum class BwdMode : int { DX = 0, DX_PARTIALS = 1, PARTIALS = 2, DROPOUT = 3, RMS = 4 };

// Row layouts of the prologue backward: three column accumulators per value
// leave room for fewer values per lane (multi-wave 16-bit rows take 2 slots
// per lane), and none for 1024-lane rows (128 registers per lane), so rows
// stop at 8192 columns there (512 lanes).
#define MBROW_LAYOUTS_DROP_F32(X)                                           \
    X(16, 1) X(16, 2) X(16, 4) X(32, 1) X(32, 2) X(32, 3) X(32, 4)          \
    X(64, 1) X(64, 2) X(64, 3) X(64, 4) X(64, 5) X(64, 6)                   \
    X(128, 4) X(256, 4) X(512, 4)
#define MBROW_LAYOUTS_DROP_16(X)                                            \
    X(16, 1) X(16, 2) X(32, 1) X(32, 2) X(32, 3)                            \
    X(64, 1) X(64, 2) X(64, 3) X(128, 2) X(256, 2) X(512, 2)

// Threads per workgroup of the backward for G lanes per row.
constexpr int bwd_threads(int g) { return g <= 512 ? 512 : g; }

// Row partitions of the dgamma/dbeta stage-1 pass: a pure function of
// (rows, cols).  Partition p owns the blocks of rows p, p + P, p + 2P, ...
// of the backward's row blocks; a partition without rows writes zeros.
int64_t bwd_partitions(int64_t rows, int64_t cols);

// Path selection from (dtype, cols, alignment); honours the test-only
// override set through ln_debug_force_path.
Path pick_path(Dt dt, int64_t cols, bool vec);        // forward
Path pick_bwd_path(Dt dt, int64_t cols, bool vec, bool dropout = false);   // backward
int elems_per_slot(Dt dt);

// Workgroups for a launch of `kernel` with `threads` threads per workgroup
// over `blocks` units of work, walked with a stride of the grid: as many as
// are resident on the device at once (occupancy x CUs), never more than
// `blocks`.  With `dyn_per_cu` > 0, a kernel with at least that many
// workgroups resident per CU and at least three rounds of blocks gets one
// workgroup per block instead, so that the hardware dispatcher hands each
// block to whichever compute unit frees up first (a fixed share per
// workgroup ends at the slowest one's pace).  Callers pass it where that
// measured faster: kernels with little per-workgroup set-up and enough
// workgroups per CU to overlap one block's loads with another's arithmetic.
int64_t persistent_grid(const void* kernel, int threads, int64_t blocks, int dyn_per_cu = 0);

// Kernel launches; return hipSuccess or the launch error.
hipError_t launch_fwd(Dt dt, const Path& p, bool fused, const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd(Dt dt, const Path& p, BwdMode mode, const BwdArgs& a, hipStream_t s);
hipError_t launch_dropout_mask(const FwdArgs& a, hipStream_t s);   // a.mask_out, rows, m, thr, seed
// Attention softmax over rows of `m` scores.
struct SmArgs {
    const void* x;          // forward: scores; backward: gradient of the output
    const void* mask;       // forward: additive mask rows, or NULL
    const void* y;          // backward: the forward's softmax output
    void* out;              // forward: y; backward: dx
    void* out2;             // forward: dropped output, or NULL
    int64_t rows;
    int64_t m;
    int64_t nslots;
    int64_t rows_per_mask;  // row r adds mask row r / rows_per_mask
    float scale;            // forward: multiplies x; backward: multiplies dx
    float pscale;           // 1 / (1 - p)
    uint32_t thr;           // keep iff 16-bit uniform >= thr
    uint32_t seed_lo;
    uint32_t seed_hi;
    int causal;             // keys j > r mod m masked (square score blocks)
};

// Row layouts of the softmax kernels (1024 x 5-8 fp32, 512 x 6, 8 and
// 1024 x 3-8 16-bit keep the block packed: softmax_wide_kernel).
#define MBROW_SM_LAYOUTS_F32(X)                                             \
    X(16, 1) X(16, 2) X(16, 4) X(32, 2) X(32, 4) X(64, 2) X(64, 4) X(64, 8) \
    X(128, 4) X(256, 4) X(512, 4) X(1024, 4) X(1024, 5) X(1024, 6)          \
    X(1024, 7) X(1024, 8)
#define MBROW_SM_LAYOUTS_16(X)                                              \
    X(16, 1) X(16, 2) X(32, 1) X(32, 2) X(64, 1) X(64, 2) X(64, 4)          \
    X(128, 4) X(256, 4) X(512, 4) X(512, 6) X(512, 8) X(1024, 3) X(1024, 4) \
    X(1024, 5) X(1024, 6) X(1024, 7) X(1024, 8)

// Widest 16-bit backward layout of the softmax (1024 x this many slots).
constexpr int kSmWideBwdV16 = 6;

// Softmax layouts that keep the block packed (softmax_wide_kernel): those
// whose unpacked scores would not fit a lane's registers.
constexpr bool sm_wide_layout(int g, int v, int e) {
    return (g == 1024 && v * e > 16) || (g == 512 && v > 4);
}

Path pick_softmax_path(Dt dt, int64_t cols, bool vec, bool backward);
hipError_t launch_softmax(Dt dt, const Path& p, bool backward, const SmArgs& a, hipStream_t s);

// Residual add + RMSNorm forward over rows of `m` values.
struct RmsArgs {
    const void* x;
    const void* residual;   // NULL: plain RMSNorm of x
    const void* gamma;
    void* residual_out;     // z = x + residual (with a residual)
    void* y;
    float* rstd;            // or NULL
    int64_t rows;
    int64_t m;
    int64_t nslots;
    float eps;
    float inv_m;
};
hipError_t launch_rmsnorm_fwd(Dt dt, const Path& p, const RmsArgs& a, hipStream_t s);

// Cross-entropy with label smoothing over rows of `cols` classes stored with
// a row stride of `ld` elements (columns [cols, ld) are padding).
struct XeArgs {
    const void* x;           // logits
    const int64_t* labels;   // [rows]
    float* loss;             // [rows]
    void* dx;                // gradient, or NULL (loss only); may equal x
    int64_t rows;
    int64_t cols;
    int64_t ld;
    int64_t nvalid;          // ceil(cols / E): slots holding classes
    int64_t nslots;          // ceil(ld / E): slots of the padded row
    float alpha;             // label smoothing
    float inv_v;             // 1 / cols
    float scale;             // gradient scale
};

// Row layouts of the cross-entropy kernel: vocabulary-wide rows over up to
// 1024 lanes with up to 16 slots per lane: 65536 fp32 or 131072 16-bit
// classes.
#define MBROW_XE_LAYOUTS_F32(X)                                             \
    X(16, 1) X(16, 2) X(16, 4) X(32, 2) X(32, 4) X(64, 2) X(64, 4) X(64, 8) \
    X(128, 4) X(256, 4) X(512, 4) X(512, 8) X(512, 13) X(1024, 4)          \
    X(1024, 6) X(1024, 8) X(1024, 10) X(1024, 13) X(1024, 16)
#define MBROW_XE_LAYOUTS_16(X)                                              \
    X(16, 1) X(16, 2) X(32, 1) X(32, 2) X(64, 1) X(64, 2) X(64, 4)          \
    X(128, 4) X(256, 4) X(512, 4) X(512, 7) X(512, 10) X(512, 13)          \
    X(1024, 4) X(1024, 5) X(1024, 6) X(1024, 7) X(1024, 8) X(1024, 10)     \
    X(1024, 12) X(1024, 14) X(1024, 16) X(1024, 18) X(1024, 20)

Path pick_xent_path(Dt dt, int64_t slots, bool vec);
hipError_t launch_xent(Dt dt, const Path& p, const XeArgs& a, hipStream_t s);

// Cross-entropy rows past the register layouts on the vector path
// (xent_lds_kernel): one workgroup per row holds the padded row, part of
// each lane's slots in registers and the rest in LDS, so rows of up to
// 32768 slots (131072 fp32, 262144 16-bit classes) are read once.  16-bit
// rows: 1024 lanes x (23 + 9) slots; fp32 rows: 512 lanes x (45 + 19) slots
// (fp32 needs the 256 registers a lane of a 512-lane workgroup has).
template <int E>
struct XeLds {
    static constexpr int LANES = E == 8 ? 1024 : 512;
    static constexpr int REG = E == 8 ? 23 : 45;   // slots per lane in registers
    static constexpr int LDS = E == 8 ? 9 : 19;    // slots per lane in LDS
};
constexpr int64_t kXeLdsMaxSlots = 32768;
static_assert(XeLds<8>::LANES * (XeLds<8>::REG + XeLds<8>::LDS) == kXeLdsMaxSlots, "16-bit");
static_assert(XeLds<4>::LANES * (XeLds<4>::REG + XeLds<4>::LDS) == kXeLdsMaxSlots, "fp32");
hipError_t launch_xent_lds(Dt dt, const XeArgs& a, hipStream_t s);

// LayerNorm rows wider than the register layouts (ln_wide.hip): one 1024-lane
// workgroup per row, the row staged in LDS.  The backward takes modes DX,
// DX_PARTIALS and PARTIALS.
constexpr int64_t kRegisterMaxCols = 16384;   // widest LayerNorm row of the register kernels
hipError_t launch_wide_fwd(Dt dt, bool vec, bool fused, const FwdArgs& a, hipStream_t s);
hipError_t launch_wide_bwd(Dt dt, bool vec, BwdMode mode, const BwdArgs& a, hipStream_t s);

// Rows too long for the register layouts: one workgroup per row, two passes
// over the row (stream.hip).
hipError_t launch_softmax_stream(Dt dt, bool vec, bool backward, const SmArgs& a, hipStream_t s);
hipError_t launch_xent_stream(Dt dt, bool vec, const XeArgs& a, hipStream_t s);

// Fold of [P][kinds][m] partials (kinds = 1, 2 or 3) into out[0..kinds-1].
struct FoldOut {
    float* p[3];
};
hipError_t launch_fold(const float* ws, int64_t parts, int64_t m, int kinds, FoldOut out,
                       hipStream_t s);

}  // namespace mbrow
