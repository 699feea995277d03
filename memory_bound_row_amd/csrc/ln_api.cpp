// ln_api.cpp -- the C ABI declared in include/mbrow_ln.h: argument checks,
// path selection and launches on the caller's stream.  Everything that can
// be rejected is rejected here, on the host, before anything is enqueued.
#include "mbrow_ln.h"
#include "mbrow_ln_debug.h"

#include <rocprofiler-sdk-roctx/roctx.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <limits>
#include <mutex>
#include <unordered_map>

#include "ln_launch.hpp"

namespace mbrow {

hipError_t launch_fwd_f32(const Path&, bool, const FwdArgs&, hipStream_t);
hipError_t launch_fwd_f16(const Path&, bool, const FwdArgs&, hipStream_t);
hipError_t launch_fwd_bf16(const Path&, bool, const FwdArgs&, hipStream_t);
hipError_t launch_bwd_f32(const Path&, BwdMode, const BwdArgs&, hipStream_t);
hipError_t launch_bwd_f16(const Path&, BwdMode, const BwdArgs&, hipStream_t);
hipError_t launch_bwd_bf16(const Path&, BwdMode, const BwdArgs&, hipStream_t);
hipError_t launch_softmax_f32(const Path&, bool, const SmArgs&, hipStream_t);
hipError_t launch_softmax_f16(const Path&, bool, const SmArgs&, hipStream_t);
hipError_t launch_softmax_bf16(const Path&, bool, const SmArgs&, hipStream_t);
hipError_t launch_rmsnorm_fwd_f32(const Path&, const RmsArgs&, hipStream_t);
hipError_t launch_rmsnorm_fwd_f16(const Path&, const RmsArgs&, hipStream_t);
hipError_t launch_rmsnorm_fwd_bf16(const Path&, const RmsArgs&, hipStream_t);

hipError_t launch_xent_f32(const Path&, const XeArgs&, hipStream_t);
hipError_t launch_xent_f16(const Path&, const XeArgs&, hipStream_t);
hipError_t launch_xent_bf16(const Path&, const XeArgs&, hipStream_t);

hipError_t launch_softmax_stream_f32(bool, bool, const SmArgs&, hipStream_t);
hipError_t launch_softmax_stream_f16(bool, bool, const SmArgs&, hipStream_t);
hipError_t launch_softmax_stream_bf16(bool, bool, const SmArgs&, hipStream_t);
hipError_t launch_xent_stream_f32(bool, const XeArgs&, hipStream_t);
hipError_t launch_xent_stream_f16(bool, const XeArgs&, hipStream_t);
hipError_t launch_xent_stream_bf16(bool, const XeArgs&, hipStream_t);
hipError_t launch_softmax_long_fwd_f32(int, const SmArgs&, hipStream_t);
hipError_t launch_softmax_long_fwd_f16(int, const SmArgs&, hipStream_t);
hipError_t launch_softmax_long_fwd_bf16(int, const SmArgs&, hipStream_t);
hipError_t launch_softmax_fwd_mask_lds_f32(const SmArgs&, hipStream_t);
hipError_t launch_softmax_fwd_mask_lds_f16(const SmArgs&, hipStream_t);
hipError_t launch_softmax_fwd_mask_lds_bf16(const SmArgs&, hipStream_t);
hipError_t launch_softmax_bwd_lds_f32(const SmArgs&, hipStream_t);
hipError_t launch_softmax_bwd_lds_f16(const SmArgs&, hipStream_t);
hipError_t launch_softmax_bwd_lds_bf16(const SmArgs&, hipStream_t);
hipError_t launch_xent_lds_f32(const XeArgs&, hipStream_t);
hipError_t launch_xent_lds_f16(const XeArgs&, hipStream_t);
hipError_t launch_xent_lds_bf16(const XeArgs&, hipStream_t);

hipError_t launch_softmax_stream(Dt dt, bool vec, bool backward, const SmArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_softmax_stream_f32(vec, backward, a, s);
    case Dt::F16: return launch_softmax_stream_f16(vec, backward, a, s);
    default: return launch_softmax_stream_bf16(vec, backward, a, s);
    }
}

hipError_t launch_xent_stream(Dt dt, bool vec, const XeArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_xent_stream_f32(vec, a, s);
    case Dt::F16: return launch_xent_stream_f16(vec, a, s);
    default: return launch_xent_stream_bf16(vec, a, s);
    }
}

static_assert(LN_MAX_COLS_XENT_LDS_F32 / 4 == kXeLdsMaxSlots &&
                  LN_MAX_COLS_XENT_LDS_16 / 8 == kXeLdsMaxSlots,
              "the header's on-chip cross-entropy widths are the kernel's slots");

hipError_t launch_xent_lds(Dt dt, const XeArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_xent_lds_f32(a, s);
    case Dt::F16: return launch_xent_lds_f16(a, s);
    default: return launch_xent_lds_bf16(a, s);
    }
}

hipError_t launch_xent(Dt dt, const Path& p, const XeArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_xent_f32(p, a, s);
    case Dt::F16: return launch_xent_f16(p, a, s);
    default: return launch_xent_bf16(p, a, s);
    }
}

hipError_t launch_rmsnorm_fwd(Dt dt, const Path& p, const RmsArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_rmsnorm_fwd_f32(p, a, s);
    case Dt::F16: return launch_rmsnorm_fwd_f16(p, a, s);
    default: return launch_rmsnorm_fwd_bf16(p, a, s);
    }
}

hipError_t launch_softmax(Dt dt, const Path& p, bool backward, const SmArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_softmax_f32(p, backward, a, s);
    case Dt::F16: return launch_softmax_f16(p, backward, a, s);
    default: return launch_softmax_bf16(p, backward, a, s);
    }
}

hipError_t launch_fwd(Dt dt, const Path& p, bool fused, const FwdArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_fwd_f32(p, fused, a, s);
    case Dt::F16: return launch_fwd_f16(p, fused, a, s);
    default: return launch_fwd_bf16(p, fused, a, s);
    }
}

hipError_t launch_wide_fwd_f32(bool, bool, const FwdArgs&, hipStream_t);
hipError_t launch_wide_fwd_f16(bool, bool, const FwdArgs&, hipStream_t);
hipError_t launch_wide_fwd_bf16(bool, bool, const FwdArgs&, hipStream_t);
hipError_t launch_wide_bwd_f32(bool, BwdMode, const BwdArgs&, hipStream_t);
hipError_t launch_wide_bwd_f16(bool, BwdMode, const BwdArgs&, hipStream_t);
hipError_t launch_wide_bwd_bf16(bool, BwdMode, const BwdArgs&, hipStream_t);

hipError_t launch_wide_fwd(Dt dt, bool vec, bool fused, const FwdArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_wide_fwd_f32(vec, fused, a, s);
    case Dt::F16: return launch_wide_fwd_f16(vec, fused, a, s);
    default: return launch_wide_fwd_bf16(vec, fused, a, s);
    }
}

hipError_t launch_wide_bwd(Dt dt, bool vec, BwdMode mode, const BwdArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_wide_bwd_f32(vec, mode, a, s);
    case Dt::F16: return launch_wide_bwd_f16(vec, mode, a, s);
    default: return launch_wide_bwd_bf16(vec, mode, a, s);
    }
}

hipError_t launch_bwd(Dt dt, const Path& p, BwdMode mode, const BwdArgs& a, hipStream_t s) {
    switch (dt) {
    case Dt::F32: return launch_bwd_f32(p, mode, a, s);
    case Dt::F16: return launch_bwd_f16(p, mode, a, s);
    default: return launch_bwd_bf16(p, mode, a, s);
    }
}

int elems_per_slot(Dt dt) { return dt == Dt::F32 ? 4 : 8; }

// Instances compiled in ln_fwd.hip / ln_bwd.hip.
static bool have_instance(bool f32, int g, int v) {
#define MBROW_HAVE(GG, VV) if (g == GG && v == VV) return true;
    if (f32) {
        MBROW_LAYOUTS_F32(MBROW_HAVE)
    } else {
        MBROW_LAYOUTS_16(MBROW_HAVE)
    }
#undef MBROW_HAVE
    return false;
}

static std::atomic<int> g_force_g{0}, g_force_v{0}, g_force_scalar{0}, g_force_grid{0},
    g_force_two_pass{0}, g_force_staged{0};

// The test-only override that forces the per-element path (no vector access).
bool force_scalar() { return g_force_scalar.load(std::memory_order_relaxed) != 0; }
bool force_two_pass() { return g_force_two_pass.load(std::memory_order_relaxed) != 0; }
bool force_staged() { return g_force_staged.load(std::memory_order_relaxed) != 0; }

// Row layout: among the candidate layouts, the one with the fewest slots
// (used or not); ties go to the earlier candidate.  With `wave_rows`, slots
// of a layout whose row is not exactly one wave (G != 64) count 5/4: one row
// per wave measured faster in the backward even with some lanes idle.
static bool in_list(const int (*list)[2], int n, int g, int v) {
    for (int k = 0; k < n; ++k)
        if (list[k][0] == g && list[k][1] == v) return true;
    return false;
}

// `only_listed`: a forced layout applies only if it is one of the candidates
// (the prologue backward is compiled for its own list).
static Path pick(bool f32, int64_t ns, bool vec, const int (*prefer)[2], int nprefer,
                 bool wave_rows = false, bool only_listed = false) {
    Path p;
    p.vec = vec && g_force_scalar.load(std::memory_order_relaxed) == 0;
    const int fg = g_force_g.load(std::memory_order_relaxed);
    const int fv = g_force_v.load(std::memory_order_relaxed);
    const bool known = only_listed ? in_list(prefer, nprefer, fg, fv) : have_instance(f32, fg, fv);
    if (fg > 0 && (int64_t)fg * fv >= ns && known) {
        p.g = fg;
        p.v = fv;
        return p;
    }
    int64_t best = -1;
    for (int k = 0; k < nprefer; ++k) {
        const int64_t cap = (int64_t)prefer[k][0] * prefer[k][1];
        if (cap < ns) continue;
        const int64_t cost = wave_rows ? cap * (prefer[k][0] == 64 ? 4 : 5) : cap;
        if (best < 0 || cost < best) {
            best = cost;
            p.g = prefer[k][0];
            p.v = prefer[k][1];
        }
    }
    if (best < 0) {
        p.g = f32 ? 1024 : 512;   // wider than every layout: callers cap cols
        p.v = 4;
    }
    return p;
}

// Candidate layouts in order of preference for equal cost.  Within a wave a
// lane holds at most 32 fp32 or 40 16-bit values of a row (8 or 5 slots; the
// backward also keeps two column accumulators per value); wider rows spread
// over several waves.
static const int kFwd32[][2] = {{16, 1}, {32, 1}, {16, 2}, {32, 2}, {64, 1}, {32, 3}, {64, 2},
                                {32, 4}, {64, 3}, {32, 5}, {32, 6}, {64, 4}, {32, 7}, {32, 8},
                                {64, 5}, {64, 6}, {64, 7}, {64, 8}, {128, 4}, {256, 4},
                                {512, 4}, {1024, 4}};
static const int kFwd16[][2] = {{16, 1}, {32, 1}, {16, 2}, {32, 2}, {64, 1}, {32, 3}, {64, 2},
                                {32, 4}, {64, 3}, {32, 5}, {64, 4}, {128, 4}, {256, 4},
                                {512, 4}};
static const int kBwd32[][2] = {{16, 1}, {32, 1}, {16, 2}, {32, 2}, {64, 1}, {32, 3}, {64, 2},
                                {32, 4}, {64, 3}, {32, 5}, {32, 6}, {64, 4}, {32, 7}, {32, 8},
                                {64, 5}, {64, 6}, {64, 7}, {64, 8}, {128, 4}, {256, 4},
                                {512, 4}, {1024, 4}};
static const int kDrop32[][2] = {{16, 1}, {32, 1}, {16, 2}, {32, 2}, {64, 1}, {32, 3}, {64, 2},
                                 {32, 4}, {64, 3}, {64, 4}, {64, 5}, {64, 6}, {128, 4},
                                 {256, 4}, {512, 4}};
static const int kDrop16[][2] = {{16, 1}, {32, 1}, {16, 2}, {32, 2}, {64, 1}, {32, 3}, {64, 2},
                                 {64, 3}, {128, 2}, {256, 2}, {512, 2}};
static const int kBwd16[][2] = {{16, 1}, {32, 1}, {16, 2}, {32, 2}, {64, 1}, {32, 3}, {64, 2},
                                {32, 4}, {64, 3}, {32, 5}, {64, 4}, {64, 5}, {128, 4}, {256, 4},
                                {512, 4}};

#define MBROW_N(a) (int)(sizeof(a) / sizeof(a[0]))

Path pick_path(Dt dt, int64_t cols, bool vec) {
    const int E = elems_per_slot(dt);
    const int64_t ns = (cols + E - 1) / E;
    return E == 4 ? pick(true, ns, vec, kFwd32, MBROW_N(kFwd32))
                  : pick(false, ns, vec, kFwd16, MBROW_N(kFwd16));
}

static const int kSm32[][2] = {{16, 1}, {16, 2}, {16, 4}, {32, 2}, {32, 4}, {64, 2}, {64, 4},
                               {64, 8}, {128, 4}, {256, 4}, {512, 4}, {1024, 4}, {1024, 5},
                               {1024, 6}, {1024, 7}, {1024, 8}};
static const int kSm16[][2] = {{16, 1}, {16, 2}, {32, 1}, {32, 2}, {64, 1}, {64, 2}, {64, 4},
                               {128, 4}, {256, 4}, {512, 4}, {512, 6}, {512, 8}, {1024, 3},
                               {1024, 4}, {1024, 5}, {1024, 6}, {1024, 7}, {1024, 8}};

// (the 16-bit backward stops at 1024 x kSmWideBwdV16: the last entries of
// kSm16 are forward-only)
Path pick_softmax_path(Dt dt, int64_t cols, bool vec, bool backward) {
    const int E = elems_per_slot(dt);
    const int64_t ns = (cols + E - 1) / E;
    const int n16 = backward ? MBROW_N(kSm16) - (8 - kSmWideBwdV16) : MBROW_N(kSm16);
    return E == 4 ? pick(true, ns, vec, kSm32, MBROW_N(kSm32), false, true)
                  : pick(false, ns, vec, kSm16, n16, false, true);
}

static const int kXe32[][2] = {{16, 1}, {16, 2}, {16, 4}, {32, 2}, {32, 4}, {64, 2},
                               {64, 4}, {64, 8}, {128, 4}, {256, 4}, {512, 4}, {512, 8},
                               {512, 13}, {1024, 4},
                               {1024, 6}, {1024, 8}, {1024, 10}, {1024, 13}, {1024, 16}};
static const int kXe16[][2] = {{16, 1}, {16, 2}, {32, 1}, {32, 2}, {64, 1}, {64, 2},
                               {64, 4}, {128, 4}, {256, 4}, {512, 4}, {512, 7}, {512, 10},
                               {512, 13}, {1024, 4}, {1024, 5},
                               {1024, 6}, {1024, 7}, {1024, 8}, {1024, 10}, {1024, 12},
                               {1024, 14}, {1024, 16}, {1024, 18}, {1024, 20}};

// `slots`: 16-byte slots of the padded row (ceil(ld / E)).
Path pick_xent_path(Dt dt, int64_t slots, bool vec) {
    return dt == Dt::F32 ? pick(true, slots, vec, kXe32, MBROW_N(kXe32), false, true)
                         : pick(false, slots, vec, kXe16, MBROW_N(kXe16), false, true);
}

// The same choice with and without partials, so the fused and the
// partials-only passes accumulate in the same order.  The prologue backward
// (`dropout`) chooses among the layouts compiled for it.
Path pick_bwd_path(Dt dt, int64_t cols, bool vec, bool dropout) {
    const int E = elems_per_slot(dt);
    const int64_t ns = (cols + E - 1) / E;
    if (dropout)
        return E == 4 ? pick(true, ns, vec, kDrop32, MBROW_N(kDrop32), true, true)
                      : pick(false, ns, vec, kDrop16, MBROW_N(kDrop16), true, true);
    return E == 4 ? pick(true, ns, vec, kBwd32, MBROW_N(kBwd32), true)
                  : pick(false, ns, vec, kBwd16, MBROW_N(kBwd16), true);
}

static int64_t grid_for(const void* kernel, int threads, int64_t blocks, int dyn_per_cu) {
    const int forced = g_force_grid.load(std::memory_order_relaxed);
    if (forced < 0) return blocks;
    static std::mutex mu;
    // per device: its CU count, and resident workgroups per CU of each kernel
    static std::unordered_map<int, int> cu_count;
    static std::unordered_map<int, std::unordered_map<const void*, int>> per_cu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return blocks;
    int cus = 0, n = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto c = cu_count.find(dev);
        if (c == cu_count.end()) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) !=
                    hipSuccess || v <= 0)
                v = 0;
            c = cu_count.emplace(dev, v).first;
        }
        cus = c->second;
        auto& kmap = per_cu[dev];
        auto it = kmap.find(kernel);
        if (it == kmap.end()) {
            int b = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kernel, threads, 0) !=
                    hipSuccess || b <= 0)
                b = 0;
            it = kmap.emplace(kernel, b).first;
        }
        n = it->second;
    }
    if (cus <= 0 || n <= 0) return blocks;   // unknown: one workgroup per block
    const int64_t per = forced > 0 ? forced : n;
    const int64_t g = (int64_t)cus * per;
    if (forced == 0 && dyn_per_cu > 0 && n >= dyn_per_cu && blocks >= 3 * g) return blocks;
    return g < blocks ? g : blocks;
}

int64_t persistent_grid(const void* kernel, int threads, int64_t blocks, int dyn_per_cu) {
    // a dispatch counts its work-items in 32 bits; every kernel walks its
    // blocks with a stride of the grid, so a smaller grid only loops more
    const int64_t cap = std::numeric_limits<int32_t>::max() / threads;
    const int64_t g = grid_for(kernel, threads, blocks, dyn_per_cu);
    return g < cap ? g : cap;
}

// ln_bwd_noalloc's static device scratch (noalloc.hip).
hipError_t noalloc_scratch(float** out);

int64_t bwd_partitions(int64_t rows, int64_t cols) {
    (void)cols;
    const int64_t kParts = 256;
    return rows < kParts ? rows : kParts;
}

}  // namespace mbrow

using namespace mbrow;

namespace {

constexpr int64_t kMaxRows = std::numeric_limits<int32_t>::max();

bool valid_dtype(ln_dtype_t dt) { return dt == LN_F32 || dt == LN_F16 || dt == LN_BF16; }

size_t elem_bytes(ln_dtype_t dt) { return dt == LN_F32 ? 4 : 2; }

enum class Kind { FWD, BWD, RMS };

int64_t max_cols(ln_dtype_t dt, Kind k) {
    switch (k) {
    case Kind::FWD: return LN_MAX_COLS;
    case Kind::BWD: return dt == LN_F32 ? LN_MAX_COLS_BWD_F32 : LN_MAX_COLS_BWD_16;
    default: return LN_MAX_COLS_RMSNORM;
    }
}

// widest softmax row held in registers (wider rows take the two-pass path)
int64_t softmax_max_cols(ln_dtype_t dt, bool backward) {
    if (dt == LN_F32) return LN_MAX_COLS_SOFTMAX_F32;
    return backward ? LN_MAX_COLS_SOFTMAX_BWD_16 : LN_MAX_COLS_SOFTMAX_16;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
    bool tensor2d;   // a [rows, cols] tensor (may be updated in place)
};

bool overlaps(const Span& a, const Span& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outputs may not overlap each other; an output may coincide exactly with a
// [rows, cols] input (in place) and must otherwise be disjoint from inputs.
ln_status_t check_aliasing(const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j])) return LN_ERR_UNSUPPORTED;
        for (int j = 0; j < nin; ++j) {
            if (!overlaps(outs[i], ins[j])) continue;
            const bool exact = outs[i].p == ins[j].p && outs[i].bytes == ins[j].bytes &&
                               outs[i].tensor2d && ins[j].tensor2d;
            if (!exact) return LN_ERR_UNSUPPORTED;
        }
    }
    return LN_OK;
}

ln_status_t check_shape(int64_t rows, int64_t cols, ln_dtype_t dt, Kind k) {
    if (!valid_dtype(dt)) return LN_ERR_DTYPE;
    if (rows < 0 || cols <= 0) return LN_ERR_SHAPE;
    if (cols > max_cols(dt, k) || rows > kMaxRows) return LN_ERR_UNSUPPORTED;
    return LN_OK;
}

// LayerNorm rows past the register layouts, or every row under the test hook,
// take the LDS-staged kernels.
bool staged(int64_t cols) { return cols > kRegisterMaxCols || force_staged(); }

// The plain forward of fp32 rows of 6145-16384 columns on the vector path
// runs faster staged (512 lanes x up to 8 slots, two workgroups per CU) than
// in the register layouts that hold them (512 or 1024 lanes x 4 slots, their
// last slot partly idle): measured 101.8 -> 96.4 us at 9362x7168, 98.7 ->
// 96.4 us at 8192x8192, 175 -> 149 us at 8192x12288, 102.7 -> 100.2 us at
// 4096x16384; at 6144 columns and below the registers win (105.6 against
// 128.3 us at 10922x6144).  The fused forward, 16-bit rows and the backward
// measured as fast or faster in registers.  A layout forced through the
// test hook keeps the register kernel.
bool staged_plain_fwd(Dt d, int64_t cols, bool vec) {
    return d == Dt::F32 && vec && cols > 6144 && g_force_g.load(std::memory_order_relaxed) == 0;
}

ln_status_t from_hip(hipError_t e) { return e == hipSuccess ? LN_OK : LN_ERR_HIP; }

// Shape check of the calls with a two-pass path for long rows.
ln_status_t check_shape_stream(int64_t rows, int64_t cols, ln_dtype_t dt) {
    if (!valid_dtype(dt)) return LN_ERR_DTYPE;
    if (rows < 0 || cols <= 0) return LN_ERR_SHAPE;
    if (cols > LN_MAX_COLS_STREAM || rows > kMaxRows) return LN_ERR_UNSUPPORTED;
    return LN_OK;
}

// A roctx range around each entry point, for timelines from rocprofv3
// --marker-trace: on when the environment has MBROW_ROCTX=1 (read once per
// process), off otherwise, so that by default a call costs nothing extra.
bool roctx_on() {
    static const bool on = [] {
        const char* v = std::getenv("MBROW_ROCTX");
        return v != nullptr && v[0] == '1';
    }();
    return on;
}

struct Range {
    const bool on;
    explicit Range(const char* name) : on(roctx_on()) {
        if (on) roctxRangePushA(name);
    }
    ~Range() {
        if (on) roctxRangePop();
    }
    Range(const Range&) = delete;
    Range& operator=(const Range&) = delete;
};

}  // namespace

extern "C" {

const char* ln_status_string(ln_status_t status) {
    switch (status) {
    case LN_OK: return "LN_OK: success";
    case LN_ERR_NULL: return "LN_ERR_NULL: a required pointer is NULL";
    case LN_ERR_SHAPE: return "LN_ERR_SHAPE: rows must be >= 0 and cols > 0";
    case LN_ERR_DTYPE: return "LN_ERR_DTYPE: unknown storage dtype";
    case LN_ERR_PARAM: return "LN_ERR_PARAM: eps must be >= 0; p must be in [0, 1)";
    case LN_ERR_WORKSPACE: return "LN_ERR_WORKSPACE: workspace missing or too small";
    case LN_ERR_UNSUPPORTED:
        return "LN_ERR_UNSUPPORTED: shape too large or buffers overlap in a way the call "
               "does not allow";
    case LN_ERR_HIP: return "LN_ERR_HIP: a HIP launch failed";
    case LN_ERR_SCRATCH:
        return "LN_ERR_SCRATCH: the shape needs more than the library's static scratch "
               "(LN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown ln_status_t";
    }
}

size_t ln_bwd_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)bwd_partitions(rows, cols) * 2u * (size_t)cols * sizeof(float);
}

size_t bias_dropout_residual_ln_bwd_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)bwd_partitions(rows, cols) * 3u * (size_t)cols * sizeof(float);
}

size_t add_rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)bwd_partitions(rows, cols) * (size_t)cols * sizeof(float);
}

ln_status_t ln_fwd(const void* x, const void* gamma, const void* beta, void* y, float* mean,
                   float* rstd, int64_t rows, int64_t cols, float eps, ln_dtype_t dt,
                   hipStream_t stream) {
    const Range range("ln_fwd");
    if (!x || !gamma || !beta || !y) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::FWD);
    if (st != LN_OK) return st;
    if (!(eps >= 0.0f) || std::isinf(eps)) return LN_ERR_PARAM;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float);
    const Span outs[] = {{y, tb, true}, {mean, sb, false}, {rstd, sb, false}};
    const Span ins[] = {{x, tb, true}, {gamma, vb, false}, {beta, vb, false}};
    st = check_aliasing(outs, 3, ins, 3);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(x) && aligned16(y) && aligned16(gamma) && aligned16(beta) &&
                     (cols * (int64_t)es) % 16 == 0;
    FwdArgs a{};
    a.x = x; a.gamma = gamma; a.beta = beta; a.y = y; a.mean = mean; a.rstd = rstd;
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.eps = eps;
    a.inv_m = (float)(1.0 / (double)cols);
    const bool v = vec && !force_scalar();
    if (staged(cols) || staged_plain_fwd(d, cols, v))
        return from_hip(launch_wide_fwd(d, v, false, a, stream));
    return from_hip(launch_fwd(d, pick_path(d, cols, vec), false, a, stream));
}

ln_status_t bias_dropout_residual_ln_fwd(const void* x, const void* bias, const void* residual,
                                         const void* gamma, const void* beta, void* residual_out,
                                         void* y, float* mean, float* rstd, uint8_t* mask_out,
                                         int64_t rows, int64_t cols, float eps, float p,
                                         uint64_t seed, ln_dtype_t dt, hipStream_t stream) {
    const Range range("bias_dropout_residual_ln_fwd");
    if (!x || !bias || !residual || !gamma || !beta || !residual_out || !y) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::FWD);
    if (st != LN_OK) return st;
    if (!(eps >= 0.0f) || std::isinf(eps)) return LN_ERR_PARAM;
    if (!(p >= 0.0f && p < 1.0f)) return LN_ERR_PARAM;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float);
    const Span outs[] = {{residual_out, tb, true}, {y, tb, true}, {mean, sb, false},
                         {rstd, sb, false}, {mask_out, (size_t)rows * (size_t)cols, false}};
    const Span ins[] = {{x, tb, true}, {residual, tb, true}, {bias, vb, false},
                        {gamma, vb, false}, {beta, vb, false}};
    st = check_aliasing(outs, 5, ins, 5);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(x) && aligned16(bias) && aligned16(residual) &&
                     aligned16(gamma) && aligned16(beta) && aligned16(residual_out) &&
                     aligned16(y) && (cols * (int64_t)es) % 16 == 0;
    FwdArgs a{};
    a.x = x; a.bias = bias; a.residual = residual; a.gamma = gamma; a.beta = beta;
    a.residual_out = residual_out; a.y = y; a.mean = mean; a.rstd = rstd; a.mask_out = mask_out;
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.eps = eps;
    a.inv_m = (float)(1.0 / (double)cols);
    a.thr = (uint32_t)std::floor((double)p * 65536.0 + 0.5);
    a.scale = (float)(1.0 / (1.0 - (double)p));
    a.seed_lo = (uint32_t)(seed & 0xffffffffu);
    a.seed_hi = (uint32_t)(seed >> 32);
    st = staged(cols) ? from_hip(launch_wide_fwd(d, vec && !force_scalar(), true, a, stream))
                      : from_hip(launch_fwd(d, pick_path(d, cols, vec), true, a, stream));
    if (st == LN_OK && mask_out) st = from_hip(launch_dropout_mask(a, stream));
    return st;
}

ln_status_t ln_bwd_dx(const void* dy, const void* x, const void* gamma, const float* mean,
                      const float* rstd, void* dx, float* workspace, size_t workspace_bytes,
                      int64_t rows, int64_t cols, ln_dtype_t dt, hipStream_t stream) {
    const Range range("ln_bwd_dx");
    if (!dy || !x || !gamma || !mean || !rstd || !dx) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::BWD);
    if (st != LN_OK) return st;
    const size_t need = ln_bwd_workspace_bytes(rows, cols);
    if (workspace && workspace_bytes < need) return LN_ERR_WORKSPACE;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float);
    const Span outs[] = {{dx, tb, true}, {workspace, workspace ? need : 0, false}};
    const Span ins[] = {{dy, tb, true}, {x, tb, true}, {gamma, vb, false},
                        {mean, sb, false}, {rstd, sb, false}};
    st = check_aliasing(outs, 2, ins, 5);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(dy) && aligned16(x) && aligned16(gamma) && aligned16(dx) &&
                     (cols * (int64_t)es) % 16 == 0;
    BwdArgs a{};
    a.dy = dy; a.x = x; a.gamma = gamma; a.mean = mean; a.rstd = rstd; a.dx = dx;
    a.ws = workspace; a.ws_vec = aligned16(workspace);
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.parts = bwd_partitions(rows, cols);
    a.inv_m = (float)(1.0 / (double)cols);
    const BwdMode mode = workspace ? BwdMode::DX_PARTIALS : BwdMode::DX;
    if (staged(cols)) return from_hip(launch_wide_bwd(d, vec && !force_scalar(), mode, a, stream));
    return from_hip(launch_bwd(d, pick_bwd_path(d, cols, vec), mode, a,
                               stream));
}

ln_status_t ln_bwd_dgamma_dbeta(const void* dy, const void* x, const float* mean,
                                const float* rstd, float* dgamma, float* dbeta, float* workspace,
                                size_t workspace_bytes, int partials_ready, int64_t rows,
                                int64_t cols, ln_dtype_t dt, hipStream_t stream) {
    const Range range("ln_bwd_dgamma_dbeta");
    if (!dgamma || !dbeta || !workspace) return LN_ERR_NULL;
    if (!partials_ready && (!dy || !x || !mean || !rstd)) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::BWD);
    if (st != LN_OK) return st;
    const size_t need = ln_bwd_workspace_bytes(rows, cols);
    if (workspace_bytes < need) return LN_ERR_WORKSPACE;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float), cb = (size_t)cols * sizeof(float);
    const Span outs[] = {{dgamma, cb, false}, {dbeta, cb, false},
                         {partials_ready ? nullptr : workspace, need, false}};
    const Span ins[] = {{dy, tb, true}, {x, tb, true}, {mean, sb, false}, {rstd, sb, false},
                        {partials_ready ? workspace : nullptr, need, false}};
    st = check_aliasing(outs, 3, ins, 5);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const int64_t parts = bwd_partitions(rows, cols);
    if (!partials_ready) {
        const bool vec = aligned16(dy) && aligned16(x) && (cols * (int64_t)es) % 16 == 0;
        BwdArgs a{};
        a.dy = dy; a.x = x; a.mean = mean; a.rstd = rstd; a.ws = workspace;
        a.ws_vec = aligned16(workspace);
        a.rows = rows; a.m = cols;
        a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
        a.parts = parts;
        a.inv_m = (float)(1.0 / (double)cols);
        st = staged(cols)
                 ? from_hip(launch_wide_bwd(d, vec && !force_scalar(), BwdMode::PARTIALS, a,
                                            stream))
                 : from_hip(launch_bwd(d, pick_bwd_path(d, cols, vec), BwdMode::PARTIALS, a,
                                       stream));
        if (st != LN_OK) return st;
    }
    FoldOut out{};
    out.p[0] = dgamma;
    out.p[1] = dbeta;
    return from_hip(launch_fold(workspace, parts, cols, 2, out, stream));
}

ln_status_t ln_bwd_noalloc(const void* dy, const void* x, const void* gamma, const float* mean,
                           const float* rstd, void* dx, float* dgamma, float* dbeta,
                           int64_t rows, int64_t cols, ln_dtype_t dt, hipStream_t stream) {
    const Range range("ln_bwd_noalloc");
    if (!dy || !x || !gamma || !mean || !rstd || !dx || !dgamma || !dbeta) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::BWD);
    if (st != LN_OK) return st;
    if (rows == 0) return LN_OK;
    const size_t need = ln_bwd_workspace_bytes(rows, cols);
    if (need > LN_NOALLOC_SCRATCH_BYTES) return LN_ERR_SCRATCH;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float), cb = (size_t)cols * sizeof(float);
    const Span outs[] = {{dx, tb, true}, {dgamma, cb, false}, {dbeta, cb, false}};
    const Span ins[] = {{dy, tb, true}, {x, tb, true}, {gamma, vb, false},
                        {mean, sb, false}, {rstd, sb, false}};
    st = check_aliasing(outs, 3, ins, 5);
    if (st != LN_OK) return st;
    float* ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess || !ws) return LN_ERR_HIP;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(dy) && aligned16(x) && aligned16(gamma) && aligned16(dx) &&
                     (cols * (int64_t)es) % 16 == 0;
    BwdArgs a{};
    a.dy = dy; a.x = x; a.gamma = gamma; a.mean = mean; a.rstd = rstd; a.dx = dx;
    a.ws = ws; a.ws_vec = aligned16(ws);
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.parts = bwd_partitions(rows, cols);
    a.inv_m = (float)(1.0 / (double)cols);
    st = staged(cols)
             ? from_hip(launch_wide_bwd(d, vec && !force_scalar(), BwdMode::DX_PARTIALS, a,
                                        stream))
             : from_hip(launch_bwd(d, pick_bwd_path(d, cols, vec), BwdMode::DX_PARTIALS, a,
                                   stream));
    if (st != LN_OK) return st;
    FoldOut out{};
    out.p[0] = dgamma;
    out.p[1] = dbeta;
    return from_hip(launch_fold(ws, a.parts, cols, 2, out, stream));
}

// Stage 1 of the prologue backward (dresidual, dx and the three kinds of
// column partials); with `fold`, also stage 2 into dgamma/dbeta/dbias.
static ln_status_t prologue_bwd(const void* dy, const void* dz_extra, const void* z,
                                const void* gamma, const float* mean, const float* rstd,
                                void* dresidual, void* dx, float* dgamma, float* dbeta,
                                float* dbias, float* workspace, size_t workspace_bytes,
                                int64_t rows, int64_t cols, float p, uint64_t seed,
                                ln_dtype_t dt, hipStream_t stream, bool fold) {
    if (!dy || !z || !gamma || !mean || !rstd || !dresidual || !dx || !workspace)
        return LN_ERR_NULL;
    if (fold && (!dgamma || !dbeta || !dbias)) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::FWD);
    if (st != LN_OK) return st;
    if (cols > LN_MAX_COLS_DROPOUT_BWD) return LN_ERR_UNSUPPORTED;
    if (!(p >= 0.0f && p < 1.0f)) return LN_ERR_PARAM;
    const size_t need = bias_dropout_residual_ln_bwd_workspace_bytes(rows, cols);
    if (workspace_bytes < need) return LN_ERR_WORKSPACE;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float), cb = fold ? (size_t)cols * sizeof(float) : 0;
    const Span outs[] = {{dresidual, tb, true}, {dx, tb, true}, {dgamma, cb, false},
                         {dbeta, cb, false}, {dbias, cb, false}, {workspace, need, false}};
    const Span ins[] = {{dy, tb, true}, {dz_extra, dz_extra ? tb : 0, true}, {z, tb, true},
                        {gamma, vb, false}, {mean, sb, false}, {rstd, sb, false}};
    st = check_aliasing(outs, 6, ins, 6);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(dy) && (!dz_extra || aligned16(dz_extra)) && aligned16(z) &&
                     aligned16(gamma) && aligned16(dresidual) && aligned16(dx) &&
                     (cols * (int64_t)es) % 16 == 0;
    BwdArgs a{};
    a.dy = dy; a.x = z; a.gamma = gamma; a.mean = mean; a.rstd = rstd; a.dx = dresidual;
    a.dz_extra = dz_extra; a.dx_in = dx; a.ws = workspace;
    a.ws_vec = aligned16(workspace);
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.parts = bwd_partitions(rows, cols);
    a.inv_m = (float)(1.0 / (double)cols);
    a.thr = (uint32_t)std::floor((double)p * 65536.0 + 0.5);
    a.scale = (float)(1.0 / (1.0 - (double)p));
    a.seed_lo = (uint32_t)(seed & 0xffffffffu);
    a.seed_hi = (uint32_t)(seed >> 32);
    st = from_hip(launch_bwd(d, pick_bwd_path(d, cols, vec, true), BwdMode::DROPOUT, a, stream));
    if (st != LN_OK || !fold) return st;
    FoldOut out{};
    out.p[0] = dgamma;
    out.p[1] = dbeta;
    out.p[2] = dbias;
    return from_hip(launch_fold(workspace, a.parts, cols, 3, out, stream));
}

ln_status_t bias_dropout_residual_ln_bwd(const void* dy, const void* dz_extra, const void* z,
                                         const void* gamma, const float* mean,
                                         const float* rstd, void* dresidual, void* dx,
                                         float* dgamma, float* dbeta, float* dbias,
                                         float* workspace, size_t workspace_bytes, int64_t rows,
                                         int64_t cols, float p, uint64_t seed, ln_dtype_t dt,
                                         hipStream_t stream) {
    const Range range("bias_dropout_residual_ln_bwd");
    return prologue_bwd(dy, dz_extra, z, gamma, mean, rstd, dresidual, dx, dgamma, dbeta, dbias,
                        workspace, workspace_bytes, rows, cols, p, seed, dt, stream, true);
}

ln_status_t bias_dropout_residual_ln_bwd_dx(const void* dy, const void* dz_extra, const void* z,
                                            const void* gamma, const float* mean,
                                            const float* rstd, void* dresidual, void* dx,
                                            float* workspace, size_t workspace_bytes,
                                            int64_t rows, int64_t cols, float p, uint64_t seed,
                                            ln_dtype_t dt, hipStream_t stream) {
    const Range range("bias_dropout_residual_ln_bwd_dx");
    return prologue_bwd(dy, dz_extra, z, gamma, mean, rstd, dresidual, dx, nullptr, nullptr,
                        nullptr, workspace, workspace_bytes, rows, cols, p, seed, dt, stream,
                        false);
}

ln_status_t bias_dropout_residual_ln_bwd_fold(const float* workspace, size_t workspace_bytes,
                                              float* dgamma, float* dbeta, float* dbias,
                                              int64_t rows, int64_t cols, hipStream_t stream) {
    const Range range("bias_dropout_residual_ln_bwd_fold");
    if (!workspace || !dgamma || !dbeta || !dbias) return LN_ERR_NULL;
    if (rows < 0 || cols <= 0) return LN_ERR_SHAPE;
    if (cols > LN_MAX_COLS_DROPOUT_BWD || rows > kMaxRows) return LN_ERR_UNSUPPORTED;
    const size_t need = bias_dropout_residual_ln_bwd_workspace_bytes(rows, cols);
    if (workspace_bytes < need) return LN_ERR_WORKSPACE;
    if (rows == 0) return LN_OK;
    const size_t cb = (size_t)cols * sizeof(float);
    const Span outs[] = {{dgamma, cb, false}, {dbeta, cb, false}, {dbias, cb, false}};
    const Span ins[] = {{workspace, need, false}};
    const ln_status_t st = check_aliasing(outs, 3, ins, 1);
    if (st != LN_OK) return st;
    FoldOut out{};
    out.p[0] = dgamma;
    out.p[1] = dbeta;
    out.p[2] = dbias;
    return from_hip(launch_fold(workspace, bwd_partitions(rows, cols), cols, 3, out, stream));
}

ln_status_t add_rmsnorm_fwd(const void* x, const void* residual, const void* gamma,
                            void* residual_out, void* y, float* rstd, int64_t rows, int64_t cols,
                            float eps, ln_dtype_t dt, hipStream_t stream) {
    const Range range("add_rmsnorm_fwd");
    if (!x || !gamma || !y || (residual && !residual_out)) return LN_ERR_NULL;
    if (!residual && residual_out) return LN_ERR_PARAM;
    ln_status_t st = check_shape(rows, cols, dt, Kind::RMS);
    if (st != LN_OK) return st;
    if (!(eps >= 0.0f) || std::isinf(eps)) return LN_ERR_PARAM;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float);
    const Span outs[] = {{residual_out, residual_out ? tb : 0, true}, {y, tb, true},
                         {rstd, sb, false}};
    const Span ins[] = {{x, tb, true}, {residual, residual ? tb : 0, true}, {gamma, vb, false}};
    st = check_aliasing(outs, 3, ins, 3);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(x) && (!residual || aligned16(residual)) && aligned16(gamma) &&
                     (!residual_out || aligned16(residual_out)) && aligned16(y) &&
                     (cols * (int64_t)es) % 16 == 0;
    RmsArgs a{};
    a.x = x; a.residual = residual; a.gamma = gamma; a.residual_out = residual_out; a.y = y;
    a.rstd = rstd;
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.eps = eps;
    a.inv_m = (float)(1.0 / (double)cols);
    return from_hip(launch_rmsnorm_fwd(d, pick_path(d, cols, vec), a, stream));
}

ln_status_t add_rmsnorm_bwd(const void* dy, const void* dz_extra, const void* z,
                            const void* gamma, const float* rstd, void* dz, float* dgamma,
                            float* workspace, size_t workspace_bytes, int64_t rows, int64_t cols,
                            ln_dtype_t dt, hipStream_t stream) {
    const Range range("add_rmsnorm_bwd");
    if (!dy || !z || !gamma || !rstd || !dz || !dgamma || !workspace) return LN_ERR_NULL;
    ln_status_t st = check_shape(rows, cols, dt, Kind::RMS);
    if (st != LN_OK) return st;
    const size_t need = add_rmsnorm_bwd_workspace_bytes(rows, cols);
    if (workspace_bytes < need) return LN_ERR_WORKSPACE;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es, vb = (size_t)cols * es;
    const size_t sb = (size_t)rows * sizeof(float), cb = (size_t)cols * sizeof(float);
    const Span outs[] = {{dz, tb, true}, {dgamma, cb, false}, {workspace, need, false}};
    const Span ins[] = {{dy, tb, true}, {dz_extra, dz_extra ? tb : 0, true}, {z, tb, true},
                        {gamma, vb, false}, {rstd, sb, false}};
    st = check_aliasing(outs, 3, ins, 5);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(dy) && (!dz_extra || aligned16(dz_extra)) && aligned16(z) &&
                     aligned16(gamma) && aligned16(dz) && (cols * (int64_t)es) % 16 == 0;
    BwdArgs a{};
    a.dy = dy; a.x = z; a.gamma = gamma; a.rstd = rstd; a.dx = dz; a.dz_extra = dz_extra;
    a.ws = workspace; a.ws_vec = aligned16(workspace);
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.parts = bwd_partitions(rows, cols);
    a.inv_m = (float)(1.0 / (double)cols);
    st = from_hip(launch_bwd(d, pick_bwd_path(d, cols, vec), BwdMode::RMS, a, stream));
    if (st != LN_OK) return st;
    FoldOut out{};
    out.p[0] = dgamma;
    return from_hip(launch_fold(workspace, a.parts, cols, 1, out, stream));
}

ln_status_t cross_entropy_fwd_bwd(const void* logits, const int64_t* labels, float* loss,
                                  void* dlogits, int64_t rows, int64_t cols, int64_t ld,
                                  float label_smoothing, float grad_scale, ln_dtype_t dt,
                                  hipStream_t stream) {
    const Range range("cross_entropy_fwd_bwd");
    if (!logits || !labels || !loss) return LN_ERR_NULL;
    if (!valid_dtype(dt)) return LN_ERR_DTYPE;
    if (rows < 0 || cols <= 0 || ld < cols) return LN_ERR_SHAPE;
    if (ld > LN_MAX_COLS_STREAM || rows > kMaxRows) return LN_ERR_UNSUPPORTED;
    const int64_t max_ld = dt == LN_F32 ? LN_MAX_COLS_XENT_F32 : LN_MAX_COLS_XENT_16;
    if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f)) return LN_ERR_PARAM;
    if (!std::isfinite(grad_scale)) return LN_ERR_PARAM;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)ld * es;
    const Span outs[] = {{dlogits, dlogits ? tb : 0, true}, {loss, (size_t)rows * 4, false}};
    const Span ins[] = {{logits, tb, true}, {labels, (size_t)rows * 8, false}};
    ln_status_t st = check_aliasing(outs, 2, ins, 2);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const int E = elems_per_slot(d);
    const bool vec = aligned16(logits) && (!dlogits || aligned16(dlogits)) &&
                     (ld * (int64_t)es) % 16 == 0;
    XeArgs a{};
    a.x = logits; a.labels = labels; a.loss = loss; a.dx = dlogits;
    a.rows = rows; a.cols = cols; a.ld = ld;
    a.nvalid = (cols + E - 1) / E;
    a.nslots = (ld + E - 1) / E;
    a.alpha = label_smoothing;
    a.inv_v = (float)(1.0 / (double)cols);
    a.scale = grad_scale;
    if (ld > max_ld || force_two_pass()) {
        // past the register layouts: rows that the registers and LDS of one
        // workgroup hold (vector path) are still read once; the rest take
        // the two-pass walk
        const bool vec_ok = vec && !force_scalar();
        if (vec_ok && !force_two_pass() && a.nslots <= kXeLdsMaxSlots)
            return from_hip(launch_xent_lds(d, a, stream));
        return from_hip(launch_xent_stream(d, vec_ok, a, stream));
    }
    return from_hip(launch_xent(d, pick_xent_path(d, a.nslots, vec), a, stream));
}

ln_status_t attn_softmax_fwd(const void* x, const void* mask, int64_t rows_per_mask, void* y,
                             void* y_dropped, int64_t rows, int64_t cols, float scale,
                             int causal, float p, uint64_t seed, ln_dtype_t dt,
                             hipStream_t stream) {
    const Range range("attn_softmax_fwd");
    if (!x || !y) return LN_ERR_NULL;
    ln_status_t st = check_shape_stream(rows, cols, dt);
    if (st != LN_OK) return st;
    if (!std::isfinite(scale) || (causal != 0 && causal != 1)) return LN_ERR_PARAM;
    if (!(p >= 0.0f && p < 1.0f)) return LN_ERR_PARAM;
    if (mask && rows_per_mask < 1) return LN_ERR_PARAM;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es;
    const int64_t mrows = mask ? (rows + rows_per_mask - 1) / rows_per_mask : 0;
    const Span outs[] = {{y, tb, true}, {y_dropped, y_dropped ? tb : 0, true}};
    const Span ins[] = {{x, tb, true}, {mask, (size_t)mrows * (size_t)cols * es, false}};
    st = check_aliasing(outs, 2, ins, 2);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(x) && aligned16(y) && (!mask || aligned16(mask)) &&
                     (!y_dropped || aligned16(y_dropped)) && (cols * (int64_t)es) % 16 == 0;
    SmArgs a{};
    a.x = x; a.mask = mask; a.out = y; a.out2 = y_dropped;
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.rows_per_mask = mask ? rows_per_mask : 1;
    a.scale = scale;
    a.causal = causal;
    a.thr = (uint32_t)std::floor((double)p * 65536.0 + 0.5);
    a.pscale = (float)(1.0 / (1.0 - (double)p));
    a.seed_lo = (uint32_t)(seed & 0xffffffffu);
    a.seed_hi = (uint32_t)(seed >> 32);
    if (cols > softmax_max_cols(dt, false) || force_two_pass()) {
        // past the register layouts: rows on the vector path are still held
        // on chip, with or without the dropped copy, up to
        // LN_MAX_COLS_SOFTMAX_PLAIN_FWD_16 / _F32 columns (the scores in
        // registers; a mask row in registers and LDS); the rest take the
        // two-pass walk
        const bool vec_ok = vec && !force_scalar();
        const int64_t plain_max =
            dt == LN_F32 ? LN_MAX_COLS_SOFTMAX_PLAIN_FWD_F32 : LN_MAX_COLS_SOFTMAX_PLAIN_FWD_16;
        if (vec_ok && !force_two_pass() && mask && cols <= plain_max)
            return from_hip(d == Dt::F32   ? launch_softmax_fwd_mask_lds_f32(a, stream)
                            : d == Dt::F16 ? launch_softmax_fwd_mask_lds_f16(a, stream)
                                           : launch_softmax_fwd_mask_lds_bf16(a, stream));
        if (vec_ok && !force_two_pass() && !mask && cols <= plain_max) {
            const int64_t per_lane = (a.nslots + 1023) / 1024;
            const int v = per_lane <= 10 ? 10 : per_lane <= 12 ? 12 : per_lane <= 14 ? 14 : 16;
            return from_hip(d == Dt::F32   ? launch_softmax_long_fwd_f32(v, a, stream)
                            : d == Dt::F16 ? launch_softmax_long_fwd_f16(v, a, stream)
                                           : launch_softmax_long_fwd_bf16(v, a, stream));
        }
        return from_hip(launch_softmax_stream(d, vec_ok, false, a, stream));
    }
    return from_hip(launch_softmax(d, pick_softmax_path(d, cols, vec, false), false, a, stream));
}

ln_status_t attn_softmax_bwd(const void* dy, const void* y, void* dx, int64_t rows,
                             int64_t cols, float scale, int causal, float p, uint64_t seed,
                             ln_dtype_t dt, hipStream_t stream) {
    const Range range("attn_softmax_bwd");
    if (!dy || !y || !dx) return LN_ERR_NULL;
    ln_status_t st = check_shape_stream(rows, cols, dt);
    if (st != LN_OK) return st;
    if (!std::isfinite(scale) || (causal != 0 && causal != 1)) return LN_ERR_PARAM;
    if (!(p >= 0.0f && p < 1.0f)) return LN_ERR_PARAM;
    if (rows == 0) return LN_OK;
    const size_t es = elem_bytes(dt);
    const size_t tb = (size_t)rows * (size_t)cols * es;
    const Span outs[] = {{dx, tb, true}};
    const Span ins[] = {{dy, tb, true}, {y, tb, true}};
    st = check_aliasing(outs, 1, ins, 2);
    if (st != LN_OK) return st;

    const Dt d = static_cast<Dt>(dt);
    const bool vec = aligned16(dy) && aligned16(y) && aligned16(dx) &&
                     (cols * (int64_t)es) % 16 == 0;
    SmArgs a{};
    a.x = dy; a.y = y; a.out = dx;
    a.rows = rows; a.m = cols;
    a.nslots = (cols + elems_per_slot(d) - 1) / elems_per_slot(d);
    a.rows_per_mask = 1;
    a.scale = scale;
    a.causal = causal;
    a.thr = (uint32_t)std::floor((double)p * 65536.0 + 0.5);
    a.pscale = (float)(1.0 / (1.0 - (double)p));
    a.seed_lo = (uint32_t)(seed & 0xffffffffu);
    a.seed_hi = (uint32_t)(seed >> 32);
    if (cols > softmax_max_cols(dt, true) || force_two_pass()) {
        // past the register layouts: rows on the vector path are still held
        // on chip, dy and y read once, up to LN_MAX_COLS_SOFTMAX_PLAIN_BWD_16
        // / _F32 columns; the rest take the two-pass walk
        const bool vec_ok = vec && !force_scalar();
        const int64_t plain_max =
            dt == LN_F32 ? LN_MAX_COLS_SOFTMAX_PLAIN_BWD_F32 : LN_MAX_COLS_SOFTMAX_PLAIN_BWD_16;
        if (vec_ok && !force_two_pass() && cols <= plain_max)
            return from_hip(d == Dt::F32   ? launch_softmax_bwd_lds_f32(a, stream)
                            : d == Dt::F16 ? launch_softmax_bwd_lds_f16(a, stream)
                                           : launch_softmax_bwd_lds_bf16(a, stream));
        return from_hip(launch_softmax_stream(d, vec_ok, true, a, stream));
    }
    return from_hip(launch_softmax(d, pick_softmax_path(d, cols, vec, true), true, a, stream));
}

ln_status_t ln_debug_force_staged(int on) {
    g_force_staged.store(on ? 1 : 0, std::memory_order_relaxed);
    return LN_OK;
}

ln_status_t ln_debug_force_two_pass(int on) {
    g_force_two_pass.store(on ? 1 : 0, std::memory_order_relaxed);
    return LN_OK;
}

ln_status_t ln_debug_force_grid(int workgroups_per_cu) {
    g_force_grid.store(workgroups_per_cu, std::memory_order_relaxed);
    return LN_OK;
}

ln_status_t ln_debug_force_path(int lanes_per_row, int slots_per_lane, int scalar) {
    const int g = lanes_per_row, v = slots_per_lane;
    if (g != 0 && !have_instance(true, g, v) && !have_instance(false, g, v) &&
        !in_list(kDrop32, MBROW_N(kDrop32), g, v) && !in_list(kDrop16, MBROW_N(kDrop16), g, v) &&
        !in_list(kSm32, MBROW_N(kSm32), g, v) && !in_list(kSm16, MBROW_N(kSm16), g, v) &&
        !in_list(kXe32, MBROW_N(kXe32), g, v) && !in_list(kXe16, MBROW_N(kXe16), g, v))
        return LN_ERR_UNSUPPORTED;
    g_force_g.store(lanes_per_row, std::memory_order_relaxed);
    g_force_v.store(lanes_per_row ? slots_per_lane : 0, std::memory_order_relaxed);
    g_force_scalar.store(scalar ? 1 : 0, std::memory_order_relaxed);
    return LN_OK;
}

}  // extern "C"
