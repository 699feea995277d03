// xent.hip -- fused cross-entropy forward and backward for gfx950 (label
// smoothing, loss and gradient in one pass).  Compiled once per storage type
// (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// "Accelerating Transformer on GPU (I)" §5.2: with q = softmax(x) and the
// smoothed target p = (1 - a)[j == label] + a/V, the loss is
// log Z + m - [(1 - a) x_label + (a/V) sum x] (m the row maximum,
// Z = sum exp(x - m)) and its gradient is q - p, an elementwise difference,
// so one kernel reduces the row and writes the gradient.  "02 · llmc/ 的 CUDA
// kernel 层" §6.1: over a vocabulary-wide row the probabilities are never
// stored; the row's max and sum come from one online softmax reduction and
// the logits can be overwritten by the gradient in the same kernel.
//
// Here a row is held in registers across G lanes (up to 1024 lanes of one
// workgroup: 65536 fp32 or 131072 16-bit classes),
// so it is read from HBM once and written once.  Each lane reduces its own
// values to (max, sum of exp(x - max), sum x), the lanes merge those states
// in one butterfly (and one LDS exchange across the waves of a row), x at the
// label is read directly, and the gradient pass re-reads the registers.
// Columns in [V, ld) are padding: not used, and written as 0 in the gradient.
#include "ln_device.hpp"
#include "ln_launch.hpp"
#include "online_softmax.hpp"

#ifndef MBROW_DT
#error "compile with -DMBROW_DT=0|1|2"
#endif

namespace mbrow {

#if MBROW_DT == 0
using St = StF32;
#define MBROW_SUFFIX f32
#elif MBROW_DT == 1
using St = StF16;
#define MBROW_SUFFIX f16
#else
using St = StBF16;
#define MBROW_SUFFIX bf16
#endif

template <int G>
struct XeGeometry {
    static constexpr int NT = G <= 256 ? 256 : G;   // threads per workgroup
    static constexpr int ROWS = NT / G;              // rows per block
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
};

template <class S, int G, int V, bool VEC>
__global__ __launch_bounds__(XeGeometry<G>::NT) void xent_kernel(XeArgs a) {
    constexpr int E = S::E;
    constexpr int ROWS = XeGeometry<G>::ROWS;
    constexpr int WPR = XeGeometry<G>::WPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lg = tid % G;
    const int rloc = tid / G;
    const int ld = (int)a.ld;
    const int cols = (int)a.cols;
    const int nv = (int)a.nvalid;    // slots holding at least one class
    const int ns = (int)a.nslots;    // slots of the padded row
    const int64_t nblk = (a.rows + ROWS - 1) / ROWS;
    const bool grad = a.dx != nullptr;   // uniform

    // Slot i of this lane covers columns (i*G + lg)*E + e, e < E: column
    // c(i, e) = base + i*G*E + e with base = lg*E, so "column < cols" is
    // "i*G*E + e < cols - base" against a compile-time left side.
    const int base = lg * E;
    // vector path: byte offset of slot i in the wave's row view is
    // rbase + i*G*16 (rbase: the lane's row within the wave and its first
    // slot); slots past the classes are not read (kOob), slots past the
    // padded row are not written
    const uint32_t rbase = slot_offset<S, G>(tid, 0, ld, true);
    // per-element path: byte offset of the lane's first column in the view
    const uint32_t ebase = (uint32_t)((G <= 64 ? (tid & 63) / G : 0) * ld + base) * S::BYTES;
    auto slot_off = [&](uint32_t rb, int i, int nslot) {
        return i * G + lg < nslot ? rb + (uint32_t)(i * G * 16) : kOob;
    };
    const int wrow = wave_first_row<G>(tid);
    auto view = [&](const void* t, int64_t blk) {
        const int64_t row0 = blk * ROWS + wrow;
        const int64_t left = a.rows - row0;
        return row_view<S>(t, row0, left < WaveRows<G>::N ? left : WaveRows<G>::N, ld);
    };
    __shared__ XeState red[2][ROWS][WPR];   // cross-wave exchange, double-buffered
    const float inv_v = a.inv_v;
    const float alpha = a.alpha;

    int it = 0;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x, ++it) {
        const int64_t row = blk * ROWS + rloc;
        const bool rok = row < a.rows;
        const int64_t r = rok ? row : 0;
        const int64_t off = r * (int64_t)ld;
        const int64_t label = rok ? a.labels[row] : -1;
        const bool ignored = label < 0;
        const bool bad = label >= cols;
        // x at the label, read directly (one element per row)
        const float xl = (ignored || bad) ? 0.0f : S::load1(a.x, off + label);
        u32x4 xr[V];
        if constexpr (VEC) {
            const rsrc_t vx = view(a.x, blk);
            const uint32_t rb = (uint32_t)opaque((int)rbase);
#pragma unroll
            for (int i = 0; i < V; ++i) xr[i] = buf_load_nt(vx, slot_off(rb, i, nv));
        } else {
            const rsrc_t vx = view(a.x, blk);
            const int lim = opaque(cols - base);
            const uint32_t eb = (uint32_t)opaque((int)ebase);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int c = i * G * E + e;
                    f[e] = elem_load<S>(vx, c < lim ? eb + (uint32_t)c * S::BYTES : kOob);
                }
                xr[i] = S::pack(f);
                // wide rows: at most four slots of element loads in flight
                if constexpr (V * E > 32) {
                    if (i % 4 == 3 || i == V - 1) {
#pragma unroll
                        for (int k = i - i % 4; k <= i; ++k) hold_packed(xr[k]);
                    }
                }
            }
        }
        // This lane's state: max and sum of x, then the exp-sum against the
        // max.  Slots wholly inside the classes take no per-element test; at
        // most one slot of a row is partial, and slots past the classes are
        // skipped (per-slot branches, taken by few waves).
        XeState st{-INFINITY, 0.0f, 0.0f};
        {
            const int lim = opaque(cols - base);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                constexpr int W = G * E;
                float f[E];
                S::unpack(xr[i], f);
                if (i * W + E <= lim) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        st.mx = fmaxf(st.mx, f[e]);
                        st.sx += f[e];
                    }
                } else if (i * W < lim) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if (i * W + e < lim) {
                            st.mx = fmaxf(st.mx, f[e]);
                            st.sx += f[e];
                        }
                    }
                }
            }
        }
        keep_packed(xr);
        {
            const int lim = opaque(cols - base);
            // exp(x - m) = exp2(x log2(e) - m log2(e)), one fma and one exp2
            const float nm = st.mx == -INFINITY ? 0.0f : -st.mx * kLog2e;   // lanes past the row
#pragma unroll
            for (int i = 0; i < V; ++i) {
                constexpr int W = G * E;
                float f[E];
                S::unpack(xr[i], f);
                if (i * W + E <= lim) {
#pragma unroll
                    for (int e = 0; e < E; ++e) st.z += exp2_(fmaf(f[e], kLog2e, nm));
                } else if (i * W < lim) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (i * W + e < lim) st.z += exp2_(fmaf(f[e], kLog2e, nm));
                }
            }
        }
        if constexpr (G <= 64) {
            st = xe_group<G>(st);
        } else {
            st = xe_group<64>(st);
            const int buf = it & 1;
            if (lane == 0) red[buf][rloc][lg / 64] = st;
            __syncthreads();
            st = red[buf][rloc][0];
#pragma unroll
            for (int k = 1; k < WPR; ++k) st = xe_merge(st, red[buf][rloc][k]);
        }
        // loss = log Z + (1 - a)(m - x_label) + a (m - sum x / V)
        if (lg == 0 && rok) {
            const float l = logf(st.z) + (1.0f - alpha) * (st.mx - xl) +
                            alpha * (st.mx - st.sx * inv_v);
            a.loss[row] = ignored ? 0.0f : (bad ? NAN : l);
        }
        if (grad) {
            // dx = scale * (q - p) = exp(x - m) * (scale / Z) - scale * p with
            // p = a/V off the label and a/V + 1 - a at it
            keep_packed(xr);
            const float nm = -st.mx * kLog2e;
            const float siz = a.scale * (1.0f / st.z);
            const float pa = alpha * inv_v;
            const float nsp = -(a.scale * pa);
            const float nsl = -(a.scale * (pa + (1.0f - alpha)));
            const bool no_target = ignored || bad;
            const float fill = ignored ? 0.0f : NAN;   // rows without a target
            const int lim = opaque(cols - base);
            const int rel = opaque((int)(no_target ? -1 : label) - base);
            const rsrc_t vd = view(a.dx, blk);
            const uint32_t rb = (uint32_t)opaque((int)rbase);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                constexpr int W = G * E;
                float f[E], out[E];
                S::unpack(xr[i], f);
                if (!no_target) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        out[e] = fmaf(exp2_(fmaf(f[e], kLog2e, nm)), siz, nsp);
                    if ((unsigned)(rel - i * W) < (unsigned)E) {   // the label is here
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            if (i * W + e == rel)
                                out[e] = fmaf(exp2_(fmaf(f[e], kLog2e, nm)), siz, nsl);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) out[e] = fill;
                }
                if (!(i * W + E <= lim)) {   // padding columns get 0
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (i * W + e >= lim) out[e] = 0.0f;
                }
                if constexpr (VEC) {
                    buf_store_nt(S::pack(out), vd, slot_off(rb, i, ns));
                } else {
                    const int wl = opaque(ld - base);
                    const uint32_t eb = (uint32_t)opaque((int)ebase);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int c = i * W + e;
                        elem_store<S>(vd, c < wl ? eb + (uint32_t)c * S::BYTES : kOob, out[e]);
                    }
                }
            }
        }
    }
}

template <int G, int V, bool VEC>
static hipError_t launch_one(const XeArgs& a, hipStream_t s) {
    constexpr int ROWS = XeGeometry<G>::ROWS;
    const int64_t nblk = (a.rows + ROWS - 1) / ROWS;
    const void* k = reinterpret_cast<const void*>(&xent_kernel<St, G, V, VEC>);
    // one workgroup per block where two or more fit a compute unit (GPT-2's
    // rows 9 % faster; 1024-lane rows keep the persistent walk)
    const int64_t grid = persistent_grid(k, XeGeometry<G>::NT, nblk, 2);
    hipLaunchKernelGGL((xent_kernel<St, G, V, VEC>), dim3((unsigned)grid),
                       dim3(XeGeometry<G>::NT), 0, s, a);
    return hipGetLastError();
}

template <bool VEC>
static hipError_t dispatch(const Path& p, const XeArgs& a, hipStream_t s) {
#define MBROW_CASE(GG, VV) \
    if (p.g == GG && p.v == VV) return launch_one<GG, VV, VEC>(a, s);
#if MBROW_DT == 0
    MBROW_XE_LAYOUTS_F32(MBROW_CASE)
#else
    MBROW_XE_LAYOUTS_16(MBROW_CASE)
#endif
#undef MBROW_CASE
    return hipErrorInvalidValue;
}

// Rows past the register layouts, on the vector path: one workgroup per row
// holds the whole row, each lane's first REG slots in registers and its
// next LDS slots in LDS (XeLds), so the row is still
// read from global memory once ("02 · llmc/ 的 CUDA kernel 层" §3.1: what
// fits on chip is read once; §6.1: the vocabulary-wide row reduced by one
// online softmax and overwritten by its gradient).  The LDS slots are loaded
// straight into LDS (buffer loads with an LDS destination), so all slots
// of a lane are in flight together without staging registers; each wave's
// lanes land in consecutive 16-byte cells, and each lane reads back only the
// cells its own loads wrote.  The arithmetic is the register kernel's, slot
// by slot, in the same order.
template <class S>
__global__ __launch_bounds__(XeLds<S::E>::LANES) void xent_lds_kernel(XeArgs a) {
    constexpr int E = S::E;
    constexpr int G = XeLds<E>::LANES;
    constexpr int VR = XeLds<E>::REG;
    constexpr int VL = XeLds<E>::LDS;
    constexpr int NW = G / 64;
    constexpr int W = G * E;   // columns between consecutive slots of a lane
    __shared__ __attribute__((aligned(16))) u32x4 stage[VL][G];
    __shared__ XeState red[2][NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ld = (int)a.ld;
    const int cols = (int)a.cols;
    const int nv = (int)a.nvalid;
    const int ns = (int)a.nslots;
    const bool grad = a.dx != nullptr;   // uniform
    const int base = tid * E;            // first column of the lane's slot 0
    // Byte offset of slot i of this lane in its row's view, or kOob past
    // `nslot`: formed where it is used from an opaque copy of the lane index,
    // so that no slot's offset stays live between the loads and the stores
    // (32 of them would not fit beside the row).
    auto slot_off = [&](int i, int nslot) {
        const int t = opaque(tid);
        return i * G + t < nslot ? (uint32_t)(t * 16 + i * G * 16) : kOob;
    };
    // LDS slot j of this lane, read where it is used: one slot's registers
    // at a time (the next read is not hoisted above this one)
    auto lds_slot = [&](int j) {
        u32x4 v = stage[j][tid];
        hold_packed(v);
        return v;
    };
    // The per-row constants are formed inside the row loop from opaque
    // scalar copies of the arguments, so they are not hoisted out of it into
    // vector registers that would stay live beside the row.
    auto sreg = [](float v) {
        asm volatile("" : "+s"(v));
        return v;
    };

    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const int64_t label = a.labels[row];
        const bool ignored = label < 0;
        const bool bad = label >= cols;
        // x at the label (one element, uniform per row), loaded before the
        // row and moved to a scalar register once it arrives
        const float xl_v = (ignored || bad) ? 0.0f : S::load1(a.x, row * (int64_t)ld + label);
        const rsrc_t vx = row_view<S>(a.x, row, 1, ld);
        u32x4 xr[VR];
#pragma unroll
        for (int i = 0; i < VR; ++i) xr[i] = buf_load_nt(vx, slot_off(i, nv));
        // the wave's 64 cells of LDS slot j start at stage[j][64 * wave]
        // (the previous row's cells were consumed before its stores)
#pragma unroll
        for (int j = 0; j < VL; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vx, (__attribute__((address_space(3))) void*)&stage[j][64 * wave], 16,
                (int)slot_off(VR + j, nv), 0, 0, kNt);
        const float xl = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, xl_v)));

        // Pass 1: max and sum of x; pass 2: sum of exp(x - max).  Slots
        // wholly inside the classes take no per-element test; slots past
        // them are skipped (their values are not used).
        XeState st{-INFINITY, 0.0f, 0.0f};
        // The lane's L = cols - base columns from its first one: slots
        // i < nfull lie wholly inside the classes, slot i < npart holds at
        // least one (columns e < L - i*W of it).  Each pass forms these from
        // its own opaque copy of L, so the per-slot tests are made again
        // against small inline constants rather than kept live.
        int L, nfull, npart;
        auto limits = [&]() {
            L = opaque(cols - base);
            nfull = L >= E ? (L - E) / W + 1 : 0;
            npart = L > 0 ? (L - 1) / W + 1 : 0;
        };
        limits();
        auto sums = [&](int i, const u32x4& v) {
            float f[E];
            S::unpack(v, f);
            if (i < nfull) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    st.mx = fmaxf(st.mx, f[e]);
                    st.sx += f[e];
                }
            } else if (i < npart) {
                const int r = L - i * W;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (e < r) {
                        st.mx = fmaxf(st.mx, f[e]);
                        st.sx += f[e];
                    }
                }
            }
        };
#pragma unroll
        for (int i = 0; i < VR; ++i) sums(i, xr[i]);
#pragma unroll
        for (int j = 0; j < VL; ++j) sums(VR + j, lds_slot(j));
        keep_packed(xr);
        limits();
        {
            // exp(x - m) = exp2(x log2(e) - m log2(e)), one fma and one exp2
            const float nm = st.mx == -INFINITY ? 0.0f : -st.mx * kLog2e;   // lanes past the row
            auto expsum = [&](int i, const u32x4& v) {
                float f[E];
                S::unpack(v, f);
                if (i < nfull) {
#pragma unroll
                    for (int e = 0; e < E; ++e) st.z += exp2_(fmaf(f[e], kLog2e, nm));
                } else if (i < npart) {
                    const int r = L - i * W;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (e < r) st.z += exp2_(fmaf(f[e], kLog2e, nm));
                }
            };
#pragma unroll
            for (int i = 0; i < VR; ++i) expsum(i, xr[i]);
#pragma unroll
            for (int j = 0; j < VL; ++j) expsum(VR + j, lds_slot(j));
        }
        // the lanes' states: a butterfly per wave, then the waves in order
        // through LDS (double-buffered: one barrier per row)
        st = xe_group<64>(st);
        const int buf = it & 1;
        if (lane == 0) red[buf][wave] = st;
        __syncthreads();
        st = red[buf][0];
#pragma unroll
        for (int k = 1; k < NW; ++k) st = xe_merge(st, red[buf][k]);
        // loss = log Z + (1 - a)(m - x_label) + a (m - sum x / V)
        if (tid == 0) {
            const float alpha = sreg(a.alpha);
            const float l = logf(st.z) + (1.0f - alpha) * (st.mx - xl) +
                            alpha * (st.mx - st.sx * sreg(a.inv_v));
            a.loss[row] = ignored ? 0.0f : (bad ? NAN : l);
        }
        if (!grad) continue;
        // dx = scale * (q - p) = exp(x - m) * (scale / Z) - scale * p with
        // p = a/V off the label and a/V + 1 - a at it
        keep_packed(xr);
        const float nm = -st.mx * kLog2e;
        const float alpha = sreg(a.alpha);
        const float scale = sreg(a.scale);
        const float siz = scale * (1.0f / st.z);
        const float pa = alpha * sreg(a.inv_v);
        const float nsp = -(scale * pa);
        const float nsl = -(scale * (pa + (1.0f - alpha)));
        const bool no_target = ignored || bad;
        const float fill = ignored ? 0.0f : NAN;   // rows without a target
        const int rel = opaque((int)(no_target ? -1 : label) - base);
        limits();
        const rsrc_t vd = row_view<S>(a.dx, row, 1, ld);
        auto grad_slot = [&](int i, const u32x4& v) {
            float f[E], out[E];
            S::unpack(v, f);
            if (!no_target) {
#pragma unroll
                for (int e = 0; e < E; ++e) out[e] = fmaf(exp2_(fmaf(f[e], kLog2e, nm)), siz, nsp);
                if ((unsigned)(rel - i * W) < (unsigned)E) {   // the label is here
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (i * W + e == rel) out[e] = fmaf(exp2_(fmaf(f[e], kLog2e, nm)), siz, nsl);
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) out[e] = fill;
            }
            if (i >= nfull) {   // padding columns get 0
                const int r = L - i * W;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (e >= r) out[e] = 0.0f;
            }
            buf_store_nt(S::pack(out), vd, slot_off(i, ns));
        };
#pragma unroll
        for (int i = 0; i < VR; ++i) grad_slot(i, xr[i]);
#pragma unroll
        for (int j = 0; j < VL; ++j) grad_slot(VR + j, lds_slot(j));
    }
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_xent_, MBROW_SUFFIX)(const Path& p, const XeArgs& a, hipStream_t s) {
    return p.vec ? dispatch<true>(p, a, s) : dispatch<false>(p, a, s);
}
hipError_t MBROW_CAT(launch_xent_lds_, MBROW_SUFFIX)(const XeArgs& a, hipStream_t s) {
    const void* k = reinterpret_cast<const void*>(&xent_lds_kernel<St>);
    constexpr int lanes = XeLds<St::E>::LANES;
    const int64_t grid = persistent_grid(k, lanes, a.rows);
    hipLaunchKernelGGL((xent_lds_kernel<St>), dim3((unsigned)grid), dim3(lanes), 0, s, a);
    return hipGetLastError();
}

}  // namespace mbrow
