// stream.hip -- attention softmax (forward, backward) and cross-entropy over
// rows too long to hold in one workgroup's registers, for gfx950.  Compiled
// once per storage type (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// One workgroup of 1024 lanes per row walks the row in chunks of 64 KB
// (four 16-byte slots per lane) twice.  Pass A reduces: the online softmax
// state of "02 · llmc/ 的 CUDA kernel 层" §6.1 (a running maximum and a sum of
// exp(x - max) rescaled when the maximum grows, plus sum x for the
// cross-entropy), or the dot product sum g * y of the softmax backward
// ("Accelerating Transformer on GPU (II)" §3).  The lanes' states are merged
// in a fixed order (one butterfly per wave, then the waves in order through
// LDS).  Pass B writes the output exactly as the register kernels do (the
// same mask words, exp2 form and dropout).  Pass A keeps the row's first two
// chunks (128 KB) in LDS, each lane its own slots, and the 16-bit kernels
// with registers to spare one or two more chunks in registers, so pass B
// takes those from on chip and re-reads only the rest of the row from global
// memory ("02 · llmc/ 的 CUDA kernel 层" §3.1: what fits on chip is read
// once), last chunk first, while L2 may still hold it.  The rest is read
// twice (the backward reads dy and y), against once for rows that fit in
// registers.
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

constexpr int kSnt = 1024;            // lanes per row (one workgroup)
constexpr int kSnw = kSnt / 64;       // waves per row
// 16-byte slots per lane per chunk: four when one tensor is walked, two when
// two are (the next chunk is in flight as well, in 128 registers per lane)
constexpr int kSu1 = 4;
constexpr int kSu2 = 2;
// Chunks of a row kept in LDS between the passes (64 KB each: four slots of
// one tensor or two slots of two, per lane).
constexpr int kStaged = 2;
// Further chunks kept in registers, after the LDS-staged ones, by the 16-bit
// vector-path kernels whose registers allow it (16 per lane per chunk): two
// in the softmax backward, one in the cross-entropy and in the softmax
// forward without a mask.
template <class S>
constexpr int kRegStagedBwd = S::E == 8 ? 2 : 0;   // at most 2
template <class S>
constexpr int kRegStagedXent = S::E == 8 ? 1 : 0;  // at most 1
template <class S, bool MASK>
constexpr int kRegStagedFwd = S::E == 8 && !MASK ? 1 : 0;   // at most 1

// Merge of the row's lane states: a butterfly per wave, then the waves in
// order through LDS.  Every lane gets the row's state.
__device__ inline XeState row_merge(XeState st, XeState* lds) {
    st = xe_group<64>(st);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[w] = st;
    __syncthreads();
    XeState r = lds[0];
#pragma unroll
    for (int k = 1; k < kSnw; ++k) r = xe_merge(r, lds[k]);
    __syncthreads();   // the next row reuses lds
    return r;
}
__device__ inline float row_sum(float v, float* lds) {
    v = group_sum<64>(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[w] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int k = 1; k < kSnw; ++k) r = r + lds[k];
    __syncthreads();
    return r;
}

// One chunk of a row: slot k of this lane is s = chunk*kSnt*U + k*kSnt +
// lane (a wave covers 1 KB contiguous per k).  Slots at or past `nslot` read
// 0; on the per-element path, columns at or past `lim` read 0.  The first
// pass reads through the caches (LAST = false) so that the second pass, the
// row's last use, finds it in the 256 MB Infinity Cache; the second pass
// reads nontemporally.
template <class S, bool VEC, bool LAST, int U>
__device__ inline void load_chunk(rsrc_t v, int64_t chunk, int nslot, int lim, u32x4 (&out)[U]) {
    constexpr int E = S::E;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int s = (int)(chunk * (kSnt * U)) + k * kSnt + (int)threadIdx.x;
        if constexpr (VEC) {
            const uint32_t off = s < nslot ? (uint32_t)s * 16u : kOob;
            out[k] = LAST ? buf_load_nt(v, off) : buf_load(v, off);
        } else {
            float f[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int col = s * E + e;
                f[e] = elem_load<S>(v, col < lim ? (uint32_t)col * S::BYTES : kOob);
            }
            out[k] = S::pack(f);
            hold_packed(out[k]);   // one slot of element loads in flight at a time
        }
    }
}
template <class S, bool VEC>
__device__ inline void store_slot(rsrc_t v, int s, int nslot, int lim, const float* f) {
    constexpr int E = S::E;
    if constexpr (VEC) {
        buf_store_nt(S::pack(f), v, s < nslot ? (uint32_t)s * 16u : kOob);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int col = s * E + e;
            elem_store<S>(v, col < lim ? (uint32_t)col * S::BYTES : kOob, f[e]);
        }
    }
}

// Online update of a lane's (max, sum of exp(x - max)) by a chunk whose
// values in play have maximum cm: rescale the sum when the maximum grows.
__device__ inline void rescale(XeState& st, float cm) {
    if (cm > st.mx) {
        if (st.mx != -INFINITY) st.z = st.z * exp2_((st.mx - cm) * kLog2e);
        st.mx = cm;
    }
}

// Walk chunks [0, n) with the next chunk's loads in flight while one is used
// (two register buffers, used alternately).  A chunk at or past the end
// reads nothing (its slots are outside the row's view), so the prefetch is
// unconditional: a conditional one would make the wait for the current
// chunk also wait for it, since loads retire in order.
// (The per-element path, PREFETCH = false, has no registers for a second
// buffer and walks the chunks one at a time.)
template <class B, bool PREFETCH, class Fetch, class Use>
__device__ inline void pipelined(int64_t n, Fetch&& fetch, Use&& use) {
    if constexpr (PREFETCH) {
        B b0, b1;
        fetch(int64_t(0), b0);
        for (int64_t c = 0; c < n; c += 2) {
            fetch(c + 1, b1);
            use(c, b0);
            if (c + 1 >= n) break;
            fetch(c + 2, b0);
            use(c + 1, b1);
        }
    } else {
        B b;
        for (int64_t c = 0; c < n; ++c) {
            fetch(c, b);
            use(c, b);
        }
    }
}

// Pass B's walk.  Chunks [0, nst) are read back from the LDS stage by
// `stage`, the rest fetched from global memory.  With prefetch, the walk takes
// the last chunk first, since the chunks pass A read last are the ones most
// likely still in L2, and the staged chunks at the end; a prefetch that would
// fall on a staged chunk is sent to chunk n instead, which reads nothing.
// (The per-element path walks in order: the reverse walk costs it a spill.)
template <class B, bool PREFETCH, class Stage, class Fetch, class Use>
__device__ inline void pipelined_staged(int64_t nst, int64_t n, Stage&& stage, Fetch&& fetch,
                                        Use&& use) {
    auto next = [&](int64_t c) { return c >= nst ? c : n; };
    if constexpr (PREFETCH) {
        B b0, b1;
        fetch(next(n - 1), b0);
        for (int64_t c = n - 1; c >= nst; c -= 2) {
            fetch(next(c - 1), b1);
            use(c, b0);
            if (c - 1 < nst) break;
            fetch(next(c - 2), b0);
            use(c - 1, b1);
        }
        for (int64_t c = nst - 1; c >= 0; --c) {
            stage(c, b1);
            use(c, b1);
        }
    } else {
        B b;
        for (int64_t c = 0; c < nst; ++c) {
            stage(c, b);
            use(c, b);
        }
        for (int64_t c = nst; c < n; ++c) {
            fetch(c, b);
            use(c, b);
        }
    }
}

template <bool MASK>
struct SmChunk {
    static constexpr int U = MASK ? kSu2 : kSu1;
    u32x4 x[U];
    u32x4 m[MASK ? U : 1];
};
struct DyChunk {
    static constexpr int U = kSu2;
    u32x4 d[U];
    u32x4 y[U];
};
struct XChunk {
    static constexpr int U = kSu1;
    u32x4 x[U];
};

// ---------------------------------------------------------------------------
// Softmax forward: y = softmax(scale * x + mask, causal), optional dropped y.
// ---------------------------------------------------------------------------
template <class S, bool VEC, bool MASK>
__global__ __launch_bounds__(kSnt) void softmax_stream_fwd(SmArgs a) {
    constexpr int E = S::E;
    constexpr int kSu = SmChunk<MASK>::U;
    constexpr int kSchunk = kSnt * kSu;
    __shared__ XeState lds[kSnw];
    // pass A's first chunks, each lane its own slots (x, then the mask's)
    __shared__ u32x4 stg[kStaged][MASK ? 2 * kSu : kSu][kSnt];
    constexpr int R = VEC ? kRegStagedFwd<S, MASK> : 0;   // and the next R, in registers
    const int tid = threadIdx.x;
    const int m = (int)a.m;
    const int ns = (int)a.nslots;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const rsrc_t vx = row_view<S>(a.x, row, 1, m);
        const rsrc_t vm = MASK ? row_view<S>(a.mask, row / a.rows_per_mask, 1, m) : vx;
        // columns in play: all, or up to the query under the causal mask
        const int lim = a.causal ? (int)(row % m) + 1 : m;
        const int nlive = (lim + E - 1) / E;                       // slots in play
        const int64_t clive = (nlive + kSchunk - 1) / kSchunk;      // chunks in play
        const int64_t call = (ns + kSchunk - 1) / kSchunk;
        auto fetch = [&](auto last) {
            return [&](int64_t c, SmChunk<MASK>& b) {
                load_chunk<S, VEC, decltype(last)::value, kSu>(vx, c, nlive, lim, b.x);
                if constexpr (MASK) load_chunk<S, VEC, false, kSu>(vm, c, nlive, lim, b.m);
            };
        };
        // scaled, masked scores of a chunk (-inf outside the columns in play)
        auto scores = [&](int64_t c, const SmChunk<MASK>& b, float (&t)[kSu][E]) {
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                float xv[E], mv[E];
                S::unpack(b.x[k], xv);
                if constexpr (MASK) S::unpack(b.m[k], mv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float v = a.scale * xv[e];
                    if constexpr (MASK) v = v + mv[e];
                    t[k][e] = s * E + e < lim ? v : -INFINITY;
                }
            }
        };
        XeState st{-INFINITY, 0.0f, 0.0f};
        SmChunk<MASK> k0;   // the chunk after the staged ones (if R = 1)
        pipelined<SmChunk<MASK>, VEC>(clive, fetch(std::false_type{}),
                                 [&](int64_t c, const SmChunk<MASK>& b) {
            if (c < kStaged) {   // read back by this lane only: no barrier
#pragma unroll
                for (int k = 0; k < kSu; ++k) {
                    stg[c][k][tid] = b.x[k];
                    if constexpr (MASK) stg[c][kSu + k][tid] = b.m[k];
                }
            }
            if (R > 0 && c == kStaged) k0 = b;   // uniform
            float t[kSu][E];
            scores(c, b, t);
            float cm = -INFINITY;
#pragma unroll
            for (int k = 0; k < kSu; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) cm = fmaxf(cm, t[k][e]);
            rescale(st, cm);
            const float nm = st.mx == -INFINITY ? 0.0f : -st.mx * kLog2e;
#pragma unroll
            for (int k = 0; k < kSu; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) st.z += exp2_(fmaf(t[k][e], kLog2e, nm));
        });
        st = row_merge(st, lds);
        const bool live_row = st.mx != -INFINITY;
        const float nm = live_row ? -st.mx * kLog2e : 0.0f;
        const float inv = live_row ? 1.0f / st.z : 0.0f;
        const float inv_kept = inv * a.pscale;
        const rsrc_t vy = row_view<S>(a.out, row, 1, m);
        const rsrc_t vd = row_view<S>(a.out2 ? a.out2 : a.out, row, 1, m);
        // every chunk of the row is written; chunks past the query read
        // nothing and give y = 0
        auto staged = [&](int64_t c, SmChunk<MASK>& b) {
            if (R == 0 || c < kStaged) {   // uniform
#pragma unroll
                for (int k = 0; k < kSu; ++k) {
                    b.x[k] = stg[c][k][tid];
                    if constexpr (MASK) b.m[k] = stg[c][kSu + k][tid];
                }
            }
            if (R > 0 && c == kStaged) b = k0;
        };
        pipelined_staged<SmChunk<MASK>, VEC>(clive < kStaged + R ? clive : kStaged + R, call,
                                             staged,
                                             fetch(std::true_type{}),
                                             [&](int64_t c, const SmChunk<MASK>& b) {
            float t[kSu][E];
            scores(c, b, t);
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                float yv[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    t[k][e] = exp2_(fmaf(t[k][e], kLog2e, nm));
                    yv[e] = t[k][e] * inv;
                }
                store_slot<S, VEC>(vy, s, ns, m, yv);
                if (a.out2) {
                    const u32x4 w = dropout_words(row, s * E, a.seed_lo, a.seed_hi, a.thr);
                    float dv[E];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        dv[e] = kept<E>(w, s * E, e, a.thr) ? t[k][e] * inv_kept : 0.0f;
                    store_slot<S, VEC>(vd, s, ns, m, dv);
                }
            }
        });
    }
}

// ---------------------------------------------------------------------------
// Softmax backward: g = keep ? dy / (1 - p) : 0, s = sum g * y,
// dx = scale * y * (g - s).
// ---------------------------------------------------------------------------
template <class S, bool VEC>
__global__ __launch_bounds__(kSnt) void softmax_stream_bwd(SmArgs a) {
    constexpr int E = S::E;
    constexpr int kSu = DyChunk::U;
    constexpr int kSchunk = kSnt * kSu;
    __shared__ float lds[kSnw];
    __shared__ u32x4 stg[kStaged][2 * kSu][kSnt];   // pass A's first chunks: dy, then y
    constexpr int R = VEC ? kRegStagedBwd<S> : 0;    // and the next R, in registers
    const int tid = threadIdx.x;
    const int m = (int)a.m;
    const int ns = (int)a.nslots;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const rsrc_t vdy = row_view<S>(a.x, row, 1, m);
        const rsrc_t vyy = row_view<S>(a.y, row, 1, m);
        const int lim = a.causal ? (int)(row % m) + 1 : m;   // y = 0 past the query
        const int nlive = (lim + E - 1) / E;
        const int64_t clive = (nlive + kSchunk - 1) / kSchunk;
        const int64_t call = (ns + kSchunk - 1) / kSchunk;
        auto fetch = [&](auto last) {
            return [&](int64_t c, DyChunk& b) {
                load_chunk<S, VEC, decltype(last)::value, kSu>(vdy, c, nlive, lim, b.d);
                load_chunk<S, VEC, decltype(last)::value, kSu>(vyy, c, nlive, lim, b.y);
            };
        };
        // g and y of one chunk (0 outside the columns in play)
        auto grads = [&](int64_t c, const DyChunk& b, float (&g)[kSu][E], float (&y)[kSu][E]) {
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                const u32x4 w = dropout_words(row, s * E, a.seed_lo, a.seed_hi, a.thr);
                float dv[E];
                S::unpack(b.d[k], dv);
                S::unpack(b.y[k], y[k]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const bool in = s * E + e < lim;
                    g[k][e] = (in && kept<E>(w, s * E, e, a.thr)) ? dv[e] * a.pscale : 0.0f;
                    if (!in) y[k][e] = 0.0f;
                }
            }
        };
        float sum = 0.0f;
        DyChunk k0, k1;   // the chunks after the staged ones (R of them used)
        pipelined<DyChunk, VEC>(clive, fetch(std::false_type{}), [&](int64_t c, const DyChunk& b) {
            if (c < kStaged) {   // read back by this lane only: no barrier
#pragma unroll
                for (int k = 0; k < kSu; ++k) {
                    stg[c][k][tid] = b.d[k];
                    stg[c][kSu + k][tid] = b.y[k];
                }
            }
            if (R > 0 && c == kStaged) k0 = b;   // uniform
            if (R > 1 && c == kStaged + 1) k1 = b;
            float g[kSu][E], y[kSu][E];
            grads(c, b, g, y);
#pragma unroll
            for (int k = 0; k < kSu; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) sum = fmaf(g[k][e], y[k][e], sum);
        });
        sum = row_sum(sum, lds);
        const rsrc_t vdx = row_view<S>(a.out, row, 1, m);
        auto staged = [&](int64_t c, DyChunk& b) {
            if (R == 0 || c < kStaged) {   // uniform
#pragma unroll
                for (int k = 0; k < kSu; ++k) {
                    b.d[k] = stg[c][k][tid];
                    b.y[k] = stg[c][kSu + k][tid];
                }
            }
            if (R > 0 && c == kStaged) b = k0;
            if (R > 1 && c == kStaged + 1) b = k1;
        };
        pipelined_staged<DyChunk, VEC>(clive < kStaged + R ? clive : kStaged + R, call, staged,
                                       fetch(std::true_type{}),
                                       [&](int64_t c, const DyChunk& b) {
            float g[kSu][E], y[kSu][E];
            grads(c, b, g, y);
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                float dx[E];
#pragma unroll
                for (int e = 0; e < E; ++e) dx[e] = a.scale * (y[k][e] * (g[k][e] - sum));
                store_slot<S, VEC>(vdx, s, ns, m, dx);
            }
        });
    }
}

// ---------------------------------------------------------------------------
// Cross-entropy with label smoothing: loss and dx = scale * (q - p).
// ---------------------------------------------------------------------------
template <class S, bool VEC>
__global__ __launch_bounds__(kSnt) void xent_stream(XeArgs a) {
    constexpr int E = S::E;
    constexpr int kSu = XChunk::U;
    constexpr int kSchunk = kSnt * kSu;
    __shared__ XeState lds[kSnw];
    __shared__ u32x4 stg[kStaged][kSu][kSnt];   // pass A's first chunks
    constexpr int R = VEC ? kRegStagedXent<S> : 0;   // and the next R, in registers
    const int tid = threadIdx.x;
    const int cols = (int)a.cols;
    const int ld = (int)a.ld;
    const int nv = (int)a.nvalid;
    const int ns = (int)a.nslots;
    const int64_t cv = (nv + kSchunk - 1) / kSchunk;
    const int64_t call = (ns + kSchunk - 1) / kSchunk;
    const float alpha = a.alpha;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const rsrc_t vx = row_view<S>(a.x, row, 1, ld);
        const int64_t label = a.labels[row];
        const bool ignored = label < 0;
        const bool bad = label >= cols;
        const bool no_target = ignored || bad;
        const float xl = no_target ? 0.0f : elem_load<S>(vx, (uint32_t)label * S::BYTES);
        auto fetch = [&](auto last) {
            return [&](int64_t c, XChunk& b) {
                load_chunk<S, VEC, decltype(last)::value, kSu>(vx, c, nv, cols, b.x);
            };
        };
        XeState st{-INFINITY, 0.0f, 0.0f};
        XChunk k0;   // the chunk after the staged ones (if R = 1)
        pipelined<XChunk, VEC>(cv, fetch(std::false_type{}), [&](int64_t c, const XChunk& b) {
            if (c < kStaged) {   // read back by this lane only: no barrier
#pragma unroll
                for (int k = 0; k < kSu; ++k) stg[c][k][tid] = b.x[k];
            }
            if (R > 0 && c == kStaged) k0 = b;   // uniform
            float cm = -INFINITY;
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                float f[E];
                S::unpack(b.x[k], f);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const bool in = s * E + e < cols;
                    cm = fmaxf(cm, in ? f[e] : -INFINITY);
                    st.sx += in ? f[e] : 0.0f;
                }
            }
            rescale(st, cm);
            const float nm = st.mx == -INFINITY ? 0.0f : -st.mx * kLog2e;
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                float f[E];
                S::unpack(b.x[k], f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    st.z += s * E + e < cols ? exp2_(fmaf(f[e], kLog2e, nm)) : 0.0f;
            }
        });
        st = row_merge(st, lds);
        if (threadIdx.x == 0) {
            const float l = logf(st.z) + (1.0f - alpha) * (st.mx - xl) +
                            alpha * (st.mx - st.sx * a.inv_v);
            a.loss[row] = ignored ? 0.0f : (bad ? NAN : l);
        }
        if (a.dx == nullptr) continue;   // uniform
        const float nm = -st.mx * kLog2e;
        const float siz = a.scale * (1.0f / st.z);
        const float pa = alpha * a.inv_v;
        const float nsp = -(a.scale * pa);
        const float nsl = -(a.scale * (pa + (1.0f - alpha)));
        const float fill = ignored ? 0.0f : NAN;
        const rsrc_t vd = row_view<S>(a.dx, row, 1, ld);
        auto staged = [&](int64_t c, XChunk& b) {
            if (R == 0 || c < kStaged) {   // uniform
#pragma unroll
                for (int k = 0; k < kSu; ++k) b.x[k] = stg[c][k][tid];
            }
            if (R > 0 && c == kStaged) b = k0;
        };
        pipelined_staged<XChunk, VEC>(cv < kStaged + R ? cv : kStaged + R, call, staged,
                                      fetch(std::true_type{}), [&](int64_t c, const XChunk& b) {
#pragma unroll
            for (int k = 0; k < kSu; ++k) {
                const int s = (int)(c * kSchunk) + k * kSnt + (int)threadIdx.x;
                float f[E], out[E];
                S::unpack(b.x[k], f);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int col = s * E + e;
                    const float q = exp2_(fmaf(f[e], kLog2e, nm));
                    float d = fmaf(q, siz, col == label ? nsl : nsp);
                    if (no_target) d = fill;
                    out[e] = col < cols ? d : 0.0f;   // padding columns get 0
                }
                store_slot<S, VEC>(vd, s, ns, ld, out);
            }
        });
    }
}

template <class K, class A>
static hipError_t launch_rows(K kernel, const A& a, hipStream_t s) {
    const int64_t grid = persistent_grid(reinterpret_cast<const void*>(kernel), kSnt, a.rows);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kSnt), 0, s, a);
    return hipGetLastError();
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_softmax_stream_, MBROW_SUFFIX)(bool vec, bool backward,
                                                           const SmArgs& a, hipStream_t s) {
    if (backward)
        return vec ? launch_rows(softmax_stream_bwd<St, true>, a, s)
                   : launch_rows(softmax_stream_bwd<St, false>, a, s);
    if (a.mask)
        return vec ? launch_rows(softmax_stream_fwd<St, true, true>, a, s)
                   : launch_rows(softmax_stream_fwd<St, false, true>, a, s);
    return vec ? launch_rows(softmax_stream_fwd<St, true, false>, a, s)
               : launch_rows(softmax_stream_fwd<St, false, false>, a, s);
}
hipError_t MBROW_CAT(launch_xent_stream_, MBROW_SUFFIX)(bool vec, const XeArgs& a,
                                                        hipStream_t s) {
    return vec ? launch_rows(xent_stream<St, true>, a, s) : launch_rows(xent_stream<St, false>, a, s);
}

}  // namespace mbrow
