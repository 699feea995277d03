// softmax.hip -- attention softmax forward and backward for gfx950.
// Compiled once per storage type (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// Forward ("Accelerating Transformer on GPU (I)" §4.1): every row of scores
// is scaled and gets its additive mask row and the causal mask; then the row
// maximum (one butterfly), exp of the difference and the row sum (a second
// butterfly), and the normalised row is written.  With dropout the dropped
// copy (keep ? y / (1 - p) : 0, keep from the same Philox mask as the
// LayerNorm prologue) is written as well.  One row per group of G lanes,
// held in registers, as in the LayerNorm forward; under the causal mask a
// slot that lies wholly past the query is never read (its buffer offset is
// out of range), so the masked half of the scores costs no reads.
//
// Backward ("Accelerating Transformer on GPU (II)" §3): the dropout backward
// first, in registers (g = keep ? dy / (1 - p) : 0, the mask regenerated from
// the seed), then one dot product s = sum g * y and dx = scale * y * (g - s).
//
// Rows wider than the generic kernel's registers hold unpacked (up to 65536
// 16-bit or 32768 fp32 columns, over 512 or 1024 lanes) take
// softmax_wide_kernel: it holds the block packed, not its unpacked scores,
// and each pass recomputes what it needs from the packed block (the scores;
// in the backward g, from dy and one keep bit per value kept from the first
// pass).  The row is still read once and written once.  Being lean in
// registers it also keeps more rows in flight per CU, which makes it the
// faster forward for 16-bit rows of 512 lanes (16384 columns) as well.
//
// Past those widths, rows on the 16-byte vector path of up to 131072 16-bit
// / 65536 fp32 columns are still held on chip by one 1024-lane workgroup and
// read once: the forward without a mask row in registers (16 slots per
// lane), the forward with a mask row with the mask in registers and LDS
// (softmax_fwd_mask_lds_kernel), the backward with dy in registers and y in
// registers and LDS (softmax_bwd_lds_kernel), each with or without dropout.
// Wider rows take the two-pass walk (stream.hip).
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
struct SmGeometry {
    static constexpr int NT = G <= 256 ? 256 : G;   // threads per workgroup
    static constexpr int ROWS = NT / G;              // rows per block
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
};

template <class S, int G, int V, bool VEC, bool BWD>
__global__ __launch_bounds__(SmGeometry<G>::NT) void softmax_kernel(SmArgs a) {
    constexpr int E = S::E;
    constexpr int ROWS = SmGeometry<G>::ROWS;
    constexpr int WPR = SmGeometry<G>::WPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lg = tid % G;
    const int rloc = tid / G;
    const int m = (int)a.m;
    const int nslots = (int)a.nslots;
    const int64_t nblk = (a.rows + ROWS - 1) / ROWS;

    // slot i of this lane covers columns (i*G + lg)*E .. +E-1
    bool ok[V];
    uint32_t vo[VEC ? V : 1];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        ok[i] = i * G + lg < nslots;
        if constexpr (VEC) vo[i] = slot_offset<S, G>(tid, i, m, ok[i]);
    }
    const int wrow = wave_first_row<G>(tid);
    constexpr int64_t N = WaveRows<G>::N;   // rows of one wave
    auto view = [&](const void* t, int64_t blk) {
        const int64_t row0 = blk * ROWS + wrow;
        const int64_t left = a.rows - row0;
        return row_view<S>(t, row0, left < N ? left : N, m);
    };
    // cross-wave exchange of multi-wave rows: [buffer][max, sum][row][wave]
    __shared__ float red[2][2][ROWS][WPR];
    auto reduce_max = [&](float v, int buf) {
        if constexpr (G <= 64) {
            return group_max<G>(v);
        } else {
            v = group_max<64>(v);
            if (lane == 0) red[buf][0][rloc][lg / 64] = v;
            __syncthreads();
            float r = red[buf][0][rloc][0];
#pragma unroll
            for (int k = 1; k < WPR; ++k) r = fmaxf(r, red[buf][0][rloc][k]);
            return r;
        }
    };
    auto reduce_sum = [&](float v, int buf) {
        if constexpr (G <= 64) {
            return group_sum<G>(v);
        } else {
            v = group_sum<64>(v);
            if (lane == 0) red[buf][1][rloc][lg / 64] = v;
            __syncthreads();
            float r = red[buf][1][rloc][0];
#pragma unroll
            for (int k = 1; k < WPR; ++k) r = r + red[buf][1][rloc][k];
            return r;
        }
    };

    // Persistent walk over row blocks, uniform per workgroup (so the barriers
    // of multi-wave rows are reached by all), one block at a time.
    int it = 0;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x, ++it) {
        const int64_t row = blk * ROWS + rloc;
        const bool rok = row < a.rows;
        const int64_t r = rok ? row : 0;
        const int q = (int)(r % m);   // query position under the causal mask
        const int buf = it & 1;
        // a slot is read unless it is past the row or wholly past the query
        bool live[V];
#pragma unroll
        for (int i = 0; i < V; ++i) live[i] = ok[i] && (!a.causal || (i * G + lg) * E <= q);
        // element e of slot i takes part: inside the row and not causally masked
        auto valid = [&](int i, int e) {
            const int col = (i * G + lg) * E + e;
            return ok[i] && (VEC || col < m) && (!a.causal || col <= q);
        };

        u32x4 xr[V], yr[BWD ? V : 1], mr[BWD ? 1 : V];
        const bool has_mask = !BWD && a.mask != nullptr;   // uniform
        if constexpr (VEC) {
            const rsrc_t vx = view(a.x, blk);
            const rsrc_t vy = view(BWD ? a.y : a.x, blk);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const uint32_t off = live[i] ? vo[i] : kOob;
                xr[i] = buf_load_nt(vx, off);
                if constexpr (BWD) yr[i] = buf_load_nt(vy, off);
            }
            if constexpr (!BWD) {
                if (has_mask) {
                    // mask rows of this wave's rows: a contiguous range
                    const int64_t row0 = blk * ROWS + wrow;
                    const int64_t last = (row0 + N - 1 < a.rows ? row0 + N - 1 : a.rows - 1);
                    const int64_t m0 = row0 / a.rows_per_mask;
                    const int64_t nm = row0 < a.rows ? last / a.rows_per_mask - m0 + 1 : 0;
                    const rsrc_t vm = row_view<S>(a.mask, m0, nm, m);
                    const uint32_t mrow = (uint32_t)(r / a.rows_per_mask - m0);
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        const uint32_t off = (live[i] && rok)
                                                 ? mrow * (uint32_t)m * S::BYTES +
                                                       (uint32_t)(i * G + lg) * 16u
                                                 : kOob;
                        mr[i] = buf_load(vm, off);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                const int col0 = (i * G + lg) * E;
                load_elems<S>(a.x, r, m, col0, live[i] && rok, f);
                xr[i] = S::pack(f);
                if constexpr (BWD) {
                    load_elems<S>(a.y, r, m, col0, live[i] && rok, f);
                    yr[i] = S::pack(f);
                } else if (has_mask) {
                    load_elems<S>(a.mask, r / a.rows_per_mask, m, col0, live[i] && rok, f);
                    mr[i] = S::pack(f);
                }
            }
        }

        // The dropout mask words depend only on (row, column): formed while
        // the block's loads are in flight (forward: only with a dropped copy).
        u32x4 dw[V];
        const bool drop = BWD || a.out2 != nullptr;   // uniform
        if (drop) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                dw[i] = dropout_words(row, (i * G + lg) * E, a.seed_lo, a.seed_hi, a.thr);
            keep_packed(dw);
        }
        if constexpr (!BWD) {
            // scores: scale, mask, -inf where masked; the row maximum
            float t[V][E];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float xv[E], mv[E];
                S::unpack(xr[i], xv);
                if (has_mask) S::unpack(mr[i], mv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float v = a.scale * xv[e];
                    if (has_mask) v = v + mv[e];
                    t[i][e] = valid(i, e) ? v : -INFINITY;
                    mx = fmaxf(mx, t[i][e]);
                }
            }
            mx = reduce_max(mx, buf);
            // exp of the difference and the row sum (a row with every key
            // masked has mx = -inf: its scores are all -inf and exp2 gives 0)
            const bool live_row = mx != -INFINITY;
            const float nm = live_row ? -mx * kLog2e : 0.0f;
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < V; ++i)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    t[i][e] = exp2_(fmaf(t[i][e], kLog2e, nm));
                    s += t[i][e];
                }
            s = reduce_sum(s, buf);
            const float inv = live_row ? 1.0f / s : 0.0f;
            const float inv_kept = inv * a.pscale;   // dropped copy: y / (1 - p)
            const rsrc_t vy = view(a.out, blk);
            const rsrc_t vd = view(a.out2 ? a.out2 : a.out, blk);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int col0 = (i * G + lg) * E;
                float yv[E];
#pragma unroll
                for (int e = 0; e < E; ++e) yv[e] = t[i][e] * inv;
                if constexpr (VEC) {
                    buf_store_nt(S::pack(yv), vy, vo[i]);
                } else {
                    store_elems<S>(a.out, r, m, col0, ok[i] && rok, yv);
                }
                if (a.out2) {
                    const u32x4 w = dw[i];
                    float dv[E];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        dv[e] = kept<E>(w, col0, e, a.thr) ? t[i][e] * inv_kept : 0.0f;
                    if constexpr (VEC) {
                        buf_store_nt(S::pack(dv), vd, vo[i]);
                    } else {
                        store_elems<S>(a.out2, r, m, col0, ok[i] && rok, dv);
                    }
                }
            }
        } else {
            // dropout backward, then s = sum g * y and dx = scale * y * (g - s)
            float g[V][E], y[V][E];
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int col0 = (i * G + lg) * E;
                float dv[E];
                S::unpack(xr[i], dv);
                S::unpack(yr[i], y[i]);
                const u32x4 w = dw[i];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    g[i][e] = kept<E>(w, col0, e, a.thr) ? dv[e] * a.pscale : 0.0f;
                    s = fmaf(g[i][e], y[i][e], s);
                }
            }
            s = reduce_sum(s, buf);
            const rsrc_t vdx = view(a.out, blk);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float dx[E];
#pragma unroll
                for (int e = 0; e < E; ++e) dx[e] = a.scale * (y[i][e] * (g[i][e] - s));
                if constexpr (VEC) {
                    buf_store_nt(S::pack(dx), vdx, vo[i]);
                } else {
                    store_elems<S>(a.out, r, m, (i * G + lg) * E, ok[i] && rok, dx);
                }
            }
        }
    }
}

// One row per workgroup of G lanes, the block packed in registers (V slots of
// 16 bytes per lane).  Slot i of lane t covers columns (i*G + t)*E ..+E-1;
// element e of it is in play iff i*G*E + e < rel, rel = the columns in
// play (all, or up to the query under the causal mask) minus the lane's first
// column.  Each pass takes rel and the lane's byte offset through opaque(), so
// the compiler keeps no per-slot masks or offsets across passes, and only the
// lane's one partial slot tests elements.
// DROP = false: a forward built without the dropped copy (a.out2 must be
// NULL) and so without Philox code, a few registers leaner.
template <class S, int G, int V, bool VEC, bool BWD, bool MASK, bool DROP = true>
__global__ __launch_bounds__(G) void softmax_wide_kernel(SmArgs a) {
    constexpr int E = S::E, W = G * E, NW = G / 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int m = (int)a.m;
    const int ns = (int)a.nslots;
    const int base = tid * E;                       // the lane's first column
    const uint32_t rb0 = (uint32_t)tid * 16u;       // ... and its byte offset (vector path)
    const uint32_t eb0 = (uint32_t)base * S::BYTES;
    __shared__ float red[2][2][NW];                 // [buffer][max, sum][wave]
    auto reduce = [&](float v, int buf, int k) {
        v = k == 0 ? group_max<64>(v) : group_sum<64>(v);
        if (lane == 0) red[buf][k][tid / 64] = v;
        __syncthreads();
        float r = red[buf][k][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = k == 0 ? fmaxf(r, red[buf][k][w]) : r + red[buf][k][w];
        return r;
    };
    // the lane's slots of one tensor row: slot i is read iff it holds a
    // column in play (i*G + tid < nlive); others read 0
    auto load = [&](const void* t, int64_t trow, int nlive, int lim, u32x4 (&out)[V], bool cached) {
        const rsrc_t v = row_view<S>(t, trow, 1, m);
        if constexpr (VEC) {
            const uint32_t rb = (uint32_t)opaque((int)rb0);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const uint32_t off = i * G + tid < nlive ? rb + (uint32_t)(i * G * 16) : kOob;
                out[i] = cached ? buf_load(v, off) : buf_load_nt(v, off);
            }
        } else {
            const int rel = opaque(lim - base);
            const uint32_t eb = (uint32_t)opaque((int)eb0);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int c = i * W + e;
                    f[e] = elem_load<S>(v, c < rel ? eb + (uint32_t)c * S::BYTES : kOob);
                }
                out[i] = S::pack(f);
                hold_packed(out[i]);   // one slot of element loads in flight at a time
            }
        }
    };
    // writes slot i of a row: every slot of the row (i*G + tid < ns), and on
    // the per-element path only its columns < m
    auto store = [&](const rsrc_t v, int i, const float* f) {
        if constexpr (VEC) {
            const uint32_t rb = (uint32_t)opaque((int)rb0);
            buf_store_nt(S::pack(f), v, i * G + tid < ns ? rb + (uint32_t)(i * G * 16) : kOob);
        } else {
            const int wl = opaque(m - base);
            const uint32_t eb = (uint32_t)opaque((int)eb0);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int c = i * W + e;
                elem_store<S>(v, c < wl ? eb + (uint32_t)c * S::BYTES : kOob, f[e]);
            }
        }
    };

    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const int buf = it & 1;
        const int q = a.causal ? (int)(row % m) : m - 1;   // last key in play
        const int lim = q + 1 < m ? q + 1 : m;
        const int nlive = (lim + E - 1) / E;
        u32x4 xr[V];
        if constexpr (!BWD) {
            u32x4 mr[MASK ? V : 1];
            load(a.x, row, nlive, lim, xr, false);
            if constexpr (MASK) load(a.mask, row / a.rows_per_mask, nlive, lim, mr, true);
            // scores of slot i: scale, mask; elements out of play are skipped
            // by the callers
            auto score = [&](int i, float (&t)[E]) {
                float xv[E];
                S::unpack(xr[i], xv);
#pragma unroll
                for (int e = 0; e < E; ++e) t[e] = a.scale * xv[e];
                if constexpr (MASK) {
                    float mv[E];
                    S::unpack(mr[i], mv);
#pragma unroll
                    for (int e = 0; e < E; ++e) t[e] = t[e] + mv[e];
                }
            };
            auto repack = [&]() {
                keep_packed(xr);
                if constexpr (MASK) keep_packed(mr);
            };
            // the row maximum, then the sum of exp(score - maximum)
            float mx = -INFINITY;
            {
                const int rel = opaque(lim - base);
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float t[E];
                    score(i, t);
                    if (i * W + E <= rel) {
#pragma unroll
                        for (int e = 0; e < E; ++e) mx = fmaxf(mx, t[e]);
                    } else if (i * W < rel) {
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            if (i * W + e < rel) mx = fmaxf(mx, t[e]);
                    }
                }
            }
            mx = reduce(mx, buf, 0);
            const bool live_row = mx != -INFINITY;   // every key masked: y = 0
            const float nm = live_row ? -mx * kLog2e : 0.0f;
            repack();
            float z = 0.0f;
            {
                const int rel = opaque(lim - base);
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float t[E];
                    score(i, t);
                    if (i * W + E <= rel) {
#pragma unroll
                        for (int e = 0; e < E; ++e) z += exp2_(fmaf(t[e], kLog2e, nm));
                    } else if (i * W < rel) {
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            if (i * W + e < rel) z += exp2_(fmaf(t[e], kLog2e, nm));
                    }
                }
            }
            z = reduce(z, buf, 1);
            const float inv = live_row ? 1.0f / z : 0.0f;
            const float inv_kept = inv * a.pscale;   // dropped copy: y / (1 - p)
            repack();
            const rsrc_t vy = row_view<S>(a.out, row, 1, m);
            const rsrc_t vd = row_view<S>(a.out2 ? a.out2 : a.out, row, 1, m);
            const int rel = opaque(lim - base);
            // (seed and threshold from opaque scalar copies per row, and each
            // slot's column from an opaque lane index where it is used, so
            // that neither is hoisted out of the row loop into registers
            // held beside the row)
            uint32_t slo = a.seed_lo, shi = a.seed_hi, thr = a.thr;
            asm volatile("" : "+s"(slo), "+s"(shi), "+s"(thr));
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float t[E], yv[E];
                score(i, t);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    t[e] = exp2_(fmaf(t[e], kLog2e, nm));
                    yv[e] = t[e] * inv;
                }
                if (!(i * W + E <= rel)) {   // keys out of play get y = 0
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if (i * W + e >= rel) {
                            t[e] = 0.0f;
                            yv[e] = 0.0f;
                        }
                    }
                }
                store(vy, i, yv);
                if (DROP && a.out2) {
                    const int col0 = i * W + opaque(tid) * E;
                    const u32x4 w = dropout_words(row, col0, slo, shi, thr);
                    float dv[E];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        dv[e] = kept<E>(w, col0, e, thr) ? t[e] * inv_kept : 0.0f;
                    store(vd, i, dv);
                }
            }
        } else {
            // dy in xr, y in yr; keys out of play read 0 (y = 0 there, so
            // they add nothing and get dx = 0)
            u32x4 yr[V];
            load(a.x, row, nlive, lim, xr, false);
            load(a.y, row, nlive, lim, yr, false);
            // pass 1: g = keep ? dy / (1 - p) : 0 and s = sum g * y, with the
            // keep bits of the slots in play kept for pass 2
            constexpr int NB = (V * E + 31) / 32;
            uint32_t kb[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) kb[k] = 0u;
            float sg = 0.0f;
            const int live = opaque(nlive - tid);   // slot i in play iff i*G < live
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if (i * G < live) {
                    const int col0 = i * W + base;
                    float dv[E], yv[E];
                    S::unpack(xr[i], dv);
                    S::unpack(yr[i], yv);
                    const u32x4 w = dropout_words(row, col0, a.seed_lo, a.seed_hi, a.thr);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int b = i * E + e;
                        const bool keep = kept<E>(w, col0, e, a.thr);
                        kb[b >> 5] |= keep ? (1u << (b & 31)) : 0u;
                        sg = fmaf(keep ? dv[e] * a.pscale : 0.0f, yv[e], sg);
                    }
                }
            }
            sg = reduce(sg, buf, 1);
            keep_packed(xr);
            keep_packed(yr);
            const rsrc_t vdx = row_view<S>(a.out, row, 1, m);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float dv[E], yv[E], dx[E];
                S::unpack(xr[i], dv);
                S::unpack(yr[i], yv);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int b = i * E + e;
                    const float g = ((kb[b >> 5] >> (b & 31)) & 1u) ? dv[e] * a.pscale : 0.0f;
                    dx[e] = a.scale * (yv[e] * (g - sg));
                }
                store(vdx, i, dx);
            }
        }
    }
}

// The 16-bit backward holds dy and y packed (two tensors): up to 6 slots per
// lane fit its registers, 8 in the forward (the scores and a mask row).
template <int G, int V, bool VEC, bool BWD, bool MASK, bool DROP = true>
static hipError_t launch_wide(const SmArgs& a, hipStream_t s) {
    if constexpr (BWD && St::E == 8 && G == 1024 && V > kSmWideBwdV16) {
        return hipErrorInvalidValue;   // callers send such rows to the two-pass path
    } else {
        const void* k = reinterpret_cast<const void*>(
            &softmax_wide_kernel<St, G, V, VEC, BWD, MASK, DROP>);
        const int64_t grid = persistent_grid(k, G, a.rows, 1);
        hipLaunchKernelGGL((softmax_wide_kernel<St, G, V, VEC, BWD, MASK, DROP>),
                           dim3((unsigned)grid), dim3(G), 0, s, a);
        return hipGetLastError();
    }
}

template <int G, int V, bool VEC, bool BWD>
static hipError_t launch_one(const SmArgs& a, hipStream_t s) {
    // (the 16-bit forward over 512-lane rows also measured faster lean:
    // 16384 columns 4.2 -> 5.6 TB/s; narrower rows and fp32 did not)
    if constexpr (sm_wide_layout(G, V, St::E) || (!BWD && St::E == 8 && G == 512)) {
        if constexpr (!BWD) {
            if (a.mask) return launch_wide<G, V, VEC, BWD, true>(a, s);
            // fp32 rows without a dropped copy: the instance without Philox
            // code (1024 x 6 fp32: 148 -> 139 us at 4096 x 24576; the 16-bit
            // layouts up to 8 slots measured 1-3 % slower so)
            if constexpr (St::E == 4) {
                if (!a.out2) return launch_wide<G, V, VEC, BWD, false, false>(a, s);
            }
        }
        return launch_wide<G, V, VEC, BWD, false>(a, s);
    } else {
        constexpr int ROWS = SmGeometry<G>::ROWS;
        const int64_t nblk = (a.rows + ROWS - 1) / ROWS;
        const void* k = reinterpret_cast<const void*>(&softmax_kernel<St, G, V, VEC, BWD>);
        // one workgroup per block when there are three rounds of them:
        // 3-10 % faster at every width measured
        const int64_t grid = persistent_grid(k, SmGeometry<G>::NT, nblk, 1);
        hipLaunchKernelGGL((softmax_kernel<St, G, V, VEC, BWD>), dim3((unsigned)grid),
                           dim3(SmGeometry<G>::NT), 0, s, a);
        return hipGetLastError();
    }
}

// The forward without a mask row holds one tensor, so its rows fit 1024
// lanes x up to 16 slots (131072 16-bit / 65536 fp32 columns) packed in
// registers, with or without the dropped copy (whose Philox rounds run one
// slot at a time in the output pass); past LN_MAX_COLS_SOFTMAX_16 / _F32
// such rows (vector path) take these layouts.
template <int V>
static hipError_t launch_long_fwd(const SmArgs& a, hipStream_t s) {
    if (a.mask) return hipErrorInvalidValue;   // callers send masked rows elsewhere
    return a.out2 ? launch_wide<1024, V, true, false, false, true>(a, s)
                  : launch_wide<1024, V, true, false, false, false>(a, s);
}

// dy's packed slot with the elements that dropout dropped set to +0 (the
// keep bits from the words of the slot's 8-column group), so that
// dy * (1/(1-p)) afterwards is exactly keep ? dy / (1 - p) : 0.
template <class S>
__device__ __forceinline__ u32x4 zero_dropped(u32x4 v, const u32x4& w, int col0, uint32_t thr) {
    constexpr int E = S::E, PER = E / 4;   // elements per 32-bit word
    constexpr uint32_t FIELD = PER == 1 ? ~0u : 0xffffu;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (!kept<E>(w, col0, e, thr)) v[e / PER] &= ~(FIELD << ((e % PER) * (32 / PER)));
    return v;
}

// Backward rows past the register layouts, vector path: one 1024-lane
// workgroup per row holds dy and y on chip and reads each once
// ("02 · llmc/ 的 CUDA kernel 层" §3.1: what fits on chip is read once).
// dy's 16 slots per lane and y's first kSbYReg in registers, y's last
// kSbYLds in LDS, loaded straight into LDS (each wave's lanes fill 64
// consecutive 16-byte cells and each lane reads back only its own).  The
// arithmetic and its order are the register kernel's: s = sum g * y per lane
// in slot order, one butterfly per wave, the waves in order;
// dx = scale * (y * (g - s)).  With dropout (DROP), pass 1 regenerates each
// slot's keep bits from the seed and clears the dropped elements of dy in
// its registers, which then give g = 0 in both passes: no keep bits are held
// beside the row.  Slots out of play (past the query of a causal row) read
// as 0 in registers and are zeroed in LDS, whose cells may still hold
// another row's values.
constexpr int kSbSlots = 16;   // slots per lane of each tensor (131072 16-bit / 65536 fp32 keys)
constexpr int kSbYReg = 7;     // y's slots in registers
constexpr int kSbYLds = kSbSlots - kSbYReg;   // y's slots in LDS (144 KB)
template <class S, bool DROP>
__global__ __launch_bounds__(1024) void softmax_bwd_lds_kernel(SmArgs a) {
    constexpr int E = S::E, G = 1024, V = kSbSlots, VY = kSbYReg, VL = kSbYLds, NW = G / 64;
    static_assert(VY + VL == V, "y's slots: registers, then LDS");
    __shared__ __attribute__((aligned(16))) u32x4 stage[VL][G];
    __shared__ float red[2][NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = (int)a.m;
    const int ns = (int)a.nslots;
    // byte offset of slot i of this lane, or kOob past `nslot`, formed where
    // it is used from an opaque copy of the lane index
    auto slot_off = [&](int i, int nslot) {
        const int t = opaque(tid);
        return i * G + t < nslot ? (uint32_t)(t * 16 + i * G * 16) : kOob;
    };
    auto lds_slot = [&](int j) {
        u32x4 v = stage[j][tid];
        hold_packed(v);
        return v;
    };
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const int buf = it & 1;
        // (the division by m set up per row from an opaque scalar copy, not
        // hoisted into a vector register kept beside the row)
        int mq = m;
        asm volatile("" : "+s"(mq));
        const int q = a.causal ? (int)(row % mq) : m - 1;   // last key in play
        const int lim = q + 1 < m ? q + 1 : m;
        const int nlive = (lim + E - 1) / E;
        const rsrc_t vdy = row_view<S>(a.x, row, 1, m);
        const rsrc_t vy = row_view<S>(a.y, row, 1, m);
        u32x4 dr[V], yr[VY];
#pragma unroll
        for (int i = 0; i < V; ++i) dr[i] = buf_load_nt(vdy, slot_off(i, nlive));
#pragma unroll
        for (int i = 0; i < VY; ++i) yr[i] = buf_load_nt(vy, slot_off(i, nlive));
        // (the previous row's cells were consumed before its stores)
#pragma unroll
        for (int j = 0; j < VL; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vy, (__attribute__((address_space(3))) void*)&stage[j][64 * wave], 16,
                (int)slot_off(VY + j, nlive), 0, 0, kNt);
        // pass 1: g = keep ? dy / (1 - p) : 0 and s = sum g * y over the
        // slots in play
        float sg = 0.0f;
        int live = opaque(nlive - tid);   // slot i in play iff i*G < live
        if constexpr (DROP) {
            // (seed and threshold from opaque scalar copies per row, so that
            // no vector copy of them is hoisted out of the row loop)
            uint32_t slo = a.seed_lo, shi = a.seed_hi, thr = a.thr;
            asm volatile("" : "+s"(slo), "+s"(shi), "+s"(thr));
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if (i * G < live) {
                    const int col0 = (i * G + opaque(tid)) * E;
                    const u32x4 w = dropout_words(row, col0, slo, shi, thr);
                    dr[i] = zero_dropped<S>(dr[i], w, col0, thr);
                }
            }
        }
        auto pass1 = [&](int i, const u32x4& y4) {
            if (i * G < live) {
                float dv[E], yv[E];
                S::unpack(dr[i], dv);
                S::unpack(y4, yv);
#pragma unroll
                for (int e = 0; e < E; ++e) sg = fmaf(dv[e] * a.pscale, yv[e], sg);
            }
        };
#pragma unroll
        for (int i = 0; i < VY; ++i) pass1(i, yr[i]);
#pragma unroll
        for (int j = 0; j < VL; ++j) pass1(VY + j, lds_slot(j));
        sg = group_sum<64>(sg);
        if (lane == 0) red[buf][wave] = sg;
        __syncthreads();
        float r = red[buf][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = r + red[buf][w];
        sg = r;
        keep_packed(dr);
        keep_packed(yr);
        // pass 2: dx = scale * (y * (g - s)), every slot of the row written
        const rsrc_t vdx = row_view<S>(a.out, row, 1, m);
        live = opaque(nlive - tid);
        auto pass2 = [&](int i, const u32x4& y4) {
            float dv[E], yv[E], dx[E];
            S::unpack(dr[i], dv);
            S::unpack(y4, yv);
            if (!(i * G < live)) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    dv[e] = 0.0f;
                    yv[e] = 0.0f;
                }
            }
#pragma unroll
            for (int e = 0; e < E; ++e) dx[e] = a.scale * (yv[e] * (dv[e] * a.pscale - sg));
            buf_store_nt(S::pack(dx), vdx, slot_off(i, ns));
        };
#pragma unroll
        for (int i = 0; i < VY; ++i) pass2(i, yr[i]);
#pragma unroll
        for (int j = 0; j < VL; ++j) pass2(VY + j, lds_slot(j));
    }
}

// Forward rows with an additive mask row past the register layouts, vector
// path: one 1024-lane workgroup per row holds the scores (16 slots per lane
// in registers) and the row's mask (its first kSfMReg slots in registers,
// its last kSbYLds in LDS, loaded straight into LDS as in the backward
// above), so scores and mask are each read once ("02 · llmc/ 的 CUDA kernel
// 层" §3.1).  The arithmetic and its order are the register kernel's: score
// = scale * x + mask, the row maximum and the sum of exp2(score log2(e) -
// max log2(e)) per lane in slot order, one butterfly per wave, the waves in
// order; y = e * (1 / sum), the dropped copy from the same per-slot Philox
// words (DROP).  Keys out of play (past the row, or past the query of a
// causal row) take no part and get y = 0, whatever the LDS cells hold.
constexpr int kSfMReg = 7;   // mask slots in registers (the rest in LDS)
static_assert(kSfMReg + kSbYLds == kSbSlots, "mask slots: registers, then LDS");
template <class S, bool DROP>
__global__ __launch_bounds__(1024) void softmax_fwd_mask_lds_kernel(SmArgs a) {
    constexpr int E = S::E, G = 1024, V = kSbSlots, VM = kSfMReg, VL = kSbYLds, NW = G / 64;
    constexpr int W = G * E;   // columns between consecutive slots of a lane
    __shared__ __attribute__((aligned(16))) u32x4 stage[VL][G];
    __shared__ float red[2][2][NW];   // [buffer][max, sum][wave]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = (int)a.m;
    const int ns = (int)a.nslots;
    auto slot_off = [&](int i, int nslot) {
        const int t = opaque(tid);
        return i * G + t < nslot ? (uint32_t)(t * 16 + i * G * 16) : kOob;
    };
    auto lds_slot = [&](int j) {
        u32x4 v = stage[j][tid];
        hold_packed(v);
        return v;
    };
    auto reduce = [&](float v, int buf, int k) {
        v = k == 0 ? group_max<64>(v) : group_sum<64>(v);
        if (lane == 0) red[buf][k][wave] = v;
        __syncthreads();
        float r = red[buf][k][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = k == 0 ? fmaxf(r, red[buf][k][w]) : r + red[buf][k][w];
        return r;
    };
    int it = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, ++it) {
        const int buf = it & 1;
        int mq = m;
        asm volatile("" : "+s"(mq));
        const int q = a.causal ? (int)(row % mq) : m - 1;   // last key in play
        const int lim = q + 1 < m ? q + 1 : m;
        const int nlive = (lim + E - 1) / E;
        const rsrc_t vx = row_view<S>(a.x, row, 1, m);
        // (both divisions set up per row from opaque scalar copies, not
        // hoisted into a vector register kept beside the row)
        int64_t rpm = a.rows_per_mask;
        asm volatile("" : "+s"(rpm));
        const rsrc_t vm = row_view<S>(a.mask, row / rpm, 1, m);
        u32x4 xr[V], mr[VM];
#pragma unroll
        for (int i = 0; i < V; ++i) xr[i] = buf_load_nt(vx, slot_off(i, nlive));
#pragma unroll
        for (int i = 0; i < VM; ++i) mr[i] = buf_load(vm, slot_off(i, nlive));
        // (the previous row's cells were consumed before its stores; the
        // mask row, which rows_per_mask rows share, is read through the
        // caches)
#pragma unroll
        for (int j = 0; j < VL; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vm, (__attribute__((address_space(3))) void*)&stage[j][64 * wave], 16,
                (int)slot_off(VM + j, nlive), 0, 0, 0);
        // score of slot i: scale * x + mask (the mask slot from registers or
        // LDS, read only where it is used)
        auto score = [&](int i, float (&t)[E]) {
            const u32x4 m4 = i < VM ? mr[i < VM ? i : 0] : lds_slot(i < VM ? 0 : i - VM);
            float xv[E], mv[E];
            S::unpack(xr[i], xv);
            S::unpack(m4, mv);
#pragma unroll
            for (int e = 0; e < E; ++e) t[e] = a.scale * xv[e] + mv[e];
        };
        // rel: columns in play from the lane's first; slot i is wholly in
        // play iff i*W + E <= rel, partly iff i*W < rel, and takes no work
        // otherwise (rows shorter than 16 slots per lane skip the rest)
        int rel = opaque(lim - tid * E);
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (i * W < rel) {
                float t[E];
                score(i, t);
                if (i * W + E <= rel) {
#pragma unroll
                    for (int e = 0; e < E; ++e) mx = fmaxf(mx, t[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (i * W + e < rel) mx = fmaxf(mx, t[e]);
                }
            }
        }
        mx = reduce(mx, buf, 0);
        const bool live_row = mx != -INFINITY;   // every key masked: y = 0
        const float nm = live_row ? -mx * kLog2e : 0.0f;
        keep_packed(xr);
        keep_packed(mr);
        rel = opaque(lim - tid * E);
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (i * W < rel) {
                float t[E];
                score(i, t);
                if (i * W + E <= rel) {
#pragma unroll
                    for (int e = 0; e < E; ++e) z += exp2_(fmaf(t[e], kLog2e, nm));
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (i * W + e < rel) z += exp2_(fmaf(t[e], kLog2e, nm));
                }
            }
        }
        z = reduce(z, buf, 1);
        const float inv = live_row ? 1.0f / z : 0.0f;
        const float inv_kept = inv * a.pscale;   // dropped copy: y / (1 - p)
        keep_packed(xr);
        keep_packed(mr);
        // output pass: every slot of the row written (i*G < rs), keys out of
        // play as 0
        const rsrc_t vy = row_view<S>(a.out, row, 1, m);
        const rsrc_t vd = row_view<S>(DROP ? a.out2 : a.out, row, 1, m);
        rel = opaque(lim - tid * E);
        const int rs = opaque(ns - tid);
        uint32_t slo = a.seed_lo, shi = a.seed_hi, thr = a.thr;
        asm volatile("" : "+s"(slo), "+s"(shi), "+s"(thr));
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (i * G < rs) {
                float t[E], yv[E];
                u32x4 w{};
                int col0 = 0;
                if constexpr (DROP) {
                    col0 = (i * G + opaque(tid)) * E;
                    w = dropout_words(row, col0, slo, shi, thr);
                }
                if (i * W < rel) {
                    score(i, t);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        t[e] = exp2_(fmaf(t[e], kLog2e, nm));
                        yv[e] = t[e] * inv;
                    }
                    if (!(i * W + E <= rel)) {
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            if (i * W + e >= rel) {
                                t[e] = 0.0f;
                                yv[e] = 0.0f;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        t[e] = 0.0f;
                        yv[e] = 0.0f;
                    }
                }
                buf_store_nt(S::pack(yv), vy, slot_off(i, ns));
                if constexpr (DROP) {
                    float dv[E];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        dv[e] = kept<E>(w, col0, e, thr) ? t[e] * inv_kept : 0.0f;
                    buf_store_nt(S::pack(dv), vd, slot_off(i, ns));
                }
            }
        }
    }
}

template <bool VEC, bool BWD>
static hipError_t dispatch(const Path& p, const SmArgs& a, hipStream_t s) {
#define MBROW_CASE(GG, VV) \
    if (p.g == GG && p.v == VV) return launch_one<GG, VV, VEC, BWD>(a, s);
#if MBROW_DT == 0
    MBROW_SM_LAYOUTS_F32(MBROW_CASE)
#else
    MBROW_SM_LAYOUTS_16(MBROW_CASE)
#endif
#undef MBROW_CASE
    return hipErrorInvalidValue;
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_softmax_, MBROW_SUFFIX)(const Path& p, bool backward,
                                                    const SmArgs& a, hipStream_t s) {
    if (backward)
        return p.vec ? dispatch<true, true>(p, a, s) : dispatch<false, true>(p, a, s);
    return p.vec ? dispatch<true, false>(p, a, s) : dispatch<false, false>(p, a, s);
}
// the backward rows held on chip, with or without dropout
template <bool DROP>
static hipError_t launch_bwd_lds(const SmArgs& a, hipStream_t s) {
    const void* k = reinterpret_cast<const void*>(&softmax_bwd_lds_kernel<St, DROP>);
    const int64_t grid = persistent_grid(k, 1024, a.rows);
    hipLaunchKernelGGL((softmax_bwd_lds_kernel<St, DROP>), dim3((unsigned)grid), dim3(1024), 0, s,
                       a);
    return hipGetLastError();
}
hipError_t MBROW_CAT(launch_softmax_bwd_lds_, MBROW_SUFFIX)(const SmArgs& a, hipStream_t s) {
    return a.thr != 0u ? launch_bwd_lds<true>(a, s) : launch_bwd_lds<false>(a, s);
}
// the forward rows with a mask row held on chip, with or without the
// dropped copy
template <bool DROP>
static hipError_t launch_fwd_mask_lds(const SmArgs& a, hipStream_t s) {
    const void* k = reinterpret_cast<const void*>(&softmax_fwd_mask_lds_kernel<St, DROP>);
    const int64_t grid = persistent_grid(k, 1024, a.rows);
    hipLaunchKernelGGL((softmax_fwd_mask_lds_kernel<St, DROP>), dim3((unsigned)grid), dim3(1024),
                       0, s, a);
    return hipGetLastError();
}
hipError_t MBROW_CAT(launch_softmax_fwd_mask_lds_, MBROW_SUFFIX)(const SmArgs& a, hipStream_t s) {
    if (!a.mask) return hipErrorInvalidValue;   // callers send unmasked rows elsewhere
    return a.out2 ? launch_fwd_mask_lds<true>(a, s) : launch_fwd_mask_lds<false>(a, s);
}
// `v`: slots per lane (10, 12, 14 or 16)
hipError_t MBROW_CAT(launch_softmax_long_fwd_, MBROW_SUFFIX)(int v, const SmArgs& a,
                                                             hipStream_t s) {
    switch (v) {
    case 10: return launch_long_fwd<10>(a, s);
    case 12: return launch_long_fwd<12>(a, s);
    case 14: return launch_long_fwd<14>(a, s);
    case 16: return launch_long_fwd<16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mbrow
