// ln_bwd.hip -- LayerNorm backward for gfx950: dx from two row sums reduced
// together, fused with stage 1 of the dgamma/dbeta column reduction.
// Compiled once per storage type (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// dx ("Accelerating Transformer on GPU (II)" §2.1, x-hat form; §2.2 one
// synchronisation): with g = gamma*dy and xhat = (x - mean)*rstd, the sums
// A = sum g and B = sum g*xhat are independent, so one butterfly reduces
// both, and dx = rstd*(g - (A + xhat*B)/m).
//
// dgamma/dbeta (§2.4 of the same page): a column sum over rows cannot use the
// row-per-group layout directly; the rows are split into P partitions, one
// workgroup each.  The row blocks are dealt to the partitions in turn, so
// the workgroups stream through the tensor side by side.  Each lane
// accumulates dy*xhat and dy for the columns it owns, block after block;
// the row groups of the workgroup are folded in a fixed tree (in-wave lane
// exchanges, then LDS); the workgroup writes one [2][m] partial.  A second
// small kernel adds the P partials in a fixed order.  No floating-point
// atomics anywhere, so every run gives the same bits.
//
// RMSNorm ("GPU Performance from First Principles" §6): the same kernel with
// the mean fixed at 0 and no sum of g -- xhat = x*rstd, B = sum g*xhat,
// dx = rstd*(g - xhat*B/m) -- one column partial (dgamma), and the gradient
// reaching the normalised input from its other uses added to dx.
//
// Schedule.  One row block at a time per workgroup, its loads issued
// together at the top of the iteration; all P workgroups are resident, so
// the memory system sees P blocks in flight.  With 16-bit storage, the
// prologue and RMSNorm backwards, and every mode for rows of two to eight
// waves, also load the next block while they compute the current one.
#include "ln_device.hpp"
#include "ln_launch.hpp"

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
struct BwdGeometry {
    static constexpr int NT = bwd_threads(G);        // threads per workgroup (multiple of G)
    static constexpr int NG = NT / G;                // row groups per workgroup
    static constexpr int NW = NT / 64;               // waves per workgroup
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
    // Units whose lanes own identical columns, folded together at the end:
    // the waves of the workgroup (G <= 64) or its row groups (G > 64).
    static constexpr int NU = G <= 64 ? NW : NG;
    static constexpr int UT = G <= 64 ? 64 : G;      // threads per unit
};

__device__ inline float xor32(float v) { return __shfl_xor(v, 32, 64); }

// a or b, chosen at compile time (arrays of different lengths)
template <bool C, class A, class B>
__device__ __forceinline__ auto& select(A& a, B& b) {
    if constexpr (C) {
        return a;
    } else {
        return b;
    }
}

template <class S, int G, int V, bool VEC, int MODE>
__global__ __launch_bounds__(BwdGeometry<G>::NT) void ln_bwd_kernel(BwdArgs a) {
    constexpr int E = S::E;
    constexpr int NG = BwdGeometry<G>::NG;
    constexpr int WPR = BwdGeometry<G>::WPR;
    constexpr int NU = BwdGeometry<G>::NU;
    constexpr int UT = BwdGeometry<G>::UT;
    constexpr bool DX = MODE != (int)BwdMode::PARTIALS;
    constexpr bool PART = MODE != (int)BwdMode::DX;
    constexpr bool DROP = MODE == (int)BwdMode::DROPOUT;   // prologue backward too
    constexpr bool RMS = MODE == (int)BwdMode::RMS;         // mean 0, no sum of g
    constexpr bool EXTRA = DROP || RMS;                     // dz_extra may be given
    constexpr int NK = DROP ? 3 : (RMS ? 1 : 2);            // kinds of column partials
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lg = tid % G;
    const int grp = tid / G;
    const int m = (int)a.m;
    const int nslots = (int)a.nslots;

    // Partition `part` owns the blocks of NG consecutive rows starting at
    // rows part*NG, (part + P)*NG, (part + 2P)*NG, ...: the workgroups walk
    // the tensor side by side, one window of P*NG rows at a time.
    const int64_t part = blockIdx.x;
    const int64_t first = part * NG;
    const int64_t stride = a.parts * NG;

    // slot i of this lane covers columns (i*G + lg)*E .. +E-1; gamma stays
    // packed in T in registers
    bool ok[V];
    u32x4 gp[DX ? V : 1];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        ok[i] = i * G + lg < nslots;
        if constexpr (DX) gp[i] = load_param<S, VEC>(a.gamma, i * G + lg, m, ok[i]);
    }
    // vector path: the lane's byte offset of each slot in its wave's row view
    uint32_t vo[VEC ? V : 1];
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < V; ++i) vo[i] = slot_offset<S, G>(tid, i, m, ok[i]);
    }
    const int wrow = wave_first_row<G>(tid);
    // the rows of the block starting at `base` that this wave touches
    // (uniform across the wave)
    auto view = [&](const void* t, int64_t base) {
        const int64_t row0 = base + wrow;
        const int64_t left = a.rows - row0;
        return row_view<S>(t, row0, left < WaveRows<G>::N ? left : WaveRows<G>::N, m);
    };

    // Column accumulators: one per value of the lane's slots and kind
    // (dgamma, then dbeta, then dbias in the prologue mode; dgamma alone for
    // RMSNorm).
    constexpr int KA = PART ? V * E : 1;
    float acc[NK][KA];
#pragma unroll
    for (int kind = 0; kind < NK; ++kind) {
#pragma unroll
        for (int k = 0; k < KA; ++k) acc[kind][k] = 0.0f;
    }
    const bool has_extra = EXTRA && a.dz_extra != nullptr;   // uniform
    __shared__ float red[2][NG][WPR][2];   // cross-wave A/B exchange (multi-wave rows)

    // The block is unpacked once (x - mean in place, dy as is).  With 16-bit
    // storage its packed registers are then free during the two passes: the
    // next block's dy, x and row statistics are loaded into them there, so
    // each block's loads are in flight while the previous block's arithmetic
    // runs (the Philox rounds, the sums, the cross-wave exchange).  The
    // prologue and RMSNorm backwards do this at every layout; the plain
    // backward only for rows of more than one wave (a workgroup walks one to
    // four rows per block there; with one-wave rows, eight per block, it
    // measured no faster).  fp32 rows free nothing by unpacking (dy is kept
    // as loaded), so their prefetch costs registers: taken for rows of two
    // to eight waves, where it measured faster and fits 256 registers.
    constexpr bool MULTI = DX && G > 64 && G <= 512;
    constexpr bool PF = VEC && V <= 4 && (E == 8 ? (DROP || RMS || MULTI) : MULTI);
    u32x4 xp[PF ? V : 1], dp[PF ? V : 1];   // the prefetched block
    float mu_n = 0.0f, rs_n = 0.0f;
    auto issue = [&](int64_t b) {
        const rsrc_t vd = view(a.dy, b);
        const rsrc_t vx = view(a.x, b);
#pragma unroll
        for (int i = 0; i < (PF ? V : 1); ++i) {
            dp[i] = buf_load_nt(vd, vo[i]);
            xp[i] = buf_load_nt(vx, vo[i]);
        }
        const int64_t rw = b + grp < a.rows ? b + grp : 0;
        if constexpr (!RMS) mu_n = a.mean[rw];
        rs_n = a.rstd[rw];
    };

    // One block: its loads, the block unpacked once, pass 1 (the two row
    // sums), pass 2 (dx and the column partials).  The walk is uniform per
    // workgroup, so the barrier of a multi-wave row is reached by all.
    auto block = [&](const int64_t base, const int it) __attribute__((always_inline)) {
        // the block's dy and x: the prefetched registers, or its own
        u32x4 xr_b[PF ? 1 : V], dr_b[PF ? 1 : V];
        auto& xr = select<PF>(xp, xr_b);
        auto& dr = select<PF>(dp, dr_b);
        const int64_t row = base + grp;
        const bool rok = row < a.rows;
        const int64_t r = rok ? row : 0;   // rows past the end read row 0's statistics
        u32x4 er[EXTRA ? V : 1];
        if constexpr (PF) {
            if constexpr (EXTRA) {
                if (has_extra) {
                    const rsrc_t ve = view(a.dz_extra, base);
#pragma unroll
                    for (int i = 0; i < V; ++i) er[i] = buf_load_nt(ve, vo[i]);
                }
            }
        } else if constexpr (VEC) {
            // rows past the end read 0 and are never stored
            const rsrc_t vd = view(a.dy, base);
            const rsrc_t vx = view(a.x, base);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                dr[i] = buf_load_nt(vd, vo[i]);
                xr[i] = buf_load_nt(vx, vo[i]);
            }
            if constexpr (EXTRA) {
                if (has_extra) {
                    const rsrc_t ve = view(a.dz_extra, base);
#pragma unroll
                    for (int i = 0; i < V; ++i) er[i] = buf_load_nt(ve, vo[i]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                load_elems<S>(a.dy, r, m, (i * G + lg) * E, ok[i] && rok, f);
                dr[i] = S::pack(f);
                load_elems<S>(a.x, r, m, (i * G + lg) * E, ok[i] && rok, f);
                xr[i] = S::pack(f);
                if constexpr (EXTRA) {
                    if (has_extra) {
                        load_elems<S>(a.dz_extra, r, m, (i * G + lg) * E, ok[i] && rok, f);
                        er[i] = S::pack(f);
                    }
                }
            }
        }
        // The prologue's mask words depend only on (row, column): formed while
        // the block's loads are in flight (layouts with room for them; wider
        // ones form each slot's words where they are used).
        constexpr bool EARLY = DROP && V <= 4;
        u32x4 dw[EARLY ? V : 1];
        if constexpr (EARLY) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                dw[i] = dropout_words(row, (i * G + lg) * E, a.seed_lo, a.seed_hi, a.thr);
            keep_packed(dw);
        }
        float mu, rs;
        if constexpr (PF) {
            mu = RMS ? 0.0f : mu_n;
            rs = rs_n;
        } else {
            mu = RMS ? 0.0f : a.mean[r];
            rs = a.rstd[r];
        }
        // (the per-element path and multi-wave rows of the prologue backward
        // have no registers to spare for gamma unpacked across blocks)
        if constexpr (DX && (!VEC || (DROP && G > 64))) keep_packed(gp);
        float xm_[V][E], d_[V][E];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            S::unpack(xr[i], xm_[i]);
            S::unpack(dr[i], d_[i]);
            if constexpr (!RMS) {
#pragma unroll
                for (int e = 0; e < E; ++e) xm_[i][e] = xm_[i][e] - mu;
            }
        }
        if constexpr (PF) {
            // the next block's loads, into the registers just unpacked
            // (uniform per workgroup)
            asm volatile("" ::: "memory");
            if (base + stride < a.rows) issue(base + stride);
            asm volatile("" ::: "memory");
        }
        // x - mean and dy of slot i
        auto slot = [&](int i, float* xm, float* d) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                xm[e] = xm_[i][e];
                d[e] = d_[i][e];
            }
        };
        float c1 = 0.0f, c2 = 0.0f;
        if constexpr (DX) {
            // A = sum g, B = sum g * xhat = rstd * sum g * (x - mean)
            // (RMSNorm: A unused)
            float A = 0.0f, Bm = 0.0f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float ga[E], xm[E], d[E];
                S::unpack(gp[i], ga);
                slot(i, xm, d);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float g = ga[e] * d[e];   // zero outside the row
                    if constexpr (!RMS) A += g;
                    Bm = fmaf(g, xm[e], Bm);
                }
            }
            if constexpr (G <= 64) {
                A = group_sum<G>(A);
                Bm = group_sum<G>(Bm);
            } else {
                A = group_sum<64>(A);
                Bm = group_sum<64>(Bm);
                const int w = lg / 64;
                const int buf = it & 1;   // double buffer: one barrier per block
                if (lane == 0) {
                    red[buf][grp][w][0] = A;
                    red[buf][grp][w][1] = Bm;
                }
                __syncthreads();
                A = red[buf][grp][0][0];
                Bm = red[buf][grp][0][1];
#pragma unroll
                for (int k = 1; k < WPR; ++k) {
                    A += red[buf][grp][k][0];
                    Bm += red[buf][grp][k][1];
                }
            }
            // dx = rstd * (g - (A + xhat * B) / m) = rstd * (g - (c1 + xhat * c2));
            // g - (...) cancels exactly where it should (a one-column row
            // gets dx = 0)
            c1 = RMS ? 0.0f : A * a.inv_m;
            c2 = (Bm * rs) * a.inv_m;
        }
        // Pass 2, slot by slot: dx (when formed) and the column partials.
        // The partials use the same expressions in every mode, so the fused
        // and the partials-only passes produce the same bits.
        const rsrc_t vdx = view(DX ? a.dx : a.dy, base);
        const rsrc_t vdi = view(DROP ? a.dx_in : a.dy, base);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int col0 = (i * G + lg) * E;
            float xh[E], xm[E], d[E];
            slot(i, xm, d);
#pragma unroll
            for (int e = 0; e < E; ++e) xh[e] = xm[e] * rs;
            if constexpr (DX) {
                float ga[E], out[E];
                S::unpack(gp[i], ga);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    out[e] = rs * (ga[e] * d[e] - fmaf(xh[e], c2, c1));
                // dz = the norm's dx + the gradient from z's other uses
                if constexpr (EXTRA) {
                    if (has_extra) {
                        float ez[E];
                        S::unpack(er[i], ez);
#pragma unroll
                        for (int e = 0; e < E; ++e) out[e] = out[e] + ez[e];
                    }
                }
                if constexpr (DROP) {
                    // dresidual = dz; dx of the prologue = keep * dz / (1 - p)
                    // with the forward's mask regenerated; dbias sums it
                    u32x4 w;
                    if constexpr (EARLY) {
                        w = dw[i];
                    } else {
                        w = dropout_words(row, col0, a.seed_lo, a.seed_hi, a.thr);
                    }
                    float din[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        din[e] = kept<E>(w, col0, e, a.thr) ? out[e] * a.scale : 0.0f;
                        acc[2][i * E + e] = acc[2][i * E + e] + din[e];
                    }
                    if constexpr (VEC) {
                        buf_store_nt(S::pack(din), vdi, vo[i]);
                    } else {
                        store_elems<S>(a.dx_in, r, m, col0, ok[i] && rok, din);
                    }
                }
                if constexpr (VEC) {
                    buf_store_nt(S::pack(out), vdx, vo[i]);
                } else {
                    store_elems<S>(a.dx, r, m, col0, ok[i] && rok, out);
                }
            }
            if constexpr (PART) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    acc[0][i * E + e] = fmaf(d[e], xh[e], acc[0][i * E + e]);
                    if constexpr (!RMS) acc[1][i * E + e] = acc[1][i * E + e] + d[e];
                }
            }
        }
    };
    if constexpr (PF) {
        // the first block outside the loop, so that every entry to the loop
        // has the same memory operations in flight (the wait for a block's
        // prefetched loads then leaves the previous block's stores alone)
        if (first < a.rows) {
            issue(first);
            block(first, 0);
            int it = 1;
            for (int64_t base = first + stride; base < a.rows; base += stride, ++it)
                block(base, it);
        }
    } else {
        int it = 0;
        for (int64_t base = first; base < a.rows; base += stride, ++it) block(base, it);
    }

    if constexpr (PART) {
        // Rows of one wave that own the same columns are folded inside the
        // wave first: lanes l, l+16, l+32, l+48 (16-lane rows) or l, l+32
        // (32-lane rows).  Adds are commutative, so partners agree bit for
        // bit and every row group ends with the wave's sums.
#pragma unroll
        for (int kind = 0; kind < NK; ++kind) {
#pragma unroll
            for (int k = 0; k < KA; ++k) {
                float& v = acc[kind][k];
                if constexpr (G == 16) {
                    v = v + partner<16>(v);
                    v = v + xor32(v);
                } else if constexpr (G == 32) {
                    v = halves_sum_swap(v, v);
                }
            }
        }
        // Then the units whose lanes own the same columns (the waves of the
        // workgroup for G <= 64, its row groups otherwise) are added in unit
        // order 0, 1, ... and the workgroup writes its partition's [NK][m]
        // partial.  Lane l of a unit holds, for slot i of its row, all E
        // values of that slot, so the thread that adds slot i of lane
        // position l over the units writes E consecutive columns at once:
        // 16-byte stores, half the write time of one 4-byte store per column
        // at the end of the kernel.  Units stage their sums in LDS (lane
        // position fastest: conflict-free), in chunks of CI slot indices
        // that fit kStage bytes (gfx950 has 160 KB of LDS per workgroup);
        // unit u adds the (kind, slot) pairs u, u + NU, ...  A workgroup of
        // a single unit writes its sums directly.
        constexpr int NT = BwdGeometry<G>::NT;
        constexpr int kStage = 156 * 1024;
        constexpr int CI0 = kStage / (NT * NK * E * 4);
        constexpr int CI = CI0 < 1 ? 1 : (CI0 < V ? CI0 : V);
        static_assert(NU == 1 || NT * NK * CI * E * 4 <= kStage, "stage exceeds its budget");
        float* const pw = a.ws + part * NK * a.m;   // this partition's [NK][m] partial
        // 16-byte partial stores need the partial rows 16-byte aligned
        const bool wvec = VEC && a.ws_vec;          // uniform
        const int unit = tid / UT;
        const int pos = tid % UT;                    // lane position within the unit's row(s)
        // write the E sums of slot `sl` of one kind
        auto put = [&](int kind, int sl, const float* t) {
            float* dst = pw + kind * a.m + sl * E;
            if (wvec) {
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    f32x4 v = {t[e], t[e + 1], t[e + 2], t[e + 3]};
                    *reinterpret_cast<f32x4*>(dst + e) = v;
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (sl * E + e < m) dst[e] = t[e];
            }
        };
        if constexpr (NU == 1) {
            // one unit: lane position lg alone holds its columns
#pragma unroll
            for (int kind = 0; kind < NK; ++kind) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    if (i * G + lg < nslots) put(kind, i * G + lg, &acc[kind][i * E]);
                }
            }
            return;
        } else {
            __shared__ float stage[NU][NK][CI * E][UT];
#pragma unroll
            for (int i0 = 0; i0 < V; i0 += CI) {
                if (i0 > 0) __syncthreads();   // previous chunk fully read
#pragma unroll
                for (int c = 0; c < CI * E; ++c) {
                    if (i0 * E + c < KA) {
#pragma unroll
                        for (int kind = 0; kind < NK; ++kind)
                            stage[unit][kind][c][pos] = acc[kind][i0 * E + c];
                    }
                }
                __syncthreads();
                // positions past the row group's lanes (G < 64) hold copies
                if (pos < G) {
                    for (int cb = unit; cb < NK * CI; cb += NU) {
                        const int kind = cb / CI;
                        const int i = i0 + cb % CI;
                        const int sl = i * G + pos;
                        if (i >= V || sl >= nslots) continue;
                        float t[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const int c = (i - i0) * E + e;
                            float sum = stage[0][kind][c][pos];
#pragma unroll
                            for (int u = 1; u < NU; ++u) sum = sum + stage[u][kind][c][pos];
                            t[e] = sum;
                        }
                        put(kind, sl, t);
                    }
                }
            }
        }
    }
}

template <int G, int V, bool VEC, int MODE>
static hipError_t launch_one(const BwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((ln_bwd_kernel<St, G, V, VEC, MODE>), dim3((unsigned)a.parts),
                       dim3(BwdGeometry<G>::NT), 0, s, a);
    return hipGetLastError();
}

template <bool VEC, int MODE>
static hipError_t dispatch(const Path& p, const BwdArgs& a, hipStream_t s) {
#define MBROW_CASE(GG, VV) \
    if (p.g == GG && p.v == VV) return launch_one<GG, VV, VEC, MODE>(a, s);
    if constexpr (MODE == (int)BwdMode::DROPOUT) {
#if MBROW_DT == 0
        MBROW_LAYOUTS_DROP_F32(MBROW_CASE)
#else
        MBROW_LAYOUTS_DROP_16(MBROW_CASE)
#endif
    } else {
#if MBROW_DT == 0
        MBROW_LAYOUTS_F32(MBROW_CASE)
#else
        MBROW_LAYOUTS_16(MBROW_CASE)
#endif
    }
#undef MBROW_CASE
    return hipErrorInvalidValue;
}

template <bool VEC>
static hipError_t dispatch_mode(const Path& p, BwdMode mode, const BwdArgs& a, hipStream_t s) {
    switch (mode) {
    case BwdMode::DX: return dispatch<VEC, 0>(p, a, s);
    case BwdMode::DX_PARTIALS: return dispatch<VEC, 1>(p, a, s);
    case BwdMode::PARTIALS: return dispatch<VEC, 2>(p, a, s);
    case BwdMode::DROPOUT: return dispatch<VEC, 3>(p, a, s);
    default: return dispatch<VEC, 4>(p, a, s);
    }
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_bwd_, MBROW_SUFFIX)(const Path& p, BwdMode mode, const BwdArgs& a,
                                                 hipStream_t s) {
    return p.vec ? dispatch_mode<true>(p, mode, a, s) : dispatch_mode<false>(p, mode, a, s);
}

}  // namespace mbrow
