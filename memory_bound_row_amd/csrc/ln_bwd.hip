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
// row-per-group layout directly; rows are split into P contiguous ranges,
// one workgroup per range.  Each lane accumulates dy*xhat and dy for the
// columns it owns, row after row in ascending order; the row groups of the
// workgroup are folded in a fixed tree (in-wave swizzles, then LDS); the
// workgroup writes one [2][m] partial.  A second small kernel adds the P
// partials in a fixed order.  No floating-point atomics anywhere, so every
// run gives the same bits.
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
    static constexpr int NT = G <= 512 ? 512 : G;    // threads per workgroup (multiple of G)
    static constexpr int NG = NT / G;                // row groups per workgroup
    static constexpr int NW = NT / 64;               // waves per workgroup
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
    // Units whose lanes own identical columns, folded together at the end:
    // the waves of the workgroup (G <= 64) or its row groups (G > 64).
    static constexpr int NU = G <= 64 ? NW : NG;
    static constexpr int UT = G <= 64 ? 64 : G;      // threads per unit
};

__device__ inline float xor32(float v) { return __shfl_xor(v, 32, 64); }

template <class S, int G, int V, bool VEC, int MODE>
__global__ __launch_bounds__(BwdGeometry<G>::NT) void ln_bwd_kernel(BwdArgs a) {
    constexpr int E = S::E;
    constexpr int NT = BwdGeometry<G>::NT;
    constexpr int NG = BwdGeometry<G>::NG;
    constexpr int NW = BwdGeometry<G>::NW;
    constexpr int WPR = BwdGeometry<G>::WPR;
    constexpr int NU = BwdGeometry<G>::NU;
    constexpr int UT = BwdGeometry<G>::UT;
    constexpr bool DX = MODE != (int)BwdMode::PARTIALS;
    constexpr bool PART = MODE != (int)BwdMode::DX;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lg = tid % G;
    const int grp = tid / G;

    const int64_t part = blockIdx.x;
    const int64_t r0 = part * a.rows / a.parts;
    const int64_t r1 = (part + 1) * a.rows / a.parts;

    bool ok[V];
    int64_t col0[V];
    float ga[V][E];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t s = (int64_t)i * G + lg;
        ok[i] = s < a.nslots;
        col0[i] = s * E;
        if constexpr (DX) load_slot<S, VEC, false>(a.gamma, 0, col0[i], a.m, ok[i], ga[i]);
    }
    float acc_g[V][E], acc_b[V][E];
    if constexpr (PART) {
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) acc_g[i][e] = acc_b[i][e] = 0.0f;
    }
    __shared__ float red[2][NG][WPR][2];   // cross-wave A/B exchange (multi-wave rows)

    // Every row group runs the same number of iterations (a row past the
    // partition end is skipped but still takes part in the barriers of a
    // multi-wave row).
    int it = 0;
    for (int64_t base = r0; base < r1; base += NG, ++it) {
        const int64_t row = base + grp;
        const bool row_ok = row < r1;
        const int64_t roff = row_ok ? row * a.m : 0;
        float x[V][E], d[V][E];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            load_slot<S, VEC, true>(a.dy, roff, col0[i], a.m, ok[i] && row_ok, d[i]);
            load_slot<S, VEC, true>(a.x, roff, col0[i], a.m, ok[i] && row_ok, x[i]);
        }
        const float mu = row_ok ? a.mean[row] : 0.0f;
        const float rs = row_ok ? a.rstd[row] : 0.0f;
        float xh[V][E];
#pragma unroll
        for (int i = 0; i < V; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e) xh[i][e] = (x[i][e] - mu) * rs;
        if constexpr (DX) {
            float A = 0.0f, B = 0.0f;
            float g[V][E];
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    g[i][e] = ga[i][e] * d[i][e];   // zero outside the row
                    A += g[i][e];
                    B = fmaf(g[i][e], xh[i][e], B);
                }
            }
            if constexpr (G <= 64) {
                A = group_sum<G>(A);
                B = group_sum<G>(B);
            } else {
                A = group_sum<64>(A);
                B = group_sum<64>(B);
                const int w = lg / 64;
                const int buf = it & 1;   // double buffer: one barrier per row
                if (lane == 0) {
                    red[buf][grp][w][0] = A;
                    red[buf][grp][w][1] = B;
                }
                __syncthreads();
                A = red[buf][grp][0][0];
                B = red[buf][grp][0][1];
#pragma unroll
                for (int k = 1; k < WPR; ++k) {
                    A += red[buf][grp][k][0];
                    B += red[buf][grp][k][1];
                }
            }
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float out[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float t = fmaf(xh[i][e], B, A) * a.inv_m;
                    out[e] = rs * (g[i][e] - t);
                }
                store_slot<S, VEC, true>(a.dx, roff, col0[i], a.m, ok[i] && row_ok, out);
            }
        }
        if constexpr (PART) {
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    acc_g[i][e] = fmaf(d[i][e], xh[i][e], acc_g[i][e]);
                    acc_b[i][e] = acc_b[i][e] + d[i][e];
                }
            }
        }
    }

    if constexpr (PART) {
        if constexpr (G <= 32) {
            // Fold the row groups of each wave: lanes l, l+G, ... own the same
            // columns.  Adds are commutative, so partners agree bit for bit.
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    float& ag = acc_g[i][e];
                    float& ab = acc_b[i][e];
                    if constexpr (G <= 16) { ag = ag + partner<16>(ag); ab = ab + partner<16>(ab); }
                    ag = ag + xor32(ag);
                    ab = ab + xor32(ab);
                }
            }
        }
        // Fold the units (waves, or multi-wave row groups) through LDS in a
        // fixed tree, one slot at a time to bound the LDS footprint: at each
        // level unit u + h hands its sums to unit u.
        const int unit = tid / UT;
        const int pos = tid % UT;
        if constexpr (NU > 1) {
            __shared__ float tree[NU / 2][2][E][UT];
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int h = NU / 2; h >= 1; h /= 2) {
                    if (unit >= h && unit < 2 * h) {
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            tree[unit - h][0][e][pos] = acc_g[i][e];
                            tree[unit - h][1][e][pos] = acc_b[i][e];
                        }
                    }
                    __syncthreads();
                    if (unit < h) {
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            acc_g[i][e] = acc_g[i][e] + tree[unit][0][e][pos];
                            acc_b[i][e] = acc_b[i][e] + tree[unit][1][e][pos];
                        }
                    }
                    __syncthreads();
                }
            }
        }
        // Unit 0 holds the workgroup's partial; for G < 64 its first row
        // group writes it.
        const bool writer = (G <= 64) ? (tid < G) : (unit == 0);
        if (writer) {
            float* pg = a.ws + (part * 2 + 0) * a.m;
            float* pb = a.ws + (part * 2 + 1) * a.m;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if (!ok[i]) continue;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (col0[i] + e < a.m) {
                        pg[col0[i] + e] = acc_g[i][e];
                        pb[col0[i] + e] = acc_b[i][e];
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
    MBROW_CASE(16, 1)
    MBROW_CASE(32, 1)
    MBROW_CASE(64, 1)
    MBROW_CASE(64, 2)
    MBROW_CASE(64, 3)
    MBROW_CASE(64, 4)
    MBROW_CASE(64, 5)
    MBROW_CASE(64, 6)
    MBROW_CASE(64, 7)
    MBROW_CASE(64, 8)
    MBROW_CASE(128, 4)
    MBROW_CASE(256, 4)
    MBROW_CASE(512, 4)
    MBROW_CASE(1024, 4)
    MBROW_CASE(1024, 8)
#undef MBROW_CASE
    return hipErrorInvalidValue;
}

template <bool VEC>
static hipError_t dispatch_mode(const Path& p, BwdMode mode, const BwdArgs& a, hipStream_t s) {
    switch (mode) {
    case BwdMode::DX: return dispatch<VEC, 0>(p, a, s);
    case BwdMode::DX_PARTIALS: return dispatch<VEC, 1>(p, a, s);
    default: return dispatch<VEC, 2>(p, a, s);
    }
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_bwd_, MBROW_SUFFIX)(const Path& p, BwdMode mode, const BwdArgs& a,
                                                 hipStream_t s) {
    return p.vec ? dispatch_mode<true>(p, mode, a, s) : dispatch_mode<false>(p, mode, a, s);
}

}  // namespace mbrow
