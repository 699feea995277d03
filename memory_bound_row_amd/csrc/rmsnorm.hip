// rmsnorm.hip -- fused residual add + RMSNorm forward for gfx950.  Compiled
// once per storage type (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// "GPU Performance from First Principles" §6.1: the residual add and the
// next RMSNorm in one kernel -- read x and the residual, write the new
// residual stream z = x + residual and h = gamma * z * rstd, with
// rstd = 1 / sqrt(mean(z^2) + eps): one sum of squares, no mean.  z is
// stored in T and the norm runs on the stored value (as the fused LayerNorm
// does).  The sum of squares is float32 (§7.5 of the same page: squares of
// outliers of a few hundred overflow fp16).  One row per group of G lanes in
// registers, persistent grid, one block at a time; gamma is re-read (cached)
// per row.
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
struct RmsGeometry {
    static constexpr int NT = G <= 256 ? 256 : G;   // threads per workgroup
    static constexpr int ROWS = NT / G;              // rows per block
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
};

template <class S, int G, int V, bool VEC, bool ADD>
__global__ __launch_bounds__(RmsGeometry<G>::NT) void rmsnorm_fwd_kernel(RmsArgs a) {
    constexpr int E = S::E;
    constexpr int ROWS = RmsGeometry<G>::ROWS;
    constexpr int WPR = RmsGeometry<G>::WPR;
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
    auto view = [&](const void* t, int64_t blk) {
        const int64_t row0 = blk * ROWS + wrow;
        const int64_t left = a.rows - row0;
        return row_view<S>(t, row0, left < WaveRows<G>::N ? left : WaveRows<G>::N, m);
    };
    __shared__ float red[2][ROWS][WPR];   // cross-wave exchange, double-buffered

    int it = 0;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x, ++it) {
        const int64_t row = blk * ROWS + rloc;
        const bool rok = row < a.rows;
        const int64_t r = rok ? row : 0;
        u32x4 xr[V], rr[ADD ? V : 1];
        if constexpr (VEC) {
            const rsrc_t vx = view(a.x, blk);
            const rsrc_t vr = view(ADD ? a.residual : a.x, blk);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                xr[i] = buf_load_nt(vx, vo[i]);
                if constexpr (ADD) rr[i] = buf_load_nt(vr, vo[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                load_elems<S>(a.x, r, m, (i * G + lg) * E, ok[i] && rok, f);
                xr[i] = S::pack(f);
                if constexpr (ADD) {
                    load_elems<S>(a.residual, r, m, (i * G + lg) * E, ok[i] && rok, f);
                    rr[i] = S::pack(f);
                }
            }
        }
        // z = x + residual, stored in T; the norm runs on the stored value
        float z[V][E];
        float ss = 0.0f;
        const rsrc_t vz = view(ADD ? a.residual_out : a.x, blk);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            S::unpack(xr[i], z[i]);
            if constexpr (ADD) {
                float rv[E];
                S::unpack(rr[i], rv);
#pragma unroll
                for (int e = 0; e < E; ++e) z[i][e] = z[i][e] + rv[e];
                const u32x4 zp = S::pack(z[i]);
                if constexpr (VEC) {
                    buf_store_nt(zp, vz, vo[i]);
                } else {
                    store_elems<S>(a.residual_out, r, m, (i * G + lg) * E, ok[i] && rok, z[i]);
                }
                S::unpack(zp, z[i]);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) ss = fmaf(z[i][e], z[i][e], ss);   // 0 outside the row
        }
        if constexpr (G <= 64) {
            ss = group_sum<G>(ss);
        } else {
            ss = group_sum<64>(ss);
            const int buf = it & 1;
            if (lane == 0) red[buf][rloc][lg / 64] = ss;
            __syncthreads();
            ss = red[buf][rloc][0];
#pragma unroll
            for (int k = 1; k < WPR; ++k) ss = ss + red[buf][rloc][k];
        }
        const float rs = 1.0f / sqrtf(ss * a.inv_m + a.eps);
        if (lg == 0 && rok && a.rstd) a.rstd[row] = rs;
        const rsrc_t vy = view(a.y, blk);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float ga[E], out[E];
            S::unpack(load_param<S, VEC>(a.gamma, i * G + lg, m, ok[i]), ga);
#pragma unroll
            for (int e = 0; e < E; ++e) out[e] = (z[i][e] * rs) * ga[e];
            if constexpr (VEC) {
                buf_store_nt(S::pack(out), vy, vo[i]);
            } else {
                store_elems<S>(a.y, r, m, (i * G + lg) * E, ok[i] && rok, out);
            }
        }
    }
}

template <int G, int V, bool VEC, bool ADD>
static hipError_t launch_one(const RmsArgs& a, hipStream_t s) {
    constexpr int ROWS = RmsGeometry<G>::ROWS;
    const int64_t nblk = (a.rows + ROWS - 1) / ROWS;
    const void* k = reinterpret_cast<const void*>(&rmsnorm_fwd_kernel<St, G, V, VEC, ADD>);
    const int64_t grid = persistent_grid(k, RmsGeometry<G>::NT, nblk);
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<St, G, V, VEC, ADD>), dim3((unsigned)grid),
                       dim3(RmsGeometry<G>::NT), 0, s, a);
    return hipGetLastError();
}

template <bool VEC, bool ADD>
static hipError_t dispatch(const Path& p, const RmsArgs& a, hipStream_t s) {
#define MBROW_CASE(GG, VV) \
    if (p.g == GG && p.v == VV) return launch_one<GG, VV, VEC, ADD>(a, s);
#if MBROW_DT == 0
    MBROW_LAYOUTS_F32(MBROW_CASE)
#else
    MBROW_LAYOUTS_16(MBROW_CASE)
#endif
#undef MBROW_CASE
    return hipErrorInvalidValue;
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_rmsnorm_fwd_, MBROW_SUFFIX)(const Path& p, const RmsArgs& a,
                                                         hipStream_t s) {
    const bool add = a.residual != nullptr;
    if (p.vec) return add ? dispatch<true, true>(p, a, s) : dispatch<true, false>(p, a, s);
    return add ? dispatch<false, true>(p, a, s) : dispatch<false, false>(p, a, s);
}

}  // namespace mbrow
