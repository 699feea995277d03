// ln_fwd.hip -- LayerNorm forward and the fused bias + dropout + residual +
// LayerNorm forward for gfx950.  Compiled once per storage type
// (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// One row is owned by a group of G lanes: G <= 64 lanes of one wave
// (64/G rows per wave), or G/64 waves of one workgroup.  Lane l of a group
// owns the 16-byte slots l, l+G, l+2G, ... of the row, so consecutive lanes
// touch consecutive 16 bytes and every load and store of a wave is fully
// coalesced ("AI infra 学习记录(2)" §2.4: 16-byte accesses cut instructions,
// not bytes).  The whole row stays in VGPRs between the statistics and the
// affine pass, so HBM is read once and written once ("AI infra 学习记录(2)"
// §4: keep x on chip instead of reading it twice).
//
// Statistics take one reduction ("Accelerating Transformer on GPU (I)"
// §4.2: one synchronisation instead of two, without the cancellation of
// E[x^2] - E[x]^2): every lane reduces its own values exactly in registers
// to (count, shifted sum, M2), then the group merges those states with the
// Chan update through DPP / swizzle / readlane; a multi-wave row adds one LDS
// exchange and one barrier.
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
struct Geometry {
    static constexpr int NT = G <= 256 ? 256 : G;   // threads per workgroup
    static constexpr int ROWS = NT / G;              // rows per workgroup
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
};

template <class S, int G, int V, bool VEC, bool FUSED>
__global__ __launch_bounds__(Geometry<G>::NT) void ln_fwd_kernel(FwdArgs a) {
    constexpr int E = S::E;
    constexpr int NT = Geometry<G>::NT;
    constexpr int ROWS = Geometry<G>::ROWS;
    constexpr int WPR = Geometry<G>::WPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lg = tid % G;
    const int rloc = tid / G;
    const int64_t row = (int64_t)blockIdx.x * ROWS + rloc;
    const bool row_ok = row < a.rows;
    const int64_t roff = row_ok ? row * a.m : 0;

    float v[V][E];      // the values being normalised (x, or the stored z)
    float ga[V][E], be[V][E];
    bool ok[V];
    int64_t col0[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int64_t s = (int64_t)i * G + lg;
        ok[i] = row_ok && s < a.nslots;
        col0[i] = s * E;
        load_slot<S, VEC, true>(a.x, roff, col0[i], a.m, ok[i], v[i]);
    }
    if constexpr (FUSED) {
        float r[V][E], b[V][E];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            load_slot<S, VEC, true>(a.residual, roff, col0[i], a.m, ok[i], r[i]);
            load_slot<S, VEC, false>(a.bias, 0, col0[i], a.m, ok[i], b[i]);
        }
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (!ok[i]) continue;
            const uint32_t bits = keep_bits<E>(row, col0[i], a.seed_lo, a.seed_hi, a.thr);
            float z[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float t = v[i][e] + b[i][e];
                const float d = ((bits >> e) & 1u) ? t * a.scale : 0.0f;
                z[e] = r[i][e] + d;
            }
            // z is stored in T; the LayerNorm runs on the stored value.
            if constexpr (VEC) {
                u32x4 zp = S::pack(z);
                u32x4* p = reinterpret_cast<u32x4*>(static_cast<char*>(a.residual_out) +
                                                    (roff + col0[i]) * S::BYTES);
                __builtin_nontemporal_store(zp, p);
                S::unpack(zp, v[i]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    v[i][e] = S::round(z[e]);
                    if (col0[i] + e < a.m) S::store1(a.residual_out, roff + col0[i] + e, z[e]);
                }
            }
            if (a.mask_out) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (col0[i] + e < a.m)
                        a.mask_out[roff + col0[i] + e] = (uint8_t)((bits >> e) & 1u);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
        load_slot<S, VEC, false>(a.gamma, 0, col0[i], a.m, ok[i], ga[i]);
        load_slot<S, VEC, false>(a.beta, 0, col0[i], a.m, ok[i], be[i]);
    }

    // Shift: the first value of the wave's part of the row (lane 0 of the
    // group, or of the wave for a multi-wave row), common to every lane that
    // merges with it.
    float c;
    if constexpr (G <= 64) c = group_broadcast_first<G>(v[0][0], lane);
    else c = lane_read(v[0][0], 0);

    // This lane's exact local state: count, sum of (v - c), and M2 about its
    // own mean (two passes over registers).
    float n_l = 0.0f, s_l = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool in = ok[i] && (VEC || col0[i] + e < a.m);
            if (in) {
                n_l += 1.0f;
                s_l += v[i][e] - c;
            }
        }
    }
    const float mu_l = n_l > 0.0f ? s_l / n_l : 0.0f;
    float q_l = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool in = ok[i] && (VEC || col0[i] + e < a.m);
            const float d = (v[i][e] - c) - mu_l;
            if (in) q_l = fmaf(d, d, q_l);
        }
    }
    Stats st{n_l, s_l, q_l};
    if constexpr (G <= 64) {
        st = group_stats<G>(st);
    } else {
        // One wave-level merge, then one LDS exchange between the WPR waves
        // of the row and a fixed-order merge (wave 0, 1, ...) in every lane.
        __shared__ float lds[ROWS][WPR][4];
        st = group_stats<64>(st);
        const int w = (tid % G) / 64;
        if (lane == 0) {
            lds[rloc][w][0] = st.n;
            lds[rloc][w][1] = st.s;
            lds[rloc][w][2] = st.q;
            lds[rloc][w][3] = c;
        }
        __syncthreads();
        const float c0 = lds[rloc][0][3];
        Stats tot{lds[rloc][0][0], lds[rloc][0][1], lds[rloc][0][2]};
#pragma unroll
        for (int k = 1; k < WPR; ++k) {
            Stats sk{lds[rloc][k][0], lds[rloc][k][1], lds[rloc][k][2]};
            tot = merge(tot, reshift(sk, lds[rloc][k][3], c0));
        }
        st = tot;
        c = c0;
    }
    const float mu_s = st.s / st.n;          // mean of (v - c)
    const float var = st.q / st.n;
    const float rs = 1.0f / sqrtf(var + a.eps);
    if (lg == 0 && row_ok) {
        if (a.mean) a.mean[row] = c + mu_s;
        if (a.rstd) a.rstd[row] = rs;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
        float out[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float xh = ((v[i][e] - c) - mu_s) * rs;
            out[e] = fmaf(xh, ga[i][e], be[i][e]);
        }
        store_slot<S, VEC, true>(a.y, roff, col0[i], a.m, ok[i], out);
    }
}

template <int G, int V, bool VEC, bool FUSED>
static hipError_t launch_one(const FwdArgs& a, hipStream_t s) {
    using Geo = Geometry<G>;
    const int64_t blocks = (a.rows + Geo::ROWS - 1) / Geo::ROWS;
    hipLaunchKernelGGL((ln_fwd_kernel<St, G, V, VEC, FUSED>), dim3((unsigned)blocks),
                       dim3(Geo::NT), 0, s, a);
    return hipGetLastError();
}

template <bool VEC, bool FUSED>
static hipError_t dispatch(const Path& p, const FwdArgs& a, hipStream_t s) {
#define MBROW_CASE(GG, VV) \
    if (p.g == GG && p.v == VV) return launch_one<GG, VV, VEC, FUSED>(a, s);
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

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_fwd_, MBROW_SUFFIX)(const Path& p, bool fused, const FwdArgs& a,
                                                 hipStream_t s) {
    if (p.vec) return fused ? dispatch<true, true>(p, a, s) : dispatch<true, false>(p, a, s);
    return fused ? dispatch<false, true>(p, a, s) : dispatch<false, false>(p, a, s);
}

}  // namespace mbrow
