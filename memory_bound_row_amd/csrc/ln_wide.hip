// ln_wide.hip -- LayerNorm forward (plain and fused with bias + dropout +
// residual) and backward for rows wider than the register layouts hold
// (more than 16384 columns), for gfx950.  Compiled once per storage type
// (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// One workgroup owns a row at a time.  The row is staged in LDS as it is
// read ("02 · llmc/ 的 CUDA kernel 层" §3.1: a row past the register budget
// goes to shared memory, so global memory is read once), and the statistics,
// the normalisation and, in the backward, the dx pass read it back from
// there.  160 KB of LDS hold 9984 16-byte slots: 39936 fp32 or 79872 16-bit
// columns of one tensor, half that per tensor for the backward's two (dy and
// x).  Slots past that capacity are read again from global memory in each
// later pass (the fused forward reads back the z it wrote for them).  The
// forward's workgroup has 1024 lanes and the whole LDS, or, for rows of at
// most 4992 slots, 512 lanes and half of it, so that two workgroups share a
// compute unit and one reads its row while the other normalises and writes
// its own.
//
// Lane t of T owns the 16-byte slots t, t + T, t + 2T, ... of the row, so
// each wave-wide access covers 1 KB of consecutive bytes.  Reductions: a
// butterfly within each wave, then the wave sums added through LDS in wave
// order, the same bits in every lane.  Arithmetic follows the register
// kernels: statistics of values shifted by the row's first value, two exact
// passes (mean, then squared deviations), y = ((v - c - mean) * rstd) * gamma
// + beta; dx = rstd * (gamma*dy - (A + xhat * B) / m) from the two row sums
// reduced together ("Accelerating Transformer on GPU (II)" §2.1-§2.2).
//
// The backward's workgroup is a row partition (rows p, p + P, ...), as in the
// register kernel: each lane accumulates dgamma and dbeta for the columns of
// its slots over the partition's rows, and, every column being owned by one
// lane, writes its partial directly ("(II)" §2.4, stage 1 of two).
#include <type_traits>

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

constexpr int kWideT = 1024;                 // lanes per workgroup (and per row)
constexpr int kWideW = kWideT / 64;          // waves
constexpr int kWideLds = 156 * 1024;         // LDS bytes for staged slots
constexpr int kWideGroup = 4;                // slots whose loads are issued together

// Slot s of a row of a [rows, m] tensor, packed in T: one 16-byte load on the
// vector path, else per element (columns past m read 0).
template <class S, bool VEC>
__device__ __forceinline__ u32x4 wide_load(const void* base, int64_t row, int m, int s) {
    if constexpr (VEC) {
        const char* p = static_cast<const char*>(base) +
                        (row * (int64_t)m + (int64_t)s * S::E) * S::BYTES;
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    } else {
        float f[S::E];
        load_elems<S>(base, row, m, s * S::E, true, f);
        return S::pack(f);   // exact: the values are representable in T
    }
}

template <class S, bool VEC>
__device__ __forceinline__ void wide_store(void* base, int64_t row, int m, int s,
                                           const float* f) {
    if constexpr (VEC) {
        char* p = static_cast<char*>(base) + (row * (int64_t)m + (int64_t)s * S::E) * S::BYTES;
        __builtin_nontemporal_store(S::pack(f), reinterpret_cast<u32x4*>(p));
    } else {
        store_elems<S>(base, row, m, s * S::E, true, f);
    }
}

// Sum of one value per lane over a workgroup of W waves, identical in every
// lane: wave butterflies, then the wave sums in wave order.  `red` is [W]
// floats of LDS that no other reduction in flight uses.
template <int W>
__device__ __forceinline__ float wide_sum(float v, float* red, int tid) {
    v = group_sum<64>(v);
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) t = t + red[w];
    return t;
}

// Columns of slot s inside the row (E for every slot but a partial last one).
template <int E>
__device__ __forceinline__ int wide_cols(int s, int m) {
    const int left = m - s * E;
    return left < E ? left : E;
}

// ---------------------------------------------------------------------------
// Forward.
// ---------------------------------------------------------------------------
// T lanes per workgroup, LB bytes of LDS for the stage: 1024 lanes and the
// whole LDS, or, for rows that fit half of it, 512 lanes and half, so that two
// workgroups share a compute unit and one reads its row while the other
// normalises and writes its own (four waves per SIMD either way: at most 128
// registers per lane).
template <class S, bool FUSED, int T, int LB>
__global__ __launch_bounds__(T, 4) void ln_wide_fwd_kernel(FwdArgs a) {
    constexpr bool VEC = false;   // the per-element path (rows of any width and alignment)
    constexpr int E = S::E;
    constexpr int G = 2;          // slots per group (E loads each)
    constexpr int W = T / 64;
    constexpr int LCAP = LB / 16;
    __shared__ u32x4 stage[LCAP];
    __shared__ float red[2][W];
    const int tid = threadIdx.x;
    const int m = (int)a.m;
    const int nslots = (int)a.nslots;
    const int J = (nslots + T - 1) / T;   // slots per lane (at most)

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        __syncthreads();   // the previous row's reads of the stage are done

        // The values of slot s being normalised, packed in T: x, or z as
        // stored.  The first pass forms z from x, the residual, the bias and
        // the mask and writes it out; later passes read the staged slots from
        // LDS and the rest back from global memory (z as written: with
        // residual_out == residual the residual is gone by then).
        auto fetch = [&](int j0, u32x4 (&v)[G], bool first) {
            u32x4 xv[G], rv[FUSED ? G : 1];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int s = tid + (j0 + u) * T;
                const bool need = j0 + u < J && s < nslots && (first || s >= LCAP);
                if (need) {
                    if (FUSED && !first) {
                        xv[u] = wide_load<S, VEC>(a.residual_out, row, m, s);
                    } else {
                        xv[u] = wide_load<S, VEC>(a.x, row, m, s);
                        if constexpr (FUSED) rv[u] = wide_load<S, VEC>(a.residual, row, m, s);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int s = tid + (j0 + u) * T;
                if (!(j0 + u < J && s < nslots)) continue;
                if (!first && s < LCAP) {
                    v[u] = stage[s];
                    continue;
                }
                if (FUSED && !first) {
                    v[u] = xv[u];
                    continue;
                }
                if constexpr (FUSED) {
                    float xf[E], rf[E], bf[E], z[E];
                    S::unpack(xv[u], xf);
                    S::unpack(rv[u], rf);
                    S::unpack(load_param<S, VEC>(a.bias, s, m, true), bf);
                    const u32x4 w =
                        dropout_words(row, s * E, a.seed_lo, a.seed_hi, a.thr);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float t = kept<E>(w, s * E, e, a.thr) ? xf[e] + bf[e] : 0.0f;
                        z[e] = fmaf(t, a.scale, rf[e]);
                    }
                    v[u] = S::pack(z);
                    if (first) {
                        float zs[E];
                        S::unpack(v[u], zs);
                        wide_store<S, VEC>(a.residual_out, row, m, s, zs);
                    }
                } else {
                    v[u] = xv[u];
                }
            }
        };

        // pass 1: read (and form z), stage
        for (int j0 = 0; j0 < J; j0 += G) {
            u32x4 v[G];
            fetch(j0, v, true);
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int s = tid + (j0 + u) * T;
                if (j0 + u < J && s < nslots && s < LCAP) stage[s] = v[u];
            }
        }
        __syncthreads();
        // shift: the row's first value (fp32 rows whose mean dwarfs their
        // spread keep their precision; harmless for 16-bit rows)
        const float c = S::template elem<0>(stage[0]);

        // passes 2-4 over the lane's slots: f(s, values, columns)
        auto over = [&](auto&& f) {
            for (int j0 = 0; j0 < J; j0 += G) {
                u32x4 v[G];
                fetch(j0, v, false);
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    const int s = tid + (j0 + u) * T;
                    if (!(j0 + u < J && s < nslots)) continue;
                    float fv[E];
                    S::unpack(v[u], fv);
                    f(s, fv, wide_cols<E>(s, m));
                }
            }
        };
        float sl = 0.0f;
        over([&](int, const float* fv, int n) {
#pragma unroll
            for (int e = 0; e < E; ++e) sl += e < n ? fv[e] - c : 0.0f;
        });
        const float mu = wide_sum<W>(sl, red[0], tid) * a.inv_m;   // mean of v - c
        float ql = 0.0f;
        over([&](int, const float* fv, int n) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = (fv[e] - c) - mu;
                ql = e < n ? fmaf(d, d, ql) : ql;
            }
        });
        const float var = wide_sum<W>(ql, red[1], tid) * a.inv_m;
        const float rs = 1.0f / sqrtf(var + a.eps);
        if (tid == 0) {
            if (a.mean) a.mean[row] = c + mu;
            if (a.rstd) a.rstd[row] = rs;
        }
        over([&](int s, const float* fv, int) {
            float ga[E], be[E], out[E];
            S::unpack(load_param<S, VEC>(a.gamma, s, m, true), ga);
            S::unpack(load_param<S, VEC>(a.beta, s, m, true), be);
#pragma unroll
            for (int e = 0; e < E; ++e) out[e] = fmaf(((fv[e] - c) - mu) * rs, ga[e], be[e]);
            wide_store<S, VEC>(a.y, row, m, s, out);
        });
    }
}

// The vector path (rows of whole 16-byte slots): the same passes with loads
// and stores through buffer views of the row, where a slot past the row
// reads 0 and its store is dropped, so no lane branches on its own slot.
// Whether a slot is in the stage is the same for its whole wave (the stage
// holds whole waves of slots), so that test is a uniform branch.  A lane's
// slots are walked in groups of G, then one at a time for the last J mod G.
// Every load of a group is issued before the group's first store (a store
// may alias a later load, so loads are not moved above it).
template <class S, bool FUSED, int T, int LB>
__global__ __launch_bounds__(T, 4) void ln_wide_fwd_vec_kernel(FwdArgs a) {
    constexpr int E = S::E;
    constexpr int W = T / 64;
    constexpr int G = kWideGroup;
    constexpr int LCAP = LB / 16;
    static_assert(LCAP % 64 == 0, "the stage holds whole waves of slots");
    __shared__ u32x4 stage[LCAP];
    __shared__ float red[2][W];
    const int tid = threadIdx.x;
    const int wbase = tid & ~63;   // the wave's first lane
    const int m = (int)a.m;
    const int nslots = (int)a.nslots;
    const int J = (nslots + T - 1) / T;   // slots per lane (at most)
    const rsrc_t vg = row_view<S>(a.gamma, 0, 1, m);
    const rsrc_t vbe = row_view<S>(a.beta, 0, 1, m);
    const rsrc_t vbi = row_view<S>(FUSED ? a.bias : a.gamma, 0, 1, m);
    auto off = [&](int s) { return s < nslots ? (uint32_t)s * 16u : kOob; };
    auto staged = [&](int j) { return wbase + j * T < LCAP; };   // uniform
    // body(j0, N) over the lane's slots j0 .. j0+N-1
    auto groups = [&](auto&& body) {
        int j0 = 0;
        for (; j0 + G <= J; j0 += G) body(j0, std::integral_constant<int, G>{});
        for (; j0 < J; ++j0) body(j0, std::integral_constant<int, 1>{});
    };

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        __syncthreads();   // the previous row's reads of the stage are done
        const rsrc_t vx = row_view<S>(a.x, row, 1, m);
        const rsrc_t vr = row_view<S>(FUSED ? a.residual : a.x, row, 1, m);
        const rsrc_t vz = row_view<S>(FUSED ? a.residual_out : a.y, row, 1, m);
        const rsrc_t vy = row_view<S>(a.y, row, 1, m);

        // The values of the lane's slots j0 .. j0+N-1 being normalised,
        // packed in T: x, or z as stored.  `first` reads every slot, forms z
        // from x, the residual, the bias and the mask and writes it out;
        // later passes read the staged slots from LDS and the rest back from
        // global memory (z as written: with residual_out == residual the
        // residual is gone by then).
        auto values = [&](int j0, auto& v, bool first) {
            constexpr int N = sizeof(v) / sizeof(v[0]);
            u32x4 xv[N], rv[FUSED ? N : 1], bv[FUSED ? N : 1];
#pragma unroll
            for (int u = 0; u < N; ++u) {
                const int s = tid + (j0 + u) * T;
                if (FUSED && !first && !staged(j0 + u)) {
                    xv[u] = buf_load_nt(vz, off(s));
                } else if (first || !staged(j0 + u)) {
                    xv[u] = buf_load_nt(vx, off(s));
                    if constexpr (FUSED) {
                        rv[u] = buf_load_nt(vr, off(s));
                        bv[u] = buf_load(vbi, off(s));
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < N; ++u) {
                const int s = tid + (j0 + u) * T;
                if (!first && staged(j0 + u)) {
                    v[u] = stage[s];
                    continue;
                }
                if (FUSED && !first) {
                    v[u] = xv[u];
                    continue;
                }
                if constexpr (FUSED) {
                    float xf[E], rf[E], bf[E], z[E];
                    S::unpack(xv[u], xf);
                    S::unpack(rv[u], rf);
                    S::unpack(bv[u], bf);
                    const u32x4 w = dropout_words(row, s * E, a.seed_lo, a.seed_hi, a.thr);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float t = kept<E>(w, s * E, e, a.thr) ? xf[e] + bf[e] : 0.0f;
                        z[e] = fmaf(t, a.scale, rf[e]);
                    }
                    v[u] = S::pack(z);
                    if (first) buf_store_nt(v[u], vz, off(s));
                } else {
                    v[u] = xv[u];
                }
            }
        };

        // pass 1: read (and form z), stage (slots past the row stage 0).
        // Slots past the stage are not read again for the statistics: pass
        // 1 keeps their count, sum and sum of squares shifted by the wave's
        // first value cw (on the row's scale, so the sums stay small), and
        // passes 2 and 3 add them in with the shift moved to c and mean.
        float cw = 0.0f, s_ov = 0.0f, q_ov = 0.0f, n_ov = 0.0f;
        groups([&](int j0, auto n) {
            constexpr int N = decltype(n)::value;
            u32x4 v[N];
            values(j0, v, true);
            if (j0 == 0) cw = lane_read(S::template elem<0>(v[0]), 0);   // uniform
#pragma unroll
            for (int u = 0; u < N; ++u) {
                if (staged(j0 + u)) {
                    stage[tid + (j0 + u) * T] = v[u];
                } else {
                    float fv[E];
                    S::unpack(v[u], fv);
                    float t = 0.0f, q = 0.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float d = fv[e] - cw;
                        t += d;
                        q = fmaf(d, d, q);
                    }
                    const bool in = tid + (j0 + u) * T < nslots;
                    s_ov += in ? t : 0.0f;
                    q_ov += in ? q : 0.0f;
                    n_ov += in ? (float)E : 0.0f;
                }
            }
        });
        __syncthreads();
        // shift: the row's first value (fp32 rows whose mean dwarfs their
        // spread keep their precision; harmless for 16-bit rows)
        const float c = S::template elem<0>(stage[0]);

        // passes 2-3: f(values, in row) over the lane's staged slots
        auto over = [&](auto&& f) {
            groups([&](int j0, auto n) {
                constexpr int N = decltype(n)::value;
#pragma unroll
                for (int u = 0; u < N; ++u) {
                    if (!staged(j0 + u)) continue;
                    float fv[E];
                    S::unpack(stage[tid + (j0 + u) * T], fv);
                    f(fv, tid + (j0 + u) * T < nslots);
                }
            });
        };
        // the slots past the stage: sum of (v - c) = s_ov + n_ov (cw - c)
        // (lanes without such slots start from 0, as rows within the stage)
        float sl = n_ov > 0.0f ? fmaf(n_ov, cw - c, s_ov) : 0.0f;
        over([&](const float* fv, bool in) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) t += fv[e] - c;
            sl += in ? t : 0.0f;
        });
        const float mu = wide_sum<W>(sl, red[0], tid) * a.inv_m;   // mean of v - c
        // and sum of (v - c - mu)^2 = q_ov - 2 dc s_ov + n_ov dc^2,
        // dc = c + mu - cw
        const float dc = (c - cw) + mu;
        float ql = n_ov > 0.0f ? fmaf(n_ov * dc, dc, fmaf(-2.0f * dc, s_ov, q_ov)) : 0.0f;
        over([&](const float* fv, bool in) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = (fv[e] - c) - mu;
                t = fmaf(d, d, t);
            }
            ql += in ? t : 0.0f;
        });
        const float var = wide_sum<W>(ql, red[1], tid) * a.inv_m;
        const float rs = 1.0f / sqrtf(var + a.eps);
        if (tid == 0) {
            if (a.mean) a.mean[row] = c + mu;
            if (a.rstd) a.rstd[row] = rs;
        }
        // pass 4: y, with gamma and beta loaded with the group
        groups([&](int j0, auto n) {
            constexpr int N = decltype(n)::value;
            u32x4 gv[N], bv[N], v[N];
#pragma unroll
            for (int u = 0; u < N; ++u) {
                const int s = tid + (j0 + u) * T;
                gv[u] = buf_load(vg, off(s));
                bv[u] = buf_load(vbe, off(s));
            }
            values(j0, v, false);
#pragma unroll
            for (int u = 0; u < N; ++u) {
                const int s = tid + (j0 + u) * T;
                float fv[E], ga[E], be[E], out[E];
                S::unpack(v[u], fv);
                S::unpack(gv[u], ga);
                S::unpack(bv[u], be);
#pragma unroll
                for (int e = 0; e < E; ++e) out[e] = fmaf(((fv[e] - c) - mu) * rs, ga[e], be[e]);
                buf_store_nt(S::pack(out), vy, off(s));
            }
        });
    }
}

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------
// The backward holds both dy and x in LDS (no second read from global
// memory), so its rows stop at what the stage holds: 4992 slots of each,
// 19968 fp32 or 39936 16-bit columns (the library caps 16-bit rows at 32768).
// Slots per lane:
template <class S>
struct WideBwd {
    static constexpr int LCAP = kWideLds / 32;
    static constexpr int J = S::E == 4 ? (LCAP + kWideT - 1) / kWideT : 32768 / 8 / kWideT;
};

template <class S, bool VEC, int MODE>
__global__ __launch_bounds__(kWideT) void ln_wide_bwd_kernel(BwdArgs a) {
    constexpr int E = S::E;
    constexpr int JM = WideBwd<S>::J;
    constexpr bool DX = MODE != (int)BwdMode::PARTIALS;
    constexpr bool PART = MODE != (int)BwdMode::DX;
    constexpr int LCAP = WideBwd<S>::LCAP;       // slots of each of dy and x
    __shared__ u32x4 sdy[LCAP], sx[LCAP];
    __shared__ float red[2][2][kWideW];
    const int tid = threadIdx.x;
    const int m = (int)a.m;
    const int nslots = (int)a.nslots;
    const int64_t part = blockIdx.x;

    constexpr int KA = PART ? JM * E : 1;
    float acc[2][KA];
#pragma unroll
    for (int k = 0; k < KA; ++k) {
        acc[0][k] = 0.0f;
        acc[1][k] = 0.0f;
    }
    int it = 0;
    for (int64_t row = part; row < a.rows; row += a.parts, ++it) {
        __syncthreads();   // the previous row's reads of the stage are done
        const float mu = a.mean[row];
        const float rs = a.rstd[row];
        // pass 1: dy and x read (the loads of a group of slots issued
        // together) and staged; A = sum g, Bm = sum g (x - mean)
        // (groups of two slots: with the accumulators live, four would not
        // fit a lane's 128 registers)
        constexpr int GB = 2;
        float A = 0.0f, Bm = 0.0f;
#pragma unroll
        for (int j0 = 0; j0 < JM; j0 += GB) {
            u32x4 d[GB], x[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int s = tid + (j0 + u) * kWideT;
                if (j0 + u < JM && s < nslots) {
                    d[u] = wide_load<S, VEC>(a.dy, row, m, s);
                    x[u] = wide_load<S, VEC>(a.x, row, m, s);
                }
            }
#pragma unroll
            for (int u = 0; u < GB; ++u) {
                const int s = tid + (j0 + u) * kWideT;
                if (!(j0 + u < JM && s < nslots)) continue;
                sdy[s] = d[u];
                sx[s] = x[u];
                if constexpr (DX) {
                    float ga[E], df[E], xf[E];
                    S::unpack(load_param<S, VEC>(a.gamma, s, m, true), ga);
                    S::unpack(d[u], df);
                    S::unpack(x[u], xf);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float g = ga[e] * df[e];   // zero outside the row
                        A += g;
                        Bm = fmaf(g, xf[e] - mu, Bm);
                    }
                }
            }
        }
        float c1 = 0.0f, c2 = 0.0f;
        if constexpr (DX) {
            A = group_sum<64>(A);
            Bm = group_sum<64>(Bm);
            float(*r)[kWideW] = red[it & 1];
            if ((tid & 63) == 0) {
                r[0][tid >> 6] = A;
                r[1][tid >> 6] = Bm;
            }
        }
        __syncthreads();   // the stage (and the row sums) are complete
        if constexpr (DX) {
            const float(*r)[kWideW] = red[it & 1];
            A = r[0][0];
            Bm = r[1][0];
#pragma unroll
            for (int w = 1; w < kWideW; ++w) {
                A = A + r[0][w];
                Bm = Bm + r[1][w];
            }
            c1 = A * a.inv_m;
            c2 = (Bm * rs) * a.inv_m;
        }
        // pass 2, from the stage: dx and the column partials
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            {
                const int s = tid + j * kWideT;
                if (s >= nslots) continue;
                float df[E], xf[E], xh[E];
                S::unpack(sdy[s], df);
                S::unpack(sx[s], xf);
#pragma unroll
                for (int e = 0; e < E; ++e) xh[e] = (xf[e] - mu) * rs;
                if constexpr (DX) {
                    float ga[E], out[E];
                    S::unpack(load_param<S, VEC>(a.gamma, s, m, true), ga);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        out[e] = rs * (ga[e] * df[e] - fmaf(xh[e], c2, c1));
                    wide_store<S, VEC>(a.dx, row, m, s, out);
                }
                if constexpr (PART) {
                    // zero past the row (df is 0 there), so no test per element
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        acc[0][j * E + e] = fmaf(df[e], xh[e], acc[0][j * E + e]);
                        acc[1][j * E + e] = acc[1][j * E + e] + df[e];
                    }
                }
            }
        }
    }
    if constexpr (PART) {
        // every column is owned by one lane: the partition's partial directly
        float* const pw = a.ws + part * 2 * a.m;
        const bool wvec = VEC && a.ws_vec;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int s = tid + j * kWideT;
            if (s >= nslots) continue;
#pragma unroll
            for (int kind = 0; kind < 2; ++kind) {
                float* dst = pw + kind * a.m + s * E;
                if (wvec) {
#pragma unroll
                    for (int e = 0; e < E; e += 4) {
                        f32x4 v = {acc[kind][j * E + e], acc[kind][j * E + e + 1],
                                   acc[kind][j * E + e + 2], acc[kind][j * E + e + 3]};
                        *reinterpret_cast<f32x4*>(dst + e) = v;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (s * E + e < m) dst[e] = acc[kind][j * E + e];
                }
            }
        }
    }
}

template <class K>
static void launch_rows(K kern, int threads, const FwdArgs& a, hipStream_t s) {
    const int64_t grid = persistent_grid(reinterpret_cast<const void*>(kern), threads, a.rows);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, s, a);
}

template <bool VEC, bool FUSED>
static hipError_t launch_fwd_one(const FwdArgs& a, hipStream_t s) {
    constexpr int kHalf = kWideLds / 2;
    const bool half = a.nslots <= kHalf / 16;
    if constexpr (VEC) {
        if (half) launch_rows(ln_wide_fwd_vec_kernel<St, FUSED, kWideT / 2, kHalf>, kWideT / 2, a, s);
        else launch_rows(ln_wide_fwd_vec_kernel<St, FUSED, kWideT, kWideLds>, kWideT, a, s);
    } else {
        if (half) launch_rows(ln_wide_fwd_kernel<St, FUSED, kWideT / 2, kHalf>, kWideT / 2, a, s);
        else launch_rows(ln_wide_fwd_kernel<St, FUSED, kWideT, kWideLds>, kWideT, a, s);
    }
    return hipGetLastError();
}

template <bool VEC, int MODE>
static hipError_t launch_bwd_one(const BwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((ln_wide_bwd_kernel<St, VEC, MODE>), dim3((unsigned)a.parts),
                       dim3(kWideT), 0, s, a);
    return hipGetLastError();
}

template <bool VEC>
static hipError_t bwd_mode(BwdMode mode, const BwdArgs& a, hipStream_t s) {
    switch (mode) {
    case BwdMode::DX: return launch_bwd_one<VEC, 0>(a, s);
    case BwdMode::DX_PARTIALS: return launch_bwd_one<VEC, 1>(a, s);
    case BwdMode::PARTIALS: return launch_bwd_one<VEC, 2>(a, s);
    default: return hipErrorInvalidValue;
    }
}

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_wide_fwd_, MBROW_SUFFIX)(bool vec, bool fused, const FwdArgs& a,
                                                      hipStream_t s) {
    if (vec) return fused ? launch_fwd_one<true, true>(a, s) : launch_fwd_one<true, false>(a, s);
    return fused ? launch_fwd_one<false, true>(a, s) : launch_fwd_one<false, false>(a, s);
}

hipError_t MBROW_CAT(launch_wide_bwd_, MBROW_SUFFIX)(bool vec, BwdMode mode, const BwdArgs& a,
                                                      hipStream_t s) {
    return vec ? bwd_mode<true>(mode, a, s) : bwd_mode<false>(mode, a, s);
}

}  // namespace mbrow
