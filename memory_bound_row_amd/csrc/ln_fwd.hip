// ln_fwd.hip -- LayerNorm forward and the fused bias + dropout + residual +
// LayerNorm forward for gfx950.  Compiled once per storage type
// (-DMBROW_DT=0 fp32, 1 fp16, 2 bf16).
//
// Layout.  One row is owned by a group of G lanes: G <= 64 lanes of one wave
// (64/G rows per wave) or G/64 waves of one workgroup.  Lane l of a group owns
// the 16-byte slots l, l+G, l+2G, ... of the row, so consecutive lanes touch
// consecutive 16 bytes and every wave-wide load and store is fully coalesced
// ("AI infra 学习记录(2)" §2.4: 16-byte accesses cut instructions, not bytes).
// The whole row stays in VGPRs between the statistics and the affine pass,
// so HBM is read once and written once ("AI infra 学习记录(2)" §4).
//
// Schedule.  The grid is persistent (about as many workgroups as fit on the
// chip at once); each workgroup walks row blocks with a stride of the grid
// and double-buffers them: the loads of the next block are issued before the
// current block is reduced and written, so memory traffic and ALU work of
// each wave overlap.  Narrow rows with many blocks and high occupancy are
// launched one workgroup per block instead (the same loop, run once).
//
// Statistics ("Accelerating Transformer on GPU (I)" §4.2).  fp32 values are
// shifted by the first value c of the group's part of the row, so sums stay
// small when the mean is large compared with the spread (the page's
// E[x^2] - E[x]^2 collapse at mean 1e4); 16-bit values carry few enough
// significant bits that fp32 sums of them need no shift.  The values are
// unpacked once per row and held as floats through the passes; within a wave
// the mean and then the sum of squared deviations are exact two-pass sums
// over registers, each reduced by one DPP/swizzle butterfly with no barrier.  A multi-wave row
// merges the per-wave (count, sum, M2) states with the Chan update after one
// LDS exchange, so it takes a single barrier.
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
    static constexpr int ROWS = NT / G;              // rows per block
    static constexpr int WPR = G > 64 ? G / 64 : 1;  // waves per row
};

// Raw 16-byte slots of one row of the streaming inputs.
template <int V, bool FUSED>
struct RowBuf {
    u32x4 x[V];
    u32x4 r[FUSED ? V : 1];
};

template <class S, int G, int V, bool VEC, bool FUSED>
__global__ __launch_bounds__(Geometry<G>::NT) void ln_fwd_kernel(FwdArgs a) {
    constexpr int E = S::E;
    constexpr int ROWS = Geometry<G>::ROWS;
    constexpr int WPR = Geometry<G>::WPR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int lg = tid % G;
    const int rloc = tid / G;
    const int m = (int)a.m;
    const int nslots = (int)a.nslots;
    const int64_t nblk = (a.rows + ROWS - 1) / ROWS;

    // slot i of this lane covers columns (i*G + lg)*E .. +E-1
    bool ok[V];
    // The fused kernel keeps gamma, beta and bias packed in T in registers
    // across rows.  The plain one re-reads gamma and beta (from cache) in
    // its last pass: measured clearly faster on gfx950, although the wait
    // for such a load also covers the prefetched next block.
    constexpr bool PREG = FUSED;
    u32x4 gp[PREG ? V : 1], bp[PREG ? V : 1], bip[PREG ? V : 1];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int s = i * G + lg;
        ok[i] = s < nslots;
        if constexpr (PREG) {
            gp[i] = load_param<S, VEC>(a.gamma, s, m, ok[i]);
            bp[i] = load_param<S, VEC>(a.beta, s, m, ok[i]);
            bip[i] = load_param<S, VEC>(a.bias, s, m, ok[i]);
        }
    }
    auto param = [&](const void* base, const u32x4* regs, int i) -> u32x4 {
        if constexpr (PREG) return regs[i];
        else return load_param<S, VEC>(base, i * G + lg, m, ok[i]);
    };
    // vector path: the lane's byte offset of each slot in its wave's row view
    uint32_t vo[VEC ? V : 1];
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < V; ++i) vo[i] = slot_offset<S, G>(tid, i, m, ok[i]);
    }
    const int wrow = wave_first_row<G>(tid);
    // the rows of block blk that this wave touches (uniform across the wave)
    auto view = [&](const void* base, int64_t blk) {
        const int64_t row0 = blk * ROWS + wrow;
        const int64_t left = a.rows - row0;
        return row_view<S>(base, row0, left < WaveRows<G>::N ? left : WaveRows<G>::N, m);
    };

    auto load_row = [&](RowBuf<V, FUSED>& b, int64_t blk) {
        const int64_t row = blk * ROWS + rloc;
        const bool rok = row < a.rows;
        const int64_t r = rok ? row : 0;
        if constexpr (VEC) {
            const rsrc_t vx = view(a.x, blk);
            const rsrc_t vr = view(FUSED ? a.residual : a.x, blk);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                b.x[i] = buf_load_nt(vx, vo[i]);
                if constexpr (FUSED) b.r[i] = buf_load_nt(vr, vo[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                load_elems<S>(a.x, r, m, (i * G + lg) * E, ok[i] && rok, f);
                b.x[i] = S::pack(f);
                if constexpr (FUSED) {
                    load_elems<S>(a.residual, r, m, (i * G + lg) * E, ok[i] && rok, f);
                    b.r[i] = S::pack(f);
                }
            }
        }
    };

    __shared__ float lds[2][ROWS][WPR][4];

    // The streaming inputs of a block stay packed in T (16-bit types: half
    // the registers) until the block is processed; the values being
    // normalised are unpacked once and then held as floats through the
    // three passes.
    auto process = [&](const RowBuf<V, FUSED>& b, int64_t blk, int it) {
        const int64_t row = blk * ROWS + rloc;
        const bool rok = row < a.rows;
        const int64_t r = rok ? row : 0;
        if constexpr (PREG) {
            keep_packed(gp);
            keep_packed(bp);
        }
        // the values being normalised: x, or the stored z (as rounded to T)
        float v[V][E];
        // element e of slot i lies in the row
        auto inside = [&](int i, int e) { return ok[i] && (VEC || (i * G + lg) * E + e < m); };
        if constexpr (FUSED) {
            if constexpr (PREG) keep_packed(bip);
            // the mask words depend only on (row, column): formed before the
            // block's data is waited for
            u32x4 dw[V];
#pragma unroll
            for (int i = 0; i < V; ++i)
                dw[i] = dropout_words(row, (i * G + lg) * E, a.seed_lo, a.seed_hi, a.thr);
            keep_packed(dw);
            const rsrc_t vz = view(a.residual_out, blk);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const bool sok = ok[i] && rok;
                const int col0 = (i * G + lg) * E;
                float xv[E], rv[E], bv[E];
                S::unpack(b.x[i], xv);
                S::unpack(b.r[i], rv);
                S::unpack(param(a.bias, bip, i), bv);
                // (slots outside the tensor are never stored, so their
                // uniforms do not matter)
                const u32x4 w = dw[i];
                float z[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    // z = r + keep * (x + bias) / (1 - p), the scaling and the
                    // residual add rounded once
                    const float t = kept<E>(w, col0, e, a.thr) ? xv[e] + bv[e] : 0.0f;
                    z[e] = fmaf(t, a.scale, rv[e]);
                }
                // z is stored in T; the LayerNorm runs on the stored value.
                const u32x4 zp = S::pack(z);
                if constexpr (VEC) {
                    buf_store_nt(zp, vz, vo[i]);
                } else {
                    store_elems<S>(a.residual_out, r, m, col0, sok, z);
                }
                S::unpack(zp, v[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) S::unpack(b.x[i], v[i]);
        }
        // Shift c: the first value of this wave's part of the row.  fp32 rows
        // are shifted so a large mean cannot swamp the sums; 16-bit rows hold
        // at most 11 significant bits, and fp32 sums of them stay accurate far
        // beyond their storage step, so they are not shifted (c = 0).
        float c = 0.0f;
        if constexpr (S::BYTES == 4) {
            c = (G <= 64) ? group_broadcast_first<(G <= 64 ? G : 64)>(v[0][0], lane)
                          : lane_read(v[0][0], 0);
        }
        // pass 1: the sum of the shifted values (outside elements count 0; on
        // the vector path a slot is wholly inside or outside)
        float s_l = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if constexpr (VEC) {
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) ss += v[i][e] - c;
                s_l += ok[i] ? ss : 0.0f;
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) s_l += inside(i, e) ? v[i][e] - c : 0.0f;
            }
        }
        // pass 2: the sum of squared deviations from a mean m_l of the shifted
        // values; with `keep` the deviations replace the values in place
        // (the last pass needs exactly them)
        auto sq_dev = [&](float m_l, bool keep) {
            float q_l = 0.0f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float qq = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = (VEC || inside(i, e)) ? (v[i][e] - c) - m_l : 0.0f;
                    if (keep) v[i][e] = d;
                    if constexpr (VEC) qq = fmaf(d, d, qq);
                    else q_l = fmaf(d, d, q_l);
                }
                if constexpr (VEC) q_l += ok[i] ? qq : 0.0f;
            }
            return q_l;
        };
        float mu, var;   // mean of (v - c) for this wave's shift, variance
        if constexpr (G <= 64) {
            mu = group_sum<G>(s_l) * a.inv_m;
            var = group_sum<G>(sq_dev(mu, true)) * a.inv_m;
        } else {
            // this wave's exact state, then one exchange and a fixed-order
            // Chan merge (wave 0, 1, ...) done identically by every lane
            float n_l = 0.0f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if constexpr (VEC) {
                    n_l += ok[i] ? (float)E : 0.0f;
                } else {
                    const int left = m - (i * G + lg) * E;
                    n_l += ok[i] ? (float)(left < E ? left : E) : 0.0f;
                }
            }
            const float n_w = group_sum<64>(n_l);
            const float s_w = group_sum<64>(s_l);
            const float mu_w = n_w > 0.0f ? s_w / n_w : 0.0f;
            const float q_w = group_sum<64>(sq_dev(mu_w, false));
            const int w = lg / 64;
            const int buf = it & 1;   // double buffer: one barrier per block
            if (lane == 0) {
                lds[buf][rloc][w][0] = n_w;
                lds[buf][rloc][w][1] = s_w;
                lds[buf][rloc][w][2] = q_w;
                lds[buf][rloc][w][3] = c;
            }
            __syncthreads();
            const float c0 = lds[buf][rloc][0][3];
            Stats tot{lds[buf][rloc][0][0], lds[buf][rloc][0][1], lds[buf][rloc][0][2]};
#pragma unroll
            for (int k = 1; k < WPR; ++k) {
                Stats sk{lds[buf][rloc][k][0], lds[buf][rloc][k][1], lds[buf][rloc][k][2]};
                tot = merge(tot, reshift(sk, lds[buf][rloc][k][3], c0));
            }
            // mean relative to this wave's own shift c
            mu = tot.s / tot.n - (c - c0);
            var = tot.q / tot.n;
#pragma unroll
            for (int i = 0; i < V; ++i)
#pragma unroll
                for (int e = 0; e < E; ++e) v[i][e] = (v[i][e] - c) - mu;
        }
        const float rs = 1.0f / sqrtf(var + a.eps);
        if (lg == 0 && rok) {
            if (a.mean) a.mean[row] = c + mu;
            if (a.rstd) a.rstd[row] = rs;
        }
        // pass 3: normalise the deviations (now in v) and apply the affine map
        const rsrc_t vy = view(a.y, blk);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float ga[E], be[E], out[E];
            S::unpack(param(a.gamma, gp, i), ga);
            S::unpack(param(a.beta, bp, i), be);
#pragma unroll
            for (int e = 0; e < E; ++e) out[e] = fmaf(v[i][e] * rs, ga[e], be[e]);
            if constexpr (VEC) {
                buf_store_nt(S::pack(out), vy, vo[i]);
            } else {
                store_elems<S>(a.y, r, m, (i * G + lg) * E, ok[i] && rok, out);
            }
        }
    };

    // Persistent walk over row blocks, uniform per workgroup so the barrier
    // of a multi-wave row is reached by all.  Double-buffered (the next
    // block's loads are in flight while this one is reduced) except for
    // 1024-lane rows, whose 16 waves already keep enough loads in flight and
    // whose 128-VGPR budget has no room for a second buffer.  The next
    // block's loads are issued unconditionally (past the last block they
    // read nothing): a conditional prefetch would make the wait for the
    // current block also wait for the prefetch, since loads retire in order
    // and the wait must hold on the path without it.
    int64_t blk = blockIdx.x;
    const int64_t step = gridDim.x;
    int it = 0;
    if constexpr (Geometry<G>::NT <= 512) {
        RowBuf<V, FUSED> b0, b1;
        load_row(b0, blk);
        while (blk < nblk) {
            int64_t nxt = blk + step;
            load_row(b1, nxt);
            process(b0, blk, it++);
            blk = nxt;
            if (blk >= nblk) break;
            nxt = blk + step;
            load_row(b0, nxt);
            process(b1, blk, it++);
            blk = nxt;
        }
    } else {
        RowBuf<V, FUSED> b0;
        for (; blk < nblk; blk += step) {
            load_row(b0, blk);
            process(b0, blk, it++);
        }
    }
}

#if MBROW_DT == 0
// The dropout keep mask of a [rows, m] tensor as bytes (1 = kept), from the
// same function of (seed, row, column, p) the fused forward uses.  Tests and
// debugging only: the forward never stores the mask.  (One copy, in the fp32
// unit: it does not depend on the storage type.)
__global__ __launch_bounds__(256) void ln_dropout_mask_kernel(uint8_t* __restrict__ mask,
                                                              int64_t rows, int m, uint32_t thr,
                                                              uint32_t seed_lo,
                                                              uint32_t seed_hi) {
    const int groups = (m + 7) / 8;   // 8-column groups per row
    const int64_t total = rows * groups;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = q / groups;
        const int col0 = (int)(q - row * groups) * 8;
        const u32x4 w = dropout_words(row, col0, seed_lo, seed_hi, thr);
        uint8_t* dst = mask + row * (int64_t)m + col0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col0 + e < m) dst[e] = kept<8>(w, col0, e, thr) ? 1 : 0;
    }
}
#endif

template <int G, int V, bool VEC, bool FUSED>
static hipError_t launch_one(const FwdArgs& a, hipStream_t s) {
    using Geo = Geometry<G>;
    auto kern = ln_fwd_kernel<St, G, V, VEC, FUSED>;
    const int64_t nblk = (a.rows + Geo::ROWS - 1) / Geo::ROWS;
    // one workgroup per block for rows of one wave or less with up to 4
    // slots per lane, where three or more workgroups fit a compute unit
    // (narrow rows: 512-1024 columns 3-12 % faster so), and for the plain
    // forward's rows of two or four waves with every slot used (4096 16-bit
    // / 2048 fp32 columns and twice that: 3-8 % faster so; 512-lane rows,
    // rows with a partly used slot, and the fused kernel, whose workgroups
    // load gamma, beta and bias once, measured slower and keep the
    // persistent walk)
    constexpr int dyn = G <= 64 && V <= 4 ? 3 : (!FUSED && (G == 128 || G == 256) && V == 4 ? 1 : 0);
    const int64_t grid = persistent_grid(reinterpret_cast<const void*>(kern), Geo::NT, nblk, dyn);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Geo::NT), 0, s, a);
    return hipGetLastError();
}

template <bool VEC, bool FUSED>
static hipError_t dispatch(const Path& p, const FwdArgs& a, hipStream_t s) {
#define MBROW_CASE(GG, VV) \
    if (p.g == GG && p.v == VV) return launch_one<GG, VV, VEC, FUSED>(a, s);
#if MBROW_DT == 0
    MBROW_LAYOUTS_F32(MBROW_CASE)
#else
    MBROW_LAYOUTS_16(MBROW_CASE)
#endif
#undef MBROW_CASE
    return hipErrorInvalidValue;
}

#if MBROW_DT == 0
hipError_t launch_dropout_mask(const FwdArgs& a, hipStream_t s) {
    const int64_t groups = (a.m + 7) / 8;
    const int64_t total = a.rows * groups;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(ln_dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       a.mask_out, a.rows, (int)a.m, a.thr, a.seed_lo, a.seed_hi);
    return hipGetLastError();
}
#endif

#define MBROW_CAT2(a, b) a##b
#define MBROW_CAT(a, b) MBROW_CAT2(a, b)
hipError_t MBROW_CAT(launch_fwd_, MBROW_SUFFIX)(const Path& p, bool fused, const FwdArgs& a,
                                                 hipStream_t s) {
    if (p.vec) return fused ? dispatch<true, true>(p, a, s) : dispatch<true, false>(p, a, s);
    return fused ? dispatch<false, true>(p, a, s) : dispatch<false, false>(p, a, s);
}

}  // namespace mbrow
