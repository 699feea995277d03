// ln_device.hpp -- device-side building blocks of the fused LayerNorm kernels
// for gfx950 (CDNA4, wave64).
//
// Sources ("the pages"):
//   [L10]  "Accelerating Transformer on GPU (I): Kernel Fusion and LightSeq
//          Inference" (CMU 11-868 lecture-10 notes)
//   [L11]  "Accelerating Transformer on GPU (II): Training with LightSeq2"
//   [BLOG] "AI infra 学习记录(2): 从 LayerNorm 算子熟悉常见的算子优化方法"
//   [LLMC] "02 · llmc/ 的 CUDA kernel 层"
//
// Contents: storage-type traits (16-byte slot load/unpack/pack/store with
// round-to-nearest-even), the lane -> slot -> column map shared by every
// kernel, wave-level reductions built on DPP / ds_swizzle / readlane, the
// shifted (count, sum, M2) merge used for row statistics, and Philox4x32-10.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

// No implicit multiply-add contraction anywhere in the kernels: every fused
// multiply-add is written out with fmaf, so that two kernels that share an
// expression round it identically (the partials of the fused and standalone
// dgamma/dbeta paths must match bit for bit) and so that symmetric merges
// stay symmetric.
#pragma clang fp contract(off)

namespace mbrow {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Call f(std::integral_constant<int, I>) for I = 0 .. N-1 (compile-time
// indices, e.g. to pick a packed element).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Storage types.  A "slot" is 16 bytes of a row: E consecutive elements.
// ---------------------------------------------------------------------------
struct StF32 {
    static constexpr int E = 4;
    static constexpr int BYTES = 4;
    __device__ static inline float to_f(uint32_t bits) { return __uint_as_float(bits); }
    __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
    __device__ static inline u32x4 pack(const float* f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
        return v;
    }
    __device__ static inline float load1(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ static inline void store1(void* p, int64_t i, float f) {
        static_cast<float*>(p)[i] = f;
    }
    // value as it would be stored (RNE to T), back in float
    __device__ static inline float round(float f) { return f; }
    template <int e>
    __device__ static inline float elem(const u32x4& v) { return __uint_as_float(v[e]); }
};

struct StBF16 {
    static constexpr int E = 8;
    static constexpr int BYTES = 2;
    __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    __device__ static inline uint32_t pack2(float a, float b) {
        bf16x2 h = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, RNE
        return __builtin_bit_cast(uint32_t, h);
    }
    __device__ static inline u32x4 pack(const float* f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack2(f[2 * i], f[2 * i + 1]);
        return v;
    }
    __device__ static inline float load1(const void* p, int64_t i) {
        uint32_t b = static_cast<const uint16_t*>(p)[i];
        return __uint_as_float(b << 16);
    }
    __device__ static inline void store1(void* p, int64_t i, float f) {
        static_cast<__bf16*>(p)[i] = (__bf16)f;
    }
    __device__ static inline float round(float f) { return (float)(__bf16)f; }
    template <int e>
    __device__ static inline float elem(const u32x4& v) {
        const uint32_t w = v[e / 2];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

struct StF16 {
    static constexpr int E = 8;
    static constexpr int BYTES = 2;
    __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // copy the word out first: a bit_cast applied directly to the
            // vector element v[i] is miscompiled (every i reads element 0)
            const uint32_t word = v[i];
            f16x2 h = __builtin_bit_cast(f16x2, word);
            f[2 * i] = (float)h[0];
            f[2 * i + 1] = (float)h[1];
        }
    }
    __device__ static inline uint32_t pack2(float a, float b) {
        f16x2 h = {(_Float16)a, (_Float16)b};  // v_cvt_f16_f32, RNE
        return __builtin_bit_cast(uint32_t, h);
    }
    __device__ static inline u32x4 pack(const float* f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack2(f[2 * i], f[2 * i + 1]);
        return v;
    }
    __device__ static inline float load1(const void* p, int64_t i) {
        return (float)static_cast<const _Float16*>(p)[i];
    }
    __device__ static inline void store1(void* p, int64_t i, float f) {
        static_cast<_Float16*>(p)[i] = (_Float16)f;
    }
    __device__ static inline float round(float f) { return (float)(_Float16)f; }
    template <int e>
    __device__ static inline float elem(const u32x4& v) {
        const uint32_t w = v[e / 2];
        f16x2 h = __builtin_bit_cast(f16x2, w);
        return (float)h[e & 1];
    }
};

// ---------------------------------------------------------------------------
// Slot access.  VEC (row starts 16-byte aligned, cols*sizeof(T) a multiple
// of 16): one 16-byte buffer access per slot.  A wave addresses its rows
// through a buffer resource based at its first row whose size covers only
// the rows that exist, so the hardware range check returns 0 for a load and
// drops a store past the end of the tensor: no branch and no zeroing per
// access.  A lane's byte offset of slot i is fixed for the whole kernel;
// slots past the end of a row are given kOob, outside every view.
// Otherwise one access per element, each predicated on its column.
// Streaming tensors use nontemporal accesses; gamma/beta/bias (re-read by
// every row) use ordinary cached loads.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;        // beyond any view (views are < 2^31 bytes)
constexpr int kRsrcWord3 = 0x00020000;        // raw buffer, 32-bit data format
constexpr int kNt = 2;                        // nontemporal cache policy

// View of rows [row0, row0 + nrows) of a [rows, m] tensor; nrows <= 0 gives
// an empty view (every access out of range).  row0 and nrows must be
// uniform across the wave.
template <class S>
__device__ __forceinline__ rsrc_t row_view(const void* base, int64_t row0, int64_t nrows, int m) {
    const int64_t n = nrows > 0 ? nrows : 0;
    char* p = const_cast<char*>(static_cast<const char*>(base)) + row0 * (int64_t)m * S::BYTES;
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)(n * m * S::BYTES), kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load_nt(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNt);
}
__device__ __forceinline__ u32x4 buf_load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store_nt(u32x4 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kNt);
}

// Rows of one wave: a group of G <= 64 lanes owns one row, so a wave spans
// 64/G consecutive rows; wider rows span G/64 waves.
template <int G>
struct WaveRows {
    static constexpr int N = G <= 64 ? 64 / G : 1;
};

// The wave's first row within its block of NT/G rows (wave-uniform).
template <int G>
__device__ __forceinline__ int wave_first_row(int tid) {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    return G <= 64 ? w * (64 / G) : w / (G / 64);
}

// Byte offset of slot i of this lane within its wave's row view, or kOob for
// a slot past the end of the row.
template <class S, int G>
__device__ __forceinline__ uint32_t slot_offset(int tid, int i, int m, bool ok) {
    const int lg = tid % G;
    const uint32_t row_in_wave = G <= 64 ? (uint32_t)((tid & 63) / G) : 0u;
    return ok ? row_in_wave * (uint32_t)m * S::BYTES + (uint32_t)(i * G + lg) * 16u : kOob;
}

// Per-element path: E elements of row `row` starting at column col0 (< m
// checked per element), unpacked to float; outside the row reads as 0.
template <class S>
__device__ inline void load_elems(const void* base, int64_t row, int m, int col0, bool ok,
                                  float* f) {
    const int64_t off = row * (int64_t)m;
#pragma unroll
    for (int e = 0; e < S::E; ++e) f[e] = (ok && col0 + e < m) ? S::load1(base, off + col0 + e) : 0.0f;
}
template <class S>
__device__ inline void store_elems(void* base, int64_t row, int m, int col0, bool ok,
                                   const float* f) {
    const int64_t off = row * (int64_t)m;
#pragma unroll
    for (int e = 0; e < S::E; ++e)
        if (ok && col0 + e < m) S::store1(base, off + col0 + e, f[e]);
}

// One slot of a [cols] parameter vector, packed in T (cached load).
template <class S, bool VEC>
__device__ __forceinline__ u32x4 load_param(const void* base, int s, int m, bool ok) {
    if constexpr (VEC) {
        // slots past the end of the vector fall outside the view and read 0
        return buf_load(row_view<S>(base, 0, 1, m), (uint32_t)s * 16u);
    } else {
        float f[S::E];
        load_elems<S>(base, 0, m, s * S::E, ok, f);
        return S::pack(f);   // exact: the values are representable in T
    }
}

// exp(x - m) as exp2(x log2(e) - m log2(e)): one fma and the hardware exp2
// (v_exp_f32) per element, with -m log2(e) formed once per row.
constexpr float kLog2e = 1.44269504088896340736f;
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Keep a packed register array packed: the empty asm tells the compiler the
// values may have changed, so unpacking them is not hoisted out of a loop
// (which would hold the unpacked floats, twice the registers, across it).
template <int N>
__device__ __forceinline__ void keep_packed(u32x4 (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t a0 = v[i][0], a1 = v[i][1], a2 = v[i][2], a3 = v[i][3];
        asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
        v[i] = u32x4{a0, a1, a2, a3};
    }
}

// ---------------------------------------------------------------------------
// Wave-level data movement (wave64).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ inline float swz_xor16(float v) {
    // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 (stays inside 32 lanes)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
// gfx950 v_permlane32_swap: the upper 32 lanes of x trade places with the
// lower 32 lanes of y; returns (x', y') = ([x_lo, y_lo], [x_hi, y_hi]).  So
// x' + y' holds x_lo + x_hi in the lower half and y_lo + y_hi in the upper.
__device__ inline float halves_sum_swap(float x, float y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float lane_read(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

constexpr int DPP_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;       // lane i <-> 15-i within 16

// Partner of the butterfly step at distance D (lanes stay in their group of
// 2D): quad permutes for 1 and 2, mirrors for 4 and 8, swizzle for 16.  The
// mirrors pair each lane with one in the other half of its group, which is
// all a symmetric merge needs.
template <int D>
__device__ inline float partner(float v) {
    if constexpr (D == 1) return dpp<DPP_XOR1>(v);
    else if constexpr (D == 2) return dpp<DPP_XOR2>(v);
    else if constexpr (D == 4) return dpp<DPP_HALF_MIRROR>(v);
    else if constexpr (D == 8) return dpp<DPP_MIRROR>(v);
    else return swz_xor16(v);
}

// Sum over aligned groups of G lanes (G = 1..64), result in every lane of the
// group.  Adds are commutative, so both partners of a step compute the same
// bits and every lane ends with the identical sum.
template <int G>
__device__ inline float group_sum(float v) {
    if constexpr (G >= 2) v = v + partner<1>(v);
    if constexpr (G >= 4) v = v + partner<2>(v);
    if constexpr (G >= 8) v = v + partner<4>(v);
    if constexpr (G >= 16) v = v + partner<8>(v);
    if constexpr (G >= 32) v = v + partner<16>(v);
    if constexpr (G >= 64) v = lane_read(v, 0) + lane_read(v, 32);
    return v;
}

// Maximum over aligned groups of G lanes (G = 1..64), in every lane of the
// group (the same butterfly as group_sum).
template <int G>
__device__ inline float group_max(float v) {
    if constexpr (G >= 2) v = fmaxf(v, partner<1>(v));
    if constexpr (G >= 4) v = fmaxf(v, partner<2>(v));
    if constexpr (G >= 8) v = fmaxf(v, partner<4>(v));
    if constexpr (G >= 16) v = fmaxf(v, partner<8>(v));
    if constexpr (G >= 32) v = fmaxf(v, partner<16>(v));
    if constexpr (G >= 64) v = fmaxf(lane_read(v, 0), lane_read(v, 32));
    return v;
}

// ---------------------------------------------------------------------------
// Row statistics.  Each lane holds (n, s, q): its element count, the sum of
// its values minus a shift c shared by the whole group, and the sum of
// squared deviations from its own mean.  Two such states with the same shift
// merge as ([L10] §4.2, the Chan et al. pairwise update, written with sums):
//   n = na + nb,  s = sa + sb,  q = qa + qb + (nb*sa - na*sb)^2 / (na*nb*n).
// Every operation is commutative in (a, b) and no product is contracted, so
// both partners of a butterfly step get the same bits.  The shift keeps the
// sums small when the row mean is large compared with its spread ([L10]
// §4.2: E[x^2] - E[x]^2 collapses at mean 1e4).
// ---------------------------------------------------------------------------
struct Stats {
    float n, s, q;
};

__device__ inline Stats merge(const Stats& a, const Stats& b) {
    if (a.n == 0.0f) return b;
    if (b.n == 0.0f) return a;
    Stats r;
    r.n = a.n + b.n;
    r.s = a.s + b.s;
    float d = b.n * a.s - a.n * b.s;
    float w = (a.n * b.n) * r.n;
    r.q = (a.q + b.q) + (d * d) / w;
    return r;
}

template <int D>
__device__ inline Stats merge_step(const Stats& a) {
    Stats b{partner<D>(a.n), partner<D>(a.s), partner<D>(a.q)};
    // merge(a, b) and merge(b, a) coincide bit for bit: sums and products are
    // commutative, and fl(p - q) = -fl(q - p) under round-to-nearest-even, so
    // d differs only in sign and d*d is identical.
    return merge(a, b);
}

template <int G>
__device__ inline Stats group_stats(Stats st) {
    if constexpr (G >= 2) st = merge_step<1>(st);
    if constexpr (G >= 4) st = merge_step<2>(st);
    if constexpr (G >= 8) st = merge_step<4>(st);
    if constexpr (G >= 16) st = merge_step<8>(st);
    if constexpr (G >= 32) st = merge_step<16>(st);
    if constexpr (G >= 64) {
        Stats lo{lane_read(st.n, 0), lane_read(st.s, 0), lane_read(st.q, 0)};
        Stats hi{lane_read(st.n, 32), lane_read(st.s, 32), lane_read(st.q, 32)};
        st = merge(lo, hi);
    }
    return st;
}

// Re-express a state whose values were shifted by cb relative to shift ca.
__device__ inline Stats reshift(const Stats& b, float cb, float ca) {
    Stats r = b;
    r.s = b.s + b.n * (cb - ca);
    return r;
}

// Broadcast lane (group base) value to every lane of its group of G lanes.
template <int G>
__device__ inline float group_broadcast_first(float v, int lane) {
    if constexpr (G >= 64) {
        return lane_read(v, 0);
    } else if constexpr (G == 32) {
        float a = lane_read(v, 0), b = lane_read(v, 32);
        return lane < 32 ? a : b;
    } else if constexpr (G == 16) {
        float a = lane_read(v, 0), b = lane_read(v, 16);
        float c = lane_read(v, 32), d = lane_read(v, 48);
        float lo = lane < 16 ? a : b, hi = lane < 48 ? c : d;
        return lane < 32 ? lo : hi;
    } else {
        return __shfl(v, lane & ~(G - 1), 64);
    }
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of two
// 32x32->64 multiplies and xors with a Weyl-sequence key schedule.
// ---------------------------------------------------------------------------
__device__ inline u32x4 philox4x32_10(u32x4 ctr, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)ctr[0] * 0xD2511F53u;
        uint64_t p2 = (uint64_t)ctr[2] * 0xCD9E8D57u;
        u32x4 nx;
        // three-input xor in one v_bitop3_b32 (truth table 0x96)
        nx[0] = __builtin_amdgcn_bitop3_b32((uint32_t)(p2 >> 32), ctr[1], k0, 0x96);
        nx[1] = (uint32_t)p2;
        nx[2] = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), ctr[3], k1, 0x96);
        nx[3] = (uint32_t)p0;
        ctr = nx;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return ctr;
}

// Dropout uniforms of the 8-column group holding column col0 of a row:
// Philox4x32-10 with counter (col >> 3, row lo, row hi, 0) and key
// (seed lo, seed hi); column k = col & 7 of the group takes the 16-bit half
// (k & 1) of word k >> 1.  With thr == 0 every column is kept, so the
// generator is skipped and every half reads 0xffff.
__device__ inline u32x4 dropout_words(int64_t row, int col0, uint32_t seed_lo, uint32_t seed_hi,
                                      uint32_t thr) {
    if (thr == 0u) return u32x4{~0u, ~0u, ~0u, ~0u};
    u32x4 c;
    c[0] = (uint32_t)col0 >> 3;
    c[1] = (uint32_t)((uint64_t)row & 0xffffffffu);
    c[2] = (uint32_t)((uint64_t)row >> 32);
    c[3] = 0u;
    return philox4x32_10(c, seed_lo, seed_hi);
}

// Whether element e of a slot of E columns starting at col0 is kept (its
// 16-bit uniform is >= thr), from the words of its 8-column group.  E == 8:
// the slot is the whole group; E == 4: the low or the high half of one
// (col0 & 4), i.e. words 0-1 or words 2-3.
template <int E>
__device__ __forceinline__ bool kept(const u32x4& w, int col0, int e, uint32_t thr) {
    const bool high = (E == 4) && ((col0 & 4) != 0);
    const uint32_t word = high ? w[2 + (e >> 1)] : w[e >> 1];
    const uint32_t u = (e & 1) ? (word >> 16) : (word & 0xffffu);
    return u >= thr;
}

}  // namespace mbrow
