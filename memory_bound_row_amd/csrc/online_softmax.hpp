// online_softmax.hpp -- device helpers shared by the cross-entropy and the
// streaming row kernels: the online softmax state and its merge, per-element
// buffer accesses for unaligned rows, and register-pressure barriers.
#pragma once

#include "ln_device.hpp"

namespace mbrow {

// Online softmax state of a set of values: their maximum, the sum of
// exp(x - max) and the sum of x.
struct XeState {
    float mx, z, sx;
};

// Merge of two states.  Every operation is commutative in (a, b), so both
// partners of a butterfly step get the same bits.  A side with no values
// (max -inf, sum 0) contributes 0 without forming exp(-inf + inf).
__device__ inline XeState xe_merge(const XeState& a, const XeState& b) {
    XeState r;
    r.mx = fmaxf(a.mx, b.mx);
    const float ta = a.mx == r.mx ? a.z : a.z * __expf(a.mx - r.mx);
    const float tb = b.mx == r.mx ? b.z : b.z * __expf(b.mx - r.mx);
    r.z = ta + tb;
    r.sx = a.sx + b.sx;
    return r;
}

template <int D>
__device__ inline XeState xe_partner(const XeState& s) {
    return XeState{partner<D>(s.mx), partner<D>(s.z), partner<D>(s.sx)};
}

// Merge over aligned groups of G lanes (G = 1..64), result in every lane.
template <int G>
__device__ inline XeState xe_group(XeState s) {
    if constexpr (G >= 2) s = xe_merge(s, xe_partner<1>(s));
    if constexpr (G >= 4) s = xe_merge(s, xe_partner<2>(s));
    if constexpr (G >= 8) s = xe_merge(s, xe_partner<4>(s));
    if constexpr (G >= 16) s = xe_merge(s, xe_partner<8>(s));
    if constexpr (G >= 32) s = xe_merge(s, xe_partner<16>(s));
    if constexpr (G >= 64) {
        const XeState lo{lane_read(s.mx, 0), lane_read(s.z, 0), lane_read(s.sx, 0)};
        const XeState hi{lane_read(s.mx, 32), lane_read(s.z, 32), lane_read(s.sx, 32)};
        s = xe_merge(lo, hi);
    }
    return s;
}

// Per-element access for rows that are not 16-byte aligned: one 2- or
// 4-byte buffer access per element through the same wave row views (a 32-bit
// offset per element instead of a 64-bit address; offsets past the view read
// 0 and drop stores).
template <class S>
__device__ __forceinline__ float elem_load(rsrc_t r, uint32_t off) {
    if constexpr (S::BYTES == 4) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    } else {
        const uint16_t b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
        if constexpr (std::is_same<S, StBF16>::value) {
            return __uint_as_float((uint32_t)b << 16);
        } else {
            return (float)__builtin_bit_cast(_Float16, b);
        }
    }
}
template <class S>
__device__ __forceinline__ void elem_store(rsrc_t r, uint32_t off, float f) {
    if constexpr (S::BYTES == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), r, (int)off, 0, 0);
    } else if constexpr (std::is_same<S, StBF16>::value) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)f), r,
                                              (int)off, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)f), r,
                                              (int)off, 0, 0);
    }
}

// Packed slots that must be formed before any later memory access is issued
// (the memory clobber orders them): bounds the per-element loads in flight
// to one group of slots, each of which holds a whole register until packed.
__device__ __forceinline__ void hold_packed(u32x4& v) {
    uint32_t a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3) : : "memory");
    v = u32x4{a0, a1, a2, a3};
}

// An integer the compiler must treat as changed: per-element comparisons
// against it are formed where they are used instead of being hoisted out of
// the row loop and held (one lane mask per element) across the passes.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

}  // namespace mbrow
