// Shared device/host helpers of libdiagmm: element types, conversions, the key-index
// map, and the launch descriptor every kernel family receives.
//
// The index map (TVM Discuss, "Developing a faster schedule for Longformer's kernel",
// posts 1, 3, 5): slot k of row i reads key j = i + (k - w) * s with s = max(dilation, 1);
// K = w + w_upper + 1 slots per row; a slot is in range when 0 <= j < n.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diagmm {

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// ------------------------------------------------------------------ element types
// Storage is raw bits for the 16-bit types; arithmetic is always float.

struct F32 {
    using T = float;
    static constexpr int code = kF32;
    __device__ __forceinline__ static float to_f32(T x) { return x; }
    __device__ __forceinline__ static T from_f32(float x) { return x; }
};

struct F16 {
    using T = uint16_t;
    static constexpr int code = kF16;
    __device__ __forceinline__ static float to_f32(T x) {
        return static_cast<float>(__builtin_bit_cast(_Float16, x));
    }
    // v_cvt_f16_f32 rounds to nearest even in the default float mode.
    __device__ __forceinline__ static T from_f32(float x) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
};

struct BF16 {
    using T = uint16_t;
    static constexpr int code = kBF16;
    __device__ __forceinline__ static float to_f32(T x) {
        return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
    }
    // Round to nearest even on the upper 16 bits; NaN stays a quiet NaN.
    __device__ __forceinline__ static T from_f32(float x) {
        uint32_t u = __builtin_bit_cast(uint32_t, x);
        if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<T>(((u >> 16) & 0x8000u) | 0x7fc0u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return static_cast<T>(u >> 16);
    }
};

// ------------------------------------------------------------------ 16-byte pieces
// Band rows are moved as aligned 16-byte pieces; a row's first and last piece may be
// shared with the neighbouring row.  These helpers touch only elements [a, b) of such a
// piece.  Each dword is handled as a named scalar with per-element branches: per-element
// insertion into or extraction from a vector register inside divergent branches is
// avoided on purpose (it has been miscompiled for 32-bit elements).

// Dword j (0..3) of a partial piece: own elements loaded, the others zero.
template <class ST>
__device__ __forceinline__ uint32_t load_part_dword(const ST* gp, int j, int a, int b) {
    if constexpr (sizeof(ST) == 4) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(gp);
        return (a <= j && j < b) ? p[j] : 0u;
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(gp);
        const uint32_t lo = (a <= 2 * j && 2 * j < b) ? p[2 * j] : 0u;
        const uint32_t hi = (a <= 2 * j + 1 && 2 * j + 1 < b) ? p[2 * j + 1] : 0u;
        return lo | (hi << 16);
    }
}

// Mask of the elements of dword j that lie in [a, b) (all ones / zeros per element).
template <class ST>
__device__ __forceinline__ uint32_t keep_mask(int j, int a, int b) {
    if constexpr (sizeof(ST) == 4) return (a <= j && j < b) ? 0xffffffffu : 0u;
    return ((a <= 2 * j && 2 * j < b) ? 0x0000ffffu : 0u) |
           ((a <= 2 * j + 1 && 2 * j + 1 < b) ? 0xffff0000u : 0u);
}

typedef uint32_t piece_t __attribute__((ext_vector_type(4)));

// Keep elements [a, b) of a loaded 16-byte piece, zero the others.  Kept apart from the
// load itself so that a prefetch can issue whole-piece loads and mask them only when the
// data is consumed: using a loaded value right away would wait for every load in flight.
template <class ST>
__device__ __forceinline__ piece_t mask_piece(const piece_t& v, int a, int b) {
    return piece_t{v[0] & keep_mask<ST>(0, a, b), v[1] & keep_mask<ST>(1, a, b),
                   v[2] & keep_mask<ST>(2, a, b), v[3] & keep_mask<ST>(3, a, b)};
}

// Whether a piece of `vec` elements whose element 0 is slot `base` of its band row holds
// any slot of the row's in-range interval [lo, hi): a piece that holds none is never read
// (its values are masked whatever they are), which near the ends of the sequence, where
// part of the window falls outside it, saves that part of the read.
__device__ __forceinline__ bool in_reach(int base, int vec, int lo, int hi) {
    return base + vec > lo && base < hi;
}

// Elements [a, b) of a piece read one by one (for a piece that runs past the end of its
// tensor); the others read as zero.
template <class ST>
__device__ __forceinline__ piece_t load_piece_elems(const ST* gp, int a, int b) {
    return piece_t{load_part_dword<ST>(gp, 0, a, b), load_part_dword<ST>(gp, 1, a, b),
                   load_part_dword<ST>(gp, 2, a, b), load_part_dword<ST>(gp, 3, a, b)};
}

// Store elements [a, b) of a piece whose dwords are d0..d3.
template <class ST>
__device__ __forceinline__ void store_part(ST* gp, uint32_t d0, uint32_t d1, uint32_t d2,
                                           uint32_t d3, int a, int b) {
    if constexpr (sizeof(ST) == 4) {
        uint32_t* p = reinterpret_cast<uint32_t*>(gp);
        if (a <= 0 && 0 < b) p[0] = d0;
        if (a <= 1 && 1 < b) p[1] = d1;
        if (a <= 2 && 2 < b) p[2] = d2;
        if (a <= 3 && 3 < b) p[3] = d3;
    } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(gp);
        if (a <= 0 && 0 < b) p[0] = static_cast<uint16_t>(d0);
        if (a <= 1 && 1 < b) p[1] = static_cast<uint16_t>(d0 >> 16);
        if (a <= 2 && 2 < b) p[2] = static_cast<uint16_t>(d1);
        if (a <= 3 && 3 < b) p[3] = static_cast<uint16_t>(d1 >> 16);
        if (a <= 4 && 4 < b) p[4] = static_cast<uint16_t>(d2);
        if (a <= 5 && 5 < b) p[5] = static_cast<uint16_t>(d2 >> 16);
        if (a <= 6 && 6 < b) p[6] = static_cast<uint16_t>(d3);
        if (a <= 7 && 7 < b) p[7] = static_cast<uint16_t>(d3 >> 16);
    }
}

// Wait until every vector memory operation of this wave has completed (s_waitcnt with
// vmcnt 0 and the other counters left at their maxima: expcnt 7, lgkmcnt 15).
//
// The compiler's wait insertion tracks loads per register, and a load whose value is
// only used under a condition it cannot match to the load's own stays "pending" on the
// other path.  A later write of the same register anywhere downstream - an LDS read in a
// compute loop, say - then gets a full vmcnt(0), which also waits for loads issued just
// before (a prefetch meant to overlap that loop).  Calling this where such loads are
// known to be consumed clears them from the tracking at no cost.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ------------------------------------------------------------------ problem descriptor

struct Problem {
    int64_t b, n, h, d, w, wu, s;  // s = max(dilation, 1)
    int64_t K;                     // w + wu + 1
    __host__ __device__ int64_t rows() const { return b * n; }
};

// Persistent workgroups per launch: the compute units of the current device (cached per
// device; 256 on MI355X), capped by DIAGMM_MAX_WORKGROUPS when that is set.
int device_cus();

// Host-side rounding of the padding constant to the output type (nearest even),
// so every out-of-range slot receives the same bit pattern.
uint32_t pad_bits(float value, int out_dtype);

}  // namespace diagmm
