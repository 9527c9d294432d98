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

// ------------------------------------------------------------------ problem descriptor

struct Problem {
    int64_t b, n, h, d, w, wu, s;  // s = max(dilation, 1)
    int64_t K;                     // w + wu + 1
    __host__ __device__ int64_t rows() const { return b * n; }
};

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cus();

// Host-side rounding of the padding constant to the output type (nearest even),
// so every out-of-range slot receives the same bit pattern.
uint32_t pad_bits(float value, int out_dtype);

}  // namespace diagmm
