// Row-major LDS rings read through gfx950's transposing LDS reads.
//
// A ring holds rows of D 16-bit channels by slot.  ds_read_b64_tr_b16 returns to lane t
// of each 16-lane group element t mod 4 of the 8-byte chunks read by lanes 4 v + t / 4,
// v = 0..3: lanes pointing at slots r + c / 4, channels c0 + 4 (c mod 4) hand lane t the
// four slots r .. r + 3 of channel c0 + t - one MFMA operand fragment of 4 consecutive
// K-values.  Two such reads give the 8 K-values of a 16x16x32 operand.
#pragma once

#include <stdint.h>

namespace diagmm {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Row-major ring of D-channel rows: byte offset of 16-byte piece ch of slot r.  Pieces are
// XOR-swizzled by slot so that the four consecutive slots of a transposed read, two
// pieces each, fall on eight distinct 16-byte bank groups (rows of 128 or 256 bytes: by
// slot mod 4; rows of 64 bytes, two per 128 bytes: by slot / 2 mod 2).
template <int D>
__device__ __forceinline__ int ring_piece(int r, int ch) {
    const int sw = D == 32 ? 2 * ((r >> 1) & 1) : 2 * (r & 3);
    return r * (2 * D) + 16 * (ch ^ sw);
}
// Offset of this lane's transposed read within a 4-slot group starting at a multiple of
// 4: slot c / 4 of the group, channels 16 cb + 4 (c mod 4) .. +3 (lane c of its 16-lane
// group).
template <int D>
__device__ __forceinline__ int tr_lane_off(int c, int cb) {
    const int r = c >> 2;
    return ring_piece<D>(r, 2 * cb + ((c & 3) >> 1)) + 8 * (c & 1);
}
// Eight consecutive slots (two groups of four) of one channel per lane, as an MFMA
// operand.  (C-style casts: the LDS address of a generic pointer into the kernel's LDS.)
template <class V, int D>
__device__ __forceinline__ V tr_read8(const unsigned char* p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 2 * D));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(V, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

}  // namespace diagmm
