// Banded softmax with the per-key additive attention mask of the first fusion repro on
// the csarofeen/pytorch issue 2096 page: a mask m[b][n] (1 keeps key j, 0 masks it; used
// linearly) adds (1 - m[b, j]) * mask_value (-10000 there) to the scaled score of every
// slot whose key is j, before the row max:
//
//   x_k = scale * S_k + (1 - m[b, i + (k - w) s]) * mask_value   (in-range slots),
//   P_k = exp(x_k - max x) / sum exp(x - max x),   out-of-range slots exactly +0.
//
// The work is laid out as in the unmasked softmax: L lanes per band row, here with at
// most 3 pieces of 16 bytes per lane (a 513-slot f16 row on 32 lanes), every piece loaded
// whole, then the mask values of the lane's slots gathered (16-byte loads for a piece
// wholly in range without dilation; otherwise element by element, the index of an
// out-of-range slot clamped to the row's own key, so every gather is in bounds), then the
// reductions and the stores (row ends element by element, so the
// softmax may run in place).  Other shapes, dtype pairs and alignments go to a
// workgroup-per-row kernel.  The gradient needs no variant: the added term does not
// depend on the scores, so the banded softmax backward applies as it is.
#include "launch.hpp"
#include "tiles.hpp"

namespace diagmm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;
// The group kernel takes G waves: 8 with dilation, so that more rows share one staged run
// of mask values, else 4.
constexpr int kPer = 3;                        // pieces per lane in the group kernel
constexpr int kMaskWin = 4096;                 // mask floats a workgroup stages (dilated rows)

template <class T> struct Elem;
template <> struct Elem<F16> {
    __device__ __forceinline__ static float get(uint32_t d, int half) {
        return F16::to_f32(static_cast<uint16_t>(half ? (d >> 16) : (d & 0xffffu)));
    }
    __device__ __forceinline__ static uint32_t bits(float x) { return F16::from_f32(x); }
};
template <> struct Elem<BF16> {
    __device__ __forceinline__ static float get(uint32_t d, int half) {
        return BF16::to_f32(static_cast<uint16_t>(half ? (d >> 16) : (d & 0xffffu)));
    }
    __device__ __forceinline__ static uint32_t bits(float x) { return BF16::from_f32(x); }
};
template <> struct Elem<F32> {
    __device__ __forceinline__ static float get(uint32_t d, int) { return __builtin_bit_cast(float, d); }
    __device__ __forceinline__ static uint32_t bits(float x) { return __builtin_bit_cast(uint32_t, x); }
};

template <int L>
__device__ __forceinline__ float group_max(float v) {
    for (int off = L / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    for (int off = L / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

struct RowDiv {
    Div32 h, n, s;
};

// Row (b * n + i) * h + hh: its position i, the flat key-mask index b * n + i of key i,
// and its in-range slot interval [k_lo, k_hi).
struct RowGeo {
    int64_t i, mrow;
    int k_lo, k_hi;
};
__device__ __forceinline__ RowGeo row_geo(const Problem& p, const RowDiv& rd, int64_t row) {
    const uint32_t bn = div32(rd.h, static_cast<uint32_t>(row));          // b * n + i
    const int64_t i = bn - div32(rd.n, bn) * rd.n.d;
    const int64_t lo_off = div32(rd.s, static_cast<uint32_t>(i));
    const int64_t hi_off = div32(rd.s, static_cast<uint32_t>(p.n - 1 - i));
    return RowGeo{i, static_cast<int64_t>(bn),
                  static_cast<int>(p.w - (lo_off < p.w ? lo_off : p.w)),
                  static_cast<int>(p.w + (hi_off < p.wu ? hi_off : p.wu) + 1)};
}

template <class T, int L, int G>
__global__ void __launch_bounds__(G * 64)
softmax_masked_group_kernel(const typename T::T* scores, typename T::T* probs,
                            const float* __restrict__ key_mask, Problem p, float scale,
                            float mask_value, int64_t nrows, RowDiv rd) {
    using ST = typename T::T;
    constexpr int kVec = 16 / sizeof(ST);
    constexpr int kRowsPerWave = 64 / L;
    const int lane = threadIdx.x & 63;
    const int t = lane % L;
    const int64_t row_raw = (int64_t(blockIdx.x) * G + (threadIdx.x >> 6)) *
                                kRowsPerWave + lane / L;
    const bool row_ok = row_raw < nrows;
    const int64_t row = row_ok ? row_raw : nrows - 1;   // idle groups compute a real row
    const RowGeo rg = row_geo(p, rd, row);
    const int K = static_cast<int>(p.K);
    const int64_t total = nrows * p.K;
    const int64_t g = row * p.K;
    const int sh = static_cast<int>(g & (kVec - 1));
    const int nc = (sh + K + kVec - 1) / kVec;
    const ST* src = scores + (g - sh);                  // 16-byte aligned
    ST* dst = probs + (g - sh);

    u32x4 raw[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int c = t + L * q;
        raw[q] = u32x4{0u, 0u, 0u, 0u};
        if (c < nc && g - sh + (c + 1) * kVec <= total)
            raw[q] = *reinterpret_cast<const u32x4*>(src + c * kVec);
    }
    if (g + K + kVec > total) {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int c = t + L * q;
            if (c < nc && g - sh + (c + 1) * kVec > total) {
                const int b = K - (c * kVec - sh);
                raw[q] = load_piece_elems<ST>(src + c * kVec, 0, b < kVec ? b : kVec);
            }
        }
    }
    // Mask values of this lane's slots (key i + (k - w) s; the row's own key when the slot
    // is out of range, whose value is then not used).
    // Without dilation a piece's slots have consecutive keys: a piece wholly in range reads
    // its mask values as one run (the loads merge into wide ones), the others element by
    // element.
    // With dilation the keys of a piece are s apart: the workgroup first copies the
    // contiguous run of mask values its rows can reach (flat positions mrow - w s ..
    // mrow + w_upper s of its first and last row) into LDS with coalesced loads, when the
    // run fits, and gathers from there.
    __shared__ float mwin[kMaskWin];
    int64_t lo = 0;
    bool staged = false;
    if (p.s > 1) {
        const int64_t r0 = int64_t(blockIdx.x) * G * kRowsPerWave;
        const int64_t r1 = (r0 + G * kRowsPerWave - 1 < nrows - 1)
                               ? r0 + G * kRowsPerWave - 1 : nrows - 1;
        const int64_t m0 = div32(rd.h, static_cast<uint32_t>(r0));
        const int64_t m1 = div32(rd.h, static_cast<uint32_t>(r1));
        lo = m0 - p.w * p.s;
        lo = lo < 0 ? 0 : lo;
        int64_t hi = m1 + p.wu * p.s;
        hi = hi > p.b * p.n - 1 ? p.b * p.n - 1 : hi;
        staged = hi - lo + 1 <= kMaskWin;            // the same for every thread
        if (staged) {
            for (int64_t x = threadIdx.x; x <= hi - lo; x += G * 64) mwin[x] = key_mask[lo + x];
            __syncthreads();
        }
    }
    // LDS index of this row's slot k: ibase + k s, clamped into the staged run (the value
    // of an out-of-range slot is not used)
    const int ibase = static_cast<int>(rg.mrow - lo - p.w * p.s);
    const int imax = static_cast<int>(kMaskWin - 1);
    const int si = static_cast<int>(p.s);
    float mk[kPer][kVec];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int base = (t + L * q) * kVec - sh;
        if (staged) {
            const int i0 = ibase + base * si;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int ix = i0 + e * si;
                mk[q][e] = mwin[ix < 0 ? 0 : (ix > imax ? imax : ix)];
            }
        } else if (p.s == 1 && base >= rg.k_lo && base + kVec <= rg.k_hi) {
            const float* mp = key_mask + rg.mrow + (base - p.w);   // consecutive, merged
#pragma unroll
            for (int e = 0; e < kVec; ++e) mk[q][e] = mp[e];
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int k = base + e;
                const bool in = k >= rg.k_lo && k < rg.k_hi;
                const int64_t off = in ? static_cast<int64_t>(k - p.w) * p.s : 0;
                mk[q][e] = key_mask[rg.mrow + off];
            }
        }
    }
    float x[kPer][kVec];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int c = t + L * q;
        const int base = c * kVec - sh;
        const uint32_t d0 = raw[q][0], d1 = raw[q][1], d2 = raw[q][2], d3 = raw[q][3];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = c < nc && k >= rg.k_lo && k < rg.k_hi;
            const uint32_t d = kVec == 8 ? (e < 2 ? d0 : e < 4 ? d1 : e < 6 ? d2 : d3)
                                         : (e == 0 ? d0 : e == 1 ? d1 : e == 2 ? d2 : d3);
            const float v = scale * Elem<T>::get(d, e & 1) + (1.f - mk[q][e]) * mask_value;
            x[q][e] = in ? v : -INFINITY;
            m = fmaxf(m, x[q][e]);
        }
    }
    m = group_max<L>(m);
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            x[q][e] = __expf(x[q][e] - m);              // exp(-inf) = +0 for masked slots
            sum += x[q][e];
        }
    sum = group_sum<L>(sum);
    const float inv = 1.f / sum;
    if (!row_ok) return;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int c = t + L * q;
        const int base = c * kVec - sh;
        uint32_t o0, o1, o2, o3;
        if constexpr (kVec == 8) {
            o0 = Elem<T>::bits(x[q][0] * inv) | (Elem<T>::bits(x[q][1] * inv) << 16);
            o1 = Elem<T>::bits(x[q][2] * inv) | (Elem<T>::bits(x[q][3] * inv) << 16);
            o2 = Elem<T>::bits(x[q][4] * inv) | (Elem<T>::bits(x[q][5] * inv) << 16);
            o3 = Elem<T>::bits(x[q][6] * inv) | (Elem<T>::bits(x[q][7] * inv) << 16);
        } else {
            o0 = Elem<T>::bits(x[q][0] * inv);
            o1 = Elem<T>::bits(x[q][1] * inv);
            o2 = Elem<T>::bits(x[q][2] * inv);
            o3 = Elem<T>::bits(x[q][3] * inv);
        }
        if (c >= nc) continue;
        if (base >= 0 && base + kVec <= K) {
            *reinterpret_cast<u32x4*>(dst + c * kVec) = u32x4{o0, o1, o2, o3};
        } else {
            const int a = base < 0 ? -base : 0;
            const int b = K - base < kVec ? K - base : kVec;
            store_part<ST>(dst + c * kVec, o0, o1, o2, o3, a, b);
        }
    }
}

// One workgroup per row: row max, sum, then the probabilities, each pass over the row's
// in-range slots with the mask term; any dtype pair, alignment and row length.
template <class In, class Out>
__global__ void __launch_bounds__(kThreads)
softmax_masked_rows_kernel(const typename In::T* scores, typename Out::T* probs,
                           const float* __restrict__ key_mask, Problem p, float scale,
                           float mask_value, int64_t nrows, RowDiv rd) {
    __shared__ float red[kWavesPerBlock];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const RowGeo rg = row_geo(p, rd, row);
        const typename In::T* src = scores + row * p.K;
        typename Out::T* dst = probs + row * p.K;
        auto xval = [&](int k) {
            return scale * In::to_f32(src[k]) +
                   (1.f - key_mask[rg.mrow + static_cast<int64_t>(k - p.w) * p.s]) * mask_value;
        };
        float m = -INFINITY;
        for (int k = rg.k_lo + static_cast<int>(threadIdx.x); k < rg.k_hi; k += kThreads)
            m = fmaxf(m, xval(k));
        m = group_max<64>(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = red[0];
        for (int v = 1; v < kWavesPerBlock; ++v) m = fmaxf(m, red[v]);
        __syncthreads();
        float sum = 0.f;
        for (int k = rg.k_lo + static_cast<int>(threadIdx.x); k < rg.k_hi; k += kThreads)
            sum += __expf(xval(k) - m);
        sum = group_sum<64>(sum);
        if (lane == 0) red[wave] = sum;
        __syncthreads();
        sum = 0.f;
        for (int v = 0; v < kWavesPerBlock; ++v) sum += red[v];
        __syncthreads();
        const float inv = 1.f / sum;
        // (in place is safe: each element is read and rewritten by the same thread, after
        // both reductions have finished reading the row)
        for (int k = static_cast<int>(threadIdx.x); k < p.K; k += kThreads) {
            float pk = 0.f;
            if (k >= rg.k_lo && k < rg.k_hi) pk = __expf(xval(k) - m) * inv;
            dst[k] = Out::from_f32(pk);
        }
    }
}

bool is16(const void* a) { return (reinterpret_cast<uintptr_t>(a) & 15) == 0; }

int group_lanes_masked(int64_t pieces) {
    for (int l = 1; l <= 32; l *= 2)
        if (pieces <= kPer * l) return l;
    return 0;
}

template <class T, int L, int G>
hipError_t launch_gw(const void* scores, void* probs, const float* key_mask, const Problem& p,
                     float scale, float mv, const RowDiv& rd, hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t per_block = G * (64 / L);
    const int64_t grid = (nrows + per_block - 1) / per_block;
    launch_kernel((softmax_masked_group_kernel<T, L, G>), dim3(static_cast<uint32_t>(grid)),
                  dim3(G * 64), 0, stream, static_cast<const typename T::T*>(scores),
                  static_cast<typename T::T*>(probs), key_mask, p, scale, mv, nrows, rd);
    return hipGetLastError();
}
template <class T, int L>
hipError_t launch_g(const void* scores, void* probs, const float* key_mask, const Problem& p,
                    float scale, float mv, const RowDiv& rd, hipStream_t stream) {
    if (p.s > 1) return launch_gw<T, L, 8>(scores, probs, key_mask, p, scale, mv, rd, stream);
    return launch_gw<T, L, 4>(scores, probs, key_mask, p, scale, mv, rd, stream);
}

template <class T>
hipError_t launch_group(const void* scores, void* probs, const float* key_mask,
                        const Problem& p, float scale, float mv, int l, const RowDiv& rd,
                        hipStream_t stream) {
    switch (l) {
    case 1: return launch_g<T, 1>(scores, probs, key_mask, p, scale, mv, rd, stream);
    case 2: return launch_g<T, 2>(scores, probs, key_mask, p, scale, mv, rd, stream);
    case 4: return launch_g<T, 4>(scores, probs, key_mask, p, scale, mv, rd, stream);
    case 8: return launch_g<T, 8>(scores, probs, key_mask, p, scale, mv, rd, stream);
    case 16: return launch_g<T, 16>(scores, probs, key_mask, p, scale, mv, rd, stream);
    default: return launch_g<T, 32>(scores, probs, key_mask, p, scale, mv, rd, stream);
    }
}

template <class In, class Out>
hipError_t launch_rows(const void* scores, void* probs, const float* key_mask, const Problem& p,
                       float scale, float mv, const RowDiv& rd, hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t grid = nrows < (int64_t(1) << 20) ? nrows : (int64_t(1) << 20);
    launch_kernel((softmax_masked_rows_kernel<In, Out>), dim3(static_cast<uint32_t>(grid)),
                  dim3(kThreads), 0, stream, static_cast<const typename In::T*>(scores),
                  static_cast<typename Out::T*>(probs), key_mask, p, scale, mv, nrows, rd);
    return hipGetLastError();
}

}  // namespace

bool softmax_masked_supported(const Problem& p) {
    return p.rows() * p.h < (int64_t(1) << 31) && p.rows() < (int64_t(1) << 31) &&
           p.K < (int64_t(1) << 30);
}

hipError_t launch_softmax_masked(const void* scores, void* probs, const float* key_mask,
                                 const Problem& p, float scale, float mask_value, int in_dt,
                                 int out_dt, hipStream_t stream) {
    const RowDiv rd{make_div32(static_cast<uint32_t>(p.h)), make_div32(static_cast<uint32_t>(p.n)),
                    make_div32(static_cast<uint32_t>(p.s))};
    const int64_t kvec = in_dt == kF32 ? 4 : 8;
    const int l = group_lanes_masked((p.K + 2 * kvec - 2) / kvec);
    if (!force_simple() && in_dt == out_dt && l != 0 && is16(scores) && is16(probs)) {
        if (in_dt == kF16) return launch_group<F16>(scores, probs, key_mask, p, scale, mask_value, l, rd, stream);
        if (in_dt == kBF16) return launch_group<BF16>(scores, probs, key_mask, p, scale, mask_value, l, rd, stream);
        return launch_group<F32>(scores, probs, key_mask, p, scale, mask_value, l, rd, stream);
    }
    if (in_dt == kF16 && out_dt == kF16) return launch_rows<F16, F16>(scores, probs, key_mask, p, scale, mask_value, rd, stream);
    if (in_dt == kF16 && out_dt == kF32) return launch_rows<F16, F32>(scores, probs, key_mask, p, scale, mask_value, rd, stream);
    if (in_dt == kBF16 && out_dt == kBF16) return launch_rows<BF16, BF16>(scores, probs, key_mask, p, scale, mask_value, rd, stream);
    if (in_dt == kBF16 && out_dt == kF32) return launch_rows<BF16, F32>(scores, probs, key_mask, p, scale, mask_value, rd, stream);
    if (in_dt == kF32 && out_dt == kF32) return launch_rows<F32, F32>(scores, probs, key_mask, p, scale, mask_value, rd, stream);
    return hipErrorInvalidValue;
}

}  // namespace diagmm
