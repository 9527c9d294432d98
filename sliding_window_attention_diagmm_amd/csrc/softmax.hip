// Banded softmax: a group of lanes per band row (a wavefront, or a workgroup of four,
// for long rows).
//
// The row (K slots, contiguous in [b][n][h][K]) is read once as aligned 16-byte pieces
// into registers; the at most two pieces it shares with the neighbouring rows are read
// and written element by element for this row's own slots only, so rows never touch
// each other's data and the softmax may run in place.  Slots whose key lies outside the
// sequence are masked by index (they hold -inf before the max and exactly +0 after).
// The row max and the sum of exponentials are group reductions; each exponential
// is computed once and kept in registers until the normalised values are written.
//
// Recipe (csarofeen/pytorch issue 2096, first fusion repro): scale, row max, subtract,
// exp, row sum, divide.  The in-range slot interval of row i is
// [w - min(w, floor(i/s)), w + min(w_upper, floor((n-1-i)/s))], slot w being the row's
// own position, so no row is ever empty.
#include "launch.hpp"
#include "tiles.hpp"

namespace diagmm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;

// Element e (0..kVec-1) of a piece held as dwords d0..d3, as float; and the raw bits of
// a float rounded to the element type.
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

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// P = pieces per lane (the row has at most 64 P pieces).
// Row geometry without device division: row -> position i = (row / h) mod n, and the
// in-range slot interval through i / s and (n - 1 - i) / s (exact multiply-based
// divisions for 31-bit operands, reciprocals from the host).
struct RowDiv {
    Div32 h, n, s;
};

template <class T, int P>
__global__ void __launch_bounds__(kThreads)
softmax_wave_kernel(const typename T::T* scores, typename T::T* probs, Problem p, float scale,
                    int64_t nrows, RowDiv rd) {
    using ST = typename T::T;
    constexpr int kVec = 16 / sizeof(ST);
    const int lane = threadIdx.x & 63;
    const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= nrows) return;
    const uint32_t bn = div32(rd.h, static_cast<uint32_t>(row));          // b * n + i
    const int64_t i = bn - div32(rd.n, bn) * rd.n.d;
    const int64_t lo_off = div32(rd.s, static_cast<uint32_t>(i));
    const int64_t hi_off = div32(rd.s, static_cast<uint32_t>(p.n - 1 - i));
    const int k_lo = static_cast<int>(p.w - (lo_off < p.w ? lo_off : p.w));
    const int k_hi = static_cast<int>(p.w + (hi_off < p.wu ? hi_off : p.wu) + 1);
    const int K = static_cast<int>(p.K);
    const int64_t g = row * p.K;                       // first element of the row
    const int sh = static_cast<int>(g & (kVec - 1));
    const int nc = (sh + K + kVec - 1) / kVec;
    const ST* src = scores + (g - sh);                 // 16-byte aligned
    ST* dst = probs + (g - sh);

    // x[q][e]: scaled score of element e of piece c = lane + 64 q (slot c*kVec + e - sh)
    float x[P][kVec];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = lane + 64 * q;
        const int base = c * kVec - sh;                // slot of element 0
        uint32_t dw[4] = {0u, 0u, 0u, 0u};   // the piece as dwords (static indices only)
        if (c < nc && in_reach(base, kVec, k_lo, k_hi)) {
            if (base >= 0 && base + kVec <= K) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(src + c * kVec);
                dw[0] = v[0];
                dw[1] = v[1];
                dw[2] = v[2];
                dw[3] = v[3];
            } else {
                const int a = base < 0 ? -base : 0;
                const int b = K - base < kVec ? K - base : kVec;
                dw[0] = load_part_dword<ST>(src + c * kVec, 0, a, b);
                dw[1] = load_part_dword<ST>(src + c * kVec, 1, a, b);
                dw[2] = load_part_dword<ST>(src + c * kVec, 2, a, b);
                dw[3] = load_part_dword<ST>(src + c * kVec, 3, a, b);
            }
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = c < nc && k >= k_lo && k < k_hi;
            const uint32_t d = kVec == 8 ? dw[e >> 1] : dw[e];
            x[q][e] = in ? scale * Elem<T>::get(d, e & 1) : -INFINITY;
            m = fmaxf(m, x[q][e]);
        }
    }
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            x[q][e] = __expf(x[q][e] - m);             // exp(-inf) = +0 for masked slots
            sum += x[q][e];
        }
    sum = wave_sum(sum);
    const float inv = 1.f / sum;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = lane + 64 * q;
        if (c >= nc) continue;
        const int base = c * kVec - sh;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (kVec == 8)
                o[j] = Elem<T>::bits(x[q][2 * j] * inv) | (Elem<T>::bits(x[q][2 * j + 1] * inv) << 16);
            else
                o[j] = Elem<T>::bits(x[q][j] * inv);
        }
        if (base >= 0 && base + kVec <= K) {
            *reinterpret_cast<u32x4*>(dst + c * kVec) = u32x4{o[0], o[1], o[2], o[3]};
        } else {
            const int a = base < 0 ? -base : 0;
            const int b = K - base < kVec ? K - base : kVec;
            store_part<ST>(dst + c * kVec, o[0], o[1], o[2], o[3], a, b);
        }
    }
}

// Reduction within aligned groups of L lanes.
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

// Rows of moderate length: L lanes per row (64 / L rows per wavefront), lane t of a group
// holding the row's pieces t, t + L, .., t + 8 L.  Every piece is loaded whole (elements
// of the neighbouring rows are read and ignored; only a piece running past the end of
// the tensor is read element by element), so the loads issue back to back; stores write
// whole pieces except the at most two a row shares with its neighbours, which are
// written element by element for the row's own slots.
template <class T, int L>
__global__ void __launch_bounds__(kThreads)
softmax_group_kernel(const typename T::T* scores, typename T::T* probs, Problem p, float scale,
                     int64_t nrows, RowDiv rd) {
    using ST = typename T::T;
    constexpr int kVec = 16 / sizeof(ST);
    constexpr int P = 9;
    constexpr int kRowsPerWave = 64 / L;
    const int lane = threadIdx.x & 63;
    const int t = lane % L;
    const int64_t row_raw = (int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6)) *
                                kRowsPerWave + lane / L;
    const bool row_ok = row_raw < nrows;
    const int64_t row = row_ok ? row_raw : nrows - 1;   // idle groups compute a real row
    const uint32_t bn = div32(rd.h, static_cast<uint32_t>(row));          // b * n + i
    const int64_t i = bn - div32(rd.n, bn) * rd.n.d;
    const int64_t lo_off = div32(rd.s, static_cast<uint32_t>(i));
    const int64_t hi_off = div32(rd.s, static_cast<uint32_t>(p.n - 1 - i));
    const int k_lo = static_cast<int>(p.w - (lo_off < p.w ? lo_off : p.w));
    const int k_hi = static_cast<int>(p.w + (hi_off < p.wu ? hi_off : p.wu) + 1);
    const int K = static_cast<int>(p.K);
    const int64_t total = nrows * p.K;
    const int64_t g = row * p.K;                       // first element of the row
    const int sh = static_cast<int>(g & (kVec - 1));
    const int nc = (sh + K + kVec - 1) / kVec;
    const ST* src = scores + (g - sh);                 // 16-byte aligned
    ST* dst = probs + (g - sh);

    // All loads first (whole pieces; the data is not touched until every load is
    // issued), then the tensor's last piece element by element if this row holds it.
    u32x4 raw[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + L * q;
        raw[q] = u32x4{0u, 0u, 0u, 0u};
        if (c < nc && in_reach(c * kVec - sh, kVec, k_lo, k_hi) && g - sh + (c + 1) * kVec <= total)
            raw[q] = *reinterpret_cast<const u32x4*>(src + c * kVec);
    }
    if (g + K + kVec > total) {                        // the row ends within a piece of the end
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int c = t + L * q;
            if (c < nc && in_reach(c * kVec - sh, kVec, k_lo, k_hi) && g - sh + (c + 1) * kVec > total) {
                const int b = K - (c * kVec - sh);
                raw[q] = load_piece_elems<ST>(src + c * kVec, 0, b < kVec ? b : kVec);
            }
        }
    }
    float x[P][kVec];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + L * q;
        const int base = c * kVec - sh;                // slot of element 0
        const uint32_t d0 = raw[q][0], d1 = raw[q][1], d2 = raw[q][2], d3 = raw[q][3];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = c < nc && k >= k_lo && k < k_hi;
            const uint32_t d = kVec == 8 ? (e < 2 ? d0 : e < 4 ? d1 : e < 6 ? d2 : d3)
                                         : (e == 0 ? d0 : e == 1 ? d1 : e == 2 ? d2 : d3);
            x[q][e] = in ? scale * Elem<T>::get(d, e & 1) : -INFINITY;
            m = fmaxf(m, x[q][e]);
        }
    }
    m = group_max<L>(m);
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            x[q][e] = __expf(x[q][e] - m);             // exp(-inf) = +0 for masked slots
            sum += x[q][e];
        }
    sum = group_sum<L>(sum);
    const float inv = 1.f / sum;
    if (!row_ok) return;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + L * q;
        if (c >= nc) continue;
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
        if (base >= 0 && base + kVec <= K) {
            *reinterpret_cast<u32x4*>(dst + c * kVec) = u32x4{o0, o1, o2, o3};
        } else {
            const int a = base < 0 ? -base : 0;
            const int b = K - base < kVec ? K - base : kVec;
            store_part<ST>(dst + c * kVec, o0, o1, o2, o3, a, b);
        }
    }
}

template <class T, int L>
hipError_t launch_g(const void* scores, void* probs, const Problem& p, float scale,
                    hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t per_block = kRowsPerBlock * (64 / L);
    const int64_t grid = (nrows + per_block - 1) / per_block;
    launch_kernel((softmax_group_kernel<T, L>), dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream, static_cast<const typename T::T*>(scores),
                       static_cast<typename T::T*>(probs), p, scale, nrows,
                       RowDiv{make_div32(static_cast<uint32_t>(p.h)),
                              make_div32(static_cast<uint32_t>(p.n)),
                              make_div32(static_cast<uint32_t>(p.s))});
    return hipGetLastError();
}

// Long rows: a workgroup of 256 lanes per row, lane t holding pieces t, t + 256, ..
// (P of them), loaded whole as in the group kernel.  The row max and sum combine the four
// wavefronts through LDS.  A wavefront per row would hold 8 P' = 136 values a lane at
// 8193 slots and run one wavefront per SIMD; here P = 5 and several rows share a SIMD.
template <class T, int P>
__global__ void __launch_bounds__(kThreads)
softmax_block_kernel(const typename T::T* scores, typename T::T* probs, Problem p, float scale,
                     int64_t nrows, RowDiv rd) {
    using ST = typename T::T;
    constexpr int kVec = 16 / sizeof(ST);
    constexpr int kWaves = kThreads / 64;
    __shared__ float red[2][kWaves];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t row = blockIdx.x;
    const uint32_t bn = div32(rd.h, static_cast<uint32_t>(row));          // b * n + i
    const int64_t i = bn - div32(rd.n, bn) * rd.n.d;
    const int64_t lo_off = div32(rd.s, static_cast<uint32_t>(i));
    const int64_t hi_off = div32(rd.s, static_cast<uint32_t>(p.n - 1 - i));
    const int k_lo = static_cast<int>(p.w - (lo_off < p.w ? lo_off : p.w));
    const int k_hi = static_cast<int>(p.w + (hi_off < p.wu ? hi_off : p.wu) + 1);
    const int K = static_cast<int>(p.K);
    const int64_t total = nrows * p.K;
    const int64_t g = row * p.K;                       // first element of the row
    const int sh = static_cast<int>(g & (kVec - 1));
    const int nc = (sh + K + kVec - 1) / kVec;
    const ST* src = scores + (g - sh);                 // 16-byte aligned
    ST* dst = probs + (g - sh);

    u32x4 raw[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + kThreads * q;
        raw[q] = u32x4{0u, 0u, 0u, 0u};
        if (c < nc && in_reach(c * kVec - sh, kVec, k_lo, k_hi) && g - sh + (c + 1) * kVec <= total)
            raw[q] = *reinterpret_cast<const u32x4*>(src + c * kVec);
    }
    if (g + K + kVec > total) {                        // the row ends within a piece of the end
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int c = t + kThreads * q;
            if (c < nc && in_reach(c * kVec - sh, kVec, k_lo, k_hi) && g - sh + (c + 1) * kVec > total) {
                const int b = K - (c * kVec - sh);
                raw[q] = load_piece_elems<ST>(src + c * kVec, 0, b < kVec ? b : kVec);
            }
        }
    }
    float x[P][kVec];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + kThreads * q;
        const int base = c * kVec - sh;                // slot of element 0
        const uint32_t d0 = raw[q][0], d1 = raw[q][1], d2 = raw[q][2], d3 = raw[q][3];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = c < nc && k >= k_lo && k < k_hi;
            const uint32_t d = kVec == 8 ? (e < 2 ? d0 : e < 4 ? d1 : e < 6 ? d2 : d3)
                                         : (e == 0 ? d0 : e == 1 ? d1 : e == 2 ? d2 : d3);
            x[q][e] = in ? scale * Elem<T>::get(d, e & 1) : -INFINITY;
            m = fmaxf(m, x[q][e]);
        }
    }
    m = wave_max(m);
    if (lane == 0) red[0][wave] = m;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < kWaves; ++v) m = fmaxf(m, red[0][v]);
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            x[q][e] = __expf(x[q][e] - m);             // exp(-inf) = +0 for masked slots
            sum += x[q][e];
        }
    sum = wave_sum(sum);
    if (lane == 0) red[1][wave] = sum;
    __syncthreads();
    sum = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) sum += red[1][v];
    const float inv = 1.f / sum;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + kThreads * q;
        if (c >= nc) continue;
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
        if (base >= 0 && base + kVec <= K) {
            *reinterpret_cast<u32x4*>(dst + c * kVec) = u32x4{o0, o1, o2, o3};
        } else {
            const int a = base < 0 ? -base : 0;
            const int b = K - base < kVec ? K - base : kVec;
            store_part<ST>(dst + c * kVec, o0, o1, o2, o3, a, b);
        }
    }
}

template <class T, int P>
hipError_t launch_b(const void* scores, void* probs, const Problem& p, float scale,
                    hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    launch_kernel((softmax_block_kernel<T, P>), dim3(static_cast<uint32_t>(nrows)),
                  dim3(kThreads), 0, stream, static_cast<const typename T::T*>(scores),
                  static_cast<typename T::T*>(probs), p, scale, nrows,
                  RowDiv{make_div32(static_cast<uint32_t>(p.h)),
                         make_div32(static_cast<uint32_t>(p.n)),
                         make_div32(static_cast<uint32_t>(p.s))});
    return hipGetLastError();
}

template <class T, int P>
hipError_t launch_p(const void* scores, void* probs, const Problem& p, float scale,
                    hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t grid = (nrows + kRowsPerBlock - 1) / kRowsPerBlock;
    launch_kernel((softmax_wave_kernel<T, P>), dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream, static_cast<const typename T::T*>(scores),
                       static_cast<typename T::T*>(probs), p, scale, nrows,
                       RowDiv{make_div32(static_cast<uint32_t>(p.h)),
                              make_div32(static_cast<uint32_t>(p.n)),
                              make_div32(static_cast<uint32_t>(p.s))});
    return hipGetLastError();
}

template <class T>
hipError_t launch_t(const void* scores, void* probs, const Problem& p, float scale,
                    hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(typename T::T);
    const int64_t pieces = (p.K + 2 * kVec - 2) / kVec;   // worst-case alignment
    // up to 9 pieces per lane: the fewest lanes per row
    if (pieces <= 9 * 1) return launch_g<T, 1>(scores, probs, p, scale, stream);
    if (pieces <= 9 * 2) return launch_g<T, 2>(scores, probs, p, scale, stream);
    if (pieces <= 9 * 4) return launch_g<T, 4>(scores, probs, p, scale, stream);
    if (pieces <= 9 * 8) return launch_g<T, 8>(scores, probs, p, scale, stream);
    if (pieces <= 9 * 16) return launch_g<T, 16>(scores, probs, p, scale, stream);
    if (pieces <= 9 * 32) return launch_g<T, 32>(scores, probs, p, scale, stream);
    if (pieces <= 64 * 2) return launch_p<T, 2>(scores, probs, p, scale, stream);
    if (pieces <= 64 * 4) return launch_p<T, 4>(scores, probs, p, scale, stream);
    if (pieces <= 64 * 8) return launch_p<T, 8>(scores, probs, p, scale, stream);
    if (pieces <= kThreads * 5) return launch_b<T, 5>(scores, probs, p, scale, stream);
    if (pieces <= kThreads * 9) return launch_b<T, 9>(scores, probs, p, scale, stream);
    return hipErrorInvalidValue;
}

}  // namespace

bool softmax_wave_supported(const Problem& p, int in_dt, int out_dt) {
    if (in_dt != out_dt) return false;
    const int64_t kvec = in_dt == kF32 ? 4 : 8;
    const int64_t pieces = (p.K + 2 * kvec - 2) / kvec;
    const int64_t grid = (p.rows() * p.h + kRowsPerBlock - 1) / kRowsPerBlock;
    return pieces <= kThreads * 9 && grid < (int64_t(1) << 31) && p.K < (int64_t(1) << 30) &&
           p.rows() * p.h < (int64_t(1) << 31);
}

hipError_t launch_softmax_wave(const void* scores, void* probs, const Problem& p, float scale,
                               int dt, hipStream_t stream) {
    switch (dt) {
    case kF32: return launch_t<F32>(scores, probs, p, scale, stream);
    case kF16: return launch_t<F16>(scores, probs, p, scale, stream);
    case kBF16: return launch_t<BF16>(scores, probs, p, scale, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace diagmm
