// Banded softmax backward: the gradient with respect to the stored scores S of the banded
// softmax P (x_k = scale * S_k, P = softmax(x) over the in-range slots), given P and the
// gradient dP with respect to P:
//
//   dS_k = scale * P_k * (dP_k - sum_m P_m dP_m)   (in-range slots k, m; 0 elsewhere).
//
// The pages print only the forward recipe (csarofeen/pytorch issue 2096, first fusion
// repro: scale, max, subtract, exp, sum, divide) and say that the kernel has two backward
// functions (TVM Discuss, "Developing a faster schedule for Longformer's kernel", post 6)
// that multiply a band gradient; this is the chain rule through that recipe, the step
// that turns dP = qk(dO, V) into the band those functions take for dQ and dK.
//
// Rows are laid out as in the forward softmax ([b][n][h][K], contiguous), and so is the
// work: a group of L lanes per band row (a whole wavefront for long rows), every piece
// of P and dP loaded whole as an aligned 16-byte piece before any is used, the masked dot
// product reduced within the group, and the output written as whole pieces except the at
// most two a row shares with its neighbours, which are written element by element for the
// row's own slots (so dS may overwrite P or dP in place).  Slots whose key lies outside
// the sequence are masked by index: they never enter the dot product, whatever P and dP
// hold there, and their gradient is exactly +0.
//
// Rows longer than a wavefront's registers hold well take a workgroup per row with the
// same one-read layout; rows of other alignments, or longer still, go to a
// workgroup-per-row kernel that reads the row twice.
#include "launch.hpp"
#include "tiles.hpp"

namespace diagmm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / 64;

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
__device__ __forceinline__ float group_sum(float v) {
    for (int off = L / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

struct RowDiv {
    Div32 h, n, s;
};

// In-range slot interval [k_lo, k_hi) of band row `row` (b * n + i) * h + hh.
struct Range {
    int k_lo, k_hi;
};
__device__ __forceinline__ Range row_range(const Problem& p, const RowDiv& rd, int64_t row) {
    const uint32_t bn = div32(rd.h, static_cast<uint32_t>(row));          // b * n + i
    const int64_t i = bn - div32(rd.n, bn) * rd.n.d;
    const int64_t lo_off = div32(rd.s, static_cast<uint32_t>(i));
    const int64_t hi_off = div32(rd.s, static_cast<uint32_t>(p.n - 1 - i));
    return Range{static_cast<int>(p.w - (lo_off < p.w ? lo_off : p.w)),
                 static_cast<int>(p.w + (hi_off < p.wu ? hi_off : p.wu) + 1)};
}

// L lanes per row (64 / L rows per wavefront), lane t of a group holding the row's pieces
// t, t + L, .., t + (P - 1) L of both P and dP.
template <class T, int L, int P>
__global__ void __launch_bounds__(kThreads)
softmax_bwd_group_kernel(const typename T::T* probs, const typename T::T* dprobs,
                         typename T::T* dscores, Problem p, float scale, int64_t nrows,
                         RowDiv rd) {
    using ST = typename T::T;
    constexpr int kVec = 16 / sizeof(ST);
    constexpr int kRowsPerWave = 64 / L;
    const int lane = threadIdx.x & 63;
    const int t = lane % L;
    const int64_t row_raw = (int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6)) *
                                kRowsPerWave + lane / L;
    const bool row_ok = row_raw < nrows;
    const int64_t row = row_ok ? row_raw : nrows - 1;   // idle groups compute a real row
    const Range rg = row_range(p, rd, row);
    const int K = static_cast<int>(p.K);
    const int64_t total = nrows * p.K;
    const int64_t g = row * p.K;                       // first element of the row
    const int sh = static_cast<int>(g & (kVec - 1));
    const int nc = (sh + K + kVec - 1) / kVec;         // pieces the row touches
    const ST* ps = probs + (g - sh);                   // 16-byte aligned
    const ST* ds = dprobs + (g - sh);
    ST* dst = dscores + (g - sh);

    // All loads first: whole pieces, except a piece that runs past the end of the tensor,
    // which is read element by element.
    u32x4 rp[P], rd_[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + L * q;
        rp[q] = rd_[q] = u32x4{0u, 0u, 0u, 0u};
        if (c < nc && in_reach(c * kVec - sh, kVec, rg.k_lo, rg.k_hi) &&
            g - sh + (c + 1) * kVec <= total) {
            rp[q] = *reinterpret_cast<const u32x4*>(ps + c * kVec);
            rd_[q] = *reinterpret_cast<const u32x4*>(ds + c * kVec);
        }
    }
    if (g + K + kVec > total) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int c = t + L * q;
            if (c < nc && in_reach(c * kVec - sh, kVec, rg.k_lo, rg.k_hi) &&
                g - sh + (c + 1) * kVec > total) {
                const int b = K - (c * kVec - sh);
                rp[q] = load_piece_elems<ST>(ps + c * kVec, 0, b < kVec ? b : kVec);
                rd_[q] = load_piece_elems<ST>(ds + c * kVec, 0, b < kVec ? b : kVec);
            }
        }
    }
    // Element e of a piece held as dwords d0..d3 (named scalars, static selection).
    auto elem = [&](uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3, int e) {
        const uint32_t d = kVec == 8 ? (e < 2 ? d0 : e < 4 ? d1 : e < 6 ? d2 : d3)
                                     : (e == 0 ? d0 : e == 1 ? d1 : e == 2 ? d2 : d3);
        return Elem<T>::get(d, e & 1);
    };
    // The masked dot product sum_m P_m dP_m (a select, so non-finite values in
    // out-of-range slots never reach it).
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + L * q;
        const int base = c * kVec - sh;                // slot of element 0
        const uint32_t a0 = rp[q][0], a1 = rp[q][1], a2 = rp[q][2], a3 = rp[q][3];
        const uint32_t b0 = rd_[q][0], b1 = rd_[q][1], b2 = rd_[q][2], b3 = rd_[q][3];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = c < nc && k >= rg.k_lo && k < rg.k_hi;
            const float pd = elem(a0, a1, a2, a3, e) * elem(b0, b1, b2, b3, e);
            dot += in ? pd : 0.f;
        }
    }
    dot = group_sum<L>(dot);
    if (!row_ok) return;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + L * q;
        const int base = c * kVec - sh;
        const uint32_t a0 = rp[q][0], a1 = rp[q][1], a2 = rp[q][2], a3 = rp[q][3];
        const uint32_t b0 = rd_[q][0], b1 = rd_[q][1], b2 = rd_[q][2], b3 = rd_[q][3];
        float gv[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = k >= rg.k_lo && k < rg.k_hi;
            const float r = scale * elem(a0, a1, a2, a3, e) * (elem(b0, b1, b2, b3, e) - dot);
            gv[e] = in ? r : 0.f;
        }
        uint32_t o0, o1, o2, o3;
        if constexpr (kVec == 8) {
            o0 = Elem<T>::bits(gv[0]) | (Elem<T>::bits(gv[1]) << 16);
            o1 = Elem<T>::bits(gv[2]) | (Elem<T>::bits(gv[3]) << 16);
            o2 = Elem<T>::bits(gv[4]) | (Elem<T>::bits(gv[5]) << 16);
            o3 = Elem<T>::bits(gv[6]) | (Elem<T>::bits(gv[7]) << 16);
        } else {
            o0 = Elem<T>::bits(gv[0]);
            o1 = Elem<T>::bits(gv[1]);
            o2 = Elem<T>::bits(gv[2]);
            o3 = Elem<T>::bits(gv[3]);
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

// One workgroup per row for rows longer than a wavefront's registers hold well (a wave
// kernel with 17 pieces per lane needs every VGPR and runs one wave per SIMD): thread t
// holds pieces t, t + 256, .., t + 256 (P - 1) of P and dP, the dot product is reduced
// within each wavefront and then across the four through LDS, and every read completes
// before the barrier that ends that reduction, so the kernel may run in place.
template <class T, int P>
__global__ void __launch_bounds__(kThreads)
softmax_bwd_block_kernel(const typename T::T* probs, const typename T::T* dprobs,
                         typename T::T* dscores, Problem p, float scale, int64_t nrows,
                         RowDiv rd) {
    using ST = typename T::T;
    constexpr int kVec = 16 / sizeof(ST);
    __shared__ float part[kWavesPerBlock];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const Range rg = row_range(p, rd, row);
    const int K = static_cast<int>(p.K);
    const int64_t total = nrows * p.K;
    const int64_t g = row * p.K;
    const int sh = static_cast<int>(g & (kVec - 1));
    const int nc = (sh + K + kVec - 1) / kVec;
    const ST* ps = probs + (g - sh);
    const ST* ds = dprobs + (g - sh);
    ST* dst = dscores + (g - sh);

    u32x4 rp[P], rd_[P];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + kThreads * q;
        rp[q] = rd_[q] = u32x4{0u, 0u, 0u, 0u};
        if (c < nc && in_reach(c * kVec - sh, kVec, rg.k_lo, rg.k_hi) &&
            g - sh + (c + 1) * kVec <= total) {
            rp[q] = *reinterpret_cast<const u32x4*>(ps + c * kVec);
            rd_[q] = *reinterpret_cast<const u32x4*>(ds + c * kVec);
        }
    }
    if (g + K + kVec > total) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int c = t + kThreads * q;
            if (c < nc && in_reach(c * kVec - sh, kVec, rg.k_lo, rg.k_hi) &&
                g - sh + (c + 1) * kVec > total) {
                const int b = K - (c * kVec - sh);
                rp[q] = load_piece_elems<ST>(ps + c * kVec, 0, b < kVec ? b : kVec);
                rd_[q] = load_piece_elems<ST>(ds + c * kVec, 0, b < kVec ? b : kVec);
            }
        }
    }
    auto elem = [&](uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3, int e) {
        const uint32_t d = kVec == 8 ? (e < 2 ? d0 : e < 4 ? d1 : e < 6 ? d2 : d3)
                                     : (e == 0 ? d0 : e == 1 ? d1 : e == 2 ? d2 : d3);
        return Elem<T>::get(d, e & 1);
    };
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + kThreads * q;
        const int base = c * kVec - sh;
        const uint32_t a0 = rp[q][0], a1 = rp[q][1], a2 = rp[q][2], a3 = rp[q][3];
        const uint32_t b0 = rd_[q][0], b1 = rd_[q][1], b2 = rd_[q][2], b3 = rd_[q][3];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = c < nc && k >= rg.k_lo && k < rg.k_hi;
            const float pd = elem(a0, a1, a2, a3, e) * elem(b0, b1, b2, b3, e);
            dot += in ? pd : 0.f;
        }
    }
    dot = group_sum<64>(dot);
    if ((t & 63) == 0) part[t >> 6] = dot;
    __syncthreads();
    dot = 0.f;
#pragma unroll
    for (int wv = 0; wv < kWavesPerBlock; ++wv) dot += part[wv];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int c = t + kThreads * q;
        if (c >= nc) continue;
        const int base = c * kVec - sh;
        const uint32_t a0 = rp[q][0], a1 = rp[q][1], a2 = rp[q][2], a3 = rp[q][3];
        const uint32_t b0 = rd_[q][0], b1 = rd_[q][1], b2 = rd_[q][2], b3 = rd_[q][3];
        float gv[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int k = base + e;
            const bool in = k >= rg.k_lo && k < rg.k_hi;
            const float r = scale * elem(a0, a1, a2, a3, e) * (elem(b0, b1, b2, b3, e) - dot);
            gv[e] = in ? r : 0.f;
        }
        uint32_t o0, o1, o2, o3;
        if constexpr (kVec == 8) {
            o0 = Elem<T>::bits(gv[0]) | (Elem<T>::bits(gv[1]) << 16);
            o1 = Elem<T>::bits(gv[2]) | (Elem<T>::bits(gv[3]) << 16);
            o2 = Elem<T>::bits(gv[4]) | (Elem<T>::bits(gv[5]) << 16);
            o3 = Elem<T>::bits(gv[6]) | (Elem<T>::bits(gv[7]) << 16);
        } else {
            o0 = Elem<T>::bits(gv[0]);
            o1 = Elem<T>::bits(gv[1]);
            o2 = Elem<T>::bits(gv[2]);
            o3 = Elem<T>::bits(gv[3]);
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

// One workgroup per row, any alignment and length: the dot product over the row's
// in-range slots (strided over the threads, then reduced across the workgroup), then the
// gradient element by element.  Every read of the row completes before the first write
// (the reduction's barriers separate them), so it too may run in place.
template <class T>
__global__ void __launch_bounds__(kThreads)
softmax_bwd_row_kernel(const typename T::T* probs, const typename T::T* dprobs,
                       typename T::T* dscores, Problem p, float scale, int64_t nrows,
                       RowDiv rd) {
    __shared__ float part[kWavesPerBlock];
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const Range rg = row_range(p, rd, row);
        const int64_t g = row * p.K;
        float dot = 0.f;
        for (int k = rg.k_lo + static_cast<int>(threadIdx.x); k < rg.k_hi; k += kThreads)
            dot += T::to_f32(probs[g + k]) * T::to_f32(dprobs[g + k]);
        dot = group_sum<64>(dot);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = dot;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWavesPerBlock; ++wv) tot += part[wv];
        __syncthreads();                                // part is reused by the next row
        for (int k = static_cast<int>(threadIdx.x); k < p.K; k += kThreads) {
            float r = 0.f;
            if (k >= rg.k_lo && k < rg.k_hi)
                r = scale * T::to_f32(probs[g + k]) * (T::to_f32(dprobs[g + k]) - tot);
            dscores[g + k] = T::from_f32(r);
        }
    }
}

template <class T, int L, int P>
hipError_t launch_g(const void* probs, const void* dprobs, void* dscores, const Problem& p,
                    float scale, const RowDiv& rd, hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t per_block = kWavesPerBlock * (64 / L);
    const int64_t grid = (nrows + per_block - 1) / per_block;
    launch_kernel((softmax_bwd_group_kernel<T, L, P>), dim3(static_cast<uint32_t>(grid)),
                  dim3(kThreads), 0, stream, static_cast<const typename T::T*>(probs),
                  static_cast<const typename T::T*>(dprobs),
                  static_cast<typename T::T*>(dscores), p, scale, nrows, rd);
    return hipGetLastError();
}

// Lanes per row for a row touching `pieces` 16-byte pieces: the fewest lanes holding at
// most 3 pieces each (a 513-slot f16 row on 32 lanes: one load instruction then covers two
// rows of 512 contiguous bytes), a whole wavefront with up to 8 each, or (returned as 256)
// a whole workgroup with up to 5 or 9 each; 0 = the row kernel.
int group_lanes(int64_t pieces, int* per_lane) {
    for (int l = 1; l <= 32; l *= 2)
        if (pieces <= 3 * l) {
            *per_lane = 3;
            return l;
        }
    for (int pl : {2, 4, 8})
        if (pieces <= 64 * pl) {
            *per_lane = pl;
            return 64;
        }
    for (int pl : {5, 9})
        if (pieces <= kThreads * pl) {
            *per_lane = pl;
            return kThreads;
        }
    return 0;
}

template <class T, int P>
hipError_t launch_b(const void* probs, const void* dprobs, void* dscores, const Problem& p,
                    float scale, const RowDiv& rd, hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    launch_kernel((softmax_bwd_block_kernel<T, P>), dim3(static_cast<uint32_t>(nrows)),
                  dim3(kThreads), 0, stream, static_cast<const typename T::T*>(probs),
                  static_cast<const typename T::T*>(dprobs),
                  static_cast<typename T::T*>(dscores), p, scale, nrows, rd);
    return hipGetLastError();
}

template <class T>
hipError_t launch_t(const void* probs, const void* dprobs, void* dscores, const Problem& p,
                    float scale, bool fast, hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(typename T::T);
    const RowDiv rd{make_div32(static_cast<uint32_t>(p.h)), make_div32(static_cast<uint32_t>(p.n)),
                    make_div32(static_cast<uint32_t>(p.s))};
    const int64_t pieces = (p.K + 2 * kVec - 2) / kVec;   // worst-case alignment
    int per = 0;
    const int l = fast ? group_lanes(pieces, &per) : 0;
    switch (l) {
    case 1: return launch_g<T, 1, 3>(probs, dprobs, dscores, p, scale, rd, stream);
    case 2: return launch_g<T, 2, 3>(probs, dprobs, dscores, p, scale, rd, stream);
    case 4: return launch_g<T, 4, 3>(probs, dprobs, dscores, p, scale, rd, stream);
    case 8: return launch_g<T, 8, 3>(probs, dprobs, dscores, p, scale, rd, stream);
    case 16: return launch_g<T, 16, 3>(probs, dprobs, dscores, p, scale, rd, stream);
    case 32: return launch_g<T, 32, 3>(probs, dprobs, dscores, p, scale, rd, stream);
    case 64:
        if (per == 2) return launch_g<T, 64, 2>(probs, dprobs, dscores, p, scale, rd, stream);
        if (per == 4) return launch_g<T, 64, 4>(probs, dprobs, dscores, p, scale, rd, stream);
        return launch_g<T, 64, 8>(probs, dprobs, dscores, p, scale, rd, stream);
    case kThreads:
        if (per == 5) return launch_b<T, 5>(probs, dprobs, dscores, p, scale, rd, stream);
        return launch_b<T, 9>(probs, dprobs, dscores, p, scale, rd, stream);
    default: {
        const int64_t nrows = p.rows() * p.h;
        const int64_t grid = nrows < (int64_t(1) << 20) ? nrows : (int64_t(1) << 20);
        launch_kernel((softmax_bwd_row_kernel<T>), dim3(static_cast<uint32_t>(grid)),
                      dim3(kThreads), 0, stream, static_cast<const typename T::T*>(probs),
                      static_cast<const typename T::T*>(dprobs),
                      static_cast<typename T::T*>(dscores), p, scale, nrows, rd);
        return hipGetLastError();
    }
    }
}

bool is16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// The fast kernels need 16-byte aligned tensors, rows of at most 256 x 9 pieces and
// 32-bit row arithmetic; the row kernel takes the rest (32-bit row counts).
bool softmax_bwd_fast(const Problem& p, int dt, const void* a, const void* b, const void* c) {
    const int64_t kvec = dt == kF32 ? 4 : 8;
    const int64_t pieces = (p.K + 2 * kvec - 2) / kvec;
    int per = 0;
    return group_lanes(pieces, &per) != 0 && is16(a) && is16(b) && is16(c) &&
           p.rows() * p.h < (int64_t(1) << 31) && p.K < (int64_t(1) << 30);
}

bool softmax_bwd_supported(const Problem& p) {
    return p.rows() * p.h < (int64_t(1) << 31) && p.n < (int64_t(1) << 31) &&
           p.K < (int64_t(1) << 30);
}

int64_t softmax_bwd_workgroups(const Problem& p, int dt, bool fast) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t kvec = dt == kF32 ? 4 : 8;
    int per = 0;
    const int l = fast ? group_lanes((p.K + 2 * kvec - 2) / kvec, &per) : 0;
    if (l == 0) return nrows < (int64_t(1) << 20) ? nrows : (int64_t(1) << 20);
    if (l == kThreads) return nrows;
    const int64_t per_block = kWavesPerBlock * (64 / l);
    return (nrows + per_block - 1) / per_block;
}

const char* softmax_bwd_kernel_name(const Problem& p, int dt, bool fast) {
    if (!fast) return "softmax_bwd_rows";
    const int64_t kvec = dt == kF32 ? 4 : 8;
    int per = 0;
    const int l = group_lanes((p.K + 2 * kvec - 2) / kvec, &per);
    return l == kThreads ? "softmax_bwd_block" : l == 64 ? "softmax_bwd_wave" : "softmax_bwd_group";
}

hipError_t launch_softmax_bwd(const void* probs, const void* dprobs, void* dscores,
                              const Problem& p, float scale, int dt, bool fast,
                              hipStream_t stream) {
    switch (dt) {
    case kF16: return launch_t<F16>(probs, dprobs, dscores, p, scale, fast, stream);
    case kBF16: return launch_t<BF16>(probs, dprobs, dscores, p, scale, fast, stream);
    case kF32: return launch_t<F32>(probs, dprobs, dscores, p, scale, fast, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace diagmm
