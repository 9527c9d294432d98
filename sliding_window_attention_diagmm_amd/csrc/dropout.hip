// Dropout on a probability band (csarofeen/pytorch issue 2096, first fusion repro: a
// uniform random tensor of the band's shape, a comparison with the drop probability, and
// the kept probabilities scaled by 1 / (1 - p)):
//
//   out_k = P_k / (1 - p)   if slot k is in range and rand_k > p,   else +0.
//
// The random numbers are an input (float32, the band's shape), so the keep decision is
// one float32 comparison that any implementation of the definition takes the same way.
// Run over dP with the same random numbers it is also the backward of the same dropout.
//
// The band is one flat array of b n h K elements; the kernel streams it in aligned
// 16-byte pieces of P and out (8 elements of a 16-bit type, 4 of float32) with the
// matching 32 or 16 bytes of rand, every load of a thread issued before any is used.  A
// piece may straddle two band rows (K is rarely a multiple of 8): each thread finds the
// row of its piece's first element and the in-range slot intervals of that row and the
// next one by multiply-based division, so nothing but the index arithmetic depends on
// the row structure.  Tensors that are not 16-byte aligned, or rows shorter than a piece,
// take the same kernel with one element per piece.
#include "launch.hpp"
#include "tiles.hpp"

namespace diagmm {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // pieces per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row (b * n + i) * h + hh -> position i -> in-range slots [k_lo, k_hi), with divisions
// by h, n and s done by multiplication (operands below 2^31).
struct RowDiv {
    Div32 h, n, s;
};
struct Range {
    int k_lo, k_hi;
};
__device__ __forceinline__ Range row_range(const Problem& p, const RowDiv& rd, uint32_t row) {
    const uint32_t bn = div32(rd.h, row);                                 // b * n + i
    const int64_t i = bn - div32(rd.n, bn) * rd.n.d;
    const int64_t lo_off = div32(rd.s, static_cast<uint32_t>(i));
    const int64_t hi_off = div32(rd.s, static_cast<uint32_t>(p.n - 1 - i));
    return Range{static_cast<int>(p.w - (lo_off < p.w ? lo_off : p.w)),
                 static_cast<int>(p.w + (hi_off < p.wu ? hi_off : p.wu) + 1)};
}

// Element e of a piece held as four named dwords (16-bit types: dword e / 2, half
// e % 2).  The piece is kept in a plain array rather than a vector register: indexing
// a loaded vector by element here has been compiled to read element 0 for every e.
template <class T>
__device__ __forceinline__ float elem(const uint32_t (&pw)[4], int e) {
    if constexpr (sizeof(typename T::T) == 4) return __builtin_bit_cast(float, pw[e]);
    else {
        const uint32_t d = pw[e >> 1];
        return T::to_f32(static_cast<uint16_t>((e & 1) ? (d >> 16) : (d & 0xffffu)));
    }
}

// V elements per piece: 16 / sizeof(element) on the aligned path, 1 otherwise.  A
// workgroup takes kThreads * kUnroll consecutive pieces, thread t the pieces
// t, t + kThreads, ...
template <class T, int V>
__global__ void __launch_bounds__(kThreads)
dropout_kernel(const typename T::T* probs, const float* rand, typename T::T* out, Problem p,
               float thr, float scale, int64_t total, Div32 dk, RowDiv rd) {
    using ST = typename T::T;
    constexpr bool kWide = V * sizeof(ST) == 16;
    constexpr int64_t kChunk = int64_t(kThreads) * kUnroll * V;
    const int K = static_cast<int>(p.K);
    const int64_t base = int64_t(blockIdx.x) * kChunk;
    const int64_t row_base = base / p.K;                  // one division per workgroup
    const int kb = static_cast<int>(base - row_base * p.K);

    uint32_t pw[kUnroll][4];   // P's piece as dwords
    float rv[kUnroll][V];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t e = base + int64_t(u * kThreads + threadIdx.x) * V;
#pragma unroll
        for (int c = 0; c < 4; ++c) pw[u][c] = 0u;
#pragma unroll
        for (int j = 0; j < V; ++j) rv[u][j] = 0.0f;
        if (e + V <= total) {
            if constexpr (kWide) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(probs + e);
                pw[u][0] = x.x;
                pw[u][1] = x.y;
                pw[u][2] = x.z;
                pw[u][3] = x.w;
#pragma unroll
                for (int q = 0; q < V / 4; ++q) {
                    const f32x4 r = *reinterpret_cast<const f32x4*>(rand + e + 4 * q);
                    rv[u][4 * q] = r.x;
                    rv[u][4 * q + 1] = r.y;
                    rv[u][4 * q + 2] = r.z;
                    rv[u][4 * q + 3] = r.w;
                }
            } else {
                if constexpr (sizeof(ST) == 4) pw[u][0] = __builtin_bit_cast(uint32_t, probs[e]);
                else pw[u][0] = static_cast<uint32_t>(probs[e]);
                rv[u][0] = rand[e];
            }
        } else if (e < total) {
            // the last, partial piece of the tensor: element by element
            const int m = static_cast<int>(total - e);
#pragma unroll
            for (int c = 0; c < 4; ++c) pw[u][c] = load_part_dword<ST>(probs + e, c, 0, m);
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (j < m) rv[u][j] = rand[e + j];
        }
    }

#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t e = base + int64_t(u * kThreads + threadIdx.x) * V;
        if (e >= total) continue;
        const int x = kb + (u * kThreads + static_cast<int>(threadIdx.x)) * V;
        const uint32_t q = div32(dk, static_cast<uint32_t>(x));
        const int k0 = x - static_cast<int>(q) * K;
        const uint32_t row = static_cast<uint32_t>(row_base) + q;
        const Range r0 = row_range(p, rd, row);
        // the next row, for pieces that run past the end of this one (K >= V)
        const Range r1 = V > 1 ? row_range(p, rd, row + 1) : r0;
        uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int k = k0 + j;
            const bool next = V > 1 && k >= K;
            const int kk = next ? k - K : k;
            const int lo = next ? r1.k_lo : r0.k_lo;
            const int hi = next ? r1.k_hi : r0.k_hi;
            const bool keep = kk >= lo && kk < hi && rv[u][j] > thr;
            const float val = keep ? elem<T>(pw[u], j) * scale : 0.0f;
            if constexpr (sizeof(ST) == 4) o[j] = __builtin_bit_cast(uint32_t, val);
            else o[j >> 1] |= static_cast<uint32_t>(T::from_f32(val)) << (16 * (j & 1));
        }
        if (e + V <= total) {
            if constexpr (kWide) *reinterpret_cast<u32x4*>(out + e) = u32x4{o[0], o[1], o[2], o[3]};
            else if constexpr (sizeof(ST) == 4) out[e] = __builtin_bit_cast(float, o[0]);
            else out[e] = static_cast<ST>(o[0]);
        } else {
            store_part<ST>(out + e, o[0], o[1], o[2], o[3], 0, static_cast<int>(total - e));
        }
    }
}

bool is16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <class T>
hipError_t launch_t(const void* probs, const float* rand, void* out, const Problem& p, float thr,
                    bool wide, hipStream_t stream) {
    using ST = typename T::T;
    constexpr int kV = 16 / sizeof(ST);
    const int64_t total = p.rows() * p.h * p.K;
    const RowDiv rd{make_div32(static_cast<uint32_t>(p.h)), make_div32(static_cast<uint32_t>(p.n)),
                    make_div32(static_cast<uint32_t>(p.s))};
    const Div32 dk = make_div32(static_cast<uint32_t>(p.K));
    // 1 / (1 - p) in double, rounded once to float
    const float scale = static_cast<float>(1.0 / (1.0 - static_cast<double>(thr)));
    const int v = wide ? kV : 1;
    const int64_t chunk = int64_t(kThreads) * kUnroll * v;
    const dim3 grid(static_cast<uint32_t>((total + chunk - 1) / chunk));
    if (wide)
        launch_kernel(dropout_kernel<T, kV>, grid, dim3(kThreads), 0, stream,
                      static_cast<const ST*>(probs), rand, static_cast<ST*>(out), p, thr, scale,
                      total, dk, rd);
    else
        launch_kernel(dropout_kernel<T, 1>, grid, dim3(kThreads), 0, stream,
                      static_cast<const ST*>(probs), rand, static_cast<ST*>(out), p, thr, scale,
                      total, dk, rd);
    return hipGetLastError();
}

}  // namespace

// 32-bit rows and slot offsets (a workgroup's chunk plus one row stays below 2^31), and a
// grid of at most 2^31 - 1 workgroups.
bool dropout_supported(const Problem& p) {
    const int64_t total = p.rows() * p.h * p.K;
    return p.rows() * p.h < (int64_t(1) << 31) - 1 && p.n < (int64_t(1) << 31) &&
           p.K < (int64_t(1) << 30) && total / (int64_t(kThreads) * kUnroll) < (int64_t(1) << 31);
}

bool dropout_wide(const Problem& p, int dt, const void* probs, const void* rand,
                  const void* out) {
    return p.K >= (dt == kF32 ? 4 : 8) && is16(probs) && is16(rand) && is16(out);
}

int64_t dropout_chunk(int dt, bool wide) {
    return int64_t(kThreads) * kUnroll * (wide ? (dt == kF32 ? 4 : 8) : 1);
}

int64_t dropout_workgroups(const Problem& p, int dt, bool wide) {
    const int64_t total = p.rows() * p.h * p.K;
    const int64_t chunk = dropout_chunk(dt, wide);
    return (total + chunk - 1) / chunk;
}

hipError_t launch_dropout(const void* probs, const float* rand, void* out, const Problem& p,
                          float drop_p, int dt, bool wide, hipStream_t stream) {
    switch (dt) {
    case kF16: return launch_t<F16>(probs, rand, out, p, drop_p, wide, stream);
    case kBF16: return launch_t<BF16>(probs, rand, out, p, drop_p, wide, stream);
    case kF32: return launch_t<F32>(probs, rand, out, p, drop_p, wide, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace diagmm
