// Element-per-thread kernels for qk, pv and pvT, and a workgroup-per-row banded softmax.
//
// These run any shape and dtype pair the ABI accepts.  They read operands straight from
// global memory (no tiling), so they are the general fallback and the on-device
// cross-check for the tiled MFMA kernels, not the fast path.
#include "launch.hpp"

namespace diagmm {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = int64_t(1) << 20;  // grid-stride beyond this

int64_t blocks_for(int64_t total) {
    int64_t nb = (total + kThreads - 1) / kThreads;
    return nb < kMaxBlocks ? nb : kMaxBlocks;
}

// band[row, k] with row = (bb * n + i) * h + hh.
template <class In, class Out>
__global__ void __launch_bounds__(kThreads)
qk_simple_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ kx,
                 typename Out::T* __restrict__ band, Problem p, typename Out::T pad,
                 int64_t total) {
    const int64_t step = int64_t(gridDim.x) * kThreads;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total; idx += step) {
        const int64_t k = idx % p.K, row = idx / p.K;
        const int64_t hh = row % p.h, bi = row / p.h;
        const int64_t i = bi % p.n, bb = bi / p.n;
        const int64_t j = i + (k - p.w) * p.s;
        if (j < 0 || j >= p.n) {
            band[idx] = pad;
            continue;
        }
        const typename In::T* qr = q + row * p.d;
        const typename In::T* kr = kx + ((bb * p.n + j) * p.h + hh) * p.d;
        float acc = 0.f;
        for (int64_t c = 0; c < p.d; ++c) acc = fmaf(In::to_f32(qr[c]), In::to_f32(kr[c]), acc);
        band[idx] = Out::from_f32(acc);
    }
}

// out[row, c] = sum over in-range k of band[row, k] * v[key row of slot k, c].
template <class In, class Out>
__global__ void __launch_bounds__(kThreads)
pv_simple_kernel(const typename In::T* __restrict__ band, const typename In::T* __restrict__ v,
                 typename Out::T* __restrict__ out, Problem p, int64_t total) {
    const int64_t step = int64_t(gridDim.x) * kThreads;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total; idx += step) {
        const int64_t c = idx % p.d, row = idx / p.d;
        const int64_t hh = row % p.h, bi = row / p.h;
        const int64_t i = bi % p.n, bb = bi / p.n;
        float acc = 0.f;
        for (int64_t k = 0; k < p.K; ++k) {
            const int64_t j = i + (k - p.w) * p.s;
            if (j < 0 || j >= p.n) continue;
            acc = fmaf(In::to_f32(band[row * p.K + k]),
                       In::to_f32(v[((bb * p.n + j) * p.h + hh) * p.d + c]), acc);
        }
        out[idx] = Out::from_f32(acc);
    }
}

// out[row_j, c] = sum over k of band[row_i, k] * x[row_i, c] with i = j - (k - w) * s.
template <class In, class Out>
__global__ void __launch_bounds__(kThreads)
pvT_simple_kernel(const typename In::T* __restrict__ band, const typename In::T* __restrict__ x,
                  typename Out::T* __restrict__ out, Problem p, int64_t total) {
    const int64_t step = int64_t(gridDim.x) * kThreads;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total; idx += step) {
        const int64_t c = idx % p.d, row = idx / p.d;
        const int64_t hh = row % p.h, bj = row / p.h;
        const int64_t j = bj % p.n, bb = bj / p.n;
        float acc = 0.f;
        for (int64_t k = 0; k < p.K; ++k) {
            const int64_t i = j - (k - p.w) * p.s;
            if (i < 0 || i >= p.n) continue;
            const int64_t ri = (bb * p.n + i) * p.h + hh;
            acc = fmaf(In::to_f32(band[ri * p.K + k]), In::to_f32(x[ri * p.d + c]), acc);
        }
        out[idx] = Out::from_f32(acc);
    }
}

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One workgroup per band row (grid-stride over rows).  Only the in-range slot interval
// [k_lo, k_hi) is read; the rest of the row is written as +0.
template <class In, class Out>
__global__ void __launch_bounds__(kThreads)
softmax_rows_kernel(const typename In::T* scores, typename Out::T* probs, Problem p,
                    float scale, int64_t nrows) {
    __shared__ float red[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t row = blockIdx.x; row < nrows; row += gridDim.x) {
        const int64_t i = (row / p.h) % p.n;
        // in range: 0 <= i + (k - w) s < n  <=>  w - floor(i/s) <= k <= w + floor((n-1-i)/s)
        const int64_t lo_off = i / p.s, hi_off = (p.n - 1 - i) / p.s;
        const int64_t k_lo = p.w - (lo_off < p.w ? lo_off : p.w);
        const int64_t k_hi = p.w + (hi_off < p.wu ? hi_off : p.wu) + 1;
        const typename In::T* src = scores + row * p.K;
        typename Out::T* dst = probs + row * p.K;

        float m = -INFINITY;
        for (int64_t k = k_lo + threadIdx.x; k < k_hi; k += kThreads)
            m = fmaxf(m, scale * In::to_f32(src[k]));
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = red[0];
        for (int t = 1; t < kThreads / 64; ++t) m = fmaxf(m, red[t]);
        __syncthreads();

        float sum = 0.f;
        for (int64_t k = k_lo + threadIdx.x; k < k_hi; k += kThreads)
            sum += __expf(scale * In::to_f32(src[k]) - m);
        sum = wave_sum(sum);
        if (lane == 0) red[wave] = sum;
        __syncthreads();
        sum = 0.f;
        for (int t = 0; t < kThreads / 64; ++t) sum += red[t];
        __syncthreads();

        const float inv = 1.f / sum;
        for (int64_t k = threadIdx.x; k < p.K; k += kThreads) {
            float pk = 0.f;
            if (k >= k_lo && k < k_hi) pk = __expf(scale * In::to_f32(src[k]) - m) * inv;
            dst[k] = Out::from_f32(pk);
        }
        // In place (dst == src) is safe: each element is read and rewritten by the same
        // thread, after both reductions have finished reading the row.
    }
}

// Calls f(In{}, Out{}) for a supported (in, out) dtype pair.
template <class F>
hipError_t dispatch(int in_dt, int out_dt, F&& f) {
    if (in_dt == kF32 && out_dt == kF32) return f(F32{}, F32{});
    if (in_dt == kF16 && out_dt == kF16) return f(F16{}, F16{});
    if (in_dt == kF16 && out_dt == kF32) return f(F16{}, F32{});
    if (in_dt == kBF16 && out_dt == kBF16) return f(BF16{}, BF16{});
    if (in_dt == kBF16 && out_dt == kF32) return f(BF16{}, F32{});
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qk_simple(const void* q, const void* k, void* band, const Problem& p,
                            int in_dt, int out_dt, uint32_t pad, hipStream_t stream) {
    const int64_t total = p.rows() * p.h * p.K;
    return dispatch(in_dt, out_dt, [&](auto in, auto out) {
        using In = decltype(in);
        using Out = decltype(out);
        typename Out::T padv;
        if constexpr (Out::code == kF32) padv = __builtin_bit_cast(float, pad);
        else padv = static_cast<uint16_t>(pad);
        launch_kernel((qk_simple_kernel<In, Out>), dim3(blocks_for(total)), dim3(kThreads),
                           0, stream, static_cast<const typename In::T*>(q),
                           static_cast<const typename In::T*>(k),
                           static_cast<typename Out::T*>(band), p, padv, total);
        return hipGetLastError();
    });
}

hipError_t launch_pv_simple(const void* band, const void* v, void* out, const Problem& p,
                            int in_dt, int out_dt, hipStream_t stream) {
    const int64_t total = p.rows() * p.h * p.d;
    return dispatch(in_dt, out_dt, [&](auto in, auto o) {
        using In = decltype(in);
        using Out = decltype(o);
        launch_kernel((pv_simple_kernel<In, Out>), dim3(blocks_for(total)), dim3(kThreads),
                           0, stream, static_cast<const typename In::T*>(band),
                           static_cast<const typename In::T*>(v),
                           static_cast<typename Out::T*>(out), p, total);
        return hipGetLastError();
    });
}

hipError_t launch_pvT_simple(const void* band, const void* x, void* out, const Problem& p,
                             int in_dt, int out_dt, hipStream_t stream) {
    const int64_t total = p.rows() * p.h * p.d;
    return dispatch(in_dt, out_dt, [&](auto in, auto o) {
        using In = decltype(in);
        using Out = decltype(o);
        launch_kernel((pvT_simple_kernel<In, Out>), dim3(blocks_for(total)),
                           dim3(kThreads), 0, stream, static_cast<const typename In::T*>(band),
                           static_cast<const typename In::T*>(x),
                           static_cast<typename Out::T*>(out), p, total);
        return hipGetLastError();
    });
}

hipError_t launch_softmax_rows(const void* scores, void* probs, const Problem& p, float scale,
                               int in_dt, int out_dt, hipStream_t stream) {
    const int64_t nrows = p.rows() * p.h;
    const int64_t grid = nrows < kMaxBlocks ? nrows : kMaxBlocks;
    return dispatch(in_dt, out_dt, [&](auto in, auto o) {
        using In = decltype(in);
        using Out = decltype(o);
        launch_kernel((softmax_rows_kernel<In, Out>), dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const typename In::T*>(scores),
                           static_cast<typename Out::T*>(probs), p, scale, nrows);
        return hipGetLastError();
    });
}

}  // namespace diagmm
