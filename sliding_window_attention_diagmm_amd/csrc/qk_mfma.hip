// diagmm_qk on MFMA: Q.K^T on the dense 16x16 sub-tiles that cover a band tile, the
// band assembled in LDS, and stored to HBM with aligned 16-byte stores.
//
// One workgroup (4 waves) owns a tile: M = 64 consecutive rows t0..t0+63 of one residue
// class of one (batch, head), and a block of KB consecutive slots k0..k0+KB-1.  The keys
// those slots reach form a window of M + KB - 1 consecutive keys of the class; the
// kernel walks it in 16-key column blocks jb and, for each, the 16-row blocks rb that
// the band crosses:
//
//   acc(rb, jb)[i][j] = sum_c Q[t0 + 16 rb + i][c] * K[u0 + 16 jb + j][c]
//
// on v_mfma_f32_16x16x32_{f16,bf16} (A = 16 Q rows, B = 16 K rows, depth 32 per
// instruction, d / 32 instructions).  Both operands come straight from global memory
// in 16-byte pieces per lane (a key row is 128 bytes at d = 64; the window's rows are
// re-read by neighbouring tiles from L2).  Each accumulator element (row t, key u)
// belongs to slot k = u - t + w; those inside the tile's slot block are converted
// (round to nearest even) and written into an LDS staging copy of the tile's band rows.
// Slots whose key lies outside the sequence get the padding constant instead.
//
// LDS staging row il starts at il * RS + shift(il), where shift(il) is the output row's
// global offset modulo 16 bytes, so LDS and HBM agree on 16-byte alignment.  After a
// barrier the workgroup streams the staged rows out: every full aligned 16-byte piece
// of a band row is one global_store_dwordx4; the at most two partial pieces at a row's
// ends (shared with the neighbouring head's band row) are stored element by element.
#include "launch.hpp"
#include "tiles.hpp"

namespace diagmm {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class In> struct Mfma;
template <> struct Mfma<F16> {
    using V = f16x8;
    __device__ __forceinline__ static f32x4 run(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<BF16> {
    using V = bf16x8;
    __device__ __forceinline__ static f32x4 run(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <class V>
__device__ __forceinline__ V load16(const void* p) {
    return __builtin_bit_cast(V, *reinterpret_cast<const uint4*>(p));
}

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct QkArgs {
    int64_t n, h, K, w;
    TileGrid g;
    int64_t rs;       // LDS staging row stride (elements)
    uint32_t pad;     // padding constant, already rounded to the output type
};

template <class In, class Out, int D, int M>
__global__ void __launch_bounds__(kThreads, 2)
qk_mfma_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ kx,
               typename Out::T* __restrict__ band, QkArgs a) {
    using OT = typename Out::T;
    using V = typename Mfma<In>::V;
    constexpr int kVec = 16 / sizeof(OT);   // elements per 16-byte piece
    constexpr int kRB = M / 16;             // row blocks per tile
    constexpr int kDC = D / 32;             // depth chunks
    extern __shared__ __align__(16) unsigned char lds_raw[];
    OT* stage = reinterpret_cast<OT*>(lds_raw);

    TileId t;
    if (!tile_of(a.g, a.h, blockIdx.x, &t)) return;
    const int64_t n = a.n, h = a.h, K = a.K, s = a.g.s;
    const int64_t n_r = class_len(n, s, t.r);
    const int64_t t0 = t.tb * M;
    if (t0 >= n_r) return;
    const int rows_here = static_cast<int>(n_r - t0 < M ? n_r - t0 : M);
    const int64_t k0 = t.kb * a.g.kb;
    const int kbeff = static_cast<int>(K - k0 < a.g.kb ? K - k0 : a.g.kb);
    const int64_t u0 = t0 + k0 - a.w;             // class-local key of window column 0
    const int nj = (M + kbeff - 1 + 15) / 16;     // 16-key column blocks in the window
    const int span = (kbeff + 14) / 16;           // jb - rb ranges over [0, span]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    // element offset of (class row t, head) in a [b][n][h][*] tensor, per unit of last dim
    const int64_t row0 = (t.bb * n + t.r) * h + t.hh;   // row index of class row 0
    const int64_t row_step = s * h;                      // rows between class rows

    // A operands: the tile's Q rows (clamped inside the class; rows past the end are
    // computed but never stored).
    V qf[kRB][kDC];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        int64_t tq = t0 + 16 * rb + col;
        if (tq > n_r - 1) tq = n_r - 1;
        const typename In::T* qrow = q + (row0 + tq * row_step) * D + grp * 8;
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) qf[rb][dc] = load16<V>(qrow + dc * 32);
    }

    // Output geometry: global element of (tile row il, tile slot 0) is g0 + il * gstep.
    const int64_t g0 = (row0 + t0 * row_step) * K + k0;
    const int64_t gstep = row_step * K;
    const int g0mod = static_cast<int>(g0 & (kVec - 1));
    const int gstepmod = static_cast<int>(gstep & (kVec - 1));
    const OT pad = [&] {
        if constexpr (sizeof(OT) == 4) return __builtin_bit_cast(OT, a.pad);
        else return static_cast<OT>(a.pad);
    }();

    auto load_keys = [&](int jb, V (&kf)[kDC]) {
        int64_t u = u0 + 16 * jb + col;
        u = u < 0 ? 0 : (u > n_r - 1 ? n_r - 1 : u);
        const typename In::T* krow = kx + (row0 + u * row_step) * D + grp * 8;
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) kf[dc] = load16<V>(krow + dc * 32);
    };

    V kf[kDC], kn[kDC];
    int jb = wave;
    if (jb < nj) load_keys(jb, kf);
    for (; jb < nj; jb += kWaves) {
        if (jb + kWaves < nj) load_keys(jb + kWaves, kn);
        const int64_t ucol = u0 + 16 * jb + col;          // this lane's output key
        const bool key_ok = ucol >= 0 && ucol < n_r;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            if (jb - rb < 0 || jb - rb > span) continue;    // wave-uniform
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc) acc = Mfma<In>::run(qf[rb][dc], kf[dc], acc);
            // acc[v] = D[row 16 rb + 4 grp + v][key column col]
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int il = 16 * rb + 4 * grp + v;
                const int kl = 16 * jb + col - il;          // slot within the tile
                if (il < rows_here && kl >= 0 && kl < kbeff) {
                    const int sh = (g0mod + il * gstepmod) & (kVec - 1);
                    stage[il * a.rs + sh + kl] = key_ok ? Out::from_f32(acc[v]) : pad;
                }
            }
        }
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) kf[dc] = kn[dc];
    }
    __syncthreads();

    // Stream the staged rows out in aligned 16-byte pieces.
    const int ncmax = (kVec - 1 + kbeff + kVec - 1) / kVec;
    const int total = rows_here * ncmax;
    for (int idx = threadIdx.x; idx < total; idx += kThreads) {
        const int il = idx / ncmax, c = idx - il * ncmax;
        const int sh = (g0mod + il * gstepmod) & (kVec - 1);
        const int nc = (sh + kbeff + kVec - 1) / kVec;
        if (c >= nc) continue;
        const int64_t gstart = g0 + il * gstep;            // first element of the row
        OT* gp = band + (gstart - sh) + c * kVec;           // 16-byte aligned
        const OT* lp = stage + il * a.rs + c * kVec;        // 16-byte aligned
        const int lo = c * kVec, hi = lo + kVec;            // staged positions covered
        if (lo >= sh && hi <= sh + kbeff) {
            *reinterpret_cast<uint4*>(gp) = *reinterpret_cast<const uint4*>(lp);
        } else {
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                if (lo + e >= sh && lo + e < sh + kbeff) gp[e] = lp[e];
        }
    }
}

template <class In, class Out, int D>
hipError_t launch_typed(const void* q, const void* k, void* band, const Problem& p,
                        const QkTilePlan& tp, uint32_t pad, hipStream_t stream) {
    QkArgs a{p.n, p.h, p.K, p.w, tp.grid, tp.rs, pad};
    const size_t lds = static_cast<size_t>(tp.lds_bytes);
    auto kern = qk_mfma_kernel<In, Out, D, kQkRows>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(tp.grid.per_xcd * kXcds)), dim3(kThreads),
                       lds, stream, static_cast<const typename In::T*>(q),
                       static_cast<const typename In::T*>(k),
                       static_cast<typename Out::T*>(band), a);
    return hipGetLastError();
}

template <class In, class Out>
hipError_t launch_d(const void* q, const void* k, void* band, const Problem& p,
                    const QkTilePlan& tp, uint32_t pad, hipStream_t stream) {
    switch (p.d) {
    case 32: return launch_typed<In, Out, 32>(q, k, band, p, tp, pad, stream);
    case 64: return launch_typed<In, Out, 64>(q, k, band, p, tp, pad, stream);
    case 128: return launch_typed<In, Out, 128>(q, k, band, p, tp, pad, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

QkTilePlan plan_qk_mfma(const Problem& p, int out_dt) {
    QkTilePlan tp;
    const int64_t esize = out_dt == kF32 ? 4 : 2;
    const int64_t vec = 16 / esize;
    // Staging budget ~66 KB per workgroup: two workgroups per CU fit in 160 KB of LDS.
    const int64_t max_slots = (kQkStageBytes / (kQkRows * esize)) - (vec - 1);
    tp.grid = make_grid(p.b, p.n, p.h, p.K, p.s, kQkRows, max_slots);
    tp.rs = ceil_div(tp.grid.kb + vec - 1, vec) * vec;
    tp.lds_bytes = kQkRows * tp.rs * esize;
    return tp;
}

hipError_t launch_qk_mfma(const void* q, const void* k, void* band, const Problem& p,
                          const QkTilePlan& tp, int in_dt, int out_dt, uint32_t pad,
                          hipStream_t stream) {
    if (in_dt == kF16 && out_dt == kF16) return launch_d<F16, F16>(q, k, band, p, tp, pad, stream);
    if (in_dt == kF16 && out_dt == kF32) return launch_d<F16, F32>(q, k, band, p, tp, pad, stream);
    if (in_dt == kBF16 && out_dt == kBF16) return launch_d<BF16, BF16>(q, k, band, p, tp, pad, stream);
    if (in_dt == kBF16 && out_dt == kF32) return launch_d<BF16, F32>(q, k, band, p, tp, pad, stream);
    return hipErrorInvalidValue;
}

}  // namespace diagmm
