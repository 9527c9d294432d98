// diagmm_qk on MFMA with persistent, sliding workgroups.
//
// Tiles.  A tile is M = 64 consecutive rows t0..t0+63 of one residue class of one
// (batch, head) and a block of KB consecutive slots k0..k0+KB-1 (KB <= 513, fixed per
// call by the LDS budget).  Its slots reach the W = M + KB - 1 consecutive keys
// u0 = t0 + k0 - w .. u0 + W - 1 of the class.  Tiles are numbered with the row block
// fastest, so consecutive tiles of one strip slide down the class by 64 rows and share
// all but 64 of their keys.
//
// Workgroups.  One 512-thread workgroup per compute unit walks a contiguous range of
// tile ids.  It keeps the key window of the current tile in an LDS ring (rows swizzled by
// 16-byte chunk), so a tile that continues a strip only brings in 64 new key rows and
// its 64 query rows; both are fetched into registers at the start of the previous tile
// and written to LDS after its MFMAs, so their latency hides behind compute.
//
// Compute.  The window is cut into 16-key column blocks jb, dealt round-robin to the 8
// waves; for each, the 16-row blocks rb the band crosses are computed as the transposed
// product on v_mfma_f32_16x16x32_{f16,bf16}:
//
//   acc(jb, rb)[j][i] = sum_c K[u0 + 16 jb + j][c] * Q[t0 + 16 rb + i][c]
//
// (A = 16 key rows read from the ring, B = 16 query rows held in registers).  Lane
// (i = lane % 16, g = lane / 16) holds keys 16 jb + 4 g + v, v = 0..3, of query row
// 16 rb + i: four consecutive band slots k = key - row + w of one row.  They are
// rounded (nearest even, two packed conversions) and written with one 8-byte LDS
// store; the staging row of tile row il begins il mod 4 elements past its base, which
// makes every such store 8-byte aligned whatever the row.  Slots whose key lies outside
// the sequence get the padding constant.
//
// Store.  The staged rows leave in aligned 16-byte pieces of the band in HBM.  Staging
// and HBM disagree on alignment by ((il mod 4) - (row offset mod 8)) elements, one
// value per row: each piece is assembled from three aligned 8-byte LDS reads with a
// funnel shift.  The at most two partial pieces of a row (shared with the neighbouring
// head's band row) are written element by element.
#include "launch.hpp"
#include "tiles.hpp"

namespace diagmm {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Four accumulators -> the staged representation (two packed dwords for 16-bit outputs,
// four for f32), rounding to nearest even.
template <class Out> struct Pack;
template <> struct Pack<F16> {
    using P = u32x2;
    __device__ __forceinline__ static P run(f32x4 a) {
        return __builtin_bit_cast(P, __builtin_convertvector(a, f16x4));
    }
    __device__ __forceinline__ static P splat(uint32_t pad) {
        const uint32_t x = (pad & 0xffffu) | (pad << 16);
        return P{x, x};
    }
};
template <> struct Pack<BF16> {
    using P = u32x2;
    __device__ __forceinline__ static P run(f32x4 a) {
        return __builtin_bit_cast(P, __builtin_convertvector(a, bf16x4));
    }
    __device__ __forceinline__ static P splat(uint32_t pad) {
        const uint32_t x = (pad & 0xffffu) | (pad << 16);
        return P{x, x};
    }
};
template <> struct Pack<F32> {
    using P = u32x4;
    __device__ __forceinline__ static P run(f32x4 a) { return __builtin_bit_cast(P, a); }
    __device__ __forceinline__ static P splat(uint32_t pad) { return P{pad, pad, pad, pad}; }
};

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kQkRows;                // 64
constexpr int kMaxSlots = 513;
constexpr int kMaxWindow = kRows + kMaxSlots - 1;
constexpr int kMargin = 16;                   // staging row lead-in (elements)
constexpr int kBlocksPerWave = (kMaxWindow + 16 * kWaves - 1) / (16 * kWaves);  // 5

struct QkArgs {
    int64_t n, h, K, w, s;
    TileGrid g;
    int32_t rs;        // staging row stride (elements, multiple of 4)
    int32_t ring;      // key rows in the LDS ring (= 2 * kRows + KB - 1)
    int32_t ring_off;  // LDS byte offset of the ring
    int32_t q_off;     // LDS byte offset of the query tile
    uint32_t nwg;      // persistent workgroups
    uint32_t pad;      // padding constant, already rounded to the output type
    TileDecode dc;     // tiles over workgroups, tile -> coordinates
};

// Byte offset of (row, 16-byte chunk) in a swizzled block of D-element rows.  The chunk
// index is XORed with bits 1..3 of the row, so 16 consecutive rows read at one logical
// chunk land on distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
    constexpr int kChunks = D / 8;
    constexpr int kMask = (kChunks < 8 ? kChunks : 8) - 1;
    return row * (D * 2) + ((chunk ^ ((row >> 1) & kMask)) << 4);
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

template <class In, class Out, int D>
__global__ void __launch_bounds__(kThreads)
qk_mfma_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ kx,
               typename Out::T* __restrict__ band, QkArgs a) {
    using OT = typename Out::T;
    using V = typename Mfma<In>::V;
    using P = typename Pack<Out>::P;
    constexpr int kVec = 16 / sizeof(OT);                 // elements per 16-byte piece
    constexpr int kRB = kRows / 16;
    constexpr int kDC = D / 32;
    constexpr int kChunks = D / 8;                        // 16-byte chunks per row
    constexpr int kRowChunks = kRows * kChunks;           // chunks of a 64-row block
    constexpr int kPer64 = (kRowChunks + kThreads - 1) / kThreads;
    constexpr int kPerWin = (kMaxWindow * kChunks + kThreads - 1) / kThreads;

    extern __shared__ __align__(16) unsigned char lds[];
    OT* stage = reinterpret_cast<OT*>(lds);
    unsigned char* ring = lds + a.ring_off;
    unsigned char* qlds = lds + a.q_off;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;                       // [b][n][h] rows per class row
    const int rs = a.rs, ringc = a.ring;
    const P padv = Pack<Out>::splat(a.pad);

    uint32_t tile, tend;
    unit_range(a.dc, xcd_rank(blockIdx.x, a.nwg), &tile, &tend);

    // Registers carrying the next tile's new key rows and query rows.
    u32x4 kn[kPer64], qn[kPer64];
    bool prefetched = false;
    int s0 = 0;                     // ring slot of the current window's first key

    // Staging write base of this lane (row col of block 0, keys 4 grp .. 4 grp + 3).
    const int ebase = col * rs + kMargin + (col & 3) - col + 4 * grp;

    for (; tile < tend; ++tile) {
        const TileId t = decode_fast(a.dc, tile);
        const int n_r = class_len_fast(a.dc, t.r);
        const int t0 = t.tb * kRows;
        if (t0 >= n_r) {           // empty tail block of a shorter residue class
            prefetched = false;
            continue;
        }
        const int rows_here = n_r - t0 < kRows ? n_r - t0 : kRows;
        const int64_t k0 = static_cast<int64_t>(t.kb) * a.g.kb;
        const int kbeff = static_cast<int>(K - k0 < a.g.kb ? K - k0 : a.g.kb);
        const int u0 = static_cast<int>(t0 + k0 - a.w);
        const int W = kRows + kbeff - 1;
        const int nj = (W + 15) / 16;
        const int span = (kbeff + 14) / 16;
        const int64_t row0 = (static_cast<int64_t>(t.bb) * n + t.r) * h + t.hh;

        if (!prefetched) {
            // First tile of a strip: the whole key window and the query tile.
            s0 = 0;
            u32x4 buf[kPerWin];
#pragma unroll
            for (int x = 0; x < kPerWin; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (rr < W) {
                    int u = u0 + rr;
                    u = u < 0 ? 0 : (u < n_r ? u : n_r - 1);
                    buf[x] = ld_global16(kx + (row0 + u * row_step) * D + ch * 8);
                }
            }
#pragma unroll
            for (int x = 0; x < kPer64; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) {
                    int tq = t0 + rr;
                    tq = tq < n_r ? tq : n_r - 1;
                    qn[x] = ld_global16(q + (row0 + tq * row_step) * D + ch * 8);
                }
            }
#pragma unroll
            for (int x = 0; x < kPerWin; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (rr < W) *reinterpret_cast<u32x4*>(ring + swz<D>(rr, ch)) = buf[x];
            }
#pragma unroll
            for (int x = 0; x < kPer64; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) *reinterpret_cast<u32x4*>(qlds + swz<D>(rr, ch)) = qn[x];
            }
            __syncthreads();
        }

        // Does the next tile continue this strip?  Then fetch its new rows now.
        bool next = false;
        if (tile + 1 < tend) {
            const TileId tn = decode_fast(a.dc, tile + 1);
            next = tn.tb == t.tb + 1 && tn.kb == t.kb && tn.r == t.r && tn.hh == t.hh &&
                   tn.bb == t.bb && t0 + kRows < n_r;
        }
        if (next) {
#pragma unroll
            for (int x = 0; x < kPer64; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) {
                    int u = u0 + W + rr;
                    u = u < 0 ? 0 : (u < n_r ? u : n_r - 1);
                    kn[x] = ld_global16(kx + (row0 + u * row_step) * D + ch * 8);
                    int tq = t0 + kRows + rr;
                    tq = tq < n_r ? tq : n_r - 1;
                    qn[x] = ld_global16(q + (row0 + tq * row_step) * D + ch * 8);
                }
            }
        }

        // B operands: the tile's 64 query rows.
        V qf[kRB][kDC];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc)
                qf[rb][dc] = *reinterpret_cast<const V*>(qlds + swz<D>(16 * rb + col, 4 * dc + grp));

        const bool key_edge = u0 < 0 || u0 + W > n_r;     // window touches a sequence end
#pragma unroll
        for (int x = 0; x < kBlocksPerWave; ++x) {
            const int jb = wave + kWaves * x;
            if (jb >= nj) break;
            int slot = s0 + 16 * jb + col;
            slot = slot < ringc ? slot : slot - ringc;
            V kf[kDC];
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc)
                kf[dc] = *reinterpret_cast<const V*>(ring + swz<D>(slot, 4 * dc + grp));
            // keys of this lane's four accumulators: u0 + 16 jb + 4 grp + v
            const int ukey = u0 + 16 * jb + 4 * grp;
            bool kok[4] = {true, true, true, true};
            if (key_edge) {
#pragma unroll
                for (int v = 0; v < 4; ++v) kok[v] = ukey + v >= 0 && ukey + v < n_r;
            }
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const int dj = jb - rb;                     // wave-uniform
                if (dj < 0 || dj > span) continue;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dc = 0; dc < kDC; ++dc) acc = Mfma<In>::run(kf[dc], qf[rb][dc], acc);
                P val = Pack<Out>::run(acc);
                if (key_edge) {
                    const P pv = padv;
                    if constexpr (sizeof(OT) == 4) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) val[v] = kok[v] ? val[v] : pv[v];
                    } else {
                        const uint32_t m0 = (kok[0] ? 0xffffu : 0u) | (kok[1] ? 0xffff0000u : 0u);
                        const uint32_t m1 = (kok[2] ? 0xffffu : 0u) | (kok[3] ? 0xffff0000u : 0u);
                        val[0] = (val[0] & m0) | (pv[0] & ~m0);
                        val[1] = (val[1] & m1) | (pv[1] & ~m1);
                    }
                }
                *reinterpret_cast<P*>(stage + ebase + 16 * rb * rs + 16 * dj) = val;
            }
        }

        // New key rows of the next tile go to ring slots outside the current window.
        if (next) {
#pragma unroll
            for (int x = 0; x < kPer64; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) {
                    int slot = s0 + W + rr;
                    slot = slot < ringc ? slot : slot - ringc;
                    *reinterpret_cast<u32x4*>(ring + swz<D>(slot, ch)) = kn[x];
                }
            }
        }
        __syncthreads();
        if (next) {
#pragma unroll
            for (int x = 0; x < kPer64; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) *reinterpret_cast<u32x4*>(qlds + swz<D>(rr, ch)) = qn[x];
            }
        }

        // Stream the staged rows out in aligned 16-byte pieces.
        const int64_t g0 = (row0 + static_cast<int64_t>(t0) * row_step) * K + k0;
        const int64_t gstep = row_step * K;
        const int g0mod = static_cast<int>(g0 & (kVec - 1));
        const int gstepmod = static_cast<int>(gstep & (kVec - 1));
        const int ncmax = (kVec - 1 + kbeff + kVec - 1) / kVec;
        int il = tid / ncmax;
        int c = tid - il * ncmax;
        const int step_rows = kThreads / ncmax, step_c = kThreads - step_rows * ncmax;
        while (il < rows_here) {
            const int sh = (g0mod + il * gstepmod) & (kVec - 1);
            const int nc = (sh + kbeff + kVec - 1) / kVec;
            if (c < nc) {
                // staged element of the piece's first slot, and its misalignment
                const int e = il * rs + kMargin + (il & 3) + kVec * c - sh;
                const int m = e & 3;
                const unsigned char* lp = reinterpret_cast<const unsigned char*>(stage + (e - m));
                // o0..o3: the piece's four dwords, named scalars throughout (no arrays)
                uint32_t o0, o1, o2, o3;
                if constexpr (sizeof(OT) == 2) {
                    const u32x2 wa = *reinterpret_cast<const u32x2*>(lp);
                    const u32x2 wb = *reinterpret_cast<const u32x2*>(lp + 8);
                    const u32x2 wc = *reinterpret_cast<const u32x2*>(lp + 16);
                    const bool hi = m & 2;
                    const uint32_t l0 = hi ? wa[1] : wa[0];
                    const uint32_t l1 = hi ? wb[0] : wa[1];
                    const uint32_t l2 = hi ? wb[1] : wb[0];
                    const uint32_t l3 = hi ? wc[0] : wb[1];
                    const uint32_t l4 = hi ? wc[1] : wc[0];
                    if (m & 1) {
                        o0 = __builtin_amdgcn_alignbit(l1, l0, 16);
                        o1 = __builtin_amdgcn_alignbit(l2, l1, 16);
                        o2 = __builtin_amdgcn_alignbit(l3, l2, 16);
                        o3 = __builtin_amdgcn_alignbit(l4, l3, 16);
                    } else {
                        o0 = l0;
                        o1 = l1;
                        o2 = l2;
                        o3 = l3;
                    }
                } else {
                    const u32x4 wa = *reinterpret_cast<const u32x4*>(lp);
                    const u32x4 wb = *reinterpret_cast<const u32x4*>(lp + 16);
                    const bool odd = m & 1, hi = m & 2;
                    const uint32_t t0_ = odd ? wa[1] : wa[0], u0_ = odd ? wa[3] : wa[2];
                    const uint32_t t1_ = odd ? wa[2] : wa[1], u1_ = odd ? wb[0] : wa[3];
                    const uint32_t t2_ = odd ? wa[3] : wa[2], u2_ = odd ? wb[1] : wb[0];
                    const uint32_t t3_ = odd ? wb[0] : wa[3], u3_ = odd ? wb[2] : wb[1];
                    o0 = hi ? u0_ : t0_;
                    o1 = hi ? u1_ : t1_;
                    o2 = hi ? u2_ : t2_;
                    o3 = hi ? u3_ : t3_;
                }
                OT* gp = band + (g0 + il * gstep - sh) + c * kVec;     // 16-byte aligned
                const int lo = c * kVec;
                if (lo >= sh && lo + kVec <= sh + kbeff) {
                    *reinterpret_cast<u32x4*>(gp) = u32x4{o0, o1, o2, o3};
                } else {
                    // partial piece: only this row's elements [a, b) of the piece
                    const int pa = sh - lo > 0 ? sh - lo : 0;
                    const int pb = sh + kbeff - lo < kVec ? sh + kbeff - lo : kVec;
                    store_part<OT>(gp, o0, o1, o2, o3, pa, pb);
                }
            }
        il += step_rows;
            c += step_c;
            if (c >= ncmax) {
                c -= ncmax;
                ++il;
            }
        }
        __syncthreads();
        prefetched = next;
        if (next) {
            s0 += kRows;
            s0 = s0 < ringc ? s0 : s0 - ringc;
        }
    }
}

struct Layout {
    int64_t kb = 0, rs = 0, ring = 0, ring_off = 0, q_off = 0, bytes = 0;
};

// LDS layout for a slot block of kb slots: staging, then the key ring, then the queries.
Layout layout_for(int64_t kb, int64_t d, int64_t esize) {
    Layout l;
    l.kb = kb;
    l.rs = ceil_div(kb + 3 * kMargin + 1, 4) * 4;
    l.ring = 2 * kRows + kb - 1;
    l.ring_off = ceil_div(kRows * l.rs * esize, 16) * 16;
    l.q_off = l.ring_off + l.ring * d * 2;
    l.bytes = l.q_off + kRows * d * 2;
    return l;
}

template <class In, class Out, int D>
hipError_t launch_typed(const void* q, const void* k, void* band, const Problem& p,
                        const QkTilePlan& tp, uint32_t pad, hipStream_t stream) {
    const Layout l = layout_for(tp.grid.kb, D, sizeof(typename Out::T));
    QkArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.rs),
             static_cast<int32_t>(l.ring), static_cast<int32_t>(l.ring_off),
             static_cast<int32_t>(l.q_off), static_cast<uint32_t>(tp.workgroups), pad,
             make_decode(tp.grid, p.h, p.n, p.s, tp.grid.tiles, tp.workgroups)};
    auto kern = qk_mfma_kernel<In, Out, D>;
    // Once per instantiation (thread-safe static initialisation): allow all of the
    // compute unit's LDS as dynamic LDS.
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(kQkLdsBytes));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(tp.workgroups)), dim3(kThreads),
                       static_cast<size_t>(l.bytes), stream,
                       static_cast<const typename In::T*>(q),
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
    // The widest slot block (at most 513) whose staging + ring + query tile fit in LDS.
    int64_t max_slots = kMaxSlots;
    while (max_slots > 16 && layout_for(max_slots, p.d, esize).bytes > kQkLdsBytes) --max_slots;
    tp.grid = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, max_slots);
    const Layout l = layout_for(tp.grid.kb, p.d, esize);
    tp.rs = l.rs;
    tp.lds_bytes = l.bytes;
    const int64_t cus = device_cus();
    tp.workgroups = tp.grid.tiles < cus ? tp.grid.tiles : cus;
    tp.ok = tp.grid.tiles <= kMaxTiles && ceil_div(p.n, p.s) < (int64_t(1) << 30) &&
            p.K < (int64_t(1) << 30) && l.bytes <= kQkLdsBytes && tp.workgroups >= 1;
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
