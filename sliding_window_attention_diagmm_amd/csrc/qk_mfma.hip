// diagmm_qk on MFMA with persistent, sliding workgroups, storing straight from registers.
//
// Tiles.  A tile is M = 128 consecutive rows t0..t0+127 of one residue class of one
// (batch, head) and a chunk of KB consecutive slots k0..k0+KB-1.  Its slots reach the
// W = M + KB - 1 consecutive keys u0 = t0 + k0 - w .. u0 + W - 1 of the class ("window
// columns" x = 0 .. W-1; row il of the tile holds its slots at columns il .. il + KB - 1).
// Tiles are numbered with the row block fastest, so consecutive tiles of one strip slide
// down the class by 128 rows and share all but 128 of their keys.
//
// Workgroups.  One 512-thread workgroup per compute unit walks a contiguous range of
// tile ids.  It keeps the key window of the current tile in an LDS ring (rows swizzled by
// 16-byte chunk) and the query tile in one of two LDS buffers; a tile that continues a
// strip only brings in 128 new key rows and its 128 query rows, fetched into registers at
// the start of the previous tile and written to LDS at its end.
//
// Alignment.  Band rows are not 16-byte aligned in HBM (row r starts at r K elements),
// and misaligned stores run at half the bandwidth of aligned ones.  Column x of tile row
// il sits at element A(il) + x with A(il) = A(0) + il (row stride - 1), so its offset
// against 16-byte pieces depends on il mod 8 only.  Wave c therefore owns the 16 rows
// il = c, c + 8, ..., c + 120, which share one offset, and cuts the window into 16-column
// blocks starting at a column o (0 <= o < 8, one per wave and tile) where those rows'
// pieces start: every block then covers whole pieces of all 16 rows.
//
// Compute.  For each block jb (columns 16 jb + o ..) the wave computes the transposed
// product on v_mfma_f32_16x16x32_{f16,bf16}:
//
//   acc(jb)[j][k] = sum_c K[u0 + 16 jb + o + j][c] * Q[t0 + c + 8 k][c']
//
// (A = 16 key rows read from the ring, B = the wave's 16 query rows held in registers).
// Lane (k = lane % 16, g = lane / 16) holds columns 16 jb + o + 4 g .. +3 of row c + 8 k.
// Slots whose key lies outside the sequence take the padding constant; results are
// rounded to the output type (nearest even).
//
// Store.  For 16-bit outputs two blocks are combined with v_permlane16_swap so that each
// lane holds 8 consecutive columns, one aligned 16-byte piece; for f32 each block already
// gives 4 columns = 16 bytes per lane.  Whole pieces go straight to HBM.  The at most two
// pieces per row that also hold slots of the neighbouring band row in HBM are parked in
// LDS and written element by element after the sweep.
#include <type_traits>

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
constexpr int kRows = kQkRows;                // 128 = 8 waves x 16 rows
constexpr int kMaxSlots = 513;
constexpr int kMaxWindow = kRows + kMaxSlots - 1;
constexpr int kRingDup = 48;                  // ring rows mirrored past its end

struct QkArgs {
    int64_t n, h, K, w, s;
    TileGrid g;
    int32_t ring;      // key rows in the LDS ring (2 * kRows + KB - 1, rounded up to 16)
    int32_t q_off;     // LDS byte offset of the two query tiles
    int32_t p_off;     // LDS byte offset of the parked row-end pieces
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
    constexpr bool k16 = sizeof(OT) == 2;
    constexpr int kVec = 16 / sizeof(OT);                 // elements per 16-byte piece
    constexpr int kDC = D / 32;
    constexpr int kChunks = D / 8;                        // 16-byte chunks per row
    constexpr int kRowChunks = kRows * kChunks;           // chunks of a row block
    constexpr int kPerRows = (kRowChunks + kThreads - 1) / kThreads;
    constexpr int kPerWin = (kMaxWindow * kChunks + kThreads - 1) / kThreads;
    constexpr int kQBytes = kRows * D * 2;
    constexpr int kBPS = k16 ? 2 : 1;                     // blocks per step

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* ring = lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int il = wave + 8 * col;                        // this lane's tile row
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;                       // [b][n][h] rows per class row
    const int64_t gstep = row_step * K;                   // band elements per class row
    const int ringc = a.ring;
    const P padv = Pack<Out>::splat(a.pad);
    // Column offset of this lane's four (after pairing: eight) columns in a step.
    const int off_g = k16 ? (grp == 1 ? 16 : (grp == 2 ? 8 : (grp == 3 ? 24 : 0))) : 4 * grp;
    // Parked row-end pieces of this wave: [row k][head, tail] x 16 bytes.
    unsigned char* park = lds + a.p_off + wave * (16 * 2 * 16);

    uint32_t tile, tend;
    unit_range(a.dc, xcd_rank(blockIdx.x, a.nwg), &tile, &tend);

    // Registers carrying the next tile's new key rows and query rows.
    u32x4 kn[kPerRows], qn[kPerRows];
    bool prefetched = false;
    int s0 = 0;                     // ring slot of the current window's first key
    int qsel = 0;                   // query buffer of the current tile

    // Ring rows below kRingDup are written twice, the second time past the ring's end,
    // so that two blocks starting at any row r < ringc (rows r .. r + 16 + 22) are read
    // unwrapped.
    auto put_ring = [&](int slot, int ch, const u32x4& v) {
        *reinterpret_cast<u32x4*>(ring + swz<D>(slot, ch)) = v;
        if (slot < kRingDup) *reinterpret_cast<u32x4*>(ring + swz<D>(slot + ringc, ch)) = v;
    };

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
        const int64_t row0 = (static_cast<int64_t>(t.bb) * n + t.r) * h + t.hh;
        unsigned char* qlds = lds + a.q_off + qsel * kQBytes;

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
            for (int x = 0; x < kPerRows; ++x) {
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
                if (rr < W) put_ring(rr, ch, buf[x]);
            }
#pragma unroll
            for (int x = 0; x < kPerRows; ++x) {
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
            for (int x = 0; x < kPerRows; ++x) {
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

        // B operands: this wave's 16 query rows.
        V qf[kDC];
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc)
            qf[dc] = *reinterpret_cast<const V*>(qlds + swz<D>(il, 4 * dc + grp));

        // Row il: global element of window column 0 (column x sits at rowA + x); the
        // wave's rows share rowA mod kVec, and column o starts their pieces.
        const int64_t rowA = (row0 + static_cast<int64_t>(t0) * row_step) * K + k0 +
                             static_cast<int64_t>(il) * (gstep - 1);
        const int o = __builtin_amdgcn_readfirstlane(
            static_cast<int>((kVec - (rowA & (kVec - 1))) & (kVec - 1)));
        const bool row_ok = il < rows_here;
        const bool key_edge = u0 < 0 || u0 + W > n_r;     // window touches a sequence end

        // Blocks: from the one holding the first piece of row `wave` (it starts at the
        // largest column <= wave that is = o mod kVec, so at least wave - kVec + 1) to the
        // one holding column wave + 120 + kbeff - 1, the last column of the last row.
        const int x_first = wave - ((wave - o + kVec) & (kVec - 1));
        const int jb_lo = (x_first - o) >> 4;             // floor division (may be -1)
        const int jb_hi = (wave + 119 + kbeff - o) >> 4;
        const int nsteps = (jb_hi - jb_lo + kBPS) / kBPS;
        // Ring swizzle of this lane's key row within a block (blocks start at ring rows
        // that are multiples of 16, so it does not depend on the block).
        const int krow = o + col;                          // 0 .. 22
        int roff[kDC];
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) roff[dc] = swz<D>(krow, 4 * dc + grp);

        // Block reads start at ring row (s0 + 16 jb) mod ringc; the step loop advances one
        // such base by 16 kBPS per step (the second block of a step reads base + 16 ..,
        // inside the mirrored rows).
        auto ring_row = [&](int jb) {
            int r0 = s0 + 16 * jb;
            return r0 < 0 ? r0 + ringc : (r0 < ringc ? r0 : r0 - ringc);
        };
        auto fetch = [&](int base, V* kf) {
            const unsigned char* rp = ring + base * (2 * D);
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc) kf[dc] = *reinterpret_cast<const V*>(rp + roff[dc]);
        };
        auto mma = [&](const V* kf) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc) acc = Mfma<In>::run(kf[dc], qf[dc], acc);
            return acc;
        };
        // Round four accumulators; on tiles whose window reaches past a sequence end, keys
        // outside it take the padding constant.
        auto pack = [&](auto edge, int jb, const f32x4& acc) {
            P val = Pack<Out>::run(acc);
            if constexpr (decltype(edge)::value) {
                // keys of this lane's four columns: u0 + 16 jb + o + 4 grp + v
                const int ukey = u0 + 16 * jb + o + 4 * grp;
                bool kok[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) kok[v] = ukey + v >= 0 && ukey + v < n_r;
                const P pv = padv;
                if constexpr (!k16) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) val[v] = kok[v] ? val[v] : pv[v];
                } else {
                    const uint32_t m0 = (kok[0] ? 0xffffu : 0u) | (kok[1] ? 0xffff0000u : 0u);
                    const uint32_t m1 = (kok[2] ? 0xffffu : 0u) | (kok[3] ? 0xffff0000u : 0u);
                    val[0] = (val[0] & m0) | (pv[0] & ~m0);
                    val[1] = (val[1] & m1) | (pv[1] & ~m1);
                }
            }
            return val;
        };
        // Step st: this lane's piece starts at column x0 = 16 (jb_lo + kBPS st) + o + off_g,
        // i.e. slot x0 - il; whole pieces lie at slots 0 .. kbeff - kVec.
        const int slot_base = 16 * jb_lo + o + off_g - il;
        const int full_max = kbeff - kVec;
        OT* const gbase = band + (rowA + 16 * jb_lo + o + off_g);   // 16-byte aligned
        // A step holds a row's partial piece only near the ends of the sweep: slot0 >=
        // 16 kBPS st - 143 (jb_lo >= -1, o >= 0, off_g >= 0, il <= 127) and slot0 <=
        // 16 kBPS st + 24 (16 jb_lo + o <= x_first <= il), so only steps below st_h or from
        // st_t on look for them.
        const int st_h = (143 + 16 * kBPS) / (16 * kBPS);
        const int st_t = (kbeff - kVec - 24) >= 0 ? (kbeff - kVec - 24) / (16 * kBPS) + 1 : 0;
        auto finish = [&](auto edge, int st, const f32x4* acc) {
            const int jb = jb_lo + kBPS * st;
            u32x4 own;
            if constexpr (k16) {
                const P va = pack(edge, jb, acc[0]), vb = pack(edge, jb + 1, acc[1]);
                const auto sx = __builtin_amdgcn_permlane16_swap(va[0], vb[0], false, false);
                const auto sy = __builtin_amdgcn_permlane16_swap(va[1], vb[1], false, false);
                own = u32x4{sx[0], sy[0], sx[1], sy[1]};
            } else {
                own = pack(edge, jb, acc[0]);
            }
            const int sst = 16 * kBPS * st;
            const int slot0 = slot_base + sst;
            if (row_ok && full_max >= 0 &&
                static_cast<unsigned>(slot0) <= static_cast<unsigned>(full_max))
                *reinterpret_cast<u32x4*>(gbase + sst) = own;
            if (st < st_h || st >= st_t) {
                const bool part = row_ok && slot0 < kbeff && slot0 + kVec > 0 &&
                                  !(slot0 >= 0 && slot0 <= full_max);
                if (part)   // head piece (holds slot 0) or tail piece
                    *reinterpret_cast<u32x4*>(park + (2 * col + (slot0 < 0 ? 0 : 1)) * 16) = own;
            }
        };

        // Software pipeline: the MFMAs of step st + 1 and the key fragment reads of step
        // st + 2 are issued before step st is finished (past the last step they work on
        // ring rows nobody stores).  The scheduling barriers keep that order; the empty asm
        // with a memory clobber keeps the compiler from folding the loop-carried fragment
        // reads back into reads at their use.
        auto sweep = [&](auto edge) {
            V kf[kBPS][kDC];
            f32x4 acc_cur[kBPS], acc_nx[kBPS];
            int base = ring_row(jb_lo);                    // block jb_lo + kBPS st
            auto advance = [&]() {
                base += 16 * kBPS;
                base = base < ringc ? base : base - ringc;
            };
#pragma unroll
            for (int bq = 0; bq < kBPS; ++bq) fetch(base + 16 * bq, kf[bq]);
#pragma unroll
            for (int bq = 0; bq < kBPS; ++bq) acc_cur[bq] = mma(kf[bq]);
            advance();
#pragma unroll
            for (int bq = 0; bq < kBPS; ++bq) fetch(base + 16 * bq, kf[bq]);
            for (int st = 0; st < nsteps; ++st) {
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) acc_nx[bq] = mma(kf[bq]);
                __builtin_amdgcn_sched_barrier(0);
                advance();
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) fetch(base + 16 * bq, kf[bq]);
                __builtin_amdgcn_sched_barrier(0);
                finish(edge, st, acc_cur);
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) acc_cur[bq] = acc_nx[bq];
            }
        };
        if (key_edge)
            sweep(std::true_type{});
        else
            sweep(std::false_type{});

        // Parked row-end pieces, element by element: lane (k, g), g < 2, takes row k's head
        // (g = 0) or tail (g = 1) piece.  A row's head piece starts at column x_first + 8 k
        // (slot -((il - o) mod kVec)); its tail piece holds slot kbeff - 1.  The piece is
        // read into named scalars before the per-element stores (store_part), which keeps
        // the element selection out of divergent vector code.
        if (grp < 2) {
            const int sh = x_first + 8 * col - il;         // head piece: slot0 in (-kVec, 0]
            const int xl = il + kbeff - 1;                 // last column of the row
            const int st_ = xl - ((xl - o + kVec) & (kVec - 1)) - il;   // tail piece slot0
            const int slot0 = grp ? st_ : sh;
            // The head piece is parked when it starts before slot 0; the tail piece when it
            // starts at or after slot 0 and runs past the last slot.
            const bool parked = row_ok && (grp ? (st_ >= 0 && st_ + kVec > kbeff) : sh < 0);
            if (parked) {
                const u32x4 pc = *reinterpret_cast<const u32x4*>(park + (2 * col + grp) * 16);
                const uint32_t d0 = pc[0], d1 = pc[1], d2 = pc[2], d3 = pc[3];
                const int pa = slot0 < 0 ? -slot0 : 0;
                const int pe = kbeff - slot0 < kVec ? kbeff - slot0 : kVec;
                store_part<OT>(band + (rowA + il + slot0), d0, d1, d2, d3, pa, pe);
            }
        }

        // The next tile's new key rows go to ring slots outside the current window (only
        // columns no row stores are read there), its query rows to the other buffer.
        if (next) {
            unsigned char* qnext = lds + a.q_off + (qsel ^ 1) * kQBytes;
#pragma unroll
            for (int x = 0; x < kPerRows; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) {
                    int slot = s0 + W + rr;
                    slot = slot < ringc ? slot : slot - ringc;
                    put_ring(slot, ch, kn[x]);
                    *reinterpret_cast<u32x4*>(qnext + swz<D>(rr, ch)) = qn[x];
                }
            }
        }
        __syncthreads();
        prefetched = next;
        if (next) {
            s0 += kRows;
            s0 = s0 < ringc ? s0 : s0 - ringc;
            qsel ^= 1;
        }
    }
}

struct Layout {
    int64_t kb = 0, ring = 0, q_off = 0, p_off = 0, bytes = 0;
};

// LDS layout for a chunk of kb slots: the key ring (plus its mirrored rows), two query
// tiles, the parked row-end pieces.
Layout layout_for(int64_t kb, int64_t d) {
    Layout l;
    l.kb = kb;
    l.ring = ceil_div(2 * kRows + kb - 1, 16) * 16;
    l.q_off = ceil_div((l.ring + kRingDup) * d * 2, 16) * 16;
    l.p_off = l.q_off + 2 * kRows * d * 2;
    l.bytes = l.p_off + kWaves * 16 * 2 * 16;
    return l;
}

template <class In, class Out, int D>
hipError_t launch_typed(const void* q, const void* k, void* band, const Problem& p,
                        const QkTilePlan& tp, uint32_t pad, hipStream_t stream) {
    const Layout l = layout_for(tp.grid.kb, D);
    QkArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.ring),
             static_cast<int32_t>(l.q_off), static_cast<int32_t>(l.p_off),
             static_cast<uint32_t>(tp.workgroups), pad,
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
    (void)out_dt;
    QkTilePlan tp;
    // The widest chunk (at most 513 slots) whose ring + query tiles fit in LDS ...
    int64_t max_slots = kMaxSlots;
    while (max_slots > 16 && layout_for(max_slots, p.d).bytes > kQkLdsBytes) --max_slots;
    // ... then the chunk count that balances the tiles over the compute units best: the
    // busiest unit's work ~ ceil(tiles / units) x (rows + chunk + a fixed cost per tile).
    const int64_t cus = device_cus();
    TileGrid best = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, max_slots);
    int64_t best_cost = -1;
    for (int64_t extra = 0; extra < 4; ++extra) {
        const int64_t nkb = ceil_div(p.K, max_slots) + extra;
        if (nkb > p.K) break;
        const TileGrid g = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, ceil_div(p.K, nkb));
        const int64_t cost = ceil_div(g.tiles, cus) * (kRows + g.kb + 32);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = g;
        }
    }
    tp.grid = best;
    const Layout l = layout_for(tp.grid.kb, p.d);
    tp.rs = 0;
    tp.lds_bytes = l.bytes;
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
