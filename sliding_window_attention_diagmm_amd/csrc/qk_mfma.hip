// diagmm_qk on MFMA with persistent, sliding workgroups, storing straight from registers.
//
// Tiles.  A tile is M = 128 consecutive rows t0..t0+127 of one residue class of one
// (batch, head) and a chunk of KB consecutive slots k0..k0+KB-1.  Its slots reach the
// W = M + KB - 1 consecutive keys u0 = t0 + k0 - w .. u0 + W - 1 of the class ("window
// columns" x = 0 .. W-1; row il of the tile holds its slots at columns il .. il + KB - 1).
// Tiles are numbered with the row block fastest, so consecutive tiles of one strip slide
// down the class by 128 rows and share all but 128 of their keys.
//
// Workgroups.  One workgroup per compute unit walks a contiguous range of tile ids.  It
// keeps the key window of the current tile in an LDS ring (rows swizzled by 16-byte chunk)
// and the query tile in one of two LDS buffers.  Its waves have two roles.  Eight compute
// waves sweep the tile and store the band; they never load from HBM, so nothing makes
// them wait for their stores to drain (a wave's vector memory counter covers its loads
// and stores alike, in issue order).  Four load waves bring the next tile's rows into LDS
// meanwhile: for a tile that continues the strip (same batch, class, head and slot chunk,
// next row block) its 128 new key rows and its query rows; for one that starts a strip,
// its whole window, when the ring holds two windows.  Slots outside the current window
// only ever feed discarded columns of the sweep, so those writes race with nothing that
// is stored.  A tile that was not prefetched is loaded by all waves before its sweep.

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
// gives 4 columns = 16 bytes per lane.  Whole pieces go straight to HBM through a buffer
// resource (pieces that are not whole get an out-of-range offset and are dropped).  A
// lane's at most two pieces that also hold slots of the neighbouring band row in HBM (the
// row's head and tail) are kept in registers and written element by element after the
// sweep.  (An optional lane trade, kTradeStores, gives each group of four consecutive
// lanes one row's 64 consecutive bytes, which the memory pipeline writes as one run; the
// trade's LDS round trip costs more than it gains here, so it is off.)
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

constexpr int kComputeThreads = 512;          // 8 waves: the sweep and every band store
constexpr int kLoadThreads = 256;             // 4 waves: the global loads of the next tile
constexpr int kThreads = kComputeThreads + kLoadThreads;
constexpr int kComputeWaves = kComputeThreads / 64;
constexpr int kRows = kQkRows;                // 128 = 8 waves x 16 rows
constexpr int kMaxSlots = 513;
constexpr int kRingDup = 80;                  // ring rows mirrored past its end
constexpr bool kTradeStores = false;          // lane trades before band stores
constexpr int kStagePer = 8;                  // 16-byte chunks per thread per load batch
                                              // (2 for d = 128, whose sweep needs the registers)

// Band stores: raw buffer resource (stride 0, range in bytes; word 3 of the gfx9 buffer
// descriptor for untyped 32-bit access).  Offsets at or past kBufRange are dropped.
constexpr int kBufRange = 0x7ffffff0;
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufDrop = static_cast<int>(0x80000000u);
// Largest tile band span the 32-bit store offsets must cover (checked by the planner).
constexpr int64_t kMaxTileSpan = (int64_t(1) << 31) - (int64_t(1) << 20);

struct QkArgs {
    int64_t n, h, K, w, s;
    TileGrid g;
    int32_t ring;      // key rows in the LDS ring (a multiple of 16, >= 2 kRows + KB - 1)
    int32_t q_off;     // LDS byte offset of the two query tiles
    uint32_t nwg;      // persistent workgroups
    uint32_t pad;      // padding constant, already rounded to the output type
    TileDecode dc;     // tiles over workgroups, tile -> coordinates
};

// Byte offset of (row, 16-byte chunk) in a swizzled block of D-element rows.  A 16-byte
// LDS read is served eight lanes at a time, 128 bytes across all banks; the chunk index
// is XORed with the row's position among the rows sharing a 128-byte stretch of banks
// (rows of 128 bytes or more: row mod 8; rows of 64 bytes, two per 128 bytes: row / 2
// mod 4), so eight consecutive rows read at one logical chunk hit eight distinct 16-byte
// bank groups.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
    constexpr int kShift = D == 32 ? 1 : 0;
    constexpr int kMask = D == 32 ? 3 : 7;
    return row * (D * 2) + ((chunk ^ ((row >> kShift) & kMask)) << 4);
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Ring rows between the end of a window of W keys and the next multiple of 16.
__device__ __forceinline__ int align_gap(int W) { return (16 - (W & 15)) & 15; }

// Rows one tile needs in LDS beyond what is already there: nk key rows of a class (keys
// u_first .., clamped into the class) for ring slots slot_first .., and nq of the tile's
// query rows (tq0 ..; all kRows of them, or none) for a query buffer.
struct Stage {
    int64_t row0;      // [b][n][h] row of class row 0 of the tile's (batch, class, head)
    int u_first, nk, slot_first, tq0, n_r;
    int qbuf;          // LDS byte offset of the query buffer
    int nq;
};

template <class In, class Out, int D>
__global__ void __launch_bounds__(kThreads)
qk_mfma_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ kx,
               typename Out::T* __restrict__ band, QkArgs a) {
    using OT = typename Out::T;
    using IT = typename In::T;
    using V = typename Mfma<In>::V;
    using P = typename Pack<Out>::P;
    constexpr bool k16 = sizeof(OT) == 2;
    constexpr int kVec = 16 / sizeof(OT);                 // elements per 16-byte piece
    constexpr int kDC = D / 32;
    constexpr int kChunks = D / 8;                        // 16-byte chunks per row
    constexpr int kQBytes = kRows * D * 2;
    constexpr int kBPS = k16 ? 2 : 1;                     // blocks per step
    constexpr int kPer = D >= 128 ? kStagePer / 4 : kStagePer;

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* ring = lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool computes = wave < kComputeWaves;
    const int col = lane & 15, grp = lane >> 4;
    const int cw = wave & (kComputeWaves - 1);            // compute wave index
    const int il = cw + 8 * col;                          // this lane's tile row
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;                       // [b][n][h] rows per class row
    const int64_t gstep = row_step * K;                   // band elements per class row
    const uint32_t row_bytes = static_cast<uint32_t>(row_step * D * 2);   // per class row
    const int ringc = a.ring;
    const P padv = Pack<Out>::splat(a.pad);

    uint32_t tile, tend;
    unit_range(a.dc, xcd_rank(blockIdx.x, a.nwg), &tile, &tend);

    // Ring rows below kRingDup are written twice, the second time past the ring's end,
    // so that a pair of steps starting at any row r < ringc (rows r .. r + 32 + 16 + 22) is
    // read unwrapped.
    auto put_ring = [&](int slot, int ch, const u32x4& v) {
        *reinterpret_cast<u32x4*>(ring + swz<D>(slot, ch)) = v;
        if (slot < kRingDup) *reinterpret_cast<u32x4*>(ring + swz<D>(slot + ringc, ch)) = v;
    };
    // Batch b0 of a Stage moved by NT threads (this one is number gt): kPer 16-byte
    // chunks per thread, chunk b0 + gt + NT x, i.e. chunk column gt mod kChunks of stage row
    // (b0 + gt) / kChunks + x NT / kChunks; stage rows are the key rows, then the query
    // rows.  Sources are addressed by 32-bit byte offsets from the strip's first row.
    // Every entry of buf is loaded (rows past the end re-read the last one), which keeps a
    // held batch in one set of registers; only the LDS writes are predicated.
    constexpr int kChunkShift = D == 32 ? 2 : (D == 64 ? 3 : 4);
    auto load_batch = [&](const Stage& sg, int gt, int b0, u32x4* buf, auto nt_c) {
        constexpr int kRowsX = decltype(nt_c)::value >> kChunkShift;
        const int ch = gt & (kChunks - 1);
        const int rr0 = (b0 + gt) >> kChunkShift;
        const int last = sg.nk + sg.nq - 1;
        const int dq = sg.tq0 - sg.nk - sg.u_first;       // query row of stage row rr: rr + dq
        const unsigned char* kb8 =
            reinterpret_cast<const unsigned char*>(kx + sg.row0 * D) + ch * 16;
        const unsigned char* qb8 =
            reinterpret_cast<const unsigned char*>(q + sg.row0 * D) + ch * 16;
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            int rr = rr0 + kRowsX * x;
            rr = rr < last ? rr : last;
            const bool isk = rr < sg.nk;
            int u = sg.u_first + rr + (isk ? 0 : dq);
            u = u < 0 ? 0 : (u < sg.n_r ? u : sg.n_r - 1);
            const uint32_t off = __umul24(static_cast<uint32_t>(u), row_bytes);
            buf[x] = ld_global16((isk ? kb8 : qb8) + off);
        }
    };
    auto write_batch = [&](const Stage& sg, int gt, int b0, const u32x4* buf, auto nt_c) {
        constexpr int kRowsX = decltype(nt_c)::value >> kChunkShift;
        const int ch = gt & (kChunks - 1);
        const int rr0 = (b0 + gt) >> kChunkShift;
        const int rows = sg.nk + sg.nq;
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            const int rr = rr0 + kRowsX * x;
            if (rr < rows) {
                if (rr < sg.nk) {
                    int slot = sg.slot_first + rr;
                    slot = slot < ringc ? slot : slot - ringc;
                    put_ring(slot, ch, buf[x]);
                } else {
                    *reinterpret_cast<u32x4*>(lds + sg.qbuf + swz<D>(rr - sg.nk, ch)) = buf[x];
                }
            }
        }
    };
    // The batches of a Stage from b0 on, each loaded and then written.
    auto stage_from = [&](const Stage& sg, int gt, int b0, auto nt_c) {
        constexpr int NT = decltype(nt_c)::value;
        const int total = (sg.nk + sg.nq) * kChunks;
        for (; b0 < total; b0 += NT * kPer) {
            u32x4 buf[kPer];
            load_batch(sg, gt, b0, buf, nt_c);
            write_batch(sg, gt, b0, buf, nt_c);
        }
    };

    // Tile coordinates and extents.
    struct TInfo {
        TileId t;
        int n_r, t0, kbeff, u0, W;
        int64_t row0;
        bool ok;                   // not an empty tail block of a shorter residue class
    };
    // Tile ids are walked in order: the next id by carrying through the grid extents.
    auto next_id = [&](TileId t) {
        if (++t.tb == static_cast<int>(a.dc.rb.d)) {
            t.tb = 0;
            if (++t.kb == static_cast<int>(a.dc.nkb.d)) {
                t.kb = 0;
                if (++t.r == static_cast<int>(a.dc.res.d)) {
                    t.r = 0;
                    if (++t.hh == static_cast<int>(a.dc.h.d)) {
                        t.hh = 0;
                        ++t.bb;
                    }
                }
            }
        }
        return t;
    };
    auto info = [&](const TileId& id) {
        TInfo f;
        f.t = id;
        f.n_r = class_len_fast(a.dc, f.t.r);
        f.t0 = f.t.tb * kRows;
        f.ok = f.t0 < f.n_r;
        const int64_t k0 = static_cast<int64_t>(f.t.kb) * a.g.kb;
        f.kbeff = static_cast<int>(K - k0 < a.g.kb ? K - k0 : a.g.kb);
        f.u0 = static_cast<int>(f.t0 + k0 - a.w);
        f.W = kRows + f.kbeff - 1;
        f.row0 = (static_cast<int64_t>(f.t.bb) * n + f.t.r) * h + f.t.hh;
        return f;
    };
    // The rows tile nn needs after tile c (window at ring slot s0c).  A tile continuing
    // c's strip needs 128 new keys, right after c's window; one starting a strip its whole
    // window, from the first multiple of 16 past c's window (block reads assume windows
    // start at such ring rows), less the first `skip` keys when those were written earlier.
    // They go to the ring while c is swept only if the ring holds both (*fits: at + the
    // keys nn adds <= ringc).
    auto link = [&](const TInfo& c, const TInfo& nn, int s0c, int qbuf, int skip, bool* cont,
                    int* at, bool* fits) {
        *cont = nn.t.tb == c.t.tb + 1 && nn.t.kb == c.t.kb && nn.t.r == c.t.r &&
                nn.t.hh == c.t.hh && nn.t.bb == c.t.bb;
        *at = *cont ? c.W : c.W + align_gap(c.W);
        const int add = *cont ? kRows : nn.W;
        *fits = *at + add <= ringc;
        skip = *cont ? 0 : skip;
        Stage sg;
        sg.row0 = nn.row0;
        sg.u_first = *cont ? c.u0 + c.W : nn.u0 + skip;
        sg.nk = add - skip;
        int sl = s0c + *at + skip;
        sg.slot_first = sl < ringc ? sl : sl - ringc;
        sg.tq0 = nn.t0;
        sg.n_r = nn.n_r;
        sg.qbuf = qbuf;
        sg.nq = kRows;
        return sg;
    };
    // The first e keys of the window of a tile x that starts a strip, as key rows only, for
    // ring slots from slot0 (the slot of x's window) on.
    auto early_stage = [&](const TInfo& x, int slot0, int e) {
        Stage sg;
        sg.row0 = x.row0;
        sg.u_first = x.u0;
        sg.nk = e;
        sg.slot_first = slot0 < ringc ? slot0 : slot0 - ringc;
        sg.tq0 = x.t0;
        sg.n_r = x.n_r;
        sg.qbuf = 0;
        sg.nq = 0;
        return sg;
    };

    bool ready = false;             // the current tile's keys and query rows are in LDS
    int s0 = 0;                     // ring slot of the current window's first key
    int qsel = 0;                   // query buffer of the current tile
    // A tile that starts a strip needs a whole window, three times the keys a continuing
    // tile adds.  When it comes two tiles after one that its predecessor continues, the
    // first keys of its window are written while that earlier tile is swept, into ring
    // rows neither window being swept then holds; the rest, with its query rows, then
    // comes one tile early like a continuing tile's rows.  (A workgroup whose range
    // crosses into a second strip would otherwise load that window within one tile and
    // finish last.)  early_tile / early_n: the tile whose first early_n keys are written.
    uint32_t early_tile = ~0u;
    int early_n = 0;
    constexpr int kEarlyCap = kLoadThreads * kPer / kChunks;   // key rows of one load batch

    // Load waves: the first batch of the rows the tile after next needs, loaded during
    // this tile and written to LDS during the next one.
    u32x4 lbuf[kPer];
    bool lheld = false;

    // This tile, the next and the one after (ids past the range decode to unused values).
    TileId id2 = decode_fast(a.dc, tile);
    TInfo inf0 = info(id2);
    id2 = next_id(id2);
    TInfo inf1 = info(id2);
    id2 = next_id(id2);

    for (; tile < tend; ++tile) {
        const TInfo cur = inf0;
        TInfo nxt = inf1;
        const TInfo nn = info(id2);
        id2 = next_id(id2);
        inf0 = inf1;
        inf1 = nn;
        if (!cur.ok) {
            ready = lheld = false;
            continue;
        }
        const int n_r = cur.n_r, t0 = cur.t0, kbeff = cur.kbeff, u0 = cur.u0, W = cur.W;
        const int rows_here = n_r - t0 < kRows ? n_r - t0 : kRows;
        const int64_t k0 = static_cast<int64_t>(cur.t.kb) * a.g.kb;
        const int64_t row0 = cur.row0;

        if (!ready) s0 = 0;

        // The next tile's rows go to LDS while this one is swept, when the ring holds both.
        bool pre = false, cont = false;
        int at = 0;
        Stage nx{};
        if (tile + 1 >= tend) nxt.ok = false;
        const int qnext = a.q_off + (qsel ^ 1) * kQBytes;
        if (nxt.ok) {
            link(cur, nxt, s0, qnext, 0, &cont, &at, &pre);
            // A cold tile followed by a strip start: the first keys of the next window are
            // loaded with this tile's rows (they go past this window, at + e <= ringc).
            if (!ready && pre && !cont) {
                const int e = min(min(nxt.W, ringc - at), kEarlyCap);
                early_tile = tile + 1;
                early_n = e;
            }
            nx = link(cur, nxt, s0, qnext, early_tile == tile + 1 ? early_n : 0, &cont, &at,
                      &pre);
        }
        // The tile after next starts a strip and the next one continues this one: the first
        // e2 keys of its window go to ring rows from s0 + kRows + at2 (its window's slot)
        // while this tile is swept.  This tile's window lies kRows before the next one's, so
        // rows up to ringc - kRows past the next window's slot are free.
        int e2 = 0, slot2 = 0;
        if (pre && cont && tile + 2 < tend && nn.ok && early_tile != tile + 2) {
            bool c2, fit2;
            int at2;
            link(nxt, nn, 0, 0, 0, &c2, &at2, &fit2);
            if (!c2 && fit2) {
                e2 = min(min(nn.W, ringc - kRows - at2), kEarlyCap);
                slot2 = s0 + kRows + at2;
                slot2 = slot2 < ringc ? slot2 : slot2 - ringc;
                if (e2 > 0) {
                    early_tile = tile + 2;
                    early_n = e2;
                }
            }
        }

        if (!ready) {
            // Nothing prefetched: every wave loads the whole key window and the query tile,
            // or, when the early keys of the next strip's window come too, the compute waves
            // the window and query tile and the load waves those keys.
            const Stage cold{row0, u0, W, 0, t0, n_r, a.q_off + qsel * kQBytes, kRows};
            const bool e1 = early_tile == tile + 1;
            if (!e1 && e2 <= 0) {
                stage_from(cold, tid, 0, std::integral_constant<int, kThreads>{});
            } else if (computes) {
                stage_from(cold, tid, 0, std::integral_constant<int, kComputeThreads>{});
            } else {
                const int lt = tid - kComputeThreads;
                constexpr auto nt = std::integral_constant<int, kLoadThreads>{};
                stage_from(e1 ? early_stage(nxt, s0 + at, early_n) : early_stage(nn, slot2, e2),
                           lt, 0, nt);
            }
            __syncthreads();
        }

        if (!computes) {
            const int lt = tid - kComputeThreads;
            constexpr auto nt = std::integral_constant<int, kLoadThreads>{};
            if (pre) {
                if (!lheld) load_batch(nx, lt, 0, lbuf, nt);
                write_batch(nx, lt, 0, lbuf, nt);
                stage_from(nx, lt, kLoadThreads * kPer, nt);
            }
            if (ready && e2 > 0) stage_from(early_stage(nn, slot2, e2), lt, 0, nt);
            lheld = false;
            if (nxt.ok && tile + 2 < tend && nn.ok) {
                bool c2, fit2;
                int at2;
                const Stage nx2 = link(nxt, nn, 0, 0, early_tile == tile + 2 ? early_n : 0,
                                       &c2, &at2, &fit2);   // rows only
                if (fit2) {
                    load_batch(nx2, lt, 0, lbuf, nt);
                    lheld = true;
                }
            }
        } else {
            unsigned char* qlds = lds + a.q_off + qsel * kQBytes;
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
            // Before a piece is stored, lanes trade pieces (ds_bpermute) so that each group of
            // four consecutive lanes holds four consecutive pieces of one row, which the memory
            // pipeline writes as one 64-byte run.  Lane 16 b + 4 a + j then stores row
            // srow = 4 a + b of the wave's 16 (tile row ils), columns off_s .. of each step.  In
            // the MFMA layout lane 16 g + c holds row c: for f32 columns 4 g .., for 16-bit
            // outputs (after pairing two blocks) columns 0, 16, 8, 24 .. for g = 0, 1, 2, 3.
            const int srow = kTradeStores ? 4 * ((lane >> 2) & 3) + (lane >> 4) : col;
            const int sj = kTradeStores ? lane & 3 : (k16 ? ((grp & 1) << 1) | (grp >> 1) : grp);
            const int ils = cw + 8 * srow;
            const bool row_ok_s = ils < rows_here;
            const int off_s = k16 ? 8 * sj : 4 * sj;
            const int src_g = k16 ? (((sj & 1) << 1) | (sj >> 1)) : sj;   // holds off_s ..
            const int bp_addr = (16 * src_g + srow) * 4;

            // Blocks: from the one holding the first piece of row `cw` (it starts at the
            // largest column <= cw that is = o mod kVec, so at least cw - kVec + 1) to the
            // one holding column cw + 120 + kbeff - 1, the last column of the last row.
            const int x_first = cw - ((cw - o + kVec) & (kVec - 1));
            const int jb_lo = (x_first - o) >> 4;             // floor division (may be -1)
            const int jb_hi = (cw + 119 + kbeff - o) >> 4;
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
            // outside it take the padding constant (checked per lane only in blocks that
            // reach past it: the block's keys are u0 + 16 jb + o .. +15 for the whole wave).
            auto pack = [&](auto edge, int jb, const f32x4& acc) {
                P val = Pack<Out>::run(acc);
                const int ublk = u0 + 16 * jb + o;
                if (!decltype(edge)::value) return val;
                if (ublk + 16 <= 0 || ublk >= n_r) return padv;     // whole block outside
                if (ublk < 0 || ublk + 16 > n_r) {
                    // keys of this lane's four columns: u0 + 16 jb + o + 4 grp + v
                    const int ukey = ublk + 4 * grp;
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
            // Step st: the piece this lane stores starts at column x0 = 16 (jb_lo + kBPS st) + o
            // + off_s, i.e. slot x0 - ils; whole pieces lie at slots 0 .. kbeff - kVec.
            const int slot_base = 16 * jb_lo + o + off_s - ils;
            const int full_max = kbeff - kVec;
            // Whole pieces are stored through a buffer resource based at the tile's band
            // origin: this lane's piece of step st sits (ils (gstep - 1) + 16 jb_lo + o + off_s
            // + kCS st) elements past it, a 16-byte aligned spot.  Pieces that are not whole
            // (or rows past the class) get an offset beyond the resource's range, whose stores
            // the hardware drops: no branch, no exec mask.
            const bool any_full = row_ok_s && full_max >= 0;
            const int sb_full = any_full ? slot_base : -(1 << 30);
            const unsigned fm_full = any_full ? static_cast<unsigned>(full_max) : 0u;
            const int lane_off = static_cast<int>(
                (static_cast<int64_t>(ils) * (gstep - 1) + 16 * jb_lo + o + off_s) *
                static_cast<int64_t>(sizeof(OT)));
            const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
                band + ((row0 + static_cast<int64_t>(t0) * row_step) * K + k0), 0, kBufRange,
                kBufWord3);
            // A step holds a row's partial piece only near the ends of the sweep: slot0 >=
            // 16 kBPS st - 143 (jb_lo >= -1, o >= 0, off_s >= 0, ils <= 127) and slot0 <=
            // 16 kBPS st + 24 (16 jb_lo + o <= x_first <= ils), so only steps below st_h or from
            // st_t on look for them.
            constexpr int kCS = 16 * kBPS;                   // columns per step
            const int st_h = (143 + kCS) / kCS;
            const int st_t = (kbeff - kVec - 24) >= 0 ? (kbeff - kVec - 24) / kCS + 1 : 0;
            // This lane's partial pieces: the one starting in slots -(kVec - 1) .. -1 (it holds
            // slot 0) and the one starting in max(0, full_max + 1) .. kbeff - 1 (it holds the
            // last slot but is not whole).  Its pieces start kCS slots apart, so each range
            // holds at most one; st_hd / st_tl are their steps (-1: none).
            auto first_step = [&](int slot) {                // first st with slot0 >= slot
                const int d = slot - slot_base;
                return d <= 0 ? 0 : (d + kCS - 1) / kCS;
            };
            int st_hd = first_step(-(kVec - 1));
            if (!row_ok_s || slot_base + kCS * st_hd > -1) st_hd = -1;
            const int lo_t = full_max + 1 > 0 ? full_max + 1 : 0;
            int st_tl = first_step(lo_t);
            if (!row_ok_s || slot_base + kCS * st_tl >= kbeff) st_tl = -1;
            // Step st's piece in the store layout: rounded (and padded), paired into 16-byte
            // pieces for 16-bit outputs, then traded between lanes.
            auto gather_ = [&](auto edge, int st, const f32x4* acc) {
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
                if constexpr (!kTradeStores) return own;
                u32x4 pc;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pc[i] = static_cast<uint32_t>(
                        __builtin_amdgcn_ds_bpermute(bp_addr, static_cast<int>(own[i])));
                return pc;
            };
            // Steps whose keys all lie inside the class: ub + kCS st .. + kCS - 1 in [0, n_r);
            // on tiles touching a sequence end, those skip the per-block padding checks.
            const int ub = u0 + 16 * jb_lo + o;
            const int st_in_lo = ub >= 0 ? 0 : (kCS - 1 - ub) / kCS;
            int st_in_n = n_r - kCS - ub >= 0 ? (n_r - kCS - ub) / kCS + 1 - st_in_lo : 0;
            st_in_n = st_in_n > 0 ? st_in_n : 0;
            auto gather = [&](auto edge, int st, const f32x4* acc) {
                if constexpr (decltype(edge)::value) {
                    if (static_cast<unsigned>(st - st_in_lo) < static_cast<unsigned>(st_in_n))
                        return gather_(std::false_type{}, st, acc);
                }
                return gather_(edge, st, acc);
            };
            // Store step st's piece: whole pieces to HBM, the row's partial ones to LDS.
            // The lane's partial pieces are kept in registers (head steps all come before
            // st_h, tail steps from st_t on) and stored element by element after the sweep.
            u32x4 hpc = {0u, 0u, 0u, 0u}, tpc = {0u, 0u, 0u, 0u};
            auto put = [&](int st, const u32x4& pc) {
                const int sst = 16 * kBPS * st;
                const bool whole = static_cast<unsigned>(sb_full + sst) <= fm_full;
                __builtin_amdgcn_raw_buffer_store_b128(
                    pc, brs, whole ? lane_off + sst * static_cast<int>(sizeof(OT)) : kBufDrop,
                    0, 0);
                if (st < st_h) {
                    const bool mine = st == st_hd;
#pragma unroll
                    for (int i = 0; i < 4; ++i) hpc[i] = mine ? pc[i] : hpc[i];
                }
                if (st >= st_t) {   // (the two ranges overlap when kbeff is small)
                    const bool mine = st == st_tl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) tpc[i] = mine ? pc[i] : tpc[i];
                }
            };

            // Software pipeline, per step st: the MFMAs of step st + 1, the lane trades of
            // step st, the key fragment reads of step st + 2 (issued after the trades, so that
            // waiting for the trades leaves them in flight), then step st's stores.  The loop
            // runs steps in pairs, the accumulators alternating between two sets (an odd count
            // gets one more step, whose columns no row stores; past the last step the reads
            // work on ring rows nobody stores).  The scheduling barriers keep that order; the
            // empty asm with a memory clobber keeps the compiler from folding the loop-carried
            // fragment reads back into reads at their use.
            auto sweep = [&](auto edge) {
                V kf[kBPS][kDC];
                f32x4 acc_a[kBPS], acc_b[kBPS];
                int base = ring_row(jb_lo);                    // block jb_lo + kBPS st
                auto advance = [&]() {
                    base += 16 * kBPS;
                    base = base < ringc ? base : base - ringc;
                };
                // The first step of a pair reads up to 70 rows past a base below ringc (inside
                // the mirrored rows), so only the second one wraps.
                auto step = [&](f32x4* acc_out, const f32x4* acc_in, int st, bool wrap) {
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int bq = 0; bq < kBPS; ++bq) acc_out[bq] = mma(kf[bq]);
                    __builtin_amdgcn_sched_barrier(0);
                    const u32x4 pc = gather(edge, st, acc_in);
                    __builtin_amdgcn_sched_barrier(0);
                    if (wrap) advance();
                    else base += 16 * kBPS;
#pragma unroll
                    for (int bq = 0; bq < kBPS; ++bq) fetch(base + 16 * bq, kf[bq]);
                    __builtin_amdgcn_sched_barrier(0);
                    put(st, pc);
                };
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) fetch(base + 16 * bq, kf[bq]);
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) acc_a[bq] = mma(kf[bq]);
                advance();
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) fetch(base + 16 * bq, kf[bq]);
                for (int st = 0; st < nsteps; st += 2) {
                    step(acc_b, acc_a, st, false);
                    step(acc_a, acc_b, st + 1, true);
                }
            };
            if (key_edge)
                sweep(std::true_type{});
            else
                sweep(std::false_type{});

            // Partial pieces, element by element: slots inside 0 .. kbeff - 1 only; the other
            // elements (and pieces the lane does not hold) get out-of-range offsets.
            // The valid elements form one stretch, bytes [a, b) of the 16-byte piece; it
            // goes out as aligned 2-, 4-, 8-, 4- and 2-byte stores taken greedily from the
            // left (at most three of them apply to a row end, and since a wave's rows share
            // their alignment, all lanes holding such a piece need the same ones).
            auto put_part = [&](int st, const u32x4& pc) {
                const int slot0 = slot_base + kCS * st;
                const int e_lo = slot0 < 0 ? -slot0 : 0;
                const int e_hi = kbeff - slot0 < kVec ? kbeff - slot0 : kVec;
                constexpr int esz = static_cast<int>(sizeof(OT));
                int a = e_lo * esz;
                const int b = e_hi * esz;
                const int off0 = lane_off + kCS * st * esz;
                auto word = [&](int byte) { return pc[byte >> 2]; };
                if ((a & 3) == 2 && a + 2 <= b) {
                    __builtin_amdgcn_raw_buffer_store_b16(
                        static_cast<unsigned short>(word(a) >> 16), brs, off0 + a, 0, 0);
                    a += 2;
                }
                if ((a & 7) == 4 && a + 4 <= b) {
                    __builtin_amdgcn_raw_buffer_store_b32(word(a), brs, off0 + a, 0, 0);
                    a += 4;
                }
                if (a + 8 <= b) {
                    const u32x2 dw = (a & 8) ? u32x2{pc[2], pc[3]} : u32x2{pc[0], pc[1]};
                    __builtin_amdgcn_raw_buffer_store_b64(dw, brs, off0 + a, 0, 0);
                    a += 8;
                }
                if (a + 4 <= b) {
                    __builtin_amdgcn_raw_buffer_store_b32(word(a), brs, off0 + a, 0, 0);
                    a += 4;
                }
                if (a + 2 <= b)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        static_cast<unsigned short>(word(a) >> (8 * (a & 2))), brs, off0 + a,
                        0, 0);
            };
            if (st_hd >= 0) put_part(st_hd, hpc);
            if (st_tl >= 0) put_part(st_tl, tpc);
        }
        __syncthreads();                                  // this tile's LDS reads are done
        ready = pre;
        if (pre) {
            s0 += cont ? kRows : at;
            s0 = s0 < ringc ? s0 : s0 - ringc;
            qsel ^= 1;
        }
    }
}

struct Layout {
    int64_t kb = 0, ring = 0, q_off = 0, bytes = 0;
};

// LDS layout for a chunk of kb slots: the key ring (plus its mirrored rows) and two query
// tiles.  The ring holds two whole windows where that fits, so
// that a tile starting a new strip is loaded while the one before it is swept, and at
// least a window plus the kRows keys a continuing tile adds.
Layout layout_for(int64_t kb, int64_t d) {
    const int64_t win = kRows + kb - 1;
    Layout l;
    for (const int64_t rows : {2 * ceil_div(win, 16) * 16, win + kRows}) {
        l.kb = kb;
        l.ring = ceil_div(rows, 16) * 16;
        l.q_off = ceil_div((l.ring + kRingDup) * d * 2, 16) * 16;
        l.bytes = l.q_off + 2 * kRows * d * 2;
        if (l.bytes <= kQkLdsBytes) break;
    }
    return l;
}

template <class In, class Out, int D>
hipError_t launch_typed(const void* q, const void* k, void* band, const Problem& p,
                        const QkTilePlan& tp, uint32_t pad, hipStream_t stream) {
    const Layout l = layout_for(tp.grid.kb, D);
    QkArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.ring),
             static_cast<int32_t>(l.q_off),
             static_cast<uint32_t>(tp.workgroups), pad,
             make_decode(tp.grid, p.h, p.n, p.s, tp.grid.tiles, tp.workgroups)};
    if (tp.strip_wgs > 0)
        set_strip_split(&a.dc, tp.grid.tiles / tp.grid.rb, tp.grid.rb, tp.strip_wgs);
    auto kern = qk_mfma_kernel<In, Out, D>;
    // Once per instantiation (thread-safe static initialisation): allow all of the
    // compute unit's LDS as dynamic LDS.
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(kQkLdsBytes));
    if (attr != hipSuccess) return attr;
    launch_kernel(kern, dim3(static_cast<uint32_t>(tp.workgroups)), dim3(kThreads),
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
    const int64_t out_bytes = out_dt == kF32 ? 4 : 2;
    // The widest chunk (at most 513 slots) whose ring + query tiles fit in LDS ...
    int64_t max_slots = kMaxSlots;
    while (max_slots > 16 && layout_for(max_slots, p.d).bytes > kQkLdsBytes) --max_slots;
    // ... as few chunks as possible: every chunk reads the query and key rows again, and
    // the whole launch is bound by HBM traffic.  With 1.5 tiles per unit (n=4096, h=12,
    // 513 slots) one chunk took 22.9 us against 24.0 us for two, although its busiest
    // units sweep twice the slots: units with one tile finish early and leave the rest
    // the bandwidth.  Only when that leaves fewer than 1.4 tiles per unit is the chunk
    // count that balances the tiles best chosen instead: the busiest unit's work ~
    // ceil(tiles / units) x (rows + chunk + a fixed cost per tile).
    const int64_t cus = device_cus();
    TileGrid best = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, max_slots);
    const bool balance = best.tiles * 10 < cus * 14;
    int64_t best_cost = -1;
    for (int64_t extra = 0; balance && extra < 4; ++extra) {
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
    // Strip split: a fixed group of workgroups per strip (the row blocks of one slot chunk
    // of one residue class of one (batch, head)) whenever it does not lengthen the longest
    // tile list.  A range that crosses into a second strip has to load that strip's whole
    // window; with one 513-slot chunk two windows do not fit in the ring, so that load is
    // not prefetched and such workgroups would end last.  (n=4096, h=12: 21 workgroups
    // per strip of 32 row blocks, 11 of them with two tiles; 252 of 256 busy.)
    {
        const int64_t per_strip = tp.grid.rb;
        const int64_t strips = per_strip > 0 ? tp.grid.tiles / per_strip : 0;
        const int64_t g = strips > 0 ? tp.workgroups / strips : 0;
        if (g >= 1 && g <= per_strip && strips * per_strip == tp.grid.tiles &&
            ceil_div(per_strip, g) <= ceil_div(tp.grid.tiles, tp.workgroups) &&
            ceil_div(tp.grid.tiles, tp.workgroups) > 1)
            tp.strip_wgs = g;
    }
    // (q and k rows of one strip are addressed by 32-bit byte offsets)
    tp.ok = tp.grid.tiles <= kMaxTiles && ceil_div(p.n, p.s) < (int64_t(1) << 30) &&
            (p.n + p.s) * p.h * p.d * 2 < (int64_t(1) << 32) &&
            kRows * p.s * p.h * p.K * out_bytes < kMaxTileSpan &&   // band store offsets
            p.s * p.h * p.d * 2 < (int64_t(1) << 24) &&             // 24-bit row offsets
            ceil_div(p.n, p.s) < (int64_t(1) << 24) &&
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
