// diagmm_pvT on MFMA with persistent workgroups.
//
//   out[j][c] = sum over (i, k) with i + k - w = j of G[i][k] * X[i][c]
//
// (class-local rows of one residue class of the dilation).  In dense form out = B^T X
// with B[i][j] = G[i][j - i + w] on the band; the kernel computes out^T = X^T B.
//
// Tiles.  A tile is 64 consecutive output rows j0..j0+63 of one residue class of one
// (batch, head), processed per slot chunk [k0, k0 + KC) (one chunk unless the band is
// wider than the LDS budget allows; the accumulators span the chunks).  The chunk's
// contributions come from the W = 64 + KC - 1 band rows i = ilo + x, x = 0 .. W-1,
// ilo = j0 - k0 - KC + 1 + w ("window rows"), and from row x only the 64 slots
// k0 + KC - 1 - x + j, j = 0..63 (a parallelogram through the band); output column j
// takes rows x = j .. j + KC - 1.
//
// LDS.  X is kept row-major in a ring over window rows (as V is in the pv kernel: pieces
// swizzled by slot, the MFMA A operand read with transposing LDS reads), sliding by 64
// rows per tile.  The parallelogram is staged row-major,
// S[x][j] = G[ilo + x][k0 + KC - 1 - x + j]: each staged row is one 128-byte row of LDS,
// filled with aligned 16-byte stores from 16-byte loads of the band tensor taken at
// 2-byte alignment (the row-dependent skew is paid in the global loads, where it costs
// little).  Elements outside the chunk, and rows outside the sequence, are stored as 0.
// 16-byte pieces of a row are XOR-swizzled by row (piece q at q ^ 2 (x mod 4)), so the
// stores of a row and the transposed reads below are free of bank conflicts.
//
// Compute.  The MFMA B operand of lane (j, g) is 8 consecutive window rows of one output
// column: a column of S.  It is read with two ds_read_b64_tr_b16 (gfx950 transposing LDS
// reads): in each 16-lane group lane t receives element t mod 4 of the 8-byte chunks read
// by lanes 4 v + t / 4, v = 0..3, so lanes pointing at rows r + c / 4, columns
// 4 (c mod 4) hand every lane 4 consecutive rows of its own column.  The 64 x d output
// tile is 4 x (d/16) blocks of 16 x 16; wave w owns column block jb = w / 2 and half of
// the channel blocks, and for every 32-row chunk of the window its columns reach issues
// one v_mfma_f32_16x16x32_{f16,bf16} per channel block.  Lane (j = lane % 16,
// g = lane / 16) accumulates out[j0 + 16 jb + j][16 cb + 4 g .. +3].
//
// Order.  Neighbouring tiles of a residue class read the same 128-byte lines of each band
// row: the parallelogram of a tile starts and ends inside a line of every row it crosses,
// and the tile next to it reads the rest of that line.  The tiles can therefore be dealt
// round-robin, on the flat split over the XCD's workgroups (tiles lo + j + m nwg / 8 for
// its j-th workgroup), on the strip split over the strip's (tiles j + m g of the strip),
// so neighbouring tiles run at the same time and the lines they share are fetched from
// HBM once while they sit in the XCD's L2; a workgroup's consecutive tiles are then
// apart, and each tile loads its whole X window.  That is done on the flat split where a
// round of tiles over the XCD reads more band lines than its L2 holds (the shared lines
// would be gone by the workgroup's next tile), and on the strip split only when asked for
// (the whole-window loads cost more time there than the band lines save).  Otherwise a
// workgroup keeps a contiguous run of tiles, its window sliding by 64 rows from one to
// the next.
//
// Pipelining.  The next tile's band pieces (and, when the window slides, its 64 new X
// rows) load into registers while the current tile computes.
#include "launch.hpp"
#include "ring.hpp"
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

constexpr int kThreads = 512;
constexpr int kRows = kPvTRows;                      // 64 output rows per tile
constexpr int kMaxChunk = 513;
constexpr int kMaxWin = kRows + kMaxChunk - 1;       // 576 window rows
// Staged rows: 0 .. XS - 1, XS = 32 ceil((63 + KC) / 32), every row a B read reaches
// (column block jb reads rows 32 floor(16 jb / 32) .. 32 ceil((16 jb + 15 + KC) / 32) - 1);
// rows at or past W are zero.
__host__ __device__ constexpr int staged_rows(int kc) { return (63 + kc + 31) / 32 * 32; }
constexpr int kRowBytes = kRows * 2;                 // 128-byte staged rows, 8 pieces
constexpr int kSegPer = (staged_rows(kMaxChunk) * 8 + kThreads - 1) / kThreads;   // 9

struct PvTArgs {
    int64_t n, h, K, w, s;
    TileGrid g;            // nkb / kb: slot chunks per tile and slots per chunk
    int32_t ring;          // X ring capacity in window rows (= 8 mod 128)
    int32_t ring_off;      // LDS byte offset of the X ring
    uint32_t nwg;
    int64_t band_elems;
    TileDecode dc;         // whole tiles (units) over workgroups, unit -> coordinates
    Div32 chunks;          // item -> (unit, chunk)
    int32_t interleave;    // units interleaved over the XCD's (flat split) or strip's workgroups
};

struct Item {
    TileId t;
    int n_r, j0, rows_here, kbeff, ilo, W;
    int64_t k0, row0;
};

// Byte offset of piece q of staged row x (pieces XOR-swizzled by row).
__device__ __forceinline__ int spiece(int x, int q) { return x * kRowBytes + 16 * (q ^ (2 * (x & 3))); }

template <class In, int D>
__global__ void __launch_bounds__(kThreads)
pvt_mfma_kernel(const typename In::T* __restrict__ band, const typename In::T* __restrict__ x,
                void* __restrict__ out_raw, int out_f32, PvTArgs a) {
    using ST = typename In::T;
    using V = typename Mfma<In>::V;
    constexpr int kChunks = D / 8;                          // 16-byte pieces per X row
    constexpr int kPerWinX = (kMaxWin * kChunks + kThreads - 1) / kThreads;
    constexpr int kPer64X = (kRows * kChunks + kThreads - 1) / kThreads;
    constexpr int kCB = D / 16;
    static_assert(kCB >= 2 && kCB % 2 == 0, "d must be a multiple of 32");
    constexpr int kCBPerWave = kCB / 2;

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* seg = lds;                               // S[x][j], swizzled pieces
    unsigned char* xr_ = lds + a.ring_off;                  // X rows by slot, swizzled

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;
    const int64_t row_k = row_step * K;                     // band elements between rows
    const int ringc = a.ring;
    const int jb = wave >> 1;                               // this wave's column block
    const int cb0 = (wave & 1) * kCBPerWave;                // first channel block

    // Items: the chunks of this workgroup's units, the units taken as a sequence
    // ufirst + ustride m (interleaved over the XCD's or the strip's workgroups).
    uint32_t item = 0, iend, ufirst, ustride;
    {
        uint32_t cnt;
        unit_seq(a.dc, blockIdx.x, a.nwg, a.interleave != 0, &ufirst, &cnt, &ustride);
        iend = cnt * a.chunks.d;
    }
    // Zero the X ring once: window rows past the current window are read (and multiplied
    // by exact zeros), so no slot may ever hold a non-finite pattern.
    for (int q = tid; q < D * ringc / 8; q += kThreads)
        reinterpret_cast<u32x4*>(xr_)[q] = u32x4{0u, 0u, 0u, 0u};

    auto describe = [&](uint32_t id, Item* it) {
        const uint32_t m = div32(a.chunks, id);
        const int kc = static_cast<int>(id - m * a.chunks.d);
        const uint32_t unit = ufirst + m * ustride;
        TileId t = decode_fast(a.dc, unit);
        t.kb = kc;
        it->t = t;
        it->n_r = class_len_fast(a.dc, t.r);
        it->j0 = t.tb * kRows;
        it->rows_here = it->n_r - it->j0 < kRows ? it->n_r - it->j0 : kRows;
        it->k0 = static_cast<int64_t>(kc) * a.g.kb;
        it->kbeff = static_cast<int>(K - it->k0 < a.g.kb ? K - it->k0 : a.g.kb);
        it->ilo = static_cast<int>(it->j0 - it->k0 - it->kbeff + 1 + a.w);
        it->W = kRows + it->kbeff - 1;
        it->row0 = (static_cast<int64_t>(t.bb) * n + t.r) * h + t.hh;
    };

    // Registers carrying the next item's band pieces and, when its window slides, its 64
    // new X rows.
    u32x4 sb[kSegPer];
    u32x4 xb[kPer64X];

    // Piece p of this thread: staged row x = idx / 8, columns 8 q .. 8 q + 7 (q = idx % 8).
    // Its elements are band elements E0 + x (row_k - 1) + 8 q + e, E0 = the element of
    // row ilo at slot k0 + kbeff - 1; row x contributes columns [x - kbeff + 1, x].
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
    auto item_e0 = [&](const Item& it, int* x_lo, int* x_hi, bool* inside) {
        const int64_t e0 = (it.row0 + static_cast<int64_t>(it.ilo) * row_step) * K + it.k0 +
                           it.kbeff - 1;
        // window rows inside the sequence: ilo + x in [0, n_r)
        *x_lo = -it.ilo > 0 ? -it.ilo : 0;
        *x_hi = it.n_r - it.ilo < it.W ? it.n_r - it.ilo : it.W;
        *inside = e0 + static_cast<int64_t>(*x_lo) * (row_k - 1) >= 0 &&
                  e0 + static_cast<int64_t>(*x_hi - 1) * (row_k - 1) + kRows <= a.band_elems;
        return e0;
    };
    auto load_seg = [&](const Item& it) {
        int x_lo, x_hi;
        bool inside;
        const int64_t e0 = item_e0(it, &x_lo, &x_hi, &inside);
#pragma unroll
        for (int p = 0; p < kSegPer; ++p) {
            const int idx = tid + p * kThreads, xr = idx >> 3, q = idx & 7;
            if (xr >= x_lo && xr < x_hi && 8 * q + 8 > xr - it.kbeff + 1 && 8 * q <= xr) {
                const int64_t off = e0 + static_cast<int64_t>(xr) * (row_k - 1) + 8 * q;
                if (inside || (off >= 0 && off + 8 <= a.band_elems))
                    sb[p] = *reinterpret_cast<const u32x4_a2*>(band + off);
            }
        }
    };
    auto store_seg = [&](const Item& it) {
        int x_lo, x_hi;
        bool inside;
        const int64_t e0 = item_e0(it, &x_lo, &x_hi, &inside);
        const int xs = staged_rows(a.g.kb);
#pragma unroll
        for (int p = 0; p < kSegPer; ++p) {
            const int idx = tid + p * kThreads, xr = idx >> 3, q = idx & 7;
            if (xr < xs) {
                u32x4 val = u32x4{0u, 0u, 0u, 0u};
                if (xr >= x_lo && xr < x_hi && 8 * q + 8 > xr - it.kbeff + 1 && 8 * q <= xr) {
                    const int64_t off = e0 + static_cast<int64_t>(xr) * (row_k - 1) + 8 * q;
                    if (inside || (off >= 0 && off + 8 <= a.band_elems)) {
                        val = sb[p];
                    } else {                                // elements [ea, eb) in the tensor
                        const int ea = off < 0 ? static_cast<int>(-off) : 0;
                        const int64_t room = a.band_elems - off;
                        const int eb = room < 8 ? static_cast<int>(room) : 8;
                        val = load_piece_elems<ST>(band + off, ea, eb);
                    }
                }
                *reinterpret_cast<u32x4*>(seg + spiece(xr, q)) = val;
            }
        }
    };
    // Row x holds columns [max(0, x - kbeff + 1), min(64, x + 1)); the pieces it stages
    // whole also carry elements of the neighbouring band rows in HBM on either side of
    // that interval.  Only rows x < 63 (right end inside the tile) and x >= kbeff (left
    // end inside) have them: task (r, k) zeroes column k of the right-end piece of row r,
    // or of the left-end piece of row kbeff + r - 63, where stray.  Runs after the pieces
    // are written (a barrier in between).
    auto clear_strays = [&](const Item& it) {
        int x_lo, x_hi;
        bool inside;
        item_e0(it, &x_lo, &x_hi, &inside);
        for (int task = tid; task < 126 * 8; task += kThreads) {
            const int r = task >> 3, k = task & 7;
            const bool right = r < 63;
            const int xr = right ? r : it.kbeff + r - 63;
            if (xr < x_lo || xr >= x_hi) continue;
            int c;
            bool stray;
            if (right) {
                const int je = xr + 1;                      // first column past the row
                c = (je & ~7) + k;
                stray = c >= je && je < kRows;
            } else {
                const int ja = xr - it.kbeff + 1;           // first column of the row
                c = (ja & ~7) + k;
                stray = c < ja;
            }
            if (stray && c < kRows)
                reinterpret_cast<uint16_t*>(seg + spiece(xr, c >> 3))[c & 7] = 0;
        }
    };

    auto put_x = [&](int slot, int ch, const u32x4& pc) {
        *reinterpret_cast<u32x4*>(xr_ + ring_piece<D>(slot, ch)) = pc;
    };
    // One 16-byte piece of X for window row xr of an item (zeros outside the sequence).
    auto get_x = [&](const Item& it, int xr, int ch) {
        const int i = it.ilo + xr;
        if (i < 0 || i >= it.n_r) return u32x4{0u, 0u, 0u, 0u};
        return *reinterpret_cast<const u32x4*>(
            x + (it.row0 + static_cast<int64_t>(i) * row_step) * D + ch * 8);
    };
    auto fill_window = [&](const Item& it) {
        constexpr int kBatch = 9;
        for (int q0 = 0; q0 < kPerWinX; q0 += kBatch) {
            u32x4 buf[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int idx = tid + (q0 + q) * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (rr < it.W) buf[q] = get_x(it, rr, ch);
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int idx = tid + (q0 + q) * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (rr < it.W) put_x(rr, ch, buf[q]);
            }
        }
        wait_vmem_all();    // every batch is consumed: keep the loads off later waits
    };
    // The 64 new rows of a sliding next item (its window columns W-64 .. W-1).  Rows past
    // the sequence are read at the nearest row inside it and zeroed when staged, so the
    // prefetch writes its registers with loads alone: no wait is due between it and the
    // staging after the next barrier.
    auto new_row = [&](const Item& nx, int rr) {
        const int i = nx.ilo + nx.W - kRows + rr;
        return i < 0 ? 0 : (i < nx.n_r ? i : nx.n_r - 1);
    };
    auto load_new_x = [&](const Item& nx) {
#pragma unroll
        for (int q = 0; q < kPer64X; ++q) {
            const int idx = tid + q * kThreads, rr = idx / kChunks, ch = idx % kChunks;
            if (rr < kRows)
                xb[q] = *reinterpret_cast<const u32x4*>(
                    x + (nx.row0 + static_cast<int64_t>(new_row(nx, rr)) * row_step) * D + ch * 8);
        }
    };
    auto store_new_x = [&](const Item& nx, int slot_first) {
#pragma unroll
        for (int q = 0; q < kPer64X; ++q) {
            const int idx = tid + q * kThreads, rr = idx / kChunks, ch = idx % kChunks;
            if (rr < kRows) {
                const int i = nx.ilo + nx.W - kRows + rr;
                int slot = slot_first + rr;
                slot = slot < ringc ? slot : slot - ringc;
                put_x(slot, ch, i >= 0 && i < nx.n_r ? xb[q] : u32x4{0u, 0u, 0u, 0u});
            }
        }
    };

    f32x4 acc[kCBPerWave];
#pragma unroll
    for (int q = 0; q < kCBPerWave; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Transposed-read address of this lane for window rows 32 ic + 8 grp + e0 .. +3:
    // row 32 ic + 8 grp + e0 + col / 4, columns 16 jb + 4 (col mod 4) .. +3 (bytes
    // 8 (col mod 4) into the block's two pieces 2 jb, 2 jb + 1).  Rows 32 ic + 8 grp + e0
    // are multiples of 4, so the swizzle depends on col / 4 only.
    const int tr_row = 8 * grp + (col >> 2);
    const int tr_off = tr_row * kRowBytes +
                       16 * ((2 * jb + ((col & 3) >> 1)) ^ (2 * ((col >> 2) & 3))) + 8 * (col & 1);

    bool seg_ready = false, x_ready = false;
    int s0 = 0;
    Item it;
    if (item < iend) describe(item, &it);
    for (; item < iend; ++item) {
        if (it.j0 >= it.n_r) {
            seg_ready = x_ready = false;
            if (item + 1 < iend) describe(item + 1, &it);
            continue;
        }
        if (!seg_ready || !x_ready) {
            if (!seg_ready) load_seg(it);
            __syncthreads();                                // previous item done with LDS
            if (!x_ready) {                                 // its loads overlap the band's
                s0 = 0;
                fill_window(it);
            }
            if (!seg_ready) {
                store_seg(it);
                __syncthreads();
                clear_strays(it);
            }
            __syncthreads();
        }
        Item nx;
        bool has_next = item + 1 < iend;
        if (has_next) {
            describe(item + 1, &nx);
            has_next = nx.j0 < nx.n_r;
        }
        const bool next_slides = has_next && a.g.nkb == 1 && nx.t.tb == it.t.tb + 1 &&
                                 nx.t.r == it.t.r && nx.t.hh == it.t.hh && nx.t.bb == it.t.bb;
        if (has_next) {
            if (next_slides) load_new_x(nx);
            load_seg(nx);
        }

        // ---- compute: out^T[c][j] += sum_x XT[c][x] * B[x][j]
        {
            const int x_lo = 16 * jb, x_hi = 16 * jb + 15 + it.kbeff;
            const int ic_lo = x_lo / 32, ic_hi = (x_hi + 31) / 32;
            int aoff[kCBPerWave];                           // A operands: transposed reads
#pragma unroll
            for (int q = 0; q < kCBPerWave; ++q) aoff[q] = tr_lane_off<D>(col, cb0 + q);
            auto fetch = [&](int ic, V* bop, V* aop) {
                unsigned char* bp = seg + ic * (32 * kRowBytes) + tr_off;
                // (a C-style cast: the LDS address of a generic pointer into `lds`)
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bp));
                const s16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bp + 4 * kRowBytes));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                *bop = __builtin_bit_cast(V, u32x4{l2[0], l2[1], h2[0], h2[1]});
                int slot0 = s0 + 32 * ic + 8 * grp;             // a multiple of 8
                slot0 = slot0 < ringc ? slot0 : slot0 - ringc;
                const unsigned char* rp = xr_ + slot0 * (2 * D);
#pragma unroll
                for (int q = 0; q < kCBPerWave; ++q) aop[q] = tr_read8<V, D>(rp + aoff[q]);
            };
            auto mma = [&](const V& bop, const V* aop) {
#pragma unroll
                for (int q = 0; q < kCBPerWave; ++q) acc[q] = Mfma<In>::run(aop[q], bop, acc[q]);
            };
            // Two operand sets in turn: the next chunk's reads are issued before the
            // current one multiplies.  The empty asm with a memory clobber keeps the
            // compiler from folding the loop-carried reads back into reads at their use;
            // the scheduling barrier keeps the reads ahead of the MFMAs.
            V b0, b1, a0[kCBPerWave], a1[kCBPerWave];
            fetch(ic_lo, &b0, a0);
            int ic = ic_lo;
            for (; ic + 1 < ic_hi; ic += 2) {
                fetch(ic + 1, &b1, a1);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                mma(b0, a0);
                fetch(ic + 2 < ic_hi ? ic + 2 : ic + 1, &b0, a0);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                mma(b1, a1);
            }
            if (ic < ic_hi) mma(b0, a0);
        }

        const bool tile_done = it.t.kb == a.g.nkb - 1;
        if (tile_done) {
            const int jl = 16 * jb + col;
            if (jl < it.rows_here) {
                const int64_t orow = (it.row0 + static_cast<int64_t>(it.j0 + jl) * row_step) * D;
#pragma unroll
                for (int q = 0; q < kCBPerWave; ++q) {
                    const int c = 16 * (cb0 + q) + 4 * grp;
                    if (out_f32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(out_raw) + orow + c) = acc[q];
                    } else {
                        u32x2 pk;
                        if constexpr (__is_same(In, F16))
                            pk = __builtin_bit_cast(u32x2, __builtin_convertvector(acc[q], f16x4));
                        else
                            pk = __builtin_bit_cast(u32x2, __builtin_convertvector(acc[q], bf16x4));
                        *reinterpret_cast<u32x2*>(static_cast<ST*>(out_raw) + orow + c) = pk;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kCBPerWave; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        __syncthreads();                                    // all LDS reads of this item done
        if (has_next) {
            store_seg(nx);
            if (next_slides) {
                store_new_x(nx, s0 + it.W);                 // slots past the current window
                s0 += kRows;
                s0 = s0 < ringc ? s0 : s0 - ringc;
            }
            __syncthreads();
            clear_strays(nx);
            __syncthreads();
            seg_ready = true;
            x_ready = next_slides;
            it = nx;
        } else {
            seg_ready = x_ready = false;
            if (item + 1 < iend) describe(item + 1, &it);
        }
    }
}

struct PvTLayout {
    int64_t kc = 0, ring = 0, ring_off = 0, bytes = 0;
};

PvTLayout pvt_layout(int64_t kc, int64_t d) {
    PvTLayout l;
    l.kc = kc;
    const int64_t need = 2 * kRows + kc - 1;               // window + 64 prefetched rows
    l.ring = ceil_div(need - 8, 128) * 128 + 8;             // = 8 mod 128
    l.ring_off = static_cast<int64_t>(staged_rows(static_cast<int>(kc))) * kRowBytes;
    l.bytes = l.ring_off + d * l.ring * 2;
    return l;
}

// Units are whole tiles (all chunks of one row block), decoded with one chunk per tile.
TileDecode unit_decode(const PvTilePlan& tp, const Problem& p) {
    const TileGrid& g = tp.grid;
    const int64_t units = g.tiles / g.nkb;
    TileDecode dc = make_decode(TileGrid{g.res, g.rb, 1, g.kb, units}, p.h, p.n, p.s, units,
                                tp.workgroups);
    if (tp.strip_wgs > 0) set_strip_split(&dc, units / g.rb, g.rb, tp.strip_wgs);
    return dc;
}

template <class In, int D>
hipError_t launch_typed(const void* band, const void* x, void* out, bool out_f32,
                        const Problem& p, const PvTilePlan& tp, hipStream_t stream) {
    const PvTLayout l = pvt_layout(tp.grid.kb, D);
    PvTArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.ring),
              static_cast<int32_t>(l.ring_off), static_cast<uint32_t>(tp.workgroups),
              p.rows() * p.h * p.K, unit_decode(tp, p),
              make_div32(static_cast<uint32_t>(tp.grid.nkb)), tp.interleave ? 1 : 0};
    auto kern = pvt_mfma_kernel<In, D>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(kPvLdsBytes));
    if (attr != hipSuccess) return attr;
    launch_kernel(kern, dim3(static_cast<uint32_t>(tp.workgroups)), dim3(kThreads),
                       static_cast<size_t>(l.bytes), stream,
                       static_cast<const typename In::T*>(band),
                       static_cast<const typename In::T*>(x), out, out_f32 ? 1 : 0, a);
    return hipGetLastError();
}

template <class In>
hipError_t launch_d(const void* band, const void* x, void* out, bool out_f32,
                    const Problem& p, const PvTilePlan& tp, hipStream_t stream) {
    switch (p.d) {
    case 32: return launch_typed<In, 32>(band, x, out, out_f32, p, tp, stream);
    case 64: return launch_typed<In, 64>(band, x, out, out_f32, p, tp, stream);
    case 128: return launch_typed<In, 128>(band, x, out, out_f32, p, tp, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

PvTilePlan plan_pvt_mfma(const Problem& p) {
    PvTilePlan tp;
    int64_t kc = kMaxChunk;
    while (kc > 16 && pvt_layout(kc, p.d).bytes > kPvLdsBytes) --kc;
    tp.grid = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, kc);
    const PvTLayout l = pvt_layout(tp.grid.kb, p.d);
    tp.lds_bytes = l.bytes;
    const int64_t cus = device_cus();
    tp.workgroups = tp.grid.tiles < cus ? tp.grid.tiles : cus;
    // A strip: the row blocks (whole tiles) of one residue class of one (batch, head).
    const int64_t per_strip = tp.grid.rb;
    if (per_strip > 0 && tp.grid.nkb > 0)
        tp.strip_wgs = pick_strip_split(tp.grid.tiles / tp.grid.nkb / per_strip, per_strip,
                                        kRows, ceil_div(p.n, p.s) - (per_strip - 1) * kRows,
                                        tp.workgroups);
    // Tile order: a workgroup's next tile shares lines with its current one, but by then
    // every workgroup of the XCD has read a whole tile's band lines (2 lines of each of its
    // 64 + KC - 1 window rows, every chunk of the tile).  Where that round exceeds the
    // XCD's L2 (4 MB), the shared lines are gone before they are read again: deal the
    // tiles round-robin instead (each tile then loads its whole X window).  That is done
    // on the flat split; on the strip split only when forced, since there the extra X
    // window loads cost more time than the band lines it saves (at n = 4096, h = 12, 513
    // slots, dilation 3: 62 instead of 90 MB fetched, but 1.5 us slower).
    const int64_t round_bytes = (tp.workgroups / kXcds) * tp.grid.nkb *
                                (kRows + tp.grid.kb - 1) * 256;
    const int forced = tile_order_forced();
    tp.interleave = tp.workgroups % kXcds == 0 &&
                    (forced ? forced == 1
                            : tp.strip_wgs == 0 && round_bytes > (int64_t(4) << 20));
    tp.ok = tp.grid.tiles <= kMaxTiles && ceil_div(p.n, p.s) < (int64_t(1) << 30) &&
            p.K < (int64_t(1) << 30) && p.w < (int64_t(1) << 30) && l.bytes <= kPvLdsBytes &&
            tp.workgroups >= 1 && (p.d == 32 || p.d == 64 || p.d == 128);
    return tp;
}

hipError_t launch_pvt_mfma(const void* band, const void* x, void* out, const Problem& p,
                           const PvTilePlan& tp, int in_dt, int out_dt, hipStream_t stream) {
    const bool f32 = out_dt == kF32;
    if (in_dt == kF16) return launch_d<F16>(band, x, out, f32, p, tp, stream);
    if (in_dt == kBF16) return launch_d<BF16>(band, x, out, f32, p, tp, stream);
    return hipErrorInvalidValue;
}

}  // namespace diagmm
