// diagmm_pv on MFMA with persistent workgroups.
//
//   out[t][c] = sum over in-range slots k of P[t][k] * V[t + k - w][c]
//
// (class-local rows t and keys u of one residue class of the dilation, as in the qk
// kernel).  In dense form out = B V with B[t][u] = P[t][u - t + w] on the band and 0
// elsewhere; the kernel computes the transposed product out^T = V^T B^T.
//
// Tiles and workgroups.  A tile is 64 consecutive rows t0..t0+63 of one residue class of
// one (batch, head); when the band is wider than a slot chunk (KC slots, set by the LDS
// budget) the tile is processed chunk by chunk with the accumulators kept in registers.
// A chunk's slots reach the W = 64 + KC - 1 keys u0 .. u0 + W - 1 (u0 = t0 + k0 - w).
// One 512-thread workgroup per compute unit walks its whole tiles chunk by chunk: a
// contiguous range, where single-chunk tiles that continue a strip slide the key window
// by 64; or, for tiles of several chunks (each chunk loads its own window, and the next
// tile's windows overlap them but for 64 keys), each XCD's tiles dealt round-robin over
// its workgroups, so that neighbouring tiles read their windows from L2 at the same time.
//
// LDS.  V is kept row-major in a ring of key slots (keys outside the sequence are
// written as zeros), each row's 16-byte pieces XOR-swizzled by slot, so new rows go in
// with aligned 16-byte stores.  The MFMA A operand (16 channels x 8 consecutive keys, a
// transposed block of V) is read with two ds_read_b64_tr_b16: in each 16-lane group lane
// t receives element t mod 4 of the 8-byte chunks read by lanes 4 v + t / 4, so lanes
// pointing at slots r + c / 4, channels 16 cb + 4 (c mod 4) hand lane t keys r .. r + 3 of
// channel 16 cb + t.  The swizzle keeps the four rows of such a read on distinct banks.  The band
// rows of the current item are staged already skewed into window coordinates,
// S[il][x] = P[il][x - il] (0 outside the chunk, and where the key lies outside the
// sequence), so that the B operand - 8 consecutive keys of one query row - is one aligned
// 16-byte LDS read as well.  The skew is paid in the global loads instead: staged piece
// (il, x .. x + 7) is the 16 bytes of the band tensor starting at slot x - il of row il,
// read at 2-byte alignment.  LDS reads at 2-byte alignment are several times slower than
// aligned ones on this hardware; global loads at that alignment cost little more.
//
// Compute.  Wave w owns query block rb = w / 2 (16 rows) and half of the channel blocks;
// for every 32-key chunk of the window that its rows reach it reads one B operand and
// issues one v_mfma_f32_16x16x32_{f16,bf16} per channel block.  Lane (i = lane % 16,
// g = lane / 16) accumulates out[16 rb + i][16 cb + 4 g .. +3].
//
// Pipelining.  While an item is computed, the band pieces and new V rows of the next
// item are already loading into registers; they are written to LDS after a barrier.
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
constexpr int kRows = kPvRows;             // 64 query rows per tile
constexpr int kMaxChunk = 513;             // slots per chunk
constexpr int kMaxWin = kRows + kMaxChunk - 1;
// Staged band row: window columns 0 .. XW - 1, XW = 32 ceil((63 + KC) / 32), which covers
// every column a B read reaches (block rb reads 32 floor(16 rb / 32) up to
// 32 ceil((16 rb + 15 + KC) / 32) - 1); 16-byte pieces per row:
__host__ __device__ constexpr int band_pieces(int kc) { return (63 + kc + 31) / 32 * 4; }
constexpr int kBandPieces = (kRows * band_pieces(kMaxChunk) + kThreads - 1) / kThreads;

struct PvArgs {
    int64_t n, h, K, w, s;
    TileGrid g;            // nkb = chunks per tile, kb = slots per chunk
    int32_t rsp;           // band staging row stride (elements, multiple of 8)
    int32_t ring;          // V ring capacity in key slots (multiple of 8)
    int32_t ring_off;      // LDS byte offset of the V ring
    uint32_t nwg;
    int64_t band_elems;    // elements of the band tensor
    TileDecode dc;         // whole tiles (units) over workgroups, unit -> coordinates
    Div32 chunks;          // item -> (unit, chunk)
    int32_t interleave;    // units interleaved over each XCD's workgroups (flat split)
};

// One work item = (tile, chunk); items run with the chunk fastest, so a tile's chunks
// are consecutive and its accumulators stay in registers.
struct Item {
    TileId t;
    int n_r, t0, rows_here, kbeff, u0, W;
    int64_t k0, row0;
};

template <class In, int D>
__global__ void __launch_bounds__(kThreads)
pv_mfma_kernel(const typename In::T* __restrict__ band, const typename In::T* __restrict__ v,
               void* __restrict__ out_raw, int out_f32, PvArgs a) {
    using ST = typename In::T;
    using V = typename Mfma<In>::V;
    constexpr int kChunks = D / 8;                          // 16-byte pieces per V row
    constexpr int kPerWinV = (kMaxWin * kChunks + kThreads - 1) / kThreads;
    constexpr int kPer64V = (kRows * kChunks + kThreads - 1) / kThreads;
    constexpr int kCB = D / 16;                             // channel blocks
    static_assert(kCB >= 2 && kCB % 2 == 0, "d must be a multiple of 32");
    constexpr int kCBPerWave = kCB / 2;

    extern __shared__ __align__(16) unsigned char lds[];
    ST* pst = reinterpret_cast<ST*>(lds);                   // band staging
    unsigned char* vr = lds + a.ring_off;                   // V rows by slot, swizzled

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;
    const int64_t row_k = row_step * K;                     // band elements between rows
    const int rsp = a.rsp, ringc = a.ring;
    const int rb = wave >> 1;                               // this wave's query block
    const int cb0 = (wave & 1) * kCBPerWave;                // first channel block

    // Whole tiles per workgroup (a tile's chunks share its accumulators), items = chunks;
    // the tiles are taken as a sequence ufirst + ustride m (interleaved over the XCD's
    // workgroups on the flat split).
    uint32_t item = 0, iend, ufirst, ustride;
    {
        uint32_t cnt;
        unit_seq(a.dc, blockIdx.x, a.nwg, a.interleave != 0, &ufirst, &cnt, &ustride);
        iend = cnt * a.chunks.d;
    }
    // Zero the V ring once: window columns past the current window are read (and
    // multiplied by exact zeros), so no slot may ever hold a non-finite pattern.
    for (int x = tid; x < D * ringc / 8; x += kThreads)
        reinterpret_cast<u32x4*>(vr)[x] = u32x4{0u, 0u, 0u, 0u};

    auto describe = [&](uint32_t id, Item* it) {
        const uint32_t m = div32(a.chunks, id);
        const int kc = static_cast<int>(id - m * a.chunks.d);
        const uint32_t unit = ufirst + m * ustride;
        TileId t = decode_fast(a.dc, unit);
        t.kb = kc;
        it->t = t;
        it->n_r = class_len_fast(a.dc, t.r);
        it->t0 = t.tb * kRows;
        it->rows_here = it->n_r - it->t0 < kRows ? it->n_r - it->t0 : kRows;
        it->k0 = static_cast<int64_t>(kc) * a.g.kb;
        it->kbeff = static_cast<int>(K - it->k0 < a.g.kb ? K - it->k0 : a.g.kb);
        it->u0 = static_cast<int>(it->t0 + it->k0 - a.w);
        it->W = kRows + it->kbeff - 1;
        it->row0 = (static_cast<int64_t>(t.bb) * n + t.r) * h + t.hh;
    };

    // Registers that carry the next item's band pieces and, when its window slides, the
    // 64 new V rows.
    u32x4 pb[kBandPieces];
    u32x4 vb[kPer64V];

    const int npw = band_pieces(a.g.kb);                    // pieces per staged row
    // Piece x of this thread is (il, q): staged row il, window columns 8q .. 8q+7, i.e.
    // slots lo .. lo+7 with lo = 8q - il, for idx = tid + x kThreads = il npw + q (the
    // same for every item, so worked out once).  idx / npw by a float reciprocal is exact
    // here: idx < 2^13, so the error is far below the 1/(2 npw) margin around the integers.
    int pil[kBandPieces], plo[kBandPieces];
    {
        const float inv_npw = 1.0f / static_cast<float>(npw);
#pragma unroll
        for (int x = 0; x < kBandPieces; ++x) {
            const int idx = tid + x * kThreads;
            const int r = static_cast<int>((static_cast<float>(idx) + 0.5f) * inv_npw);
            pil[x] = r;
            plo[x] = 8 * (idx - r * npw) - r;
        }
    }
    auto piece_of = [&](int x, int* il, int* lo) {
        *il = pil[x];
        *lo = plo[x];
    };
    // Slots of row il that take part: inside the chunk, key u0 + il + slot in [0, n_r).
    auto valid_slots = [&](const Item& it, int il, int* va, int* vb) {
        const int key0 = it.u0 + il;
        *va = -key0 > 0 ? -key0 : 0;
        *vb = it.n_r - key0 < it.kbeff ? it.n_r - key0 : it.kbeff;
    };
    // Global element of slot 0 of row 0 of an item, and whether every piece that meets
    // the chunk (slots -7 .. kbeff + 6 of its rows) lies inside the band tensor.
    auto item_base = [&](const Item& it, bool* inside) {
        const int64_t base = (it.row0 + static_cast<int64_t>(it.t0) * row_step) * K + it.k0;
        *inside = base >= 7 &&
                  base + (it.rows_here - 1) * row_k + it.kbeff + 7 <= a.band_elems;
        return base;
    };

    // Pieces that meet a row's valid slots are loaded whole (2-byte aligned) and staged
    // raw; pieces that do not are staged as zeros.  The valid slots of a row are one
    // interval, so at most two staged pieces per row (head and tail) hold stray elements;
    // clear_strays zeroes those afterwards.  So the prefetch issues no wait and staging is
    // a handful of ALU operations per piece.  On the first and last tiles of the tensor a
    // piece may reach past its ends: there, only elements inside the tensor are read, one
    // by one, when staging.
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
    // il * row_k as one 32 x 32 -> 64-bit multiply (row_k < 2^32 is a plan condition)
    auto row_off = [&](int il) {
        return static_cast<int64_t>(static_cast<uint64_t>(il) * static_cast<uint32_t>(row_k));
    };
    auto load_band = [&](const Item& it) {
        bool inside;
        const int64_t base = item_base(it, &inside);
#pragma unroll
        for (int x = 0; x < kBandPieces; ++x) {
            int il, lo;
            piece_of(x, &il, &lo);
            if (il < it.rows_here && lo + 8 > 0 && lo < it.kbeff) {
                const int64_t off = base + row_off(il) + lo;
                if (inside || (off >= 0 && off + 8 <= a.band_elems))
                    pb[x] = *reinterpret_cast<const u32x4_a2*>(band + off);
            }
        }
    };
    auto store_band = [&](const Item& it) {
        bool inside;
        const int64_t base = item_base(it, &inside);
#pragma unroll
        for (int x = 0; x < kBandPieces; ++x) {
            int il, lo, va, vb;
            piece_of(x, &il, &lo);
            if (il < it.rows_here) {
                valid_slots(it, il, &va, &vb);
                if (va >= vb) va = vb = 1 << 30;            // no valid slot: all zeros
                u32x4 val = u32x4{0u, 0u, 0u, 0u};
                if (lo + 8 > va && lo < vb) {
                    const int64_t off = base + row_off(il) + lo;
                    if (inside || (off >= 0 && off + 8 <= a.band_elems)) {
                        val = pb[x];
                    } else {                                // elements [ea, eb) in the tensor
                        const int ea = off < 0 ? static_cast<int>(-off) : 0;
                        const int64_t room = a.band_elems - off;
                        const int eb = room < 8 ? static_cast<int>(room) : 8;
                        val = load_piece_elems<ST>(band + off, ea, eb);
                    }
                }
                *reinterpret_cast<u32x4*>(pst + il * rsp + lo + il) = val;
            }
        }
    };
    // Mask the head and tail pieces of every staged row to its valid window columns
    // [xa, xb) = il + valid slots: one 16-byte read-modify-write per piece (thread 2 il
    // the head piece, 2 il + 1 the tail piece unless it is the head piece too).  A row with
    // no valid slot has all its pieces staged as zeros (store_band).  Runs after the
    // pieces are written (a barrier in between).
    auto clear_strays = [&](const Item& it) {
        if (tid >= 2 * kRows) return;
        const int il = tid >> 1, tail = tid & 1;
        if (il >= it.rows_here) return;
        int va, vb;
        valid_slots(it, il, &va, &vb);
        const int xa = il + va, xb = il + vb;
        if (xa >= xb) return;
        const int ph = xa & ~7, pt = (xb - 1) & ~7;
        if (tail && pt == ph) return;
        const int pc = tail ? pt : ph;
        u32x4* pp = reinterpret_cast<u32x4*>(pst + il * rsp + pc);
        *pp = mask_piece<ST>(*pp, xa - pc, xb - pc);
    };
    // One 16-byte piece of V row `slot` (channels ch*8 .. ch*8+7) into the ring.
    auto put_v = [&](int slot, int ch, const u32x4& pc) {
        *reinterpret_cast<u32x4*>(vr + ring_piece<D>(slot, ch)) = pc;
    };
    // One 16-byte piece of V for window column x of an item (zeros outside the sequence).
    auto get_v = [&](const Item& it, int x, int ch) {
        const int u = it.u0 + x;
        if (u < 0 || u >= it.n_r) return u32x4{0u, 0u, 0u, 0u};
        return *reinterpret_cast<const u32x4*>(
            v + (it.row0 + static_cast<int64_t>(u) * row_step) * D + ch * 8);
    };
    // The whole window of an item into ring slots 0..W-1 (synchronous; caller barriers).
    auto fill_window = [&](const Item& it) {
        constexpr int kBatch = 9;                           // pieces in flight per thread
        for (int x0 = 0; x0 < kPerWinV; x0 += kBatch) {
            u32x4 buf[kBatch];
#pragma unroll
            for (int x = 0; x < kBatch; ++x) {
                const int idx = tid + (x0 + x) * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (rr < it.W) buf[x] = get_v(it, rr, ch);
            }
#pragma unroll
            for (int x = 0; x < kBatch; ++x) {
                const int idx = tid + (x0 + x) * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (rr < it.W) put_v(rr, ch, buf[x]);
            }
        }
        wait_vmem_all();    // every batch is consumed: keep the loads off later waits
    };
    // The 64 new rows of a sliding next item (its window columns W-64 .. W-1).  Rows past
    // the sequence are read at the nearest row inside it and zeroed when staged, so the
    // prefetch writes its registers with loads alone: no wait is due between it and the
    // staging after the next barrier.
    auto new_row = [&](const Item& nx, int rr) {
        const int i = nx.u0 + nx.W - kRows + rr;
        return i < 0 ? 0 : (i < nx.n_r ? i : nx.n_r - 1);
    };
    auto load_new_v = [&](const Item& nx) {
#pragma unroll
        for (int x = 0; x < kPer64V; ++x) {
            const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
            if (rr < kRows)
                vb[x] = *reinterpret_cast<const u32x4*>(
                    v + (nx.row0 + static_cast<int64_t>(new_row(nx, rr)) * row_step) * D + ch * 8);
        }
    };
    auto store_new_v = [&](const Item& nx, int slot_first) {
#pragma unroll
        for (int x = 0; x < kPer64V; ++x) {
            const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
            if (rr < kRows) {
                const int i = nx.u0 + nx.W - kRows + rr;
                int slot = slot_first + rr;
                slot = slot < ringc ? slot : slot - ringc;
                put_v(slot, ch, i >= 0 && i < nx.n_r ? vb[x] : u32x4{0u, 0u, 0u, 0u});
            }
        }
    };

    f32x4 acc[kCBPerWave];
#pragma unroll
    for (int q = 0; q < kCBPerWave; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // band_ready: the current item's band is staged; v_ready: its key window is in the ring.
    bool band_ready = false, v_ready = false;
    int s0 = 0;                                             // ring slot of window column 0
    Item it;
    if (item < iend) describe(item, &it);
    for (; item < iend; ++item) {
        if (it.t0 >= it.n_r) {                              // empty block of a short class
            band_ready = v_ready = false;
            if (item + 1 < iend) describe(item + 1, &it);
            continue;
        }
        if (!band_ready || !v_ready) {
            if (!band_ready) load_band(it);
            __syncthreads();                                // previous item done with LDS
            if (!v_ready) {                                 // its loads overlap the band's
                s0 = 0;
                fill_window(it);
            }
            if (!band_ready) {
                store_band(it);
                __syncthreads();
                clear_strays(it);
            }
            __syncthreads();
        }
        // Next item: fetch its band pieces (and new V rows if it slides) during compute.
        Item nx;
        bool has_next = item + 1 < iend;
        if (has_next) {
            describe(item + 1, &nx);
            has_next = nx.t0 < nx.n_r;
        }
        const bool next_slides = has_next && a.g.nkb == 1 && nx.t.tb == it.t.tb + 1 &&
                                 nx.t.r == it.t.r && nx.t.hh == it.t.hh && nx.t.bb == it.t.bb;
        if (has_next) {
            if (next_slides) load_new_v(nx);
            load_band(nx);
        }

        // ---- compute: out^T[c][i] += sum_x VT[c][x] * B[x][i]
        {
            const int il = 16 * rb + col;                   // this lane's query row
            const int x_lo = 16 * rb;                       // window columns this block uses
            const int x_hi = 16 * rb + 15 + it.kbeff;       // exclusive
            const int jc_lo = x_lo / 32, jc_hi = (x_hi + 31) / 32;
            // brow[x] = B[x][il] = P[il][x - il] for every window column x this lane reads
            const ST* brow = pst + il * rsp + 8 * grp;
            // A operand of channel block cb: transposed reads of slots r .. r + 3 and
            // r + 4 .. r + 7, r = ring slot of window column 32 jc + 8 grp (a multiple of
            // 4, so the four slots of a read never wrap and their swizzle depends on this
            // lane's position in its group only).
            int aoff[kCBPerWave];
#pragma unroll
            for (int q = 0; q < kCBPerWave; ++q) aoff[q] = tr_lane_off<D>(col, cb0 + q);
            auto fetch = [&](int jc, V* bop, V* aop) {
                *bop = *reinterpret_cast<const V*>(brow + 32 * jc);
                int slot0 = s0 + 32 * jc + 8 * grp;             // ring slot of column x0
                slot0 = slot0 < ringc ? slot0 : slot0 - ringc;
                const unsigned char* rp = vr + slot0 * (2 * D);
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
            fetch(jc_lo, &b0, a0);
            int jc = jc_lo;
            for (; jc + 1 < jc_hi; jc += 2) {
                fetch(jc + 1, &b1, a1);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                mma(b0, a0);
                fetch(jc + 2 < jc_hi ? jc + 2 : jc + 1, &b0, a0);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                mma(b1, a1);
            }
            if (jc < jc_hi) mma(b0, a0);
        }

        // ---- last chunk of the tile: write the outputs and clear the accumulators
        const bool tile_done = it.t.kb == a.g.nkb - 1;
        if (tile_done) {
            const int il = 16 * rb + col;
            if (il < it.rows_here) {
                const int64_t orow = (it.row0 + static_cast<int64_t>(it.t0 + il) * row_step) * D;
#pragma unroll
                for (int q = 0; q < kCBPerWave; ++q) {
                    const int c = 16 * (cb0 + q) + 4 * grp;
                    if (out_f32) {
                        float* o = static_cast<float*>(out_raw) + orow + c;
                        *reinterpret_cast<f32x4*>(o) = acc[q];
                    } else {
                        ST* o = static_cast<ST*>(out_raw) + orow + c;
                        u32x2 pk;
                        if constexpr (sizeof(ST) == 2 && __is_same(In, F16))
                            pk = __builtin_bit_cast(u32x2, __builtin_convertvector(acc[q], f16x4));
                        else
                            pk = __builtin_bit_cast(u32x2, __builtin_convertvector(acc[q], bf16x4));
                        *reinterpret_cast<u32x2*>(o) = pk;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kCBPerWave; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        __syncthreads();                                    // all LDS reads of this item done
        if (has_next) {
            store_band(nx);
            if (next_slides) {
                store_new_v(nx, s0 + it.W);                 // slots past the current window
                s0 += kRows;
                s0 = s0 < ringc ? s0 : s0 - ringc;
            }
            __syncthreads();
            clear_strays(nx);
            __syncthreads();
            band_ready = true;
            v_ready = next_slides;
            it = nx;
        } else {
            band_ready = v_ready = false;
            if (item + 1 < iend) describe(item + 1, &it);
        }
    }
}

struct PvLayout {
    int64_t kc = 0, rsp = 0, ring = 0, ring_off = 0, bytes = 0;
};

PvLayout pv_layout(int64_t kc, int64_t d) {
    PvLayout l;
    l.kc = kc;
    l.rsp = 8 * band_pieces(static_cast<int>(kc)) + 8;    // odd multiple of 16 bytes
    const int64_t need = 2 * kRows + kc - 1;               // window + 64 prefetched keys
    l.ring = ceil_div(need - 8, 128) * 128 + 8;             // = 8 mod 128 (bank spread)
    l.ring_off = ceil_div(kRows * l.rsp * 2, 16) * 16;
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
hipError_t launch_typed(const void* band, const void* v, void* out, bool out_f32,
                        const Problem& p, const PvTilePlan& tp, hipStream_t stream) {
    const PvLayout l = pv_layout(tp.grid.kb, D);
    PvArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.rsp),
             static_cast<int32_t>(l.ring), static_cast<int32_t>(l.ring_off),
             static_cast<uint32_t>(tp.workgroups), p.rows() * p.h * p.K,
             unit_decode(tp, p), make_div32(static_cast<uint32_t>(tp.grid.nkb)),
             tp.interleave ? 1 : 0};
    auto kern = pv_mfma_kernel<In, D>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(kPvLdsBytes));
    if (attr != hipSuccess) return attr;
    launch_kernel(kern, dim3(static_cast<uint32_t>(tp.workgroups)), dim3(kThreads),
                       static_cast<size_t>(l.bytes), stream,
                       static_cast<const typename In::T*>(band),
                       static_cast<const typename In::T*>(v), out, out_f32 ? 1 : 0, a);
    return hipGetLastError();
}

template <class In>
hipError_t launch_d(const void* band, const void* v, void* out, bool out_f32,
                    const Problem& p, const PvTilePlan& tp, hipStream_t stream) {
    switch (p.d) {
    case 32: return launch_typed<In, 32>(band, v, out, out_f32, p, tp, stream);
    case 64: return launch_typed<In, 64>(band, v, out, out_f32, p, tp, stream);
    case 128: return launch_typed<In, 128>(band, v, out, out_f32, p, tp, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

PvTilePlan plan_pv_mfma(const Problem& p) {
    PvTilePlan tp;
    int64_t kc = kMaxChunk;
    while (kc > 16 && pv_layout(kc, p.d).bytes > kPvLdsBytes) --kc;
    // tiles: (b, h, res, row block) x chunks; TileGrid.nkb counts chunks
    tp.grid = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, kc);
    const PvLayout l = pv_layout(tp.grid.kb, p.d);
    tp.lds_bytes = l.bytes;
    const int64_t cus = device_cus();
    tp.workgroups = tp.grid.tiles < cus ? tp.grid.tiles : cus;
    // A strip: the row blocks (whole tiles) of one residue class of one (batch, head).
    const int64_t per_strip = tp.grid.rb;
    if (per_strip > 0 && tp.grid.nkb > 0)
        tp.strip_wgs = pick_strip_split(tp.grid.tiles / tp.grid.nkb / per_strip, per_strip,
                                        kRows, ceil_div(p.n, p.s) - (per_strip - 1) * kRows,
                                        tp.workgroups);
    // Tile order on the flat split.  A tile of one chunk continues the previous tile's key
    // window (it slides by 64 rows in LDS); a tile of several chunks loads a new window
    // per chunk, and the next tile's windows overlap them all but 64 rows.  When the
    // XCD's workgroups read more windows in one round of tiles than its L2 (4 MB) holds,
    // a workgroup's next tile finds them gone: deal the tiles round-robin instead, so
    // that neighbouring tiles read their windows at the same time.
    const int64_t round_bytes = (tp.workgroups / kXcds) * tp.grid.nkb *
                                (kRows + tp.grid.kb - 1) * p.d * 2;
    const int forced = tile_order_forced();
    tp.interleave = tp.strip_wgs == 0 && tp.workgroups % kXcds == 0 &&
                    (forced ? forced == 1
                            : tp.grid.nkb > 1 && round_bytes > (int64_t(4) << 20));
    tp.ok = tp.grid.tiles <= kMaxTiles && ceil_div(p.n, p.s) < (int64_t(1) << 30) &&
            p.K < (int64_t(1) << 30) && l.bytes <= kPvLdsBytes && tp.workgroups >= 1 &&
            p.s * p.h * p.K < (int64_t(1) << 32) &&
            (p.d == 32 || p.d == 64 || p.d == 128);
    return tp;
}

hipError_t launch_pv_mfma(const void* band, const void* v, void* out, const Problem& p,
                          const PvTilePlan& tp, int in_dt, int out_dt, hipStream_t stream) {
    const bool f32 = out_dt == kF32;
    if (in_dt == kF16) return launch_d<F16>(band, v, out, f32, p, tp, stream);
    if (in_dt == kBF16) return launch_d<BF16>(band, v, out, f32, p, tp, stream);
    return hipErrorInvalidValue;
}

}  // namespace diagmm
