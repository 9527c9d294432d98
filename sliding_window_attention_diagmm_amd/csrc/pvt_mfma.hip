// diagmm_pvT on MFMA with persistent, sliding workgroups.
//
//   out[j][c] = sum over (i, k) with i + k - w = j of G[i][k] * X[i][c]
//
// (class-local rows of one residue class of the dilation).  In dense form out = B^T X
// with B[i][j] = G[i][j - i + w] on the band; the kernel computes out^T = X^T B.
//
// Tiles.  A tile is 32 consecutive output rows j0..j0+31 of one residue class of one
// (batch, head), processed per slot chunk [k0, k0 + KC) (one chunk unless the band is
// wider than the LDS budget allows; the accumulators span the chunks).  The chunk's
// contributions come from the W = 32 + KC - 1 band rows i = ilo .. ilo + W - 1,
// ilo = j0 - k0 - KC + 1 + w, and from each such row only the 32 slots
// [j0 - i + w, j0 + 31 - i + w] (a parallelogram through the band).
//
// LDS.  X is kept transposed, XT[c][slot], in a ring over band rows (as V is in the pv
// kernel), sliding by 32 rows per tile.  The parallelogram is staged row by row: the
// segment of band row i is copied as aligned 16-byte pieces (five pieces cover 32 slots
// at any alignment) into staging row x = i - ilo, keeping the band tensor's alignment;
// elements outside the chunk, and rows outside the sequence, are stored as zeros.  For
// output column j the element of row i sits at segment position j - j0 whatever i is,
// so the MFMA B operand (8 consecutive band rows, one output column) is a fixed column
// of 8 staged rows, gathered with 2-byte LDS reads.
//
// Compute.  The 32 x d output tile is 2 x (d/16) blocks of 16 x 16; each wave owns
// blocks of one 16-row group jb and, for every 32-row chunk of the window its rows
// reach, gathers one B operand and issues one v_mfma_f32_16x16x32 per channel block.
// Lane (j = lane % 16, g = lane / 16) accumulates out[16 jb + j][16 cb + 4 g .. +3].
//
// Pipelining.  The next tile's segment pieces (and, when the window slides, its 32 new
// X rows) load into registers while the current tile computes.
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

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kPvTRows;                      // 32 output rows per tile
constexpr int kMaxChunk = 513;
constexpr int kMaxWin = kRows + kMaxChunk - 1;       // 544 band rows
constexpr int kSegPieces = (7 + kRows + 7) / 8;      // 16-byte pieces per segment (5)
constexpr int kRss = kSegPieces * 8;                 // staging row stride (elements)
constexpr int kSegPer = (kMaxWin * kSegPieces + kThreads - 1) / kThreads;

struct PvTArgs {
    int64_t n, h, K, w, s;
    TileGrid g;            // nkb / kb: slot chunks per tile and slots per chunk
    int32_t ring;          // X ring capacity in band rows (multiple of 8)
    int32_t ring_off;      // LDS byte offset of the X ring
    uint32_t nwg;
    int64_t band_elems;
    TileDecode dc;         // whole tiles (units) over workgroups, unit -> coordinates
    Div32 chunks;          // item -> (unit, chunk)
};

struct Item {
    TileId t;
    int n_r, j0, rows_here, kbeff, ilo, W;
    int64_t k0, row0;
};

template <class In, int D>
__global__ void __launch_bounds__(kThreads)
pvt_mfma_kernel(const typename In::T* __restrict__ band, const typename In::T* __restrict__ x,
                void* __restrict__ out_raw, int out_f32, PvTArgs a) {
    using ST = typename In::T;
    using V = typename Mfma<In>::V;
    constexpr int kChunks = D / 8;                          // 16-byte pieces per X row
    constexpr int kPerWinX = (kMaxWin * kChunks + kThreads - 1) / kThreads;
    constexpr int kPer32X = (kRows * kChunks + kThreads - 1) / kThreads;
    constexpr int kCB = D / 16;
    constexpr int kBlocks = (kRows / 16) * kCB;            // 16x16 output blocks
    constexpr int kBPW = (kBlocks + kWaves - 1) / kWaves;  // blocks per wave
    static_assert(kBPW == 1 || kCB % kBPW == 0, "a wave's blocks must share a row group");

    extern __shared__ __align__(16) unsigned char lds[];
    ST* seg = reinterpret_cast<ST*>(lds);                   // [kMaxWin][kRss]
    ST* xt = reinterpret_cast<ST*>(lds + a.ring_off);       // XT[c][slot]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;
    const int ringc = a.ring;
    const ST* band_end = band + a.band_elems;
    const int blk0 = wave * kBPW;
    const bool wave_busy = blk0 < kBlocks;
    const int jb = blk0 / kCB;                              // this wave's 16-row group
    const int cb0 = blk0 % kCB;

    uint32_t item, iend;
    {
        uint32_t ub, ue;
        unit_range(a.dc, xcd_rank(blockIdx.x, a.nwg), &ub, &ue);
        item = ub * a.chunks.d;
        iend = ue * a.chunks.d;
    }
    for (int q = tid; q < D * ringc / 8; q += kThreads)
        reinterpret_cast<u32x4*>(xt)[q] = u32x4{0u, 0u, 0u, 0u};

    auto describe = [&](uint32_t id, Item* it) {
        const uint32_t unit = div32(a.chunks, id);
        const int kc = static_cast<int>(id - unit * a.chunks.d);
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

    // Segment of staging row xr (band row i = ilo + xr): slots [sa, sa + 32), sa = j0 - i + w,
    // of which [max(k0, sa), min(k0 + kbeff, sa + 32)) belong to the chunk.  Its 16-byte
    // pieces start at global element gs - sh, gs = (row0 + i * row_step) * K + sa.
    u32x4 sb[kSegPer];
    // Piece q of this thread: its global address and the element range [a0, b0) that
    // belongs to the chunk; false for pieces outside the window or the sequence.
    auto seg_geom = [&](const Item& it, int q, const ST** gp, int* a0, int* b0, int* xr_out) {
        const int idx = tid + q * kThreads;
        const int xr = idx / kSegPieces, pc = idx - xr * kSegPieces;
        *xr_out = xr;
        if (xr >= it.W) return false;
        const int i = it.ilo + xr;
        if (i < 0 || i >= it.n_r) return false;
        const int64_t sa = static_cast<int64_t>(it.j0) - i + a.w;
        const int64_t gs = (it.row0 + static_cast<int64_t>(i) * row_step) * K + sa;
        const int sh = static_cast<int>(gs & 7);
        const int64_t lo_slot = sa - sh + 8 * pc;          // slot of element 0
        const int64_t va = it.k0 > sa ? it.k0 : sa;
        const int64_t vb_ = (it.k0 + it.kbeff) < (sa + kRows) ? (it.k0 + it.kbeff) : (sa + kRows);
        const int64_t pa = va - lo_slot, pe = vb_ - lo_slot;   // valid [pa, pe)
        if (pe <= 0 || pa >= 8) return false;
        *gp = band + (gs - sh) + 8 * pc;
        *a0 = pa > 0 ? static_cast<int>(pa) : 0;
        *b0 = pe < 8 ? static_cast<int>(pe) : 8;
        return true;
    };
    // Prefetch whole pieces only; masking (and any piece that runs past the end of the
    // tensor) waits for store_seg, so the loads stay in flight during compute.
    auto load_seg = [&](const Item& it) {
#pragma unroll
        for (int q = 0; q < kSegPer; ++q) {
            const ST* gp = nullptr;
            int a0 = 0, b0 = 0, xr = 0;
            if (seg_geom(it, q, &gp, &a0, &b0, &xr) && gp + 8 <= band_end)
                sb[q] = *reinterpret_cast<const u32x4*>(gp);
        }
    };
    auto store_seg = [&](const Item& it) {
#pragma unroll
        for (int q = 0; q < kSegPer; ++q) {
            const ST* gp = nullptr;
            int a0 = 0, b0 = 0, xr = 0;
            u32x4 val = u32x4{0u, 0u, 0u, 0u};
            if (seg_geom(it, q, &gp, &a0, &b0, &xr)) {
                if (gp + 8 <= band_end) {
                    val = mask_piece<ST>(sb[q], a0, b0);
                } else {
                    const int lim = static_cast<int>(band_end - gp);
                    val = load_piece_elems<ST>(gp, a0, b0 < lim ? b0 : lim);
                }
            }
            const int pc = tid + q * kThreads - xr * kSegPieces;
            if (xr < it.W) *reinterpret_cast<u32x4*>(seg + xr * kRss + 8 * pc) = val;
        }
    };

    auto put_x = [&](int slot, int ch, const u32x4& pc) {
        const uint32_t d0 = pc[0], d1 = pc[1], d2 = pc[2], d3 = pc[3];
        uint16_t* base = reinterpret_cast<uint16_t*>(xt) + (ch * 8) * ringc + slot;
        base[0 * ringc] = static_cast<uint16_t>(d0);
        base[1 * ringc] = static_cast<uint16_t>(d0 >> 16);
        base[2 * ringc] = static_cast<uint16_t>(d1);
        base[3 * ringc] = static_cast<uint16_t>(d1 >> 16);
        base[4 * ringc] = static_cast<uint16_t>(d2);
        base[5 * ringc] = static_cast<uint16_t>(d2 >> 16);
        base[6 * ringc] = static_cast<uint16_t>(d3);
        base[7 * ringc] = static_cast<uint16_t>(d3 >> 16);
    };
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
    };
    u32x4 xb[kPer32X];
    auto load_new_x = [&](const Item& nx) {
#pragma unroll
        for (int q = 0; q < kPer32X; ++q) {
            const int idx = tid + q * kThreads, rr = idx / kChunks, ch = idx % kChunks;
            if (rr < kRows) xb[q] = get_x(nx, nx.W - kRows + rr, ch);
        }
    };
    auto store_new_x = [&](int slot_first) {
#pragma unroll
        for (int q = 0; q < kPer32X; ++q) {
            const int idx = tid + q * kThreads, rr = idx / kChunks, ch = idx % kChunks;
            if (rr < kRows) {
                int slot = slot_first + rr;
                slot = slot < ringc ? slot : slot - ringc;
                put_x(slot, ch, xb[q]);
            }
        }
    };

    f32x4 acc[kBPW];
#pragma unroll
    for (int q = 0; q < kBPW; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

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
            __syncthreads();
            if (!seg_ready) store_seg(it);
            if (!x_ready) {
                s0 = 0;
                fill_window(it);
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
            load_seg(nx);
            if (next_slides) load_new_x(nx);
        }

        // ---- compute: out^T[c][j] += sum_x XT[c][x] * B[x][j]
        if (wave_busy) {
            const int x_lo = 16 * jb, x_hi = 16 * jb + 15 + it.kbeff;
            const int ic_lo = x_lo / 32, ic_hi = (x_hi + 31) / 32;
            // shift of staging row xr: (gs mod 8) = (c0 + i * d1) mod 8 with i = ilo + xr
            const int64_t c0 = (it.row0 * K + it.j0 + a.w) & 7;
            const int64_t d1 = (row_step * K - 1) & 7;
            const int jcol = 16 * jb + col;                 // segment position j - j0
            for (int ic = ic_lo; ic < ic_hi; ++ic) {
                uint32_t bw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    uint32_t lohi = 0;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int xr = 32 * ic + 8 * grp + 2 * e2 + hf;
                        const int i = it.ilo + xr;
                        const int sh = static_cast<int>((c0 + static_cast<int64_t>(i) * d1) & 7);
                        const bool ok = xr < it.W;
                        const uint32_t val = ok ? static_cast<uint32_t>(__builtin_bit_cast(
                                                      uint16_t, seg[(ok ? xr : 0) * kRss + sh + jcol]))
                                                : 0u;
                        lohi |= val << (16 * hf);
                    }
                    bw[e2] = lohi;
                }
                const V bop = __builtin_bit_cast(V, u32x4{bw[0], bw[1], bw[2], bw[3]});
                int slot0 = s0 + 32 * ic + 8 * grp;
                slot0 = slot0 < ringc ? slot0 : slot0 - ringc;
#pragma unroll
                for (int q = 0; q < kBPW; ++q) {
                    const int c = 16 * (cb0 + q) + col;
                    const V aop = *reinterpret_cast<const V*>(xt + c * ringc + slot0);
                    acc[q] = Mfma<In>::run(aop, bop, acc[q]);
                }
            }
        }

        const bool tile_done = it.t.kb == a.g.nkb - 1;
        if (tile_done) {
            const int jl = 16 * jb + col;
            if (wave_busy && jl < it.rows_here) {
                const int64_t orow = (it.row0 + static_cast<int64_t>(it.j0 + jl) * row_step) * D;
#pragma unroll
                for (int q = 0; q < kBPW; ++q) {
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
            for (int q = 0; q < kBPW; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        __syncthreads();
        if (has_next) {
            store_seg(nx);
            if (next_slides) {
                store_new_x(s0 + it.W);
                s0 += kRows;
                s0 = s0 < ringc ? s0 : s0 - ringc;
            }
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
    const int64_t need = 2 * kRows + kc - 1;               // window + 32 prefetched rows
    l.ring = ceil_div(need - 8, 128) * 128 + 8;             // = 8 mod 128
    l.ring_off = ceil_div((kRows + kc - 1) * kRss * 2, 16) * 16;
    l.bytes = l.ring_off + d * l.ring * 2;
    return l;
}

// Units are whole tiles (all chunks of one row block), decoded with one chunk per tile.
TileDecode unit_decode(const PvTilePlan& tp, const Problem& p) {
    const TileGrid& g = tp.grid;
    const int64_t units = g.tiles / g.nkb;
    return make_decode(TileGrid{g.res, g.rb, 1, g.kb, units}, p.h, p.n, p.s, units,
                       tp.workgroups);
}

template <class In, int D>
hipError_t launch_typed(const void* band, const void* x, void* out, bool out_f32,
                        const Problem& p, const PvTilePlan& tp, hipStream_t stream) {
    const PvTLayout l = pvt_layout(tp.grid.kb, D);
    PvTArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.ring),
              static_cast<int32_t>(l.ring_off), static_cast<uint32_t>(tp.workgroups),
              p.rows() * p.h * p.K, unit_decode(tp, p),
              make_div32(static_cast<uint32_t>(tp.grid.nkb))};
    auto kern = pvt_mfma_kernel<In, D>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        static_cast<int>(kPvLdsBytes));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(tp.workgroups)), dim3(kThreads),
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
