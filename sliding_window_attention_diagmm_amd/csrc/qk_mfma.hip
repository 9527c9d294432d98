// diagmm_qk on MFMA with persistent, sliding workgroups, storing straight from registers.
//
// Tiles.  A tile is M = 64 consecutive rows t0..t0+63 of one residue class of one
// (batch, head) and a block of KB consecutive slots k0..k0+KB-1 (KB <= 513, fixed per
// call by the LDS budget).  Its slots reach the W = M + KB - 1 consecutive keys
// u0 = t0 + k0 - w .. u0 + W - 1 of the class ("window columns" x = 0 .. W-1; row il of
// the tile holds its slots at columns il .. il + KB - 1).  Tiles are numbered with the
// row block fastest, so consecutive tiles of one strip slide down the class by 64 rows
// and share all but 64 of their keys.
//
// Workgroups.  One 512-thread workgroup per compute unit walks a contiguous range of
// tile ids.  It keeps the key window of the current tile in an LDS ring (rows swizzled by
// 16-byte chunk) and the query tile in one of two LDS buffers; a tile that continues a
// strip only brings in 64 new key rows and its 64 query rows, fetched into registers at
// the start of the previous tile and written to LDS at its end.
//
// Compute.  Wave (rb, half) owns query rows 16 rb .. 16 rb + 15 (B operand, held in
// registers) and sweeps half of the 16-key column blocks jb these rows reach, computing
// the transposed product on v_mfma_f32_16x16x32_{f16,bf16}:
//
//   acc(jb)[j][i] = sum_c K[u0 + 16 jb + j][c] * Q[t0 + 16 rb + i][c]
//
// Lane (i = lane % 16, g = lane / 16) holds columns 16 jb + 4 g .. +3 of row 16 rb + i,
// i.e. four consecutive band slots.  Slots whose key lies outside the sequence take the
// padding constant; results are rounded to the output type (nearest even).
//
// Store.  Rows of the band are not 16-byte aligned in HBM (row r starts at r K), and
// misaligned stores run at half the bandwidth of aligned ones, so every lane builds one
// aligned 16-byte piece per step: for 16-bit outputs two column blocks are combined with
// v_permlane16_swap so that each lane holds 8 consecutive columns (lane groups 0, 2, 1, 3
// in column order), the 8 columns before them are fetched from the lane that holds them
// with ds_bpermute (across steps through a carry register), and a per-row funnel shift
// (the row's misalignment) cuts out the aligned piece.  For f32 outputs each block
// already gives 4 columns = 16 bytes per lane.  Pieces at the two ends of a row, shared
// with the neighbouring band row in HBM, are written element by element.  The two waves
// of a row block split its steps; the second recomputes the step before its first so
// that its carry is filled.  No LDS staging: stores leave during compute.
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

struct QkArgs {
    int64_t n, h, K, w, s;
    TileGrid g;
    int32_t ring;      // key rows in the LDS ring (2 * kRows + KB - 1, rounded up to 16)
    int32_t q_off;     // LDS byte offset of the two query tiles
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

__device__ __forceinline__ uint32_t pick(bool c, uint32_t a, uint32_t b) { return c ? a : b; }

// Aligned piece from the 8 dwords E = p0..p3, o0..o3 (16-bit elements): elements
// s .. s+7 of E with s = 8 - d, d in [0, 8).  Dword rotation by s / 2 (three select
// stages), then a 16-bit funnel shift when s is odd.
__device__ __forceinline__ u32x4 funnel16(const u32x4& p, const u32x4& o, int d) {
    const int s = 8 - d;
    const int qd = s >> 1;
    const bool b0 = qd & 1, b1 = qd & 2, b2 = qd & 4;
    const uint32_t e0 = p[0], e1 = p[1], e2 = p[2], e3 = p[3];
    const uint32_t e4 = o[0], e5 = o[1], e6 = o[2], e7 = o[3];
    const uint32_t g0 = pick(b0, e1, e0), g1 = pick(b0, e2, e1), g2 = pick(b0, e3, e2);
    const uint32_t g3 = pick(b0, e4, e3), g4 = pick(b0, e5, e4), g5 = pick(b0, e6, e5);
    const uint32_t g6 = pick(b0, e7, e6);
    const uint32_t h0 = pick(b1, g2, g0), h1 = pick(b1, g3, g1), h2 = pick(b1, g4, g2);
    const uint32_t h3 = pick(b1, g5, g3), h4 = pick(b1, g6, g4);
    const uint32_t f0 = pick(b2, e4, h0), f1 = pick(b2, e5, h1), f2 = pick(b2, e6, h2);
    const uint32_t f3 = pick(b2, e7, h3), f4 = pick(b2, 0u, h4);
    const uint32_t sh = (s & 1) ? 16u : 0u;
    return u32x4{__builtin_amdgcn_alignbit(f1, f0, sh), __builtin_amdgcn_alignbit(f2, f1, sh),
                 __builtin_amdgcn_alignbit(f3, f2, sh), __builtin_amdgcn_alignbit(f4, f3, sh)};
}

// The same for 32-bit elements: dwords s .. s+3 of E with s = 4 - d, d in [0, 4).
__device__ __forceinline__ u32x4 funnel32(const u32x4& p, const u32x4& o, int d) {
    const int s = 4 - d;
    const bool b0 = s & 1, b1 = s & 2, b2 = s & 4;
    const uint32_t e0 = p[0], e1 = p[1], e2 = p[2], e3 = p[3];
    const uint32_t e4 = o[0], e5 = o[1], e6 = o[2], e7 = o[3];
    const uint32_t g0 = pick(b0, e1, e0), g1 = pick(b0, e2, e1), g2 = pick(b0, e3, e2);
    const uint32_t g3 = pick(b0, e4, e3), g4 = pick(b0, e5, e4), g5 = pick(b0, e6, e5);
    const uint32_t h0 = pick(b1, g2, g0), h1 = pick(b1, g3, g1), h2 = pick(b1, g4, g2);
    const uint32_t h3 = pick(b1, g5, g3);
    return u32x4{pick(b2, e4, h0), pick(b2, e5, h1), pick(b2, e6, h2), pick(b2, e7, h3)};
}

__device__ __forceinline__ u32x4 bperm4(int addr, const u32x4& v) {
    return u32x4{static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(v[0]))),
                 static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(v[1]))),
                 static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(v[2]))),
                 static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(v[3])))};
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
    constexpr int kRowChunks = kRows * kChunks;           // chunks of a 64-row block
    constexpr int kPer64 = (kRowChunks + kThreads - 1) / kThreads;
    constexpr int kPerWin = (kMaxWindow * kChunks + kThreads - 1) / kThreads;
    constexpr int kQBytes = kRows * D * 2;

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* ring = lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int rb = wave >> 1, half = wave & 1;            // row block, half of its steps
    const int il = 16 * rb + col;                         // this lane's tile row
    const int64_t n = a.n, h = a.h, K = a.K, s = a.s;
    const int64_t row_step = s * h;                       // [b][n][h] rows per class row
    const int64_t gstep = row_step * K;                   // band elements per class row
    const int ringc = a.ring;
    const P padv = Pack<Out>::splat(a.pad);
    // Source lane of the 8 (4) columns before this lane's own, in ds_bpermute bytes:
    // 16-bit outputs hold columns in lane groups 0, 2, 1, 3; f32 in groups 0, 1, 2, 3.
    const int src_lane = k16 ? lane + (grp == 0 ? 48 : (grp == 1 ? 16 : -32))
                             : (grp == 0 ? lane + 48 : lane - 16);
    const int src_addr = src_lane * 4;
    const int off_g = k16 ? (grp == 1 ? 16 : (grp == 2 ? 8 : (grp == 3 ? 24 : 0))) : 4 * grp;

    uint32_t tile, tend;
    unit_range(a.dc, xcd_rank(blockIdx.x, a.nwg), &tile, &tend);

    // Registers carrying the next tile's new key rows and query rows.
    u32x4 kn[kPer64], qn[kPer64];
    bool prefetched = false;
    int s0 = 0;                     // ring slot of the current window's first key
    int qsel = 0;                   // query buffer of the current tile

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

        // B operands: this wave's 16 query rows.
        V qf[kDC];
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc)
            qf[dc] = *reinterpret_cast<const V*>(qlds + swz<D>(il, 4 * dc + grp));

        // Row il of the tile: global element of window column 0 (slot x - il sits at
        // rowA + x) and its misalignment against 16-byte pieces.
        const int64_t rowA = (row0 + static_cast<int64_t>(t0) * row_step) * K + k0 +
                             static_cast<int64_t>(il) * (gstep - 1);
        const int dsh = static_cast<int>(rowA & (kVec - 1));
        const bool row_ok = il < rows_here;
        const bool key_edge = u0 < 0 || u0 + W > n_r;     // window touches a sequence end

        // One 16-key column block: four consecutive columns of row il per lane; its key
        // fragments are read (fetch), multiplied (mma) and rounded (pack) in separate
        // steps so that the loop below can overlap them across blocks.
        // The ring holds a multiple of 16 key rows and windows start at multiples of 64,
        // so block jb starts at ring row (s0 + 16 jb) mod ringc, a multiple of 16, and the
        // swizzle of its row col depends on col alone: swz(16 m + col, c) = 16 m * 2D +
        // swz(col, c).
        auto fetch = [&](int jb, V* kf) {
            int base = s0 + 16 * jb;
            base = base < ringc ? base : base - ringc;
            const unsigned char* rp = ring + base * (2 * D);
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc)
                kf[dc] = *reinterpret_cast<const V*>(rp + swz<D>(col, 4 * dc + grp));
        };
        auto mma = [&](const V* kf) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc) acc = Mfma<In>::run(kf[dc], qf[dc], acc);
            return acc;
        };
        auto pack = [&](int jb, const f32x4& acc) {
            P val = Pack<Out>::run(acc);
            if (key_edge) {
                // keys of this lane's four columns: u0 + 16 jb + 4 grp + v
                const int ukey = u0 + 16 * jb + 4 * grp;
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

        // Steps: pairs of blocks (16-bit) or single blocks (f32) from block rb on, enough
        // to cover the last piece of every row (its first column is at most 7 (3) past
        // the row's last column il + kbeff - 1 <= 16 rb + 14 + kbeff).
        constexpr int kBPS = k16 ? 2 : 1;                 // blocks per step
        constexpr int kOffMax = k16 ? 24 : 12;            // largest column offset of a lane
        const int full_max = kbeff - kVec;                // last slot0 of a whole piece
        const int nblk = (14 + kVec - 1 + kbeff) / 16 + 1;
        const int nsteps = (nblk + kBPS - 1) / kBPS;
        const int mid = (nsteps + 1) / 2;
        const int st_lo = half ? mid : 0, st_hi = half ? nsteps : mid;
        const int st_first = half && mid > 0 ? mid - 1 : st_lo;   // warm-up step first
        u32x4 carry = u32x4{0u, 0u, 0u, 0u};

        // Step st with its accumulators: round, gather 8 (4) consecutive columns per lane,
        // fetch the preceding ones, cut out the aligned piece and store it.
        auto finish = [&](int st, const f32x4* acc) {
            const int jb = rb + kBPS * st;
            u32x4 own;
            if constexpr (k16) {
                const P va = pack(jb, acc[0]), vb = pack(jb + 1, acc[1]);
                const auto sx = __builtin_amdgcn_permlane16_swap(va[0], vb[0], false, false);
                const auto sy = __builtin_amdgcn_permlane16_swap(va[1], vb[1], false, false);
                own = u32x4{sx[0], sy[0], sx[1], sy[1]};
            } else {
                own = pack(jb, acc[0]);
            }
            const int x0 = 16 * jb + off_g;                // first column of `own`
            const u32x4 provide = grp == 3 ? carry : own;
            const u32x4 pred = bperm4(src_addr, provide);
            carry = own;
            return [=](bool store) {
                if (!store) return;                        // warm-up step: carry only
                const u32x4 o = k16 ? funnel16(pred, own, dsh) : funnel32(pred, own, dsh);
                const int c0 = x0 - dsh;                   // first column of the piece
                const int slot0 = c0 - il;                 // = slot_base + 16 kBPS st
                OT* gp = band + (rowA + c0);               // 16-byte aligned
                // whole piece inside the row's slots: 0 <= slot0 <= kbeff - kVec (no such
                // piece when kbeff < kVec)
                if (row_ok && full_max >= 0 &&
                    static_cast<unsigned>(slot0) <= static_cast<unsigned>(full_max))
                    *reinterpret_cast<u32x4*>(gp) = o;
                // A piece that holds both slots of the row and others can only lie at its
                // ends: slot0 >= 16 kBPS st - 22 and slot0 <= 16 kBPS st + kOffMax, so
                // steps in between skip this wave-uniform branch.
                const int sst = 16 * kBPS * st;
                if (sst < 22 || sst + kOffMax + kVec > kbeff) {
                    const bool part = row_ok && slot0 < kbeff && slot0 + kVec > 0 &&
                                      !(slot0 >= 0 && slot0 + kVec <= kbeff);
                    if (part) {
                        const int pa = slot0 < 0 ? -slot0 : 0;
                        const int pe = kbeff - slot0 < kVec ? kbeff - slot0 : kVec;
                        store_part<OT>(gp, o[0], o[1], o[2], o[3], pa, pe);
                    }
                }
            };
        };

        // Software pipeline: the MFMAs of step st + 1 and the key fragment reads of step
        // st + 2 are issued before step st is finished.  The scheduling barriers keep that
        // order; the empty asm with a memory clobber keeps the compiler from folding the
        // loop-carried fragment reads back into reads at their use.
        if (st_first < st_hi) {
            V kf[kBPS][kDC];
            f32x4 acc_cur[kBPS], acc_nx[kBPS];
#pragma unroll
            for (int bq = 0; bq < kBPS; ++bq) fetch(rb + kBPS * st_first + bq, kf[bq]);
#pragma unroll
            for (int bq = 0; bq < kBPS; ++bq) acc_cur[bq] = mma(kf[bq]);
            if (st_first + 1 < st_hi) {
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) fetch(rb + kBPS * (st_first + 1) + bq, kf[bq]);
            }
            for (int st = st_first; st < st_hi; ++st) {
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                if (st + 1 < st_hi) {
#pragma unroll
                    for (int bq = 0; bq < kBPS; ++bq) acc_nx[bq] = mma(kf[bq]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // before the lane exchange: LDS results return in order, so waiting for
                // the exchange then costs no extra wait for these reads
                if (st + 2 < st_hi) {
#pragma unroll
                    for (int bq = 0; bq < kBPS; ++bq) fetch(rb + kBPS * (st + 2) + bq, kf[bq]);
                }
                __builtin_amdgcn_sched_barrier(0);
                auto tail = finish(st, acc_cur);
                __builtin_amdgcn_sched_barrier(0);
                tail(st >= st_lo);
#pragma unroll
                for (int bq = 0; bq < kBPS; ++bq) acc_cur[bq] = acc_nx[bq];
            }
        }

        // The next tile's new key rows go to ring slots outside the current window (only
        // columns no row stores are read there), its query rows to the other buffer.
        if (next) {
            unsigned char* qnext = lds + a.q_off + (qsel ^ 1) * kQBytes;
#pragma unroll
            for (int x = 0; x < kPer64; ++x) {
                const int idx = tid + x * kThreads, rr = idx / kChunks, ch = idx % kChunks;
                if (idx < kRowChunks) {
                    int slot = s0 + W + rr;
                    slot = slot < ringc ? slot : slot - ringc;
                    *reinterpret_cast<u32x4*>(ring + swz<D>(slot, ch)) = kn[x];
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
    int64_t kb = 0, ring = 0, q_off = 0, bytes = 0;
};

// LDS layout for a slot block of kb slots: the key ring, then two query tiles.
Layout layout_for(int64_t kb, int64_t d) {
    Layout l;
    l.kb = kb;
    l.ring = ceil_div(2 * kRows + kb - 1, 16) * 16;
    l.q_off = ceil_div(l.ring * d * 2, 16) * 16;
    l.bytes = l.q_off + 2 * kRows * d * 2;
    return l;
}

template <class In, class Out, int D>
hipError_t launch_typed(const void* q, const void* k, void* band, const Problem& p,
                        const QkTilePlan& tp, uint32_t pad, hipStream_t stream) {
    const Layout l = layout_for(tp.grid.kb, D);
    QkArgs a{p.n, p.h, p.K, p.w, p.s, tp.grid, static_cast<int32_t>(l.ring),
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
    // The widest slot block (at most 513) whose ring + query tiles fit in LDS.
    (void)out_dt;
    int64_t max_slots = kMaxSlots;
    while (max_slots > 16 && layout_for(max_slots, p.d).bytes > kQkLdsBytes) --max_slots;
    tp.grid = make_grid(p.b, p.n, p.h, p.K, p.s, kRows, max_slots);
    const Layout l = layout_for(tp.grid.kb, p.d);
    tp.rs = 0;
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
