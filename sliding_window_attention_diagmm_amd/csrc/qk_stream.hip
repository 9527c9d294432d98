// diagmm_qk on MFMA, streaming: balanced row ranges, keys streamed into an LDS window,
// band rows written straight from registers as aligned 16-byte pieces.
//
// Work split.  The rows of every strip - one residue class of one (batch, head), an
// undilated band problem on its own - are cut into g ranges of at most 208 consecutive
// class rows (g equal for all strips, so that a range id decodes with two divisions), and
// every workgroup (one per compute unit) takes one range, or a contiguous run of ranges
// when there are more ranges than units.  At n = 4096, h = 12 that is 21 ranges of ~195
// rows per head: every unit stores the same number of band bytes, and every range needs
// one key window, its rows plus the K - 1 keys around them.
//
// Offset classes.  Band rows are 2-byte aligned in HBM.  Row i of a range sits i row
// strides past the first, and column x of row i (slot x - i) at byte
// B0 + i (RB - 2) + 2 x, RB being the row stride in bytes; for the rows i = c + 8 t of one
// class c (RB even) that is B0 + c (RB - 2) + 2 x mod 16 whatever t is.  Compute wave c
// owns those rows: its 16-byte pieces start at the columns x = o_c mod 8 that make the
// address a multiple of 16, so every store of a piece inside a row is one aligned
// 16-byte write.
//
// Compute.  Wave c holds its (up to 26) query rows as two MFMA B operands in registers
// and sweeps the key columns x in steps of four 16-key blocks: for each block,
// v_mfma_f32_16x16x32_{f16,bf16} gives acc[key][query] with A = 16 keys read from the
// window.  Lane (query q, group g) then holds 4 consecutive columns of row q; two blocks
// combined with v_permlane16_swap give each lane 8 consecutive columns, one aligned
// 16-byte piece, which is stored to HBM at once.  A row's first and last piece are shared
// with the neighbouring band rows in HBM: they are kept in LDS and written element by
// element, for the row's own slots only, at the end of the range.  Keys outside the
// sequence take the padding constant; values are rounded to nearest even.
//
// Long rows.  Each step's 64 columns of a row are 128 bytes at the row's 16-byte phase, so
// they end in the middle of a 128-byte line that the next step completes.  With rows of
// more than 1000 slots the L2 no longer keeps such half-written lines until then, and they
// go to HBM twice.  There the kernel trades pieces between lane halves and holds the ones
// past the row's line boundary for one step, so that every store writes whole aligned
// lines; it also numbers the ranges head-fastest (the same rows of neighbouring heads,
// adjacent in memory, run together) and, with more ranges than workgroups, deals each
// XCD's ranges round-robin over its workgroups.  Bands larger than the Infinity Cache
// (256 MB) are stored with the non-temporal hint: no later kernel would find them cached,
// and streamed out they no longer hold the L2 until the end of the launch.
//
// Keys.  Four loader waves stream the range's key window through a ring of 1024 key
// rows (16 chunks of 64 keys, plus a copy of the chunk in ring slot 0 past slot 15, so
// that a step's 128 rows are always contiguous), up to four chunks in flight.  Each ring
// slot counts the loader waves that have written their part into it (four per chunk), and
// each compute wave, where the window is longer than the ring, the steps it has finished;
// a compute wave starts step j when slot (j + 1) mod 16 has counted chunk j + 1 in full,
// and a loader wave writes chunk c >= 16 only once every compute wave has finished step
// c - 16, the last to read the chunk c replaces (a window of up to 16 chunks never waits).
// No barrier inside a range; the waits are bounded.  Compute waves only store while
// loader waves only load (a wave's vector memory counter covers its loads and stores
// alike, in issue order, so mixing them would make loads wait behind stores).
#include <cstdlib>
#include <cstring>
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

template <class In> struct Mm;
template <> struct Mm<F16> {
    using V = f16x8;
    __device__ __forceinline__ static f32x4 run(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static u32x2 pack(f32x4 a) {
        return __builtin_bit_cast(u32x2, __builtin_convertvector(a, f16x4));
    }
};
template <> struct Mm<BF16> {
    using V = bf16x8;
    __device__ __forceinline__ static f32x4 run(V a, V b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static u32x2 pack(f32x4 a) {
        return __builtin_bit_cast(u32x2, __builtin_convertvector(a, bf16x4));
    }
};

constexpr int kComputeWaves = 8;                 // one per offset class
constexpr int kLoadWaves = 4;
constexpr int kThreads = (kComputeWaves + kLoadWaves) * 64;
constexpr int kLoadThreads = kLoadWaves * 64;
constexpr int kClassRows = 26;                   // rows of one class in a range, at most
constexpr int kMaxRange = 8 * kClassRows;        // 208 class rows per range
constexpr int kStep = 64;                        // key columns per step = keys per chunk
constexpr int kPartRows = 32;                   // rows t of a class: two query sets of 16
constexpr int kRingChunks = 16;                  // key chunks the LDS ring holds
constexpr int kRingRows = kRingChunks * kStep;   // 1024 key rows (+ 64 mirrored)
constexpr uint32_t kAllDone = 1u << 30;          // a compute wave's count once it is done
constexpr int kLdsBytes = 160 * 1024;
constexpr int kBufWord3 = 0x00020000;            // raw 32-bit buffer access (gfx9 word 3)
constexpr int kBufDrop = static_cast<int>(0x80000000u);   // offset past every range
constexpr int kPolNt = 2;                        // buffer store cache policy: non-temporal

// LDS: the key ring, the compute waves' head and tail pieces, and the progress counters
// (one per ring slot, one per compute wave).
__host__ __device__ constexpr int win_bytes(int d) { return (kRingRows + kStep) * d * 2; }
// A row's head and tail pieces (shared with the neighbouring band rows in HBM) are kept
// aside during the sweep and written element by element at the end of the range.
constexpr int kPartWave = kPartRows * 2 * 16;
__host__ __device__ constexpr int lds_bytes(int d) {
    return win_bytes(d) + kComputeWaves * kPartWave + (kRingChunks + kComputeWaves) * 4;
}
static_assert(lds_bytes(64) <= kLdsBytes, "LDS budget");

struct StreamArgs {
    int64_t n, h, K, w, s;
    int32_t res;        // residue classes enumerated
    int32_t g;          // ranges per strip
    int32_t nwg;        // workgroups launched
    int32_t rq, rrem;   // ranges per workgroup: rq, and one more for the first rrem ranks
    int32_t nq, nm;     // n = nq s + nm: class r has nq + (r < nm) rows
    uint32_t pad;       // padding constant in the output type
    int32_t order;      // range ids: 0 strip-major (a strip's parts consecutive), 1 head-fastest
    int32_t interleave; // ranges dealt round-robin over each XCD's workgroups
};

// Window offset of (key row, 16-byte chunk): chunks XOR-swizzled by the row, so that
// eight consecutive rows read at one logical chunk hit eight distinct 16-byte bank groups.
// The swizzle depends on the row mod 8 only.
template <int D>
__device__ __forceinline__ int ring_off(int row, int chunk) {
    constexpr int kShift = D == 32 ? 1 : 0;
    constexpr int kMask = D == 32 ? 3 : 7;
    return row * (D * 2) + ((chunk ^ ((row >> kShift) & kMask)) << 4);
}

template <class In, int D, bool kLines, int kPol>
__global__ void __launch_bounds__(kThreads)
qk_stream_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ kx,
                 typename In::T* __restrict__ band, StreamArgs a) {
    using V = typename Mm<In>::V;
    constexpr int kDC = D / 32;                  // MFMA depth steps
    constexpr int kChunks = D / 8;               // 16-byte chunks per key row
    constexpr int kRowBytes = D * 2;
    constexpr int kPer = 64 * kChunks / kLoadThreads;   // chunks per loader thread per step
    static_assert(kPer >= 1 && 64 * kChunks % kLoadThreads == 0, "loader split");
    constexpr int kSets = 6;                     // loader register sets (see below)

    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* const win = lds;
    unsigned char* const part_all = lds + win_bytes(D);
    uint32_t* const ready = reinterpret_cast<uint32_t*>(part_all + kComputeWaves * kPartWave);
    uint32_t* const done = ready + kRingChunks;

    // Every argument is read here, before the first branch, so that the argument block
    // arrives in one round trip rather than one per use site.
    asm volatile("" ::"s"(q), "s"(kx), "s"(band), "s"(a.n), "s"(a.h), "s"(a.K), "s"(a.w),
                 "s"(a.s), "s"(a.res), "s"(a.g), "s"(a.nwg), "s"(a.rq), "s"(a.rrem), "s"(a.nq),
                 "s"(a.nm), "s"(a.pad));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool computes = wave < kComputeWaves;
    const int64_t n = a.n, h = a.h, s = a.s;
    const int K = static_cast<int>(a.K);
    const int64_t row_elems = s * h * a.K;       // band elements between class rows
    const int RB = static_cast<int>(row_elems * 2);     // band bytes between class rows
    const int qk_bytes = static_cast<int>(s * h * D * 2);   // q / k bytes between class rows

    // This workgroup's ranges rfirst + m rstride, m < rcount: a contiguous run, or (with
    // more ranges than workgroups, on the line path) each XCD's share of the ids dealt
    // round-robin over its workgroups, so that the XCD works on consecutive ids at once.
    const uint32_t nwg = static_cast<uint32_t>(a.nwg);
    const uint32_t rq = static_cast<uint32_t>(a.rq), rrem = static_cast<uint32_t>(a.rrem);
    uint32_t rfirst, rcount, rstride;
    if (a.interleave) {
        const uint32_t ranges = rq * nwg + rrem, per = nwg / kXcds;
        const uint32_t x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
        const uint32_t lo = static_cast<uint32_t>(uint64_t(ranges) * x / kXcds);
        const uint32_t hi = static_cast<uint32_t>(uint64_t(ranges) * (x + 1) / kXcds);
        rfirst = lo + j;
        rcount = rfirst < hi ? (hi - rfirst + per - 1) / per : 0u;
        rstride = per;
    } else {
        const uint32_t rank = xcd_rank(blockIdx.x, nwg);
        rfirst = rank * rq + (rank < rrem ? rank : rrem);
        rcount = rq + (rank < rrem ? 1u : 0u);
        rstride = 1;
    }

    if (tid < kRingChunks + kComputeWaves) ready[tid] = 0u;
    __syncthreads();
    // Bounded waits on the progress counters: a wait that never ends gives up after ~2^22
    // polls rather than hang.
    auto wait_min = [&](const uint32_t* cnt, int m, uint32_t need) {
        for (int it = 0; it < (1 << 22); ++it) {
            uint32_t lo = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            for (int i = 1; i < m; ++i) {
                const uint32_t v =
                    __hip_atomic_load(cnt + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                lo = v < lo ? v : lo;
            }
            if (lo >= need) break;
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    };

    for (uint32_t m = 0; m < rcount; ++m) {
        const uint32_t rg = rfirst + m * rstride;
        // Range rg: strip sigma = rg / g (batch, head, class), part j of g.
        const uint32_t g = static_cast<uint32_t>(a.g);
        const uint32_t res = static_cast<uint32_t>(a.res), h32 = static_cast<uint32_t>(h);
        uint32_t jpart, r, hh, bb;
        if (a.order == 0) {                          // strip (batch, head, class) major
            const uint32_t sigma = rg / g, bh = sigma / res;
            jpart = rg - sigma * g;
            r = sigma - bh * res;
            hh = bh % h32;
            bb = bh / h32;
        } else {                                     // head fastest, then part, class, batch
            const uint32_t rest = rg / h32, rest2 = rest / g;
            hh = rg - rest * h32;
            jpart = rest - rest2 * g;
            r = rest2 % res;
            bb = rest2 / res;
        }
        const int n_r = a.nq + (static_cast<int>(r) < a.nm ? 1 : 0);
        const int qr = n_r / static_cast<int>(g), mr = n_r - qr * static_cast<int>(g);
        const int jp = static_cast<int>(jpart);
        const int t_lo = jp * qr + (jp < mr ? jp : mr);
        const int L = qr + (jp < mr ? 1 : 0);
        const int U0 = t_lo - static_cast<int>(a.w);       // key of column x = 0
        const int64_t strip0 = (static_cast<int64_t>(bb) * n + r) * h + hh;
        const typename In::T* qs = q + strip0 * D;
        const typename In::T* ks = kx + strip0 * D;
        typename In::T* bs = band + (strip0 + static_cast<int64_t>(t_lo) * s * h) * a.K;
        const int nr_max = L > 0 ? (L + 7) / 8 : 0;
        // Steps: every class sweeps from at most 7 columns before its first row to the end
        // of its last row; the widest class (class 0) bounds them all.  Step j reads key
        // chunks j and j + 1 (window rows 64 j .. 64 j + 127, i.e. keys U0 - 8 + row), which
        // sit in ring rows 64 (j mod 16) .. + 127 (past row 1023: the copy of slot 0).
        const int S = nr_max > 0 ? (8 * (nr_max - 1) + K + 7 + kStep - 1) / kStep : 0;
        if (S == 0) continue;
        const int C = S + 1;                                 // chunks of the window

        if (!computes) {
            // ---------------------------------------------------------------- loaders
            // Chunk c = keys U0 - 8 + 64 c .. + 63 into ring rows 64 (c mod 16) ..; a loader
            // wave writes its part of chunk c once every compute wave has finished step
            // c - 16 (chunks past the ring's first fill only), then counts it.  Chunks go in
            // order.
            const int lt = tid - kComputeWaves * 64;
            const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<typename In::T*>(ks), 0, n_r * qk_bytes, kBufWord3);
            int prow[kPer], poff[kPer];
#pragma unroll
            for (int p = 0; p < kPer; ++p) {
                const int pi = lt + kLoadThreads * p;
                prow[p] = pi / kChunks;
                poff[p] = ring_off<D>(prow[p], pi % kChunks);   // swizzle: row mod 8 only
            }
            const int chunk_byte = (lt % kChunks) * 16;
            auto load = [&](int chunk, u32x4* buf) {
                chunk = chunk < C ? chunk : C - 1;           // past the end: reload the last
#pragma unroll
                for (int p = 0; p < kPer; ++p) {
                    int u = U0 - 8 + chunk * kStep + prow[p];
                    u = u < 0 ? 0 : (u >= n_r ? n_r - 1 : u);
                    buf[p] = __builtin_amdgcn_raw_buffer_load_b128(krs, u * qk_bytes + chunk_byte,
                                                                   0, 0);
                }
            };
            auto put = [&](int chunk, const u32x4* buf) {
                if (chunk >= C) return;
                if (chunk >= kRingChunks)
                    wait_min(done, kComputeWaves, static_cast<uint32_t>(chunk - kRingChunks + 1));
                unsigned char* const base = win + (chunk & (kRingChunks - 1)) * kStep * kRowBytes;
#pragma unroll
                for (int p = 0; p < kPer; ++p) *reinterpret_cast<u32x4*>(base + poff[p]) = buf[p];
                if (chunk >= kRingChunks && (chunk & (kRingChunks - 1)) == 0) {
                    // slot 0's copy past slot 15, read by the steps that cross the ring's end
#pragma unroll
                    for (int p = 0; p < kPer; ++p)
                        *reinterpret_cast<u32x4*>(win + kRingRows * kRowBytes + poff[p]) = buf[p];
                }
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the writes are done
                if (lane == 0)
                    __hip_atomic_fetch_add(ready + (chunk & (kRingChunks - 1)), 1u,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            };
            // Register sets in rotation (chunk c in set c mod kSets).  Chunks 0 and 1 are
            // requested alone, so that they are not queued behind the rest of the window at
            // the start, when every unit loads at once; then four chunks stay in flight:
            // chunk c is written as soon as it arrives and chunk c + 4 requested.
            static_assert(kSets == 6, "rotation below");
            u32x4 buf[kSets][kPer];
            load(0, buf[0]);
            load(1, buf[1]);
            put(0, buf[0]);
            load(2, buf[2]);
            load(3, buf[3]);
            put(1, buf[1]);
            load(4, buf[4]);
            load(5, buf[5]);
            for (int c0 = 2; c0 < C; c0 += kSets) {
#pragma unroll
                for (int u = 0; u < kSets; ++u) {
                    put(c0 + u, buf[(u + 2) % kSets]);
                    load(c0 + u + 4, buf[u]);            // (c0 + u + 4) mod 6 = u
                }
            }
            wait_vmem_all();
        } else {
            // ------------------------------------------------------------------- compute
            const int c = wave;
            const int nr = L > c ? (L - c + 7) / 8 : 0;      // rows t = 0 .. nr - 1
            // Alignment origin o: pieces at columns x = o (mod 8) are 16-byte aligned in HBM.
            const int bmod = static_cast<int>(reinterpret_cast<uintptr_t>(bs) & 15);
            const int o = ((-(bmod + c * ((RB - 2) & 15))) & 15) >> 1;
            const int xs = c - ((c - o) & 7);                // first swept column
            const int xe = c + 8 * (nr - 1) + K;             // past the last row's end
            const int J = nr > 0 ? (xe - xs + kStep - 1) / kStep : 0;

            const int col = lane & 15, grp = lane >> 4;
            // B operands: rows t = col (set 0) and 16 + col (set 1) of this class.
            V qf[2][kDC];
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2) {
                const int t = 16 * b2 + col;
                // rows past this class's share read the range's first row (never stored)
                const int64_t qrow = t < nr ? t_lo + c + 8 * t : t_lo;
                const typename In::T* qp = qs + qrow * (s * h * D);
#pragma unroll
                for (int dc = 0; dc < kDC; ++dc)
                    qf[b2][dc] = *reinterpret_cast<const V*>(qp + 8 * (4 * dc + grp));
            }
            const bool ok0 = col < nr, ok1 = 16 + col < nr;
            // Lane group grp holds, after pairing, columns 8 sj .. 8 sj + 7 of a block pair.
            const int sj = ((grp & 1) << 1) | (grp >> 1);
            const uint32_t padw = (a.pad & 0xffffu) | (a.pad << 16);
            // A operands: this lane reads ring row r0 + col of a block whose first row is
            // r0 = xs + 8 (mod 8), so the swizzle of its row is fixed (row mod 8) and only
            // the block's first row moves.
            int aoff[kDC];
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc)
                aoff[dc] = ring_off<D>(((xs + 8) & 7) + col, 4 * dc + grp) -
                           (((xs + 8) & 7) * kRowBytes);

            // Store resource: this range's rows, num_records covering exactly its band bytes.
            const int span = ((L - 1) * RB) + 2 * K;
            const __amdgpu_buffer_rsrc_t brs =
                __builtin_amdgcn_make_buffer_rsrc(bs, 0, span, kBufWord3);

            // Padding: columns x of a block whose key U0 + x lies outside the class (only on
            // steps that reach a sequence end).
            auto fix = [&](int x0, u32x2 v) {
                const int u = U0 + x0;                       // first key of the block
                if (u >= 0 && u + 16 <= n_r) return v;
                if (u + 16 <= 0 || u >= n_r) return u32x2{padw, padw};
                const int uk = u + 4 * grp;                  // this lane's 4 keys
                const bool k0 = uk >= 0 && uk < n_r, k1 = uk + 1 >= 0 && uk + 1 < n_r;
                const bool k2 = uk + 2 >= 0 && uk + 2 < n_r, k3 = uk + 3 >= 0 && uk + 3 < n_r;
                const uint32_t m0 = (k0 ? 0xffffu : 0u) | (k1 ? 0xffff0000u : 0u);
                const uint32_t m1 = (k2 ? 0xffffu : 0u) | (k3 ? 0xffff0000u : 0u);
                return u32x2{(v[0] & m0) | (padw & ~m0), (v[1] & m1) | (padw & ~m1)};
            };
            // Blocks x0 and x0 + 16 rounded (and padded), paired into a 16-byte piece per lane.
            auto piece = [&](auto edge, int x0, const f32x4& lo, const f32x4& hi) {
                u32x2 va = Mm<In>::pack(lo), vb = Mm<In>::pack(hi);
                if constexpr (decltype(edge)::value) {
                    va = fix(x0, va);
                    vb = fix(x0 + 16, vb);
                }
                const auto sx = __builtin_amdgcn_permlane16_swap(va[0], vb[0], false, false);
                const auto sy = __builtin_amdgcn_permlane16_swap(va[1], vb[1], false, false);
                return u32x4{sx[0], sy[0], sx[1], sy[1]};
            };
            // Direct store of one lane's piece (row t = 16 q2 + col, columns x .. x + 7): whole
            // pieces go to HBM, a row's head and tail pieces are set aside (part).
            unsigned char* const part = part_all + c * kPartWave;
            const int prow0 = (c + 8 * col) * (RB - 2);      // row t = col: byte of column 0
            const int prow1 = prow0 + 128 * (RB - 2);        // row t = 16 + col
            auto put_direct = [&](int x, int q2, bool ok, const u32x4& v) {
                const int t = 16 * q2 + col;
                const int di = x - (c + 8 * t);              // slot of column x in row t
                const bool whole = ok && static_cast<unsigned>(di) <= static_cast<unsigned>(K - 8);
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, brs, whole ? (q2 ? prow1 : prow0) + 2 * x : kBufDrop, 0, 0);
                const bool edge =
                    ok && !whole && static_cast<unsigned>(di + 7) < static_cast<unsigned>(K + 7);
                if (edge) *reinterpret_cast<u32x4*>(part + t * 32 + (di < 0 ? 0 : 16)) = v;
            };
            // Whole-line stores (kLines).  The two query sets' pieces are traded between the
            // lane halves (col and col ^ 8, a DPP rotation by 8 within each 16-lane row), so
            // that lane (col, grp) holds row 16 q2 + 8 half + (col & 7), columns
            // 8 m .. 8 m + 7 of the step, m = 4 (col >= 8) + sj: each store instruction then
            // covers 8 rows x 128 contiguous bytes.  Those 128 bytes start at the row's
            // 16-byte phase, so they straddle two 128-byte lines; the pieces m >= lb, lb the
            // piece where the row's next line begins (the same at every step), are held one
            // step and stored with the next step's pieces m < lb, so that the 8 lanes of a row
            // always write one whole aligned line.  The pieces held after the last step are
            // stored after the sweep.
            const bool hi8 = col >= 8;
            const int r8 = col & 7;
            const int mpc = 4 * (hi8 ? 1 : 0) + sj;
            const int prow8 = (c + 8 * r8) * (RB - 2);
            auto put8 = [&](int x, int q2, int half, const u32x4& v) {
                const int t = 16 * q2 + 8 * half + r8;
                const bool ok = t < nr;
                const int di = x - (c + 8 * t);
                const bool whole = ok && static_cast<unsigned>(di) <= static_cast<unsigned>(K - 8);
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, brs, whole ? prow8 + (128 * q2 + 64 * half) * (RB - 2) + 2 * x : kBufDrop,
                    0, kPol);
                const bool edge =
                    ok && !whole && static_cast<unsigned>(di + 7) < static_cast<unsigned>(K + 7);
                if (edge) *reinterpret_cast<u32x4*>(part + t * 32 + (di < 0 ? 0 : 16)) = v;
            };
            bool late[2][2];
            u32x4 held[2][2];
            if constexpr (kLines) {
                const int bmod128 = static_cast<int>(reinterpret_cast<uintptr_t>(bs) & 127);
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int lo = c + 8 * (16 * q2 + 8 * hf + r8);
                        const int lb = ((-(bmod128 + lo * (RB - 2) + 2 * xs)) & 127) >> 4;
                        late[q2][hf] = mpc >= lb;
                        held[q2][hf] = u32x4{0u, 0u, 0u, 0u};   // (step 0: columns before every row)
                    }
            }
            auto put_line = [&](int x, int q2, int hf, const u32x4& v) {
                const bool lt = late[q2][hf];
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = lt ? held[q2][hf][e] : v[e];
                put8(lt ? x - kStep : x, q2, hf, w);
                held[q2][hf] = v;
            };
            // One step: the four blocks at columns x0 .. x0 + 63: window reads, the MFMAs of
            // both query sets (the second set's rows past the class are computed and
            // dropped), rounding, stores.
            // xr: the ring row of column x0's key minus 8 (x0 moved into the step's slot).
            auto sweep = [&](auto edge, int x0, int xr) {
                V kf[4][kDC];
#pragma unroll
                for (int bk = 0; bk < 4; ++bk) {
                    const int r0 = xr + 8 + 16 * bk;
#pragma unroll
                    for (int dc = 0; dc < kDC; ++dc)
                        kf[bk][dc] = *reinterpret_cast<const V*>(win + r0 * kRowBytes + aoff[dc]);
                }
                f32x4 acc[2][4];
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                    for (int bk = 0; bk < 4; ++bk) {
                        acc[q2][bk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int dc = 0; dc < kDC; ++dc)
                            acc[q2][bk] = Mm<In>::run(kf[bk][dc], qf[q2][dc], acc[q2][bk]);
                    }
                if constexpr (kLines) {
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        const u32x4 p0 = piece(edge, x0, acc[q2][0], acc[q2][1]);
                        const u32x4 p1 = piece(edge, x0 + 32, acc[q2][2], acc[q2][3]);
                        u32x4 ra, rb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t send = hi8 ? p0[e] : p1[e];
                            const uint32_t recv = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(
                                static_cast<int>(send), 0x128, 0xf, 0xf, false));   // row_ror:8
                            ra[e] = hi8 ? recv : p0[e];
                            rb[e] = hi8 ? p1[e] : recv;
                        }
                        put_line(x0 + 8 * mpc, q2, 0, ra);
                        put_line(x0 + 8 * mpc, q2, 1, rb);
                    }
                } else {
#pragma unroll
                    for (int pr = 0; pr < 2; ++pr) {
                        const u32x4 p0 = piece(edge, x0 + 32 * pr, acc[0][2 * pr], acc[0][2 * pr + 1]);
                        const u32x4 p1 = piece(edge, x0 + 32 * pr, acc[1][2 * pr], acc[1][2 * pr + 1]);
                        put_direct(x0 + 32 * pr + 8 * sj, 0, ok0, p0);
                        put_direct(x0 + 32 * pr + 8 * sj, 1, ok1, p1);
                    }
                }
            };
            // The head and tail pieces of rows t < nr, element by element: lane l takes row
            // l / 2, its head (l even) or tail piece.
            auto write_edges = [&]() {
                for (int l = lane; l < 2 * nr; l += 64) {
                    const int t = l >> 1, tail = l & 1;
                    const int lo = c + 8 * t;
                    // the piece holding slot 0 (head) or slot K - 1 (tail): columns x .. x + 7
                    const int xc = tail ? lo + K - 1 : lo;
                    const int x = xc - ((xc - xs) & 7);
                    const int di = x - lo;
                    if (static_cast<unsigned>(di) <= static_cast<unsigned>(K - 8)) continue;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(part + t * 32 + 16 * tail);
                    const int e_lo = di < 0 ? -di : 0;
                    const int e_hi = K - di < 8 ? K - di : 8;
                    int b0 = 2 * e_lo;
                    const int b1 = 2 * e_hi;
                    const int off0 = lo * (RB - 2) + 2 * x;  // byte of the piece's element 0
                    const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
                    auto word = [&](int byte) {
                        const int wi = byte >> 2;
                        return wi == 0 ? w0 : (wi == 1 ? w1 : (wi == 2 ? w2 : w3));
                    };
                    if ((b0 & 3) == 2 && b0 + 2 <= b1) {
                        __builtin_amdgcn_raw_buffer_store_b16(
                            static_cast<unsigned short>(word(b0) >> 16), brs, off0 + b0, 0, 0);
                        b0 += 2;
                    }
                    if ((b0 & 7) == 4 && b0 + 4 <= b1) {
                        __builtin_amdgcn_raw_buffer_store_b32(word(b0), brs, off0 + b0, 0, 0);
                        b0 += 4;
                    }
                    if (b0 + 8 <= b1) {
                        const u32x2 dw = (b0 & 8) ? u32x2{w2, w3} : u32x2{w0, w1};
                        __builtin_amdgcn_raw_buffer_store_b64(dw, brs, off0 + b0, 0, 0);
                        b0 += 8;
                    }
                    if (b0 + 4 <= b1) {
                        __builtin_amdgcn_raw_buffer_store_b32(word(b0), brs, off0 + b0, 0, 0);
                        b0 += 4;
                    }
                    if (b0 + 2 <= b1)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            static_cast<unsigned short>(word(b0) >> (8 * (b0 & 2))), brs,
                            off0 + b0, 0, 0);
                }
            };

            // Steps run as soon as their keys are in (every loader wave past chunk j + 1);
            // after the step the wave counts it (its window reads are done: the MFMAs used
            // them).  No wave waits for another compute wave.
            for (int j = 0; j < J; ++j) {
                wait_min(ready + ((j + 1) & (kRingChunks - 1)), 1,
                         static_cast<uint32_t>(kLoadWaves * ((j + 1) / kRingChunks + 1)));
                const int x0 = xs + kStep * j;
                const int xr = xs + kStep * (j & (kRingChunks - 1));
                const int u = U0 + x0;                       // keys of the step: u .. u + 63
                if (u >= 0 && u + kStep <= n_r) sweep(std::false_type{}, x0, xr);
                else sweep(std::true_type{}, x0, xr);
                if (lane == 0 && C > kRingChunks)
                    __hip_atomic_store(done + c, static_cast<uint32_t>(j + 1), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            if (lane == 0 && C > kRingChunks)
                __hip_atomic_store(done + c, kAllDone, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            if constexpr (kLines) {                  // the pieces held after the last step
                const int xl = xs + kStep * (J - 1) + 8 * mpc;
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        if (late[q2][hf]) put8(xl, q2, hf, held[q2][hf]);
            }
            write_edges();
        }
        __syncthreads();                                     // the window is free again
        if (tid < kRingChunks + kComputeWaves) ready[tid] = 0u;
        __syncthreads();
    }
}

template <class In, int D, bool kLines, int kPol>
hipError_t launch_typed(const void* q, const void* k, void* band, const StreamArgs& a,
                        hipStream_t stream) {
    auto kern = qk_stream_kernel<In, D, kLines, kPol>;
    const int lds = lds_bytes(D);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    launch_kernel(kern, dim3(static_cast<uint32_t>(a.nwg)), dim3(kThreads),
                  static_cast<size_t>(lds), stream, static_cast<const typename In::T*>(q),
                  static_cast<const typename In::T*>(k), static_cast<typename In::T*>(band), a);
    return hipGetLastError();
}

}  // namespace

QkStreamPlan plan_qk_stream(const Problem& p, int in_dt, int out_dt) {
    QkStreamPlan sp;
    if (!(in_dt == kF16 || in_dt == kBF16) || out_dt != in_dt) return sp;
    if (p.d != 64) return sp;                         // (the loader split and LDS are for 64)
    const int64_t res = p.s < p.n ? p.s : (p.n > 0 ? p.n : 1);
    const int64_t strips = p.b * p.h * res;
    const int64_t longest = ceil_div(p.n, p.s);
    if (strips < 1 || longest < 1 || p.K < 8) return sp;
    const int64_t cus = device_cus();
    int64_t g = cus / strips;
    const int64_t need = ceil_div(longest, kMaxRange);
    g = g > need ? g : need;
    g = g < longest ? g : longest;                  // no empty ranges
    sp.g = g;
    sp.ranges = strips * g;
    sp.workgroups = sp.ranges < cus ? sp.ranges : cus;
    // launch a multiple of the XCD count when that stays within the units (ranks are then
    // contiguous per XCD); spare ranks get no range
    if (sp.workgroups % kXcds != 0 && ceil_div(sp.workgroups, kXcds) * kXcds <= cus)
        sp.workgroups = ceil_div(sp.workgroups, kXcds) * kXcds;
    sp.rows_per_range = ceil_div(longest, g);
    // Whole-line stores and the head-fastest range order for rows of more than 1000 slots
    // (DIAGMM_QK_LINES=0 / 1 overrides): there a step's half-written lines no longer wait in
    // L2 for the next step (n = 8192, 1025 slots: 74 -> 61 us; n = 32768, 4097 slots:
    // 1286 -> 1027 us; long document: 2512 -> 1997 us), while at 513 slots they do, and the
    // held pieces only add work (17.6 -> 19.5 us).
    sp.lines = p.K > 1000;
    if (const char* e = std::getenv("DIAGMM_QK_LINES")) {
        if (std::strcmp(e, "0") == 0) sp.lines = false;
        if (std::strcmp(e, "1") == 0) sp.lines = true;
    }
    // Bands larger than the 256 MB Infinity Cache are stored non-temporal on the line path:
    // the band then streams out instead of filling the L2 with lines that no later kernel
    // finds there anyway (long document 1960 -> 1533 us with the ranges dealt round-robin).  Smaller
    // bands are kept cached for the call that reads them next (at 513 slots non-temporal
    // stores cost the in-place softmax after qk 21 -> 28 us).  DIAGMM_QK_NT=0 / 1 overrides.
    const int64_t band_bytes = p.b * p.n * p.h * p.K * 2;
    sp.stream_stores = sp.lines && band_bytes > (int64_t(256) << 20);
    if (const char* e = std::getenv("DIAGMM_QK_NT")) {
        if (std::strcmp(e, "0") == 0) sp.stream_stores = false;
        if (std::strcmp(e, "1") == 0) sp.stream_stores = sp.lines;
    }
    sp.order = sp.lines ? 1 : 0;
    // With more ranges than workgroups, each XCD's ranges are dealt round-robin: with
    // non-temporal stores always (n = 32768, 8193 slots: 1600 -> 1533 us), with cached ones
    // below 3000 slots (n = 16384, 2049 slots: 309 -> 259 us) but not beyond (4097 slots:
    // 509 -> 535 us at n = 16384, 1027 -> 1153 us at n = 32768).
    sp.interleave = sp.lines && sp.ranges > sp.workgroups && sp.workgroups % kXcds == 0 &&
                    (sp.stream_stores || p.K < 3000);
    sp.lds_bytes = lds_bytes(static_cast<int>(p.d));
    const int64_t row_elems = p.s * p.h * p.K;
    const int64_t span = ((sp.rows_per_range - 1) * row_elems + p.K) * 2;
    // 32-bit arithmetic: band offsets within a range (below the drop offset 2^31), key
    // offsets within a strip, columns of a sweep, positions and ranges
    const int64_t strip_bytes = (ceil_div(p.n, p.s) + 1) * p.s * p.h * p.d * 2;
    sp.ok = sp.lds_bytes <= kLdsBytes && sp.rows_per_range <= kMaxRange &&
            sp.ranges < (int64_t(1) << 31) && span < (int64_t(1) << 31) - 64 &&
            p.n < (int64_t(1) << 30) && p.w < (int64_t(1) << 30) && p.K < (int64_t(1) << 28) &&
            strip_bytes < (int64_t(1) << 31) && p.b * p.h < (int64_t(1) << 31);
    return sp;
}

hipError_t launch_qk_stream(const void* q, const void* k, void* band, const Problem& p,
                            const QkStreamPlan& sp, int in_dt, uint32_t pad,
                            hipStream_t stream) {
    StreamArgs a{p.n, p.h, p.K, p.w, p.s,
                 static_cast<int32_t>(p.s < p.n ? p.s : (p.n > 0 ? p.n : 1)),
                 static_cast<int32_t>(sp.g), static_cast<int32_t>(sp.workgroups),
                 static_cast<int32_t>(sp.ranges / sp.workgroups),
                 static_cast<int32_t>(sp.ranges % sp.workgroups),
                 static_cast<int32_t>(p.n / p.s), static_cast<int32_t>(p.n % p.s), pad,
                 sp.order, sp.interleave ? 1 : 0};
    if (in_dt == kF16) {
        switch (p.d) {
        case 64:
            return !sp.lines ? launch_typed<F16, 64, false, 0>(q, k, band, a, stream)
                   : sp.stream_stores ? launch_typed<F16, 64, true, kPolNt>(q, k, band, a, stream)
                                      : launch_typed<F16, 64, true, 0>(q, k, band, a, stream);
        }
    } else if (in_dt == kBF16) {
        switch (p.d) {
        case 64:
            return !sp.lines ? launch_typed<BF16, 64, false, 0>(q, k, band, a, stream)
                   : sp.stream_stores ? launch_typed<BF16, 64, true, kPolNt>(q, k, band, a, stream)
                                      : launch_typed<BF16, 64, true, 0>(q, k, band, a, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace diagmm
