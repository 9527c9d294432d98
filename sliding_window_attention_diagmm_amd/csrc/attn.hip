// Sliding-window attention in one pass, the band never written to HBM:
//
//   out[i] = sum_k P_k V[j_k],   P = softmax(scale * S) over the in-range slots,
//   S_k = Q[i] . K[j_k],         j_k = i + (k - w) * s
//
// (TVM Discuss, "Developing a faster schedule for Longformer's kernel", post 6: the
// forward function and the backward function with transpose_t1 = 0; csarofeen/pytorch
// issue 2096, first fusion repro: the softmax recipe between them).  The three-call path
// stores the scores and the probabilities, two band tensors of 2 (w + w_upper + 1) bytes
// per query row and head; this kernel keeps them in registers and reads only Q, K and V.
//
// Work.  Within one residue class of the dilation the window is an undilated band (rows
// t = 0 .. len - 1 of the class attend class keys t - w .. t + w_upper).  A workgroup of
// four waves takes 64 consecutive class rows of one (batch, head); wave v owns rows
// 16 v .. 16 v + 15.  It walks the keys its rows reach, t0 - w .. t0 + 63 + w_upper, in
// blocks of 64 staged in LDS, with an online softmax: when a block raises some row's
// maximum by more than a factor 2^8 the running maxima are raised and the accumulators and
// running sums rescaled by exp(old - new); then the block's probabilities, relative to the
// running maximum, are added in.
//
// MFMA layouts (v_mfma_f32_16x16x32_{f16,bf16}; A lanes hold a row and 8 K-values, B
// lanes a column and 8 K-values, C lanes a column and 4 rows).  Scores are computed
// transposed, S^T = K Q^T: A is 16 key rows read from LDS, B this wave's 16 query rows
// held in registers, and C gives lane (column = query, group g) four keys.  Two such key
// tiles per 32 keys take the key rows 8 g + e and 8 g + 4 + e (e = 0..3) for A row 4 g + e,
// so lane group g ends up with the 8 consecutive keys 8 g .. 8 g + 7 of its query - in
// the order the product with V needs as its B operand.  out^T = V^T P^T then takes
// A = V^T (16 channels x 8 consecutive keys) through gfx950's transposing LDS reads of the
// row-major V block, as the pv kernel does, and C gives lane (query, g) channels
// 4 g .. 4 g + 3 of each 16-channel block - all of one query row, so the online
// softmax's rescaling is per lane.  Row maxima and sums combine the four lane groups of a
// query with two cross-lane steps.
//
// Global tokens (onnxruntime issue 12448: the LongformerAttention op, a sliding window
// plus global tokens, with Global_Q, Global_K and Global_V beside Q, K and V).  Two
// launches.  The first holds two kinds of workgroups, and each starts by building the
// batch's global set in LDS from the position list: a bitmap of the listed positions in
// [0, n) (a repeat sets one bit) and the exclusive prefix counts of its words, so that
// the set's size is known and its r-th member (in position order) is found by a binary
// search over the counts.  Band workgroups are the one-pass kernel's with the global keys
// added: a second bitmap marks the global keys inside the workgroup's key range (left
// out of its window blocks), the global keys are staged 64 at a time in set order and
// attended first, and rows at global positions are not stored.  Global-row workgroups
// take 64 global rows (4 waves x 16, ranks 64 rb ..) of one (batch, head) over one range
// of kr keys, with the global matrices, and write the range's partial softmax state
// (running maximum, running sum, unnormalised output per row) to the workspace; they come
// first in the grid, so their short ranges run beside the band workgroups.  The second
// launch merges the nsplit states of each block of global rows and stores the rows (the
// kernel boundary orders it after every partial state; a merge inside the first launch
// would need a device-scope release per workgroup, which writes back a whole L2).
#include <type_traits>

#include "launch.hpp"
#include "ring.hpp"

namespace diagmm {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef float f32x8 __attribute__((ext_vector_type(8)));

// An MFMA operand of eight 1.0 values.
template <class In> struct Ones;
template <> struct Ones<F16> {
    __device__ __forceinline__ static f16x8 v() {
        return f16x8{1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16};
    }
};
template <> struct Ones<BF16> {
    __device__ __forceinline__ static bf16x8 v() {
        const __bf16 o = static_cast<__bf16>(1.0f);
        return bf16x8{o, o, o, o, o, o, o, o};
    }
};

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

constexpr int kRows = 64;                   // query rows per workgroup, 16 per wave
constexpr int kThreads = kRows / 16 * 64;
constexpr int kKeys = 64;                   // keys per LDS block
// Workgroups per CU the register allocation must allow: 4 (4 waves per SIMD, at most 128
// registers a lane) for d <= 64, where that needs no spills; d = 128 keeps the default.
__host__ __device__ constexpr int attn_min_groups(int d) { return d <= 64 ? 4 : 1; }
constexpr int kChunks = kKeys / 32;         // 32-key chunks per block
constexpr int64_t kMaxGlobalN = int64_t(1) << 16;   // the LDS global set: 2 n bits <= 16 KB
constexpr int kMaxSplit = 32;               // key ranges per block of global rows, at most
constexpr int kBitWords = 512;   // LDS bitmap of global keys in a workgroup's key range

struct AttnArgs {
    int64_t n, h, w, wu, s;
    int64_t cls_q, cls_m;     // n = cls_q s + cls_m: class r has cls_q + (r < cls_m) rows
    int64_t nqb_hi, nqb_lo;   // 64-row blocks of a long / short class
    int64_t per_head;         // band workgroups per (batch, head)
    int64_t groups;           // band workgroups
    float scale_log2;         // scale * log2(e)
    int32_t ng;               // entries of the position list per batch (0: no global tokens)
    int32_t nrb;              // 64-row blocks of global rows per (batch, head)
    int32_t nsplit;           // key ranges per block of global rows
    int32_t kr;               // keys per range, a multiple of 64
    int64_t rows_used;        // global-row workgroups: b h nrb nsplit
    int64_t rows_groups;      // the same rounded up to a multiple of 8 (first in the grid)
};

// The global side of a call: the position list, the global rows' matrices and the
// workspace.
template <class T> struct GlobalIn {
    const int32_t* glob;      // [b][ng] listed positions
    const T* gq;
    const T* gk;
    const T* gv;
    int32_t* gpos;            // [b h nrb][64]: position of each global row, -1 past the set
    float* part_acc;          // [b h nrb nsplit 64][d]: unnormalised outputs of a range
    float* part_ml;           // [b h nrb nsplit 64][2]: running maximum (log2), running sum
};

// The global set of batch bb in LDS: gmap (nw words, bit x = position x listed) and gpre
// (exclusive prefix popcounts of the words); returns its size.  wsum: 4 words of LDS.
// With gbits (kBitWords words), the same pass over the list also marks the listed keys u
// of residue class r (position r + s u) in [u_lo, u_hi], as bit u - u_lo.
__device__ __forceinline__ int build_set(const int32_t* __restrict__ glob, int64_t bb, int ng,
                                         int n, uint32_t* gmap, uint32_t* gpre, uint32_t* wsum,
                                         uint32_t* gbits = nullptr, int r = 0, int s = 1,
                                         int u_lo = 0, int u_hi = -1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = (n + 31) >> 5;
    for (int i = tid; i < nw; i += kThreads) gmap[i] = 0u;
    if (gbits)
        for (int i = tid; i < kBitWords; i += kThreads) gbits[i] = 0u;
    __syncthreads();
    for (int g = tid; g < ng; g += kThreads) {
        const int x = glob[bb * ng + g];
        if (x < 0 || x >= n) continue;
        atomicOr(&gmap[x >> 5], 1u << (x & 31));
        if (gbits) {
            const int u = x / s;
            if (x - u * s == r && u >= u_lo && u <= u_hi)
                atomicOr(&gbits[(u - u_lo) >> 5], 1u << ((u - u_lo) & 31));
        }
    }
    __syncthreads();
    // thread t counts words [w0, w1); a scan within each wave, then over the 4 wave totals
    const int per = (nw + kThreads - 1) / kThreads;
    const int w0 = tid * per < nw ? tid * per : nw;
    const int w1 = w0 + per < nw ? w0 + per : nw;
    int cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __builtin_popcount(gmap[i]);
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[wave] = static_cast<uint32_t>(incl);
    __syncthreads();
    int off = incl - cnt;
    for (int wv = 0; wv < wave; ++wv) off += static_cast<int>(wsum[wv]);
    for (int i = w0; i < w1; ++i) {
        gpre[i] = static_cast<uint32_t>(off);
        off += __builtin_popcount(gmap[i]);
    }
    const int total = static_cast<int>(wsum[0] + wsum[1] + wsum[2] + wsum[3]);
    __syncthreads();
    return total;
}

// Member `rank` (< the set's size) of the set in position order.
__device__ __forceinline__ int set_member(const uint32_t* gmap, const uint32_t* gpre, int nw,
                                          int rank) {
    int lo = 0, hi = nw - 1;                  // the last word whose prefix count <= rank
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int>(gpre[mid]) <= rank) lo = mid;
        else hi = mid - 1;
    }
    uint32_t word = gmap[lo];
    for (int j = rank - static_cast<int>(gpre[lo]); j > 0; --j) word &= word - 1u;
    return 32 * lo + __builtin_ctz(word);
}

// Kernel modes: the window only; the window plus the global keys for rows outside the
// global set (global query rows are not stored); global rows over one key range.
constexpr int kBand = 0, kBandGlobal = 1, kGlobalRows = 2;

// K block: row r (key), 16-byte piece ch at r * 2D + 16 (ch ^ sw(r)); the swizzle puts the
// eight rows 8 (m / 4) + (m % 4) (+ 4) read by lanes m = 0..7 of a score tile on distinct
// 16-byte bank groups.
template <int D>
__device__ __forceinline__ int kpiece(int r, int ch) {
    const int hi = (r >> 3) & 1;
    const int sw = D == 32 ? hi : D == 64 ? (((r >> 1) & 1) | (hi << 1)) : ((r & 3) | (hi << 2));
    return r * (2 * D) + 16 * (ch ^ sw);
}

__device__ __forceinline__ uint32_t pack2(float a, float b, F16) {
    return static_cast<uint32_t>(F16::from_f32(a)) | (static_cast<uint32_t>(F16::from_f32(b)) << 16);
}
__device__ __forceinline__ uint32_t pack2(float a, float b, BF16) {
    return static_cast<uint32_t>(BF16::from_f32(a)) | (static_cast<uint32_t>(BF16::from_f32(b)) << 16);
}

// XCD-aware workgroup order: the dispatcher deals workgroups to the 8 XCDs in turn, so
// XCD x gets a contiguous range of ids (neighbouring row blocks share their keys in L2).
__device__ __forceinline__ int64_t xcd_order(int64_t bid, int64_t g) {
    const int64_t per = g / 8, rem = g % 8;
    const int64_t x = bid % 8, loc = bid / 8;
    return x * per + (x < rem ? x : rem) + loc;
}

// One workgroup of any mode: `id` is its unit (band: (batch, head, class, row block);
// global rows: (batch, head, row block, key range)).  gbits: kBitWords words of LDS for
// the band-global mode; gmap, gpre: the global set (n bits each), wsum: 4 words (modes
// with global tokens only).
template <class In, int D, int kMode>
__device__ __forceinline__ void attn_body(const typename In::T* __restrict__ q,
                                          const typename In::T* __restrict__ k,
                                          const typename In::T* __restrict__ v,
                                          typename In::T* __restrict__ out,
                                          const GlobalIn<typename In::T>& gi, const AttnArgs& a,
                                          int64_t id, unsigned char* klds, unsigned char* vlds,
                                          uint32_t* gbits, uint32_t* gmap, uint32_t* gpre,
                                          uint32_t* wsum) {
    using ST = typename In::T;
    using V = typename Mfma<In>::V;
    constexpr bool kRowsMode = kMode == kGlobalRows;
    constexpr int kPieces = D / 8;                       // 16-byte pieces per row
    constexpr int kStage = kKeys * kPieces / kThreads;   // pieces per thread per tensor
    constexpr int kQk = D / 32;                          // MFMA K-steps over the channels
    constexpr int kCb = D / 16;                          // 16-channel output blocks

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int ng = a.ng;

    // ---- the unit
    int64_t bh, r = 0;
    int rb = 0, split = 0, t0, len, ngd = 0;
    if constexpr (kRowsMode) {
        split = static_cast<int>(id % a.nsplit);
        const int64_t rest = id / a.nsplit;
        rb = static_cast<int>(rest % a.nrb);
        bh = rest / a.nrb;
        t0 = kRows * rb;                                  // ranks in the global set
        len = static_cast<int>(a.n);
    } else {
        int64_t qb;
        bh = id / a.per_head;
        int64_t rest = id - bh * a.per_head;
        if (rest < a.cls_m * a.nqb_hi) {
            r = rest / a.nqb_hi;
            qb = rest - r * a.nqb_hi;
        } else {
            rest -= a.cls_m * a.nqb_hi;
            r = a.cls_m + rest / a.nqb_lo;
            qb = rest - (r - a.cls_m) * a.nqb_lo;
        }
        t0 = static_cast<int>(qb) * kRows;
        len = static_cast<int>(a.cls_q + (r < a.cls_m ? 1 : 0));
    }
    const int64_t bb = bh / a.h, hh = bh - bb * a.h;
    const int nw = static_cast<int>((a.n + 31) >> 5);
    if constexpr (kRowsMode)
        ngd = build_set(gi.glob, bb, ng, static_cast<int>(a.n), gmap, gpre, wsum);
    if constexpr (kRowsMode) {
        // the first key range's workgroup records the positions of its 64 rows
        if (split == 0 && tid < kRows)
            gi.gpos[(bh * a.nrb + rb) * kRows + tid] =
                t0 + tid < ngd ? set_member(gmap, gpre, nw, t0 + tid) : -1;
        if (t0 >= ngd) return;                            // no global rows here (uniform)
    }
    // element offset of class row t (global rows: sequence position t): base + t * step
    const int64_t base = ((bb * a.n + r) * a.h + hh) * D;
    const int64_t step = (kRowsMode ? 1 : a.s) * a.h * D;

    // ---- this lane's query row as the B operand of S^T (channels 32 kk + 8 grp .. +7)
    const int tq = t0 + 16 * wv + col;                    // class row, or rank in the set
    int tq_ld;
    if constexpr (kRowsMode) tq_ld = set_member(gmap, gpre, nw, tq < ngd ? tq : ngd - 1);
    else tq_ld = tq < len ? tq : len - 1;
    const ST* const qsrc = kRowsMode ? gi.gq : q;
    const ST* const ksrc = kRowsMode ? gi.gk : k;
    const ST* const vsrc = kRowsMode ? gi.gv : v;
    V qop[kQk];
#pragma unroll
    for (int kk = 0; kk < kQk; ++kk)
        qop[kk] = *reinterpret_cast<const V*>(qsrc + base + int64_t(tq_ld) * step + 32 * kk + 8 * grp);
    // a wave whose 16 rows are all past the rows (global rows: past the set) stages its
    // share of every block but computes nothing
    const bool wave_live = kRowsMode ? t0 + 16 * wv < ngd : t0 + 16 * wv < len;

    const int w = kRowsMode ? 0 : static_cast<int>(a.w);
    const int wu = kRowsMode ? 0 : static_cast<int>(a.wu);
    int u_lo, u_hi, nblk;
    if constexpr (kRowsMode) {
        u_lo = split * a.kr;
        u_hi = (u_lo + a.kr < len ? u_lo + a.kr : len) - 1;
    } else {
        u_lo = t0 - w > 0 ? t0 - w : 0;
        const int last_q = (t0 + kRows - 1 < len - 1) ? t0 + kRows - 1 : len - 1;
        u_hi = (last_q + wu < len - 1) ? last_q + wu : len - 1;   // inclusive
    }
    nblk = (u_hi - u_lo + kKeys) / kKeys;

    // band workgroups with global keys: the set, and the global keys of this class inside
    // the key range as bits u - u_lo, in one pass over the list (after the query loads are
    // issued, so that both latencies overlap)
    if constexpr (kMode == kBandGlobal)
        ngd = build_set(gi.glob, bb, ng, static_cast<int>(a.n), gmap, gpre, wsum, gbits,
                        static_cast<int>(r), static_cast<int>(a.s), u_lo, u_hi);
    auto is_global_key = [&](int u) {
        return ((gbits[(u - u_lo) >> 5] >> ((u - u_lo) & 31)) & 1u) != 0u;
    };

    // ---- staging of one key block: K and V rows u0 .. u0 + 63 (rows past the class are
    // loaded from its last row and written as zeros)
    u32x4 kreg[kStage], vreg[kStage];
    // this thread's pieces: row pc / kPieces of the block, channels 8 (pc % kPieces) ..;
    // the block at u0 reads class row min(u0, len - 1 - row) + row (rows past the class
    // at its last row)
    int64_t lane_off[kStage];
    int lane_lim[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
        const int pc = tid + kThreads * i, row = pc / kPieces, ch = pc % kPieces;
        lane_off[i] = base + int64_t(row) * step + 8 * ch;
        lane_lim[i] = len - 1 - row;
    }
    auto load_block = [&](int u0) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int du = u0 < lane_lim[i] ? u0 : lane_lim[i];
            const int64_t off = lane_off[i] + int64_t(du) * step;
            kreg[i] = *reinterpret_cast<const u32x4*>(ksrc + off);
            vreg[i] = *reinterpret_cast<const u32x4*>(vsrc + off);
        }
    };
    auto store_block = [&](int u0) {
        auto put = [&](auto whole) {
#pragma unroll
            for (int i = 0; i < kStage; ++i) {
                const int pc = tid + kThreads * i, row = pc / kPieces, ch = pc % kPieces;
                u32x4 kv = kreg[i], vv = vreg[i];
                if constexpr (!decltype(whole)::value) {
                    const bool ok = u0 + row < len;
                    const u32x4 z{0u, 0u, 0u, 0u};
                    kv = ok ? kv : z;
                    vv = ok ? vv : z;
                }
                *reinterpret_cast<u32x4*>(klds + kpiece<D>(row, ch)) = kv;
                *reinterpret_cast<u32x4*>(vlds + ring_piece<D>(row, ch)) = vv;
            }
        };
        if (u0 + kKeys <= len) put(std::true_type{});   // the whole block inside the class
        else put(std::false_type{});
    };

    // a block of global keys: ranks 64 gb .. 64 gb + 63 of the set (zeros past its size)
    auto load_gblock = [&](int gb) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = tid + kThreads * i, row = pc / kPieces, ch = pc % kPieces;
            const int g = kKeys * gb + row;
            const int x = set_member(gmap, gpre, nw, g < ngd ? g : ngd - 1);
            const int64_t off = ((bb * a.n + x) * a.h + hh) * D + 8 * ch;
            kreg[i] = *reinterpret_cast<const u32x4*>(k + off);
            vreg[i] = *reinterpret_cast<const u32x4*>(v + off);
        }
    };
    auto store_gblock = [&](int gb) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = tid + kThreads * i, row = pc / kPieces, ch = pc % kPieces;
            const bool ok = kKeys * gb + row < ngd;
            const u32x4 z{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(klds + kpiece<D>(row, ch)) = ok ? kreg[i] : z;
            *reinterpret_cast<u32x4*>(vlds + ring_piece<D>(row, ch)) = ok ? vreg[i] : z;
        }
    };

    f32x4 acc[kCb];
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();   // running maximum of this lane's query (log2 units)
    // Running sum of the query's probabilities, as rounded for the product with V: an
    // MFMA with an all-ones A operand sums each B column (all 32 keys of a chunk, every
    // lane group) into every element of the lane's accumulator.
    f32x4 lsum{0.f, 0.f, 0.f, 0.f};
    const V ones = Ones<In>::v();

    int aoff[kCb];
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) aoff[cb] = tr_lane_off<D>(col, cb);
    // K rows of this lane's A operand within a 32-key chunk: tile 0 and tile 1
    const int krow0 = 8 * (col >> 2) + (col & 3), krow1 = krow0 + 4;
    const float cs = a.scale_log2;

    // gl: the staged block holds global keys (ranks u0 .. u0 + 63 of the set)
    auto compute_block = [&](int u0, bool gl) {
        // 32-key chunks that hold any key: all but a block of global keys whose ranks end
        // in its first chunk (the rest are -inf before and exact zeros after the exponent,
        // so skipping them changes nothing)
        const int nck = gl && ngd - u0 <= 32 ? 1 : kChunks;

        // ---- scores: lane (col, grp) gets S[query tq][keys u0 + 32 c + 8 grp + 0..7]
        f32x4 s0[kChunks], s1[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            s0[c] = s1[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (c >= nck) continue;
#pragma unroll
            for (int kk = 0; kk < kQk; ++kk) {
                const V a0 = *reinterpret_cast<const V*>(klds + kpiece<D>(32 * c + krow0, 4 * kk + grp));
                const V a1 = *reinterpret_cast<const V*>(klds + kpiece<D>(32 * c + krow1, 4 * kk + grp));
                s0[c] = Mfma<In>::run(a0, qop[kk], s0[c]);
                s1[c] = Mfma<In>::run(a1, qop[kk], s1[c]);
            }
        }
        // ---- mask (only blocks that are not wholly inside every row's window of this
        // wave need it), block maximum in log2 units.  Inner blocks keep the raw scores
        // (the scale, when positive, commutes with the maximum and goes into the
        // exponent's fma); masked blocks replace them by scale * score or -inf.
        float mx = -__builtin_inff();
        auto sc = [&](int c, int e) { return e < 4 ? s0[c][e] : s1[c][e - 4]; };
        const int lo = tq - w, hi = tq + wu;   // in-range keys of this query (and < len)
        const int tw = t0 + 16 * wv;           // this wave's first row
        // (with global tokens: a window block none of whose keys is global; the bitmap
        // words covering keys u0 .. u0 + 63 lie inside the range when the window test holds)
        // gm: bit j = key u0 + j is global (window blocks with global tokens; words past
        // the range hold zeros, and keys past it are masked anyway)
        uint64_t gm = 0;
        if constexpr (kMode == kBandGlobal) {
            if (!gl) {
                const int o = u0 - u_lo, wa = o >> 5, sh = o & 31;
                const int w1 = wa + 1 < kBitWords ? wa + 1 : kBitWords - 1;
                const int w2 = wa + 2 < kBitWords ? wa + 2 : kBitWords - 1;
                const uint64_t lo64 = gbits[wa] | (static_cast<uint64_t>(gbits[w1]) << 32);
                gm = sh ? (lo64 >> sh) | (static_cast<uint64_t>(gbits[w2]) << (64 - sh)) : lo64;
            }
        }
        auto no_global_keys = [&]() { return gm == 0; };
        bool inner;
        if constexpr (kRowsMode) inner = u0 + kKeys - 1 < len;
        else
            inner = !gl && u0 >= tw + 15 - w && u0 + kKeys - 1 <= tw + wu &&
                    u0 + kKeys - 1 < len && (kMode == kBand || no_global_keys());
        inner = inner && cs > 0.0f;
        if (inner) {
#pragma unroll
            for (int c = 0; c < kChunks; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc(c, e));
            mx *= cs;
        } else {
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                // this lane's 8 keys' global bits
                const uint32_t g8 = static_cast<uint32_t>(gm >> (32 * c + 8 * grp)) & 0xffu;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int u = u0 + 32 * c + 8 * grp + e;
                    bool ok;
                    if constexpr (kRowsMode) ok = u < len;
                    else if constexpr (kMode == kBandGlobal)
                        ok = gl ? u < ngd : (u >= lo && u <= hi && u < len && !((g8 >> e) & 1u));
                    else ok = u >= lo && u <= hi && u < len;
                    const float sv = ok ? sc(c, e) * cs : -__builtin_inff();
                    if (e < 4) s0[c][e] = sv;               // (e is a constant here)
                    else s1[c][e - 4] = sv;
                    mx = fmaxf(mx, sv);
                }
            }
        }
        // the four lane groups of a query: swaps with lanes l ^ 16 and l ^ 32 (each swap
        // returns this lane's value and its partner's, in some order).  The halves are
        // read as integers first: bit-casting the pair's elements straight to float was
        // compiled as if both were the first one.
        {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx),
                                                            __float_as_uint(mx), false, false);
            const uint32_t r0 = r[0], r1 = r[1];
            mx = fmaxf(__uint_as_float(r0), __uint_as_float(r1));
            const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                            __float_as_uint(mx), false, false);
            const uint32_t q0 = q[0], q1 = q[1];
            mx = fmaxf(__uint_as_float(q0), __uint_as_float(q1));
        }
        // ---- rescale only when some row's maximum grew by more than 2^8: otherwise the
        // old reference stays, and the block's terms exp2(x - m) stay below 256, exact
        // in the sum and representable in the 16-bit probabilities alike
        if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(
                m_run - (m_new == -__builtin_inff() ? 0.0f : m_new));
            m_run = m_new;
            lsum *= alpha;
#pragma unroll
            for (int cb = 0; cb < kCb; ++cb) acc[cb] *= alpha;
        }
        const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;

        // ---- probabilities exp2(k s - m) (k = scale on inner blocks, 1 on masked ones)
        // as the B operand of out^T = V^T P^T, and the products
        const float k1 = inner ? cs : 1.0f;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            if (c >= nck) continue;
            f32x8 p;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc(c, e), k1, -m_use));
            const V bop = __builtin_convertvector(p, V);
            lsum = Mfma<In>::run(ones, bop, lsum);
            const unsigned char* rp = vlds + (32 * c + 8 * grp) * (2 * D);
#pragma unroll
            for (int cb = 0; cb < kCb; ++cb) {
                const V av = tr_read8<V, D>(rp + aoff[cb]);
                acc[cb] = Mfma<In>::run(av, bop, acc[cb]);
            }
        }
    };

    if constexpr (kMode == kBandGlobal) {
        const int ngb = (ngd + kKeys - 1) / kKeys;
        for (int gb = 0; gb < ngb; ++gb) {
            load_gblock(gb);
            store_gblock(gb);
            __syncthreads();
            if (wave_live) compute_block(kKeys * gb, true);
            __syncthreads();
        }
    }
    // The next block's loads overlap this block's compute (a clamped repeat of the last
    // block when there is none, so the loads are unconditional).
    load_block(u_lo);
    for (int blk = 0; blk < nblk; ++blk) {
        const int u0 = u_lo + kKeys * blk;
        store_block(u0);
        __syncthreads();
        load_block(blk + 1 < nblk ? u0 + kKeys : u0);
        if (wave_live) compute_block(u0, false);
        __syncthreads();
    }

    const float l = lsum[0];
    if constexpr (kRowsMode) {
        // ---- this range's partial state of the rows (merged by the second launch)
        if (tq < ngd) {
            const int64_t slot = ((bh * a.nrb + rb) * a.nsplit + split) * kRows + 16 * wv + col;
            float* pa = gi.part_acc + slot * D + 4 * grp;
#pragma unroll
            for (int cb = 0; cb < kCb; ++cb) *reinterpret_cast<f32x4*>(pa + 16 * cb) = acc[cb];
            if (grp == 0) *reinterpret_cast<f32x2*>(gi.part_ml + 2 * slot) = f32x2{m_run, l};
        }
        return;
    }
    // ---- normalise and store: lane (col, grp) holds channels 16 cb + 4 grp .. +3
    bool store = tq < len;
    if constexpr (kMode == kBandGlobal) {
        store = store && !is_global_key(tq);   // global rows come from the global-row units
    }
    if (store) {
        const float inv = 1.0f / l;
        ST* orow = out + base + int64_t(tq) * step + 4 * grp;
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb) {
            const u32x2 o{pack2(acc[cb][0] * inv, acc[cb][1] * inv, In{}),
                          pack2(acc[cb][2] * inv, acc[cb][3] * inv, In{})};
            *reinterpret_cast<u32x2*>(orow + 16 * cb) = o;
        }
    }
}

template <class In, int D>
__global__ void __launch_bounds__(kThreads, attn_min_groups(D))
attn_fwd_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ k,
                const typename In::T* __restrict__ v, typename In::T* __restrict__ out,
                AttnArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char klds[kKeys * 2 * D];
    __shared__ __attribute__((aligned(16))) unsigned char vlds[kKeys * 2 * D];
    __shared__ uint32_t gbits[1];
    const GlobalIn<typename In::T> none{};
    attn_body<In, D, kBand>(q, k, v, out, none, a, xcd_order(blockIdx.x, a.groups), klds, vlds,
                            gbits, nullptr, nullptr, nullptr);
}

// The global-row units (rows_groups workgroups, the padding ones idle), then the band
// workgroups with the global keys.  Dynamic LDS: the global set (2 ceil(n / 32) words).
template <class In, int D>
__global__ void __launch_bounds__(kThreads, attn_min_groups(D))
attn_global_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ k,
                   const typename In::T* __restrict__ v, typename In::T* __restrict__ out,
                   GlobalIn<typename In::T> gi, AttnArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char klds[kKeys * 2 * D];
    __shared__ __attribute__((aligned(16))) unsigned char vlds[kKeys * 2 * D];
    __shared__ uint32_t gbits[kBitWords];
    __shared__ uint32_t wsum[4];
    extern __shared__ uint32_t gdyn[];
    uint32_t* const gmap = gdyn;
    uint32_t* const gpre = gdyn + ((a.n + 31) >> 5);
    const int64_t bid = blockIdx.x;
    if (bid < a.rows_groups) {
        if (bid < a.rows_used)
            attn_body<In, D, kGlobalRows>(q, k, v, out, gi, a, bid, klds, vlds, gbits, gmap, gpre,
                                          wsum);
        return;
    }
    attn_body<In, D, kBandGlobal>(q, k, v, out, gi, a, xcd_order(bid - a.rows_groups, a.groups),
                                  klds, vlds, gbits, gmap, gpre, wsum);
}

// The global rows: block blockIdx.x = (batch, head, row block) merges its nsplit partial
// states per row and stores the rows.  Every load of a phase is independent of the others
// (the states of all rows and ranges at once, then the outputs), so the merge costs a few
// memory latencies whatever nsplit is.
template <class In, int D>
__global__ void __launch_bounds__(kThreads)
attn_gmerge_kernel(typename In::T* __restrict__ out, GlobalIn<typename In::T> gi, AttnArgs a) {
    using ST = typename In::T;
    constexpr int kQuads = D / 4;
    __shared__ float fac[kRows * kMaxSplit];             // per (row, range): exp2(m - M), then
    __shared__ float lsum[kRows * kMaxSplit];            // its running sum
    __shared__ float inv_l[kRows];
    __shared__ int pos_s[kRows];
    const int tid = threadIdx.x;
    const int ns = a.nsplit;
    const int64_t blk_id = blockIdx.x;
    const int64_t bh = blk_id / a.nrb, bb = bh / a.h, hh = bh - bb * a.h;
    const int64_t slot0 = blk_id * ns * kRows;           // row 0 of range 0
    if (tid < kRows) pos_s[tid] = gi.gpos[blk_id * kRows + tid];
    for (int i = tid; i < kRows * ns; i += kThreads) {
        const int sp = i / kRows, rr = i - sp * kRows;
        const f32x2 ml =
            *reinterpret_cast<const f32x2*>(gi.part_ml + 2 * (slot0 + int64_t(sp) * kRows + rr));
        fac[rr * kMaxSplit + sp] = ml[0];
        lsum[rr * kMaxSplit + sp] = ml[1];
    }
    __syncthreads();
    if (tid < kRows && pos_s[tid] >= 0) {
        float* f = fac + tid * kMaxSplit;
        float M = -__builtin_inff();
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, f[sp]);
        float L = 0.0f;
        for (int sp = 0; sp < ns; ++sp) {
            f[sp] = f[sp] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(f[sp] - M);
            L += lsum[tid * kMaxSplit + sp] * f[sp];
        }
        inv_l[tid] = 1.0f / L;
    }
    __syncthreads();
    for (int it = tid; it < kRows * kQuads; it += kThreads) {
        const int rr = it / kQuads, c4 = it - rr * kQuads;
        const int pos = pos_s[rr];
        if (pos < 0) continue;
        const float* f = fac + rr * kMaxSplit;
        const float* pa = gi.part_acc + (slot0 + rr) * D + 4 * c4;
        f32x4 A{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int sp = 0; sp < ns; ++sp)
            A += f[sp] * *reinterpret_cast<const f32x4*>(pa + int64_t(sp) * kRows * D);
        const float inv = inv_l[rr];
        ST* orow = out + ((bb * a.n + pos) * a.h + hh) * D + 4 * c4;
        *reinterpret_cast<u32x2*>(orow) =
            u32x2{pack2(A[0] * inv, A[1] * inv, In{}), pack2(A[2] * inv, A[3] * inv, In{})};
    }
}

AttnArgs make_args(const Problem& p, float scale, int64_t ng = 0) {
    AttnArgs a{};
    a.n = p.n;
    a.h = p.h;
    a.w = p.w;
    a.wu = p.wu;
    a.s = p.s;
    a.cls_q = p.n / p.s;
    a.cls_m = p.n % p.s;
    a.nqb_hi = (a.cls_q + 1 + kRows - 1) / kRows;
    a.nqb_lo = (a.cls_q + kRows - 1) / kRows;
    a.per_head = a.cls_m * a.nqb_hi + (p.s - a.cls_m) * a.nqb_lo;
    a.groups = p.b * p.h * a.per_head;
    a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    a.ng = static_cast<int32_t>(ng);
    if (ng > 0 && p.n > 0) {
        // key ranges about as long as a band workgroup's walk (64 + w + w_upper keys), so
        // that the global-row workgroups end with the band ones and, with them, fill one
        // round of the machine; never an empty range
        a.nrb = static_cast<int32_t>((ng + kRows - 1) / kRows);
        const int64_t units = p.b * p.h * a.nrb;
        const int64_t blocks = (p.n + kKeys - 1) / kKeys;
        const int64_t band_blocks = (kRows + p.w + p.wu + kKeys - 1) / kKeys;
        int64_t nsplit = (blocks + band_blocks - 1) / band_blocks;
        nsplit = nsplit < blocks ? nsplit : blocks;
        nsplit = nsplit < kMaxSplit ? nsplit : kMaxSplit;
        const int64_t kr = (blocks + nsplit - 1) / nsplit * kKeys;
        a.kr = static_cast<int32_t>(kr);
        a.nsplit = static_cast<int32_t>((p.n + kr - 1) / kr);
        a.rows_used = units * a.nsplit;
        a.rows_groups = (a.rows_used + 7) / 8 * 8;
    }
    return a;
}

// Workspace of the global-token form: the positions of the global rows and their
// partial states; each part 256-byte aligned.
struct GlobalWs {
    int64_t pos, acc, ml, total;
};
GlobalWs ws_layout(const Problem& p, int64_t ng) {
    GlobalWs w{};
    if (ng <= 0) return w;
    const AttnArgs a = make_args(p, 1.0f, ng);
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t blocks = p.b * p.h * a.nrb;
    const int64_t slots = blocks * int64_t(a.nsplit) * kRows;
    w.pos = 0;
    w.acc = w.pos + up(blocks * kRows * 4);
    w.ml = w.acc + up(slots * p.d * 4);
    w.total = w.ml + up(slots * 2 * 4);
    return w;
}

template <class In, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* gq,
                    const void* gk, const void* gv, void* out, const int32_t* glob,
                    unsigned char* ws, const AttnArgs& a, int64_t b, const GlobalWs& wl,
                    hipStream_t stream) {
    using ST = typename In::T;
    if (a.ng == 0) {
        launch_kernel(attn_fwd_kernel<In, D>, dim3(static_cast<uint32_t>(a.groups)),
                      dim3(kThreads), 0, stream, static_cast<const ST*>(q),
                      static_cast<const ST*>(k), static_cast<const ST*>(v),
                      static_cast<ST*>(out), a);
        return hipGetLastError();
    }
    GlobalIn<ST> gi;
    gi.glob = glob;
    gi.gq = static_cast<const ST*>(gq);
    gi.gk = static_cast<const ST*>(gk);
    gi.gv = static_cast<const ST*>(gv);
    gi.gpos = reinterpret_cast<int32_t*>(ws + wl.pos);
    gi.part_acc = reinterpret_cast<float*>(ws + wl.acc);
    gi.part_ml = reinterpret_cast<float*>(ws + wl.ml);
    const size_t set_lds = static_cast<size_t>((a.n + 31) / 32) * 2 * 4;
    launch_kernel(attn_global_kernel<In, D>,
                  dim3(static_cast<uint32_t>(a.rows_groups + a.groups)), dim3(kThreads), set_lds,
                  stream, static_cast<const ST*>(q), static_cast<const ST*>(k),
                  static_cast<const ST*>(v), static_cast<ST*>(out), gi, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(attn_gmerge_kernel<In, D>, dim3(static_cast<uint32_t>(b * a.h * a.nrb)),
                  dim3(kThreads), 0, stream, static_cast<ST*>(out), gi, a);
    return hipGetLastError();
}

template <class In>
hipError_t launch_d(const void* q, const void* k, const void* v, const void* gq,
                    const void* gk, const void* gv, void* out, const int32_t* glob,
                    unsigned char* ws, const AttnArgs& a, int64_t b, int64_t d,
                    const GlobalWs& wl, hipStream_t stream) {
    switch (d) {
    case 32: return launch_t<In, 32>(q, k, v, gq, gk, gv, out, glob, ws, a, b, wl, stream);
    case 64: return launch_t<In, 64>(q, k, v, gq, gk, gv, out, glob, ws, a, b, wl, stream);
    case 128: return launch_t<In, 128>(q, k, v, gq, gk, gv, out, glob, ws, a, b, wl, stream);
    default: return hipErrorInvalidValue;
    }
}

bool is16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// f16 / bf16, d in {32, 64, 128}, 16-byte aligned tensors, class rows and window offsets
// in 32-bit range, a grid below 2^31 workgroups.
bool attention_supported(const Problem& p, int dt, const void* q, const void* k, const void* v,
                         const void* out) {
    if (dt != kF16 && dt != kBF16) return false;
    if (p.d != 32 && p.d != 64 && p.d != 128) return false;
    if (!is16(q) || !is16(k) || !is16(v) || !is16(out)) return false;
    if (p.n >= (int64_t(1) << 30) || p.w >= (int64_t(1) << 30) || p.wu >= (int64_t(1) << 30))
        return false;
    const AttnArgs a = make_args(p, 1.0f);
    return a.groups < (int64_t(1) << 31);
}

// With global tokens: the key range of a band workgroup (64 + w + w_upper keys) must fit
// its LDS bitmap of global keys, the sequence the LDS global set (n <= 2^16), and
// the whole grid 2^31 workgroups.
bool attention_global_supported(const Problem& p, int64_t ng) {
    if (ng == 0) return true;
    if (!(64 + p.w + p.wu <= int64_t(kBitWords) * 32 && ng > 0 && ng <= p.n &&
          p.n <= kMaxGlobalN))
        return false;
    const AttnArgs a = make_args(p, 1.0f, ng);
    return a.rows_groups + a.groups < (int64_t(1) << 31) && p.b < (int64_t(1) << 31);
}

int64_t attention_global_workspace(const Problem& p, int64_t ng) {
    return ws_layout(p, ng).total;
}

int64_t attention_workgroups(const Problem& p) { return make_args(p, 1.0f).groups; }

hipError_t launch_attention(const void* q, const void* k, const void* v, const void* gq,
                            const void* gk, const void* gv, void* out, const int32_t* glob,
                            int64_t ng, void* workspace, const Problem& p, float scale,
                            int dt, hipStream_t stream) {
    const AttnArgs a = make_args(p, scale, ng);
    if (a.groups == 0) return hipSuccess;
    const GlobalWs wl = ws_layout(p, ng);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if (!gq) {
        gq = q;
        gk = k;
        gv = v;
    }
    switch (dt) {
    case kF16: return launch_d<F16>(q, k, v, gq, gk, gv, out, glob, ws, a, p.b, p.d, wl, stream);
    case kBF16: return launch_d<BF16>(q, k, v, gq, gk, gv, out, glob, ws, a, p.b, p.d, wl, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace diagmm
