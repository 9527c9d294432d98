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
#include "launch.hpp"
#include "ring.hpp"

namespace diagmm {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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

constexpr int kRows = 64;                   // class rows per workgroup, 16 per wave
constexpr int kThreads = kRows / 16 * 64;
// Workgroup size of a mode: the global-row pass splits the keys over 8 waves where their
// LDS blocks fit (d <= 64), else over 4.
__host__ __device__ constexpr int mode_threads(int mode, int d) {
    return mode == 2 && d <= 64 ? 512 : kThreads;
}
constexpr int kKeys = 64;                   // keys per LDS block
constexpr int kChunks = kKeys / 32;         // 32-key chunks per block

struct AttnArgs {
    int64_t n, h, w, wu, s;
    int64_t cls_q, cls_m;     // n = cls_q s + cls_m: class r has cls_q + (r < cls_m) rows
    int64_t nqb_hi, nqb_lo;   // 64-row blocks of a long / short class
    int64_t per_head;         // workgroups per (batch, head)
    int64_t groups;           // workgroups in the grid
    float scale_log2;         // scale * log2(e)
    int32_t ng;               // global tokens per batch (0: none)
    int64_t ngb;              // 16-row blocks of global rows per (batch, head)
};

// Kernel modes: the window only; the window plus the global keys for rows outside the
// global set (global query rows are not stored); the global rows, each over every key.
constexpr int kBand = 0, kBandGlobal = 1, kGlobalRows = 2;
constexpr int kBitWords = 512;   // LDS bitmap of global keys in a workgroup's key range

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

template <class In, int D, int kMode>
__global__ void __launch_bounds__(mode_threads(kMode, D))
attn_fwd_kernel(const typename In::T* __restrict__ q, const typename In::T* __restrict__ k,
                const typename In::T* __restrict__ v, typename In::T* __restrict__ out,
                const int32_t* __restrict__ glob, AttnArgs a) {
    using ST = typename In::T;
    using V = typename Mfma<In>::V;
    constexpr int kPieces = D / 8;                       // 16-byte pieces per row
    // the global-row mode splits the keys over the waves (8, or 4 for d = 128): each wave
    // stages its own blocks (64 threads) in its own LDS region
    constexpr int kT = mode_threads(kMode, D);
    constexpr int kSplit = kMode == kGlobalRows ? kT / 64 : 1;
    constexpr int kStageThreads = kT / kSplit;
    constexpr int kStage = kKeys * kPieces / kStageThreads;   // pieces per thread per tensor
    constexpr int kQk = D / 32;                          // MFMA K-steps over the channels
    constexpr int kCb = D / 16;                          // 16-channel output blocks
    __shared__ __attribute__((aligned(16))) unsigned char klds[kSplit * kKeys * 2 * D];
    __shared__ __attribute__((aligned(16))) unsigned char vlds[kSplit * kKeys * 2 * D];
    __shared__ uint32_t gbits[kMode == kBandGlobal ? kBitWords : 1];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;

    // ---- workgroup -> (batch, head, residue class, row block), XCD-aware: the dispatcher
    // deals workgroups to the 8 XCDs in turn, so XCD x gets a contiguous range of ids.
    int64_t id;
    {
        const int64_t g = a.groups, per = g / 8, rem = g % 8;
        const int64_t x = blockIdx.x % 8, loc = blockIdx.x / 8;
        id = x * per + (x < rem ? x : rem) + loc;
    }
    const int64_t units = kMode == kGlobalRows ? a.ngb : a.per_head;
    const int64_t bh = id / units;
    int64_t rest = id - bh * units;
    int64_t r, qb;
    if (kMode == kGlobalRows) {
        r = 0;              // the whole sequence as one undilated class, queries gathered
        qb = rest;
    } else if (rest < a.cls_m * a.nqb_hi) {
        r = rest / a.nqb_hi;
        qb = rest - r * a.nqb_hi;
    } else {
        rest -= a.cls_m * a.nqb_hi;
        r = a.cls_m + rest / a.nqb_lo;
        qb = rest - (r - a.cls_m) * a.nqb_lo;
    }
    const int64_t bb = bh / a.h, hh = bh - bb * a.h;
    const int len = kMode == kGlobalRows ? static_cast<int>(a.n)
                                         : static_cast<int>(a.cls_q + (r < a.cls_m ? 1 : 0));
    // global rows: blocks of 16, all waves on the same rows
    const int t0 = static_cast<int>(qb) * (kMode == kGlobalRows ? 16 : kRows);
    // element offset of class row t: base + t * step
    const int64_t base = ((bb * a.n + r) * a.h + hh) * D;
    const int64_t step = (kMode == kGlobalRows ? 1 : a.s) * a.h * D;
    const int ng = a.ng;
    // position of global token g of this batch, clamped into the sequence
    auto gpos = [&](int g) {
        int x = glob[bb * ng + (g < ng ? g : ng - 1)];
        return x < 0 ? 0 : (x >= a.n ? static_cast<int>(a.n) - 1 : x);
    };

    // ---- this lane's query row as the B operand of S^T (channels 32 kk + 8 grp .. +7)
    const int tq = t0 + (kMode == kGlobalRows ? 0 : 16 * wv) + col;
    const int tq_ld = kMode == kGlobalRows ? gpos(tq) : (tq < len ? tq : len - 1);
    V qop[kQk];
#pragma unroll
    for (int kk = 0; kk < kQk; ++kk)
        qop[kk] = *reinterpret_cast<const V*>(q + base + int64_t(tq_ld) * step + 32 * kk + 8 * grp);

    const int w = kMode == kGlobalRows ? 0 : static_cast<int>(a.w);
    const int wu = kMode == kGlobalRows ? 0 : static_cast<int>(a.wu);
    int u_lo = t0 - w > 0 ? t0 - w : 0;
    const int last_q = (t0 + kRows - 1 < len - 1) ? t0 + kRows - 1 : len - 1;
    int u_hi = (last_q + wu < len - 1) ? last_q + wu : len - 1;   // inclusive
    int nblk = (u_hi - u_lo + kKeys) / kKeys;
    if (kMode == kGlobalRows) {
        // wave wv sweeps the wv-th share of the key blocks; the same count for every
        // wave (blocks past the sequence are masked), so the barriers match
        const int per = ((len + kKeys - 1) / kKeys + kSplit - 1) / kSplit;
        u_lo = wv * per * kKeys;
        u_hi = len - 1;
        nblk = per;
    }
    const int stid = kMode == kGlobalRows ? lane : tid;   // staging thread index
    unsigned char* const kw = klds + (kMode == kGlobalRows ? wv : 0) * kKeys * 2 * D;
    unsigned char* const vw = vlds + (kMode == kGlobalRows ? wv : 0) * kKeys * 2 * D;

    // global keys of this class inside the key range, as bits of u - u_lo
    if constexpr (kMode == kBandGlobal) {
        for (int i = tid; i < kBitWords; i += kThreads) gbits[i] = 0u;
        __syncthreads();
        for (int g = tid; g < ng; g += kThreads) {
            const int x = gpos(g);
            const int u = x / static_cast<int>(a.s);
            if (x - u * static_cast<int>(a.s) == r && u >= u_lo && u <= u_hi)
                atomicOr(&gbits[(u - u_lo) >> 5], 1u << ((u - u_lo) & 31));
        }
        __syncthreads();
    }
    auto is_global_key = [&](int u) {
        return ((gbits[(u - u_lo) >> 5] >> ((u - u_lo) & 31)) & 1u) != 0u;
    };

    // ---- staging of one key block: K and V rows u0 .. u0 + 63 (rows past the class are
    // loaded from its last row and written as zeros)
    u32x4 kreg[kStage], vreg[kStage];
    auto load_block = [&](int u0) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = stid + kStageThreads * i, row = pc / kPieces, ch = pc % kPieces;
            int u = u0 + row;
            u = u < len ? u : len - 1;
            const int64_t off = base + int64_t(u) * step + 8 * ch;
            kreg[i] = *reinterpret_cast<const u32x4*>(k + off);
            vreg[i] = *reinterpret_cast<const u32x4*>(v + off);
        }
    };
    auto store_block = [&](int u0) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = stid + kStageThreads * i, row = pc / kPieces, ch = pc % kPieces;
            const bool ok = u0 + row < len;
            const u32x4 z{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(kw + kpiece<D>(row, ch)) = ok ? kreg[i] : z;
            *reinterpret_cast<u32x4*>(vw + ring_piece<D>(row, ch)) = ok ? vreg[i] : z;
        }
    };

    // a block of global keys: tokens 64 gb .. 64 gb + 63 of this batch (zeros past ng)
    auto load_gblock = [&](int gb) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = tid + kThreads * i, row = pc / kPieces, ch = pc % kPieces;
            const int64_t off = ((bb * a.n + gpos(kKeys * gb + row)) * a.h + hh) * D + 8 * ch;
            kreg[i] = *reinterpret_cast<const u32x4*>(k + off);
            vreg[i] = *reinterpret_cast<const u32x4*>(v + off);
        }
    };
    auto store_gblock = [&](int gb) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = tid + kThreads * i, row = pc / kPieces, ch = pc % kPieces;
            const bool ok = kKeys * gb + row < ng;
            const u32x4 z{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(klds + kpiece<D>(row, ch)) = ok ? kreg[i] : z;
            *reinterpret_cast<u32x4*>(vlds + ring_piece<D>(row, ch)) = ok ? vreg[i] : z;
        }
    };

    f32x4 acc[kCb];
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff();   // running maximum of this lane's query (log2 units)
    float l_run = 0.0f;                // this lane's share of the running sum

    int aoff[kCb];
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) aoff[cb] = tr_lane_off<D>(col, cb);
    // K rows of this lane's A operand within a 32-key chunk: tile 0 and tile 1
    const int krow0 = 8 * (col >> 2) + (col & 3), krow1 = krow0 + 4;

    // gl: the staged block holds global keys u0 .. u0 + 63 (token indices), not window keys
    auto compute_block = [&](int u0, bool gl) {

        // ---- scores: lane (col, grp) gets S[query tq][keys u0 + 32 c + 8 grp + 0..7]
        f32x4 s0[kChunks], s1[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            s0[c] = s1[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < kQk; ++kk) {
                const V a0 = *reinterpret_cast<const V*>(kw + kpiece<D>(32 * c + krow0, 4 * kk + grp));
                const V a1 = *reinterpret_cast<const V*>(kw + kpiece<D>(32 * c + krow1, 4 * kk + grp));
                s0[c] = Mfma<In>::run(a0, qop[kk], s0[c]);
                s1[c] = Mfma<In>::run(a1, qop[kk], s1[c]);
            }
        }
        // ---- scale, mask (only blocks that are not wholly inside every row's window of
        // this wave need it), block maximum
        float x[kChunks][8];
        float mx = -__builtin_inff();
        const int lo = tq - w, hi = tq + wu;   // in-range keys of this query (and < len)
        const int tw = t0 + 16 * wv;           // this wave's first row
        // (with global tokens: a window block none of whose keys is global; the bitmap
        // words covering keys u0 .. u0 + 63 lie inside the range when the window test holds)
        auto no_global_keys = [&]() {
            const int o = u0 - u_lo, wa = o >> 5, wb = (o + kKeys - 1) >> 5;
            return (gbits[wa] | gbits[wa + 1] | gbits[wb]) == 0u;
        };
        bool inner;
        if constexpr (kMode == kGlobalRows) inner = u0 + kKeys - 1 < len;
        else
            inner = !gl && u0 >= tw + 15 - w && u0 + kKeys - 1 <= tw + wu &&
                    u0 + kKeys - 1 < len && (kMode == kBand || no_global_keys());
        if (inner) {
#pragma unroll
            for (int c = 0; c < kChunks; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x[c][e] = (e < 4 ? s0[c][e] : s1[c][e - 4]) * a.scale_log2;
                    mx = fmaxf(mx, x[c][e]);
                }
        } else {
#pragma unroll
            for (int c = 0; c < kChunks; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int u = u0 + 32 * c + 8 * grp + e;
                    const float sv = e < 4 ? s0[c][e] : s1[c][e - 4];
                    bool ok;
                    if constexpr (kMode == kGlobalRows) ok = u < len;
                    else if constexpr (kMode == kBandGlobal)
                        ok = gl ? u < ng : (u >= lo && u <= hi && u < len && !is_global_key(u));
                    else ok = u >= lo && u <= hi && u < len;
                    x[c][e] = ok ? sv * a.scale_log2 : -__builtin_inff();
                    mx = fmaxf(mx, x[c][e]);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // ---- rescale only when some row's maximum grew by more than 2^8: otherwise the
        // old reference stays, and the block's terms exp2(x - m) stay below 256, exact
        // in the sum and representable in the 16-bit probabilities alike
        if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(
                m_run - (m_new == -__builtin_inff() ? 0.0f : m_new));
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < kCb; ++cb) acc[cb] *= alpha;
        }
        const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;

        // ---- probabilities as the B operand of out^T = V^T P^T, and the products
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(x[c][e] - m_use);
                l_run += p[e];
            }
            const u32x4 pb{pack2(p[0], p[1], In{}), pack2(p[2], p[3], In{}),
                           pack2(p[4], p[5], In{}), pack2(p[6], p[7], In{})};
            const V bop = __builtin_bit_cast(V, pb);
            const unsigned char* rp = vw + (32 * c + 8 * grp) * (2 * D);
#pragma unroll
            for (int cb = 0; cb < kCb; ++cb) {
                const V av = tr_read8<V, D>(rp + aoff[cb]);
                acc[cb] = Mfma<In>::run(av, bop, acc[cb]);
            }
        }
    };

    // The next block's loads overlap this block's compute (a clamped repeat of the last
    // block when there is none, so the loads are unconditional).
    if constexpr (kMode == kBandGlobal) {
        const int ngb = (ng + kKeys - 1) / kKeys;
        for (int gb = 0; gb < ngb; ++gb) {
            load_gblock(gb);
            store_gblock(gb);
            __syncthreads();
            compute_block(kKeys * gb, true);
            __syncthreads();
        }
    }
    load_block(u_lo);
    for (int blk = 0; blk < nblk; ++blk) {
        const int u0 = u_lo + kKeys * blk;
        store_block(u0);
        __syncthreads();
        load_block(blk + 1 < nblk ? u0 + kKeys : u0);
        compute_block(u0, false);
        __syncthreads();
    }

    // ---- normalise and store: lane (col, grp) holds channels 16 cb + 4 grp .. +3
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if constexpr (kMode == kGlobalRows) {
        // merge the waves' partial softmax states of the same 16 rows: scale each
        // by 2^(m_w - max m), add, divide (LDS is free: the loop ended on a barrier)
        constexpr int S = kCb * 4 + 2;
        float* mb = reinterpret_cast<float*>(klds);
        float* mine = mb + (wv * 64 + lane) * S;
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) mine[cb * 4 + e] = acc[cb][e];
        mine[kCb * 4] = m_run;
        mine[kCb * 4 + 1] = l;
        __syncthreads();
        if (wv != 0 || tq >= ng) return;
        float M = -__builtin_inff();
#pragma unroll
        for (int w4 = 0; w4 < kSplit; ++w4) M = fmaxf(M, mb[(w4 * 64 + lane) * S + kCb * 4]);
        float L = 0.0f;
        f32x4 A[kCb];
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb) A[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w4 = 0; w4 < kSplit; ++w4) {
            const float* o = mb + (w4 * 64 + lane) * S;
            const float f = o[kCb * 4] == -__builtin_inff()
                                ? 0.0f : __builtin_amdgcn_exp2f(o[kCb * 4] - M);
            L += o[kCb * 4 + 1] * f;
#pragma unroll
            for (int cb = 0; cb < kCb; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) A[cb][e] += o[cb * 4 + e] * f;
        }
        const float inv = 1.0f / L;
        ST* orow = out + base + int64_t(tq_ld) * step + 4 * grp;
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb) {
            const u32x2 o2{pack2(A[cb][0] * inv, A[cb][1] * inv, In{}),
                           pack2(A[cb][2] * inv, A[cb][3] * inv, In{})};
            *reinterpret_cast<u32x2*>(orow + 16 * cb) = o2;
        }
        return;
    }
    bool store = tq < len;
    const int64_t orow_t = tq;
    if constexpr (kMode == kBandGlobal) {
        store = store && !is_global_key(tq);   // global rows come from the global-row pass
    }
    if (store) {
        const float inv = 1.0f / l;
        ST* orow = out + base + orow_t * step + 4 * grp;
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb) {
            const u32x2 o{pack2(acc[cb][0] * inv, acc[cb][1] * inv, In{}),
                          pack2(acc[cb][2] * inv, acc[cb][3] * inv, In{})};
            *reinterpret_cast<u32x2*>(orow + 16 * cb) = o;
        }
    }
}

AttnArgs make_args(const Problem& p, float scale, int64_t ng = 0) {
    AttnArgs a;
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
    a.ngb = (ng + 15) / 16;   // global rows are taken 16 per workgroup
    return a;
}

template <class In, int D, int kMode>
void launch_mode(const void* q, const void* k, const void* v, void* out, const int32_t* glob,
                 AttnArgs a, int64_t b, hipStream_t stream) {
    using ST = typename In::T;
    if (kMode == kGlobalRows) a.groups = b * a.h * a.ngb;
    launch_kernel(attn_fwd_kernel<In, D, kMode>, dim3(static_cast<uint32_t>(a.groups)),
                  dim3(mode_threads(kMode, D)), 0, stream, static_cast<const ST*>(q), static_cast<const ST*>(k),
                  static_cast<const ST*>(v), static_cast<ST*>(out), glob, a);
}

// Without global tokens one pass; with them the rows outside the global set (window and
// global keys), then the global rows over every key - disjoint output rows, one stream.
template <class In, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, void* out, const int32_t* glob,
                    const AttnArgs& a, int64_t b, hipStream_t stream) {
    if (a.ng == 0) {
        launch_mode<In, D, kBand>(q, k, v, out, nullptr, a, b, stream);
    } else {
        launch_mode<In, D, kBandGlobal>(q, k, v, out, glob, a, b, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        launch_mode<In, D, kGlobalRows>(q, k, v, out, glob, a, b, stream);
    }
    return hipGetLastError();
}

template <class In>
hipError_t launch_d(const void* q, const void* k, const void* v, void* out, const int32_t* glob,
                    const AttnArgs& a, int64_t b, int64_t d, hipStream_t stream) {
    switch (d) {
    case 32: return launch_t<In, 32>(q, k, v, out, glob, a, b, stream);
    case 64: return launch_t<In, 64>(q, k, v, out, glob, a, b, stream);
    case 128: return launch_t<In, 128>(q, k, v, out, glob, a, b, stream);
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

// With global tokens the key range of a workgroup (64 + w + w_upper keys) must fit the
// LDS bitmap of global keys.
bool attention_global_supported(const Problem& p, int64_t ng) {
    return 64 + p.w + p.wu <= int64_t(kBitWords) * 32 && ng >= 0 && ng <= p.n &&
           p.b * p.h * ((ng + 15) / 16) < (int64_t(1) << 31);
}

int64_t attention_workgroups(const Problem& p) { return make_args(p, 1.0f).groups; }

hipError_t launch_attention(const void* q, const void* k, const void* v, void* out,
                            const int32_t* glob, int64_t ng, const Problem& p, float scale,
                            int dt, hipStream_t stream) {
    const AttnArgs a = make_args(p, scale, ng);
    if (a.groups == 0) return hipSuccess;
    switch (dt) {
    case kF16: return launch_d<F16>(q, k, v, out, glob, a, p.b, p.d, stream);
    case kBF16: return launch_d<BF16>(q, k, v, out, glob, a, p.b, p.d, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace diagmm
