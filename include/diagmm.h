/*
 * libdiagmm - the Longformer "diagonaled matmul" family on AMD Instinct MI355X (gfx950).
 *
 * The operation (TVM Discuss, "Developing a faster schedule for Longformer's kernel",
 * post 1): a banded matrix product that evaluates only selected diagonals of Q.K^T -
 * a sliding window of w diagonals to the left of the main one and w_upper to the right
 * (post 5), optionally dilated, i.e. with gaps between the selected diagonals
 * (post 3; 0 means no gaps).  Post 6 lists one forward function (result last
 * dimension 2w+1) and two backward functions selected by transpose_t1, whose first
 * operand is the band.  This library has one call per function, plus the attention
 * softmax that sits between the forward calls (csarofeen/pytorch issue 2096, first
 * fusion repro: scale, row max, subtract, exp, row sum, divide).
 *
 * Notation used below
 *   b, n, h, d   batch, sequence length, heads, head dimension
 *   w, w_upper   diagonals to the left / right of the main one (w_upper "should be 0 or
 *                w" on the pages; any value >= 0 is accepted)
 *   K            w + w_upper + 1, slots per band row
 *   s            max(dilation, 1): dilation 0 and 1 both select contiguous diagonals;
 *                dilation 3 selects every third one
 *   j(i, k)      i + (k - w) * s, the key position of slot k of row i.  Slot w is the
 *                main diagonal; slots below w look left, slots above look right.  A slot
 *                is in range when 0 <= j(i, k) < n.
 *
 * Layouts (all row-major and contiguous, element offsets are 64-bit)
 *   dense   [b][n][h][d]   (Q, K, V, X, dense outputs)
 *   band    [b][n][h][K]
 *
 * Types: inputs are f32, f16 or bf16 (both operands of one call share the type);
 * outputs are the input type or f32.  Products accumulate in f32 and are rounded
 * once, to nearest even, into the output type.
 *
 * Ownership and streams: every pointer is a device pointer owned by the caller.  The
 * library never allocates, frees or synchronises; each call only enqueues kernels on
 * `stream` (a hipStream_t; NULL is the default stream) and returns.  Calls are
 * thread-safe; the only state is the calling thread's last-error text.
 *
 * Errors: every call returns a diagmm_status_t and never aborts.  On any status other
 * than DIAGMM_OK nothing has been enqueued, except DIAGMM_ERR_HIP, which reports a
 * failed launch (the text from the HIP runtime is in diagmm_last_error()).  A call
 * with b * n * h == 0 returns DIAGMM_OK and enqueues nothing.
 */
#ifndef DIAGMM_H
#define DIAGMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIAGMM_ABI_VERSION 9

typedef enum {
    DIAGMM_F32 = 0,
    DIAGMM_F16 = 1,
    DIAGMM_BF16 = 2
} diagmm_dtype_t;

typedef enum {
    DIAGMM_OK = 0,
    DIAGMM_ERR_NULL = 1,        /* a required pointer is NULL */
    DIAGMM_ERR_SHAPE = 2,       /* negative size, d < 1, or an element count past int64 */
    DIAGMM_ERR_DTYPE = 3,       /* unknown dtype, or an unsupported in/out pair */
    DIAGMM_ERR_ALIAS = 4,       /* the output overlaps an input */
    DIAGMM_ERR_UNSUPPORTED = 5, /* valid arguments this build cannot run */
    DIAGMM_ERR_HIP = 6          /* the HIP runtime rejected a launch */
} diagmm_status_t;

/*
 * diagmm_qk - the forward function (post 6: t1 = Q, t2 = K, t3 = result, t3d3 = 2w+1).
 *   band[bb,i,hh,k] = sum_c q[bb,i,hh,c] * k[bb,j(i,k),hh,c]   for in-range slots,
 *   band[bb,i,hh,k] = padding_value                             otherwise.
 * q, k      dense [b][n][h][d] of in_dtype (read only)
 * band      band  [b][n][h][K] of out_dtype (written in full)
 * padding_value is rounded once (nearest even) to out_dtype and stored bit-exactly in
 * every out-of-range slot ("padding: any const", posts 5 and 6); -inf and -0.0 allowed.
 * The band must not overlap q or k (DIAGMM_ERR_ALIAS).
 */
diagmm_status_t diagmm_qk(const void* q, const void* k, void* band, int64_t b, int64_t n,
                          int64_t h, int64_t d, int64_t w, int64_t w_upper, int64_t dilation,
                          float padding_value, diagmm_dtype_t in_dtype,
                          diagmm_dtype_t out_dtype, void* stream);

/*
 * diagmm_pv - backward function with transpose_t1 = 0 (post 6: t1 is the band, last
 * dimension 2w+1); in the forward pass it is probabilities times V.
 *   out[bb,i,hh,c] = sum over in-range slots k of band[bb,i,hh,k] * v[bb,j(i,k),hh,c]
 * band      band  [b][n][h][K] of in_dtype; out-of-range slots are never read into the
 *           sum (skipped by index, so NaN or garbage there has no effect)
 * v         dense [b][n][h][d] of in_dtype
 * out       dense [b][n][h][d] of out_dtype (written in full)
 * padding_value is accepted for a uniform signature and ignored.
 */
diagmm_status_t diagmm_pv(const void* band, const void* v, void* out, int64_t b, int64_t n,
                          int64_t h, int64_t d, int64_t w, int64_t w_upper, int64_t dilation,
                          float padding_value, diagmm_dtype_t in_dtype,
                          diagmm_dtype_t out_dtype, void* stream);

/*
 * diagmm_pvT - backward function with transpose_t1 = 1 (post 6): the band is used
 * transposed, as for the gradients of K and V.
 *   out[bb,j,hh,c] = sum over (i, k) with j(i,k) = j of band[bb,i,hh,k] * x[bb,i,hh,c]
 * (for each j and k the only candidate is i = j - (k - w) * s, taken when 0 <= i < n).
 * band, x, out, padding_value: as for diagmm_pv.
 */
diagmm_status_t diagmm_pvT(const void* band, const void* x, void* out, int64_t b, int64_t n,
                           int64_t h, int64_t d, int64_t w, int64_t w_upper,
                           int64_t dilation, float padding_value, diagmm_dtype_t in_dtype,
                           diagmm_dtype_t out_dtype, void* stream);

/*
 * diagmm_banded_softmax - attention softmax over each band row (issue 2096 recipe).
 *   x_k = scale * scores[bb,i,hh,k] for in-range slots, -inf for the others;
 *   probs[bb,i,hh,k] = exp(x_k - max_k x) / sum_k exp(x_k - max_k x).
 * Out-of-range slots become exactly +0.  Every row holds slot w (key i), so no row is
 * empty.  scores and probs are band [b][n][h][K]; probs may be the same pointer as
 * scores (in place) when in_dtype == out_dtype; any other overlap is DIAGMM_ERR_ALIAS.
 */
diagmm_status_t diagmm_banded_softmax(const void* scores, void* probs, int64_t b, int64_t n,
                                      int64_t h, int64_t w, int64_t w_upper,
                                      int64_t dilation, float scale, diagmm_dtype_t in_dtype,
                                      diagmm_dtype_t out_dtype, void* stream);

/*
 * diagmm_banded_softmax_masked - diagmm_banded_softmax with the attention mask of the
 * issue 2096 repro: key_mask is float32 [b][n] on the device (1 keeps key j, 0 masks it;
 * any value is used linearly), and
 *   x_k = scale * scores[bb,i,hh,k] + (1 - key_mask[bb, i + (k - w) * s]) * mask_value
 * for in-range slots (mask_value -10000 on the page), -inf for the others; then max,
 * exp, sum and divide as diagmm_banded_softmax.  Its gradient with respect to scores is
 * diagmm_banded_softmax_backward's (the mask term does not depend on the scores).
 * probs may be scores itself with equal dtypes; probs overlapping key_mask, or scores
 * other than exactly, is DIAGMM_ERR_ALIAS; key_mask NULL is DIAGMM_ERR_NULL.
 */
diagmm_status_t diagmm_banded_softmax_masked(const void* scores, void* probs,
                                             const float* key_mask, int64_t b, int64_t n,
                                             int64_t h, int64_t w, int64_t w_upper,
                                             int64_t dilation, float scale, float mask_value,
                                             diagmm_dtype_t in_dtype, diagmm_dtype_t out_dtype,
                                             void* stream);

/*
 * diagmm_banded_softmax_backward - gradient of diagmm_banded_softmax with respect to its
 * stored scores, given its output probs and the gradient dprobs of a loss with respect
 * to probs (the chain rule through the issue 2096 recipe; the pages print only the
 * forward, and say the kernel's two backward functions of post 6 multiply a band
 * gradient, the one this call produces):
 *   dscores[bb,i,hh,k] = scale * probs[k] * (dprobs[k] - sum_m probs[m] * dprobs[m])
 * over the row's in-range slots k, m; out-of-range slots of dscores become exactly +0,
 * and out-of-range slots of probs and dprobs are never read into the sum (any value,
 * NaN included, is ignored).  probs, dprobs and dscores are band tensors [b][n][h][K]
 * of one dtype (f32, f16 or bf16; accumulation in f32, the result rounded to nearest
 * even).  dscores may be the same pointer as probs or as dprobs (in place); any other
 * overlap with them is DIAGMM_ERR_ALIAS.  Errors as for the other calls.
 */
diagmm_status_t diagmm_banded_softmax_backward(const void* probs, const void* dprobs,
                                               void* dscores, int64_t b, int64_t n,
                                               int64_t h, int64_t w, int64_t w_upper,
                                               int64_t dilation, float scale,
                                               diagmm_dtype_t dtype, void* stream);

/*
 * diagmm_banded_dropout - dropout on a probability band, as in the issue 2096 repro
 * (a uniform random tensor of the band's shape compared with the drop probability, the
 * kept values scaled by 1 / (1 - p)):
 *   out[bb,i,hh,k] = probs[bb,i,hh,k] / (1 - p)   if rand[bb,i,hh,k] > p and slot k is in
 *                                                 range (0 <= i + (k - w) * s < n),
 *                    +0                           otherwise.
 * The random numbers are an input: rand is float32 [b][n][h][K] on the device (any
 * values; a slot is kept when its float32 rand compares greater than p, so rand == p
 * drops), drawn by the caller.  With the same rand, the call applied to the gradient of
 * a loss with respect to out gives its gradient with respect to probs.  probs and out
 * are band tensors [b][n][h][K] of one dtype (f32, f16 or bf16; the product in f32 with
 * 1 / (1 - p) rounded to f32 once, then rounded to nearest even).  p in [0, 1), else
 * DIAGMM_ERR_SHAPE.  out may be probs itself (in place); any other overlap with probs,
 * or any overlap with rand, is DIAGMM_ERR_ALIAS.  Errors otherwise as for the other calls.
 */
diagmm_status_t diagmm_banded_dropout(const void* probs, const float* rand, void* out,
                                      int64_t b, int64_t n, int64_t h, int64_t w,
                                      int64_t w_upper, int64_t dilation, float p,
                                      diagmm_dtype_t dtype, void* stream);

/*
 * diagmm_banded_attention - sliding-window attention in one pass, the band never written:
 *   out[bb,i,hh,:] = sum_k P_k V[bb,j_k,hh,:],   j_k = i + (k - w) * s,
 *   P = softmax over the in-range slots k of x_k = scale * sum_c Q[bb,i,hh,c] K[bb,j_k,hh,c]
 * - diagmm_qk, diagmm_banded_softmax and diagmm_pv composed ([TVM] post 6 forward and
 * transpose_t1 = 0 functions, the issue 2096 softmax recipe), with the scores and
 * probabilities kept in float32 registers (the probabilities enter the second product
 * rounded to the input dtype, as the three-call path stores them).  q, k, v and out are
 * [b][n][h][d] of one dtype: f16 or bf16 with d in {32, 64, 128} and 16-byte aligned
 * pointers, else DIAGMM_ERR_UNSUPPORTED (use the three calls).  out overlapping q, k or
 * v is DIAGMM_ERR_ALIAS.  Errors otherwise as for the other calls.
 */
diagmm_status_t diagmm_banded_attention(const void* q, const void* k, const void* v, void* out,
                                        int64_t b, int64_t n, int64_t h, int64_t d, int64_t w,
                                        int64_t w_upper, int64_t dilation, float scale,
                                        diagmm_dtype_t dtype, void* stream);

/*
 * diagmm_banded_attention_global - diagmm_banded_attention with global tokens, as in the
 * LongformerAttention op of onnxruntime issue 12448 (a sliding window plus global tokens,
 * with Global_Q, Global_K and Global_V matrices beside Q, K and V: description and
 * conclusion (d)).  global_pos is int32 [b][ng] on the device; batch bb's global set is
 * the set of its entries that lie in [0, n) (a repeated position is one member, an entry
 * outside [0, n) names none).  A row outside the set attends the keys of its window and
 * every global key, each key once, with q, k and v; a global row attends every key of
 * the sequence with global_q, global_k and global_v ([b][n][h][d] like q, read at the
 * global positions and every key; all three NULL: q, k and v).  ng = 0 is
 * diagmm_banded_attention.
 *
 * workspace: device memory of at least diagmm_banded_attention_global_workspace bytes,
 * 256-byte aligned, owned by the caller, used by this call's two kernels on `stream`
 * (the positions of the global rows and their partial softmax states); its
 * contents on entry do not matter.  Calls sharing a workspace must be ordered on one
 * stream.  NULL is allowed when that size is 0 (ng = 0).
 *
 * Errors: ng outside [0, n] is DIAGMM_ERR_SHAPE, and so is workspace_bytes below the
 * size needed; a NULL pointer where data is needed, or one or two of the global matrices
 * NULL, is DIAGMM_ERR_NULL; out overlapping any input or the workspace, or the workspace
 * overlapping an input, is DIAGMM_ERR_ALIAS; besides the shapes diagmm_banded_attention
 * refuses, windows with 64 + w + w_upper > 16384, n > 65536 with ng > 0, a workspace not
 * 256-byte aligned or unaligned global matrices are DIAGMM_ERR_UNSUPPORTED.
 */
diagmm_status_t diagmm_banded_attention_global(const void* q, const void* k, const void* v,
                                               const void* global_q, const void* global_k,
                                               const void* global_v, void* out,
                                               const int32_t* global_pos, int64_t ng,
                                               int64_t b, int64_t n, int64_t h, int64_t d,
                                               int64_t w, int64_t w_upper, int64_t dilation,
                                               float scale, diagmm_dtype_t dtype,
                                               void* workspace, int64_t workspace_bytes,
                                               void* stream);

/*
 * diagmm_banded_attention_global_noalloc - diagmm_banded_attention_global for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same operation and checks, with no workspace
 * argument.  The workspace is a static 32 MiB device array of the library (one per GPU,
 * held until the process ends); the call allocates nothing.  Sizes that need more than
 * 32 MiB of workspace (diagmm_banded_attention_global_workspace) are
 * DIAGMM_ERR_UNSUPPORTED.  All calls of a process on one GPU share that GPU's array:
 * calls that may overlap in time there (on different streams, or from threads without
 * ordering between them) race and must not be issued.  The array is found on the calling
 * thread's current device, which must be the device of `stream`.
 */
diagmm_status_t diagmm_banded_attention_global_noalloc(
    const void* q, const void* k, const void* v, const void* global_q, const void* global_k,
    const void* global_v, void* out, const int32_t* global_pos, int64_t ng, int64_t b,
    int64_t n, int64_t h, int64_t d, int64_t w, int64_t w_upper, int64_t dilation, float scale,
    diagmm_dtype_t dtype, void* stream);

/*
 * Workspace bytes diagmm_banded_attention_global needs for these sizes (0 when ng = 0)
 * in *bytes.  DIAGMM_ERR_SHAPE for sizes that call would refuse as such, DIAGMM_ERR_NULL
 * for a NULL bytes.
 */
diagmm_status_t diagmm_banded_attention_global_workspace(int64_t b, int64_t n, int64_t h,
                                                         int64_t d, int64_t w, int64_t w_upper,
                                                         int64_t dilation, int64_t ng,
                                                         int64_t* bytes);

/* Static text for a status code. */
const char* diagmm_status_string(diagmm_status_t status);

/* Detail of the calling thread's most recent failure ("" if none). */
const char* diagmm_last_error(void);

/* DIAGMM_ABI_VERSION of the loaded library. */
int diagmm_abi_version(void);

/*
 * Band-tile scheduler introspection (host only, no device access).  Describes how a
 * call with these arguments is cut into workgroups: which kernel runs, the tile shape
 * (rows per tile, slots per tile), how many tiles and workgroups, the LDS bytes per
 * workgroup, and how many residue classes the dilation splits the rows into.
 * mode: 0 = qk, 1 = pv, 2 = pvT, 3 = banded softmax, 4 = banded softmax backward,
 * 6 = banded dropout, 7 = attention in one pass (the timing tags; 5, the masked softmax,
 * has no plan).  Modes 4, 6 and 7 are planned for 16-byte aligned tensors, and out_dtype
 * must equal in_dtype; for 6 rows_per_tile is 0, slots_per_tile the band elements a
 * workgroup takes and tiles the workgroups; for 7 a tile is 64 rows of one residue class
 * with keys staged 64 at a time (slots_per_tile), one workgroup per tile.  Returns DIAGMM_ERR_SHAPE /
 * DIAGMM_ERR_DTYPE for invalid arguments, as the compute calls would.
 */
typedef struct {
    char kernel[48];        /* kernel family chosen, e.g. "qk_mfma_f16" or "qk_simple" */
    int64_t rows_per_tile;  /* output rows per tile (per residue class) */
    int64_t slots_per_tile; /* band slots (or dense columns) per tile */
    int64_t tiles;          /* total tiles */
    int64_t workgroups;     /* workgroups launched */
    int64_t threads;        /* threads per workgroup */
    int64_t lds_bytes;      /* LDS per workgroup */
    int64_t residues;       /* residue classes the rows are split into (s) */
    int64_t strip_workgroups; /* pv, pvT: workgroups given to each strip (the row blocks of
                                 one residue class of one (batch, head)) when the tiles are
                                 split strip by strip; 0 when they are balanced over all
                                 workgroups at once.  qk: the row ranges each strip is cut
                                 into (a workgroup takes one range, or a run of them) */
    int64_t interleaved;    /* pv, pvT: 1 when each XCD's tiles are dealt round-robin over
                               its workgroups (neighbouring tiles run at the same time and
                               share the cache lines they both read in L2), 0 when a
                               workgroup takes a contiguous run of tiles; 0 for the other
                               modes */
} diagmm_plan_t;

diagmm_status_t diagmm_plan(int mode, int64_t b, int64_t n, int64_t h, int64_t d, int64_t w,
                            int64_t w_upper, int64_t dilation, diagmm_dtype_t in_dtype,
                            diagmm_dtype_t out_dtype, diagmm_plan_t* plan);

/*
 * Kernel timers, a measurement aid for benchmarks (not part of the method).  Between
 * diagmm_timing_begin(capacity) and diagmm_timing_end(), each of the next `capacity`
 * kernel launches by this library records a pair of HIP events at the kernel's own start
 * and end on the stream it is launched on (hipExtLaunchKernel), tagged with the entry
 * point (the diagmm_plan modes: 0 qk, 1 pv, 2 pvT, 3 banded softmax, 4 its backward;
 * 5 the masked softmax, 6 dropout, 7 attention in one pass); further launches
 * run untimed.  One session at a time, process-wide, on one device (the events are made
 * on the device current at diagmm_timing_begin; launches on another device are not to be
 * timed).  diagmm_timing_read waits for the recorded kernels and writes, for the first
 * min(max, count) launches in launch order, the entry point tag (ops[i]) and the kernel
 * time in milliseconds (ms[i]); *count receives the number of launches recorded.  The
 * arrays are host memory owned by the caller.  Errors: DIAGMM_ERR_SHAPE for capacity
 * outside 1 .. 2^20, DIAGMM_ERR_NULL for a null count (or null arrays with max > 0),
 * DIAGMM_ERR_HIP if an event call fails.
 */
diagmm_status_t diagmm_timing_begin(int64_t capacity);
diagmm_status_t diagmm_timing_end(void);
diagmm_status_t diagmm_timing_read(int64_t max, int32_t* ops, double* ms, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* DIAGMM_H */
