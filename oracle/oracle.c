/*
 * CPU oracle for the Longformer "diagonaled matmul" family and its banded softmax.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file or the library built from it; only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark do.  It shares no code with the HIP
 * library: its own element conversions, its own index arithmetic, its own loops.
 *
 * What is computed (sources are the three web pages the method is described on):
 *
 *   TVM Discuss, "Developing a faster schedule for Longformer's kernel":
 *     post 1   - the kernel is a banded matrix product that evaluates only certain
 *                diagonals of the output matrix (figures 2.b / 2.c of the
 *                Longformer paper: sliding window, optionally dilated);
 *     post 3   - dilation is the gap between the selected diagonals, 0 = none;
 *     post 5   - parameters b, n, h, m, w, w_upper, padding, transpose_t1, t1d3, t3d3;
 *                w_upper is the window to the right of the word;
 *     post 6   - one forward function (last dim of the result t3d3 = 2w+1) and two
 *                backward functions told apart by transpose_t1, whose first operand
 *                t1 is the band (last dim 2w+1); "padding" is any constant.
 *   csarofeen/pytorch issue 2096, first fusion repro: the attention softmax recipe
 *     (scale the scores, take the row max, subtract, exp, row sum, divide).
 *
 * Readings where the pages leave a step open (each is listed in the design notes):
 *   - stride s = max(dilation, 1): 0 and 1 both mean contiguous diagonals, and
 *     dilation 3 puts slot k of row i on key i + (k - w) * 3;
 *   - K = w + w_upper + 1 slots per row; slot k is key offset (k - w) * s, so slots
 *     below w look left, slot w is the main diagonal, slots above w look right;
 *   - a slot whose key index falls outside [0, n) is "out of range": qk writes the
 *     padding constant there; pv / pvT skip such terms by index, whatever the band
 *     holds; the banded softmax masks them to -inf, so their probability is 0;
 *   - dense layout [b][n][h][d], band layout [b][n][h][K], both contiguous.
 *
 * The banded softmax backward is not printed on the pages: it is the derivative of the
 * softmax recipe above with respect to the stored scores, the operation that feeds
 * the two backward functions of post 6 the band gradient they multiply.
 *
 * Arithmetic: every element is widened exactly to double, products and sums are
 * formed in double, and the result is rounded once, to nearest-even, to the output
 * type (OR_F64 keeps the unrounded double, for tolerance checks).
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 };

/* ---------------------------------------------------------------- conversions */

static double or_half_to_double(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1024 + m) * 2^(e - 15 - 10) */
    return sign ? -v : v;
}

static double or_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round x to the nearest multiple of 2^qexp, ties to even (rint in the default
 * rounding mode); scaling by a power of two is exact in double. */
static double or_round_to_quantum(double x, int qexp)
{
    return ldexp(rint(ldexp(x, -qexp)), qexp);
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits; max 65504. */
static uint16_t or_double_to_half(double x)
{
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1): unbiased exponent is e - 1 */
    int E = e - 1;
    int qexp = (E < -14) ? -24 : E - 10;
    double r = or_round_to_quantum(a, qexp);
    if (r > 65504.0) return sign | 0x7c00;
    if (r < ldexp(1.0, -14)) /* subnormal (or rounded up to exactly 2^-14, same bits) */
        return sign | (uint16_t)ldexp(r, 24);
    frexp(r, &e);
    E = e - 1;
    uint16_t mant = (uint16_t)(ldexp(r, 10 - E) - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | mant;
}

/* bfloat16: the upper half of a binary32; 8 exponent bits, 7 mantissa bits. */
static uint16_t or_double_to_bf16(double x)
{
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7f80;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    int E = e - 1;
    int qexp = (E < -126) ? -133 : E - 7;
    double r = or_round_to_quantum(a, qexp);
    if (r > 3.3895313892515355e38) return sign | 0x7f80; /* above the largest finite */
    float f = (float)r;    /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

static double or_load(const void* p, int64_t idx, int dt)
{
    switch (dt) {
    case OR_F32: return (double)((const float*)p)[idx];
    case OR_F16: return or_half_to_double(((const uint16_t*)p)[idx]);
    case OR_BF16: return or_bf16_to_double(((const uint16_t*)p)[idx]);
    default: return ((const double*)p)[idx];
    }
}

static void or_store(void* p, int64_t idx, int dt, double v)
{
    switch (dt) {
    case OR_F32: ((float*)p)[idx] = (float)v; break; /* C cast: round to nearest even */
    case OR_F16: ((uint16_t*)p)[idx] = or_double_to_half(v); break;
    case OR_BF16: ((uint16_t*)p)[idx] = or_double_to_bf16(v); break;
    default: ((double*)p)[idx] = v; break;
    }
}

/* Exposed for the tests that pin the conversions against library routines. */
void oracle_convert(const double* x, void* out, int64_t count, int dt)
{
    for (int64_t t = 0; t < count; ++t) or_store(out, t, dt, x[t]);
}

void oracle_widen(const void* x, double* out, int64_t count, int dt)
{
    for (int64_t t = 0; t < count; ++t) out[t] = or_load(x, t, dt);
}

/* ------------------------------------------------------------------ indexing */

static int64_t or_stride(int64_t dilation) { return dilation > 1 ? dilation : 1; }

static int or_check(int64_t b, int64_t n, int64_t h, int64_t d, int64_t w, int64_t wu,
                    int64_t dil, int in_dt, int out_dt)
{
    if (b < 0 || n < 0 || h < 0 || d < 1 || w < 0 || wu < 0 || dil < 0) return 1;
    if (in_dt < OR_F32 || in_dt > OR_F64 || out_dt < OR_F32 || out_dt > OR_F64) return 2;
    return 0;
}

/* Row list: rows[r] is a flattened (batch, position) index bb * n + i.  When rows is
 * NULL every row is computed, in order.  Otherwise only the listed rows are, and every
 * row-local operand (Q for qk, the band for pv and the softmax, and the output) is
 * packed: its row r belongs to position rows[r].  Operands reached through the index
 * map (K, V, X, and the band of pvT) are always the full [b][n][h][.] tensors. */
static int64_t or_row(const int64_t* rows, int64_t r) { return rows ? rows[r] : r; }

/* ------------------------------------------------------------------ qk
 * band[bb,i,hh,k] = sum_c Q[bb,i,hh,c] * K[bb,j,hh,c]   with j = i + (k - w) * s,
 * and = padding where j is outside [0, n).  The forward function of the pages'
 * kernel: t1 = Q, t2 = K, t3 = the band with last dimension w + w_upper + 1. */
int oracle_qk(const void* q, const void* kmat, void* out, int64_t b, int64_t n, int64_t h,
              int64_t d, int64_t w, int64_t wu, int64_t dil, double pad, int in_dt,
              int out_dt, const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, d, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t bi = or_row(rows, r), bb = bi / n, i = bi % n;
        for (int64_t hh = 0; hh < h; ++hh) {
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                const int64_t o = (r * h + hh) * K + k;
                if (j < 0 || j >= n) {
                    or_store(out, o, out_dt, pad);
                    continue;
                }
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc += or_load(q, (r * h + hh) * d + c, in_dt) *
                           or_load(kmat, ((bb * n + j) * h + hh) * d + c, in_dt);
                or_store(out, o, out_dt, acc);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ pv
 * out[bb,i,hh,c] = sum_k P[bb,i,hh,k] * V[bb,j,hh,c] over the slots k whose key
 * j = i + (k - w) * s is inside [0, n).  The backward function with transpose_t1 = 0:
 * t1 is the band (last dimension 2w+1 when w_upper = w), t2 is dense. */
int oracle_pv(const void* band, const void* v, void* out, int64_t b, int64_t n, int64_t h,
              int64_t d, int64_t w, int64_t wu, int64_t dil, int in_dt, int out_dt,
              const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, d, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t bi = or_row(rows, r), bb = bi / n, i = bi % n;
        for (int64_t hh = 0; hh < h; ++hh) {
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t j = i + (k - w) * s;
                    if (j < 0 || j >= n) continue;
                    acc += or_load(band, (r * h + hh) * K + k, in_dt) *
                           or_load(v, ((bb * n + j) * h + hh) * d + c, in_dt);
                }
                or_store(out, (r * h + hh) * d + c, out_dt, acc);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ pvT
 * The backward function with transpose_t1 = 1: the band is used transposed.
 * out[bb,j,hh,c] = sum over the pairs (i, k) with i + (k - w) * s = j of
 *                  G[bb,i,hh,k] * X[bb,i,hh,c];
 * for each output row j and slot k there is exactly one candidate
 * i = j - (k - w) * s, taken when it lies inside [0, n). */
int oracle_pvT(const void* band, const void* x, void* out, int64_t b, int64_t n, int64_t h,
               int64_t d, int64_t w, int64_t wu, int64_t dil, int in_dt, int out_dt,
               const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, d, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t bj = or_row(rows, r), bb = bj / n, j = bj % n;
        for (int64_t hh = 0; hh < h; ++hh) {
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t i = j - (k - w) * s;
                    if (i < 0 || i >= n) continue;
                    acc += or_load(band, ((bb * n + i) * h + hh) * K + k, in_dt) *
                           or_load(x, ((bb * n + i) * h + hh) * d + c, in_dt);
                }
                or_store(out, (r * h + hh) * d + c, out_dt, acc);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ softmax
 * Per (bb, i, hh) row of K slots: x_k = scale * S[k] for in-range slots, -inf for
 * the others; P_k = exp(x_k - max x) / sum_k exp(x_k - max x).  Out-of-range slots
 * get exactly 0.  The row always holds slot w (key i itself), so it is never empty.
 * The recipe (scale, max, subtract, exp, sum, divide) is the attention softmax of
 * the first fusion repro on the csarofeen/pytorch issue 2096 page. */
int oracle_softmax(const void* scores, void* probs, int64_t b, int64_t n, int64_t h,
                   int64_t w, int64_t wu, int64_t dil, double scale, int in_dt, int out_dt,
                   const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, 1, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = or_row(rows, r) % n;
        for (int64_t hh = 0; hh < h; ++hh) {
            const int64_t row = (r * h + hh) * K;
            double m = -INFINITY;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                if (j < 0 || j >= n) continue;
                const double x = scale * or_load(scores, row + k, in_dt);
                if (x > m) m = x;
            }
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                if (j < 0 || j >= n) continue;
                sum += exp(scale * or_load(scores, row + k, in_dt) - m);
            }
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                double p = 0.0;
                if (j >= 0 && j < n) p = exp(scale * or_load(scores, row + k, in_dt) - m) / sum;
                or_store(probs, row + k, out_dt, p);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ softmax backward
 * Per (bb, i, hh) row, with P the probabilities of the banded softmax above and dP the
 * gradient of a loss with respect to them: the gradient with respect to the stored
 * scores S is, by the chain rule through x_k = scale * S[k] and P = softmax(x),
 *     dS_k = scale * P_k * (dP_k - sum_m P_m dP_m)      for in-range slots k, m,
 *     dS_k = 0                                           for out-of-range slots,
 * out-of-range slots of P and dP never entering the sum (they are masked by index, as
 * in the forward softmax, whatever they hold). */
int oracle_softmax_bwd(const void* probs, const void* dprobs, void* dscores, int64_t b,
                       int64_t n, int64_t h, int64_t w, int64_t wu, int64_t dil, double scale,
                       int in_dt, int out_dt, const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, 1, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = or_row(rows, r) % n;
        for (int64_t hh = 0; hh < h; ++hh) {
            const int64_t row = (r * h + hh) * K;
            double dot = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                if (j < 0 || j >= n) continue;
                dot += or_load(probs, row + k, in_dt) * or_load(dprobs, row + k, in_dt);
            }
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                double g = 0.0;
                if (j >= 0 && j < n)
                    g = scale * or_load(probs, row + k, in_dt) *
                        (or_load(dprobs, row + k, in_dt) - dot);
                or_store(dscores, row + k, out_dt, g);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ masked softmax
 * The attention softmax of the first fusion repro on the csarofeen/pytorch issue 2096
 * page with its attention mask: a per-key mask m[bb, j] (1 keeps key j, 0 masks it;
 * any value is used linearly) adds (1 - m) * mask_value (-10000 there) to the scaled
 * score before the row max:
 *     x_k = scale * S[k] + (1 - m[bb, j]) * mask_value,   j = i + (k - w) * s,
 * for in-range slots; out-of-range slots are -inf as in oracle_softmax, so their
 * probability is exactly 0.  key_mask is float32 [b][n] (the full batch, also when a
 * row list is given: it is reached through the key index). */
int oracle_softmax_masked(const void* scores, void* probs, const float* key_mask, int64_t b,
                          int64_t n, int64_t h, int64_t w, int64_t wu, int64_t dil,
                          double scale, double mask_value, int in_dt, int out_dt,
                          const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, 1, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    if (!key_mask) return 1;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t bn = or_row(rows, r), i = bn % n, bb = bn / n;
        for (int64_t hh = 0; hh < h; ++hh) {
            const int64_t row = (r * h + hh) * K;
            double m = -INFINITY;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                if (j < 0 || j >= n) continue;
                const double x = scale * or_load(scores, row + k, in_dt) +
                                 (1.0 - (double)key_mask[bb * n + j]) * mask_value;
                if (x > m) m = x;
            }
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                if (j < 0 || j >= n) continue;
                sum += exp(scale * or_load(scores, row + k, in_dt) +
                           (1.0 - (double)key_mask[bb * n + j]) * mask_value - m);
            }
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                double p = 0.0;
                if (j >= 0 && j < n)
                    p = exp(scale * or_load(scores, row + k, in_dt) +
                            (1.0 - (double)key_mask[bb * n + j]) * mask_value - m) / sum;
                or_store(probs, row + k, out_dt, p);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ dropout
 * The dropout of the first fusion repro on the csarofeen/pytorch issue 2096 page, on
 * the band: a slot is kept when its uniform random number exceeds p, and a kept
 * probability is scaled by 1 / (1 - p) (1.11111 there, for p = 0.1):
 *     out[k] = rand[k] > p ? probs[k] / (1 - p) : 0     for in-range slots,
 *     out[k] = 0                                        for out-of-range slots.
 * The random numbers are an input (float32, one per band element), so the keep decision
 * is the same comparison on both sides; it is taken in float32 (rand and p as floats). */
int oracle_dropout(const void* probs, const float* rand, void* out, int64_t b, int64_t n,
                   int64_t h, int64_t w, int64_t wu, int64_t dil, float p, int in_dt,
                   int out_dt, const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, 1, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    if (!rand || !(p >= 0.0f) || !(p < 1.0f)) return 1;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    const double scale = 1.0 / (1.0 - (double)p);
    if (!rows) nrows = b * n;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = or_row(rows, r) % n;
        for (int64_t hh = 0; hh < h; ++hh) {
            const int64_t row = (r * h + hh) * K;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                double v = 0.0;
                if (j >= 0 && j < n && rand[row + k] > p)
                    v = or_load(probs, row + k, in_dt) * scale;
                or_store(out, row + k, out_dt, v);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ attention
 * Sliding-window attention with the band never stored: the forward function of [TVM]
 * post 6 (scores on the window's diagonals), the softmax of the issue 2096 repro over
 * them (scale, max, subtract, exp, sum, divide), and the backward function with
 * transpose_t1 = 0 applied to the probabilities - one row at a time, in double:
 *     x_k = scale * sum_c Q[bb,i,hh,c] K[bb,j,hh,c],   j = i + (k - w) * s in [0, n),
 *     P_k = exp(x_k - max x) / sum exp(x - max x),
 *     out[bb,i,hh,c] = sum_k P_k V[bb,j,hh,c].
 * Q, K and V are full tensors; a row list selects the output positions (packed). */
int oracle_attention(const void* q, const void* kt, const void* v, void* out, int64_t b,
                     int64_t n, int64_t h, int64_t d, int64_t w, int64_t wu, int64_t dil,
                     double scale, int in_dt, int out_dt, const int64_t* rows, int64_t nrows,
                     int nthreads)
{
    int bad = or_check(b, n, h, d, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    const int64_t K = w + wu + 1, s = or_stride(dil);
    if (!rows) nrows = b * n;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t bi = or_row(rows, r), bb = bi / n, i = bi % n;
        double* x = (double*)malloc((size_t)K * sizeof(double));
        if (!x) { failed = 1; continue; }
        for (int64_t hh = 0; hh < h; ++hh) {
            const int64_t qrow = ((bb * n + i) * h + hh) * d;
            double mx = -INFINITY;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t j = i + (k - w) * s;
                x[k] = -INFINITY;
                if (j < 0 || j >= n) continue;
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc += or_load(q, qrow + c, in_dt) *
                           or_load(kt, ((bb * n + j) * h + hh) * d + c, in_dt);
                x[k] = scale * acc;
                if (x[k] > mx) mx = x[k];
            }
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                x[k] = (x[k] == -INFINITY) ? 0.0 : exp(x[k] - mx);
                sum += x[k];
            }
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t j = i + (k - w) * s;
                    if (j < 0 || j >= n) continue;
                    acc += (x[k] / sum) * or_load(v, ((bb * n + j) * h + hh) * d + c, in_dt);
                }
                or_store(out, (r * h + hh) * d + c, out_dt, acc);
            }
        }
        free(x);
    }
    return failed ? 3 : 0;
}

/* ------------------------------------------------------------------ global tokens
 * Sliding-window attention with global tokens (onnxruntime issue 12448: the
 * LongformerAttention op, a sliding window plus global tokens, whose inputs carry the
 * Global_Q, Global_K and Global_V matrices beside Q, K and V - description, conclusion
 * (d)).  G_bb is the set of positions glob[bb * ng + g], g < ng, that lie in [0, n): a
 * position listed twice is one member, an entry outside [0, n) names no position.
 * A row i outside G_bb attends the keys of its window and every key in G_bb, each key
 * once, with Q, K and V:
 *     keys(i) = { j : j in G, or j = i + (k - w) * s for a slot k },
 *     out[i] = sum_{j in keys(i)} softmax_j(scale * Q[i] . K[j]) V[j];
 * a row i in G_bb attends every key of the sequence with the global matrices:
 *     out[i] = sum_{j < n} softmax_j(scale * GQ[i] . GK[j]) GV[j].
 * gq, gk, gv NULL: the global rows use Q, K and V.  Written directly from those sets,
 * one row at a time in double. */
int oracle_attention_global(const void* q, const void* kt, const void* v, const void* gq,
                            const void* gk, const void* gv, const int64_t* glob, int64_t ng,
                            void* out, int64_t b, int64_t n, int64_t h, int64_t d, int64_t w,
                            int64_t wu, int64_t dil, double scale, int in_dt, int out_dt,
                            const int64_t* rows, int64_t nrows, int nthreads)
{
    int bad = or_check(b, n, h, d, w, wu, dil, in_dt, out_dt);
    if (bad) return bad;
    if (ng < 0 || (ng > 0 && !glob)) return 1;
    if ((gq || gk || gv) && !(gq && gk && gv)) return 1;
    if (!gq) { gq = q; gk = kt; gv = v; }
    const int64_t s = or_stride(dil);
    if (!rows) nrows = b * n;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t bi = or_row(rows, r), bb = bi / n, i = bi % n;
        double* x = (double*)malloc((size_t)n * sizeof(double));
        char* isg = (char*)calloc((size_t)n, 1);
        if (!x || !isg) { free(x); free(isg); failed = 1; continue; }
        for (int64_t g = 0; g < ng; ++g) {
            const int64_t pos = glob[bb * ng + g];
            if (pos >= 0 && pos < n) isg[pos] = 1;
        }
        /* the matrices this row's scores and values come from */
        const void* qm = isg[i] ? gq : q;
        const void* km = isg[i] ? gk : kt;
        const void* vm = isg[i] ? gv : v;
        for (int64_t hh = 0; hh < h; ++hh) {
            const int64_t qrow = ((bb * n + i) * h + hh) * d;
            double mx = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                const int64_t off = j - i;
                const int in_window = off % s == 0 && off >= -w * s && off <= wu * s;
                x[j] = -INFINITY;
                if (!(isg[i] || isg[j] || in_window)) continue;
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc += or_load(qm, qrow + c, in_dt) *
                           or_load(km, ((bb * n + j) * h + hh) * d + c, in_dt);
                x[j] = scale * acc;
                if (x[j] > mx) mx = x[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                x[j] = (x[j] == -INFINITY) ? 0.0 : exp(x[j] - mx);
                sum += x[j];
            }
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < n; ++j)
                    if (x[j] != 0.0)
                        acc += (x[j] / sum) * or_load(vm, ((bb * n + j) * h + hh) * d + c, in_dt);
                or_store(out, (r * h + hh) * d + c, out_dt, acc);
            }
        }
        free(x);
        free(isg);
    }
    return failed ? 3 : 0;
}
