// The C ABI of libdiagmm: argument validation, dtype checks, alias checks, the
// band-tile scheduler's choice of kernel, and error reporting.  Declarations and the
// contract of every entry point are in include/diagmm.h.
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/diagmm.h"
#include "launch.hpp"
#include "sched.hpp"

namespace diagmm {

namespace {

thread_local char g_last_error[512] = "";

diagmm_status_t fail(diagmm_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
diagmm_status_t fail(diagmm_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

diagmm_status_t ok() {
    g_last_error[0] = '\0';
    return DIAGMM_OK;
}

constexpr int64_t kLimit = int64_t(1) << 62;

// a * b without overflow past kLimit; returns -1 on overflow (all operands >= 0).
int64_t mul_checked(int64_t a, int64_t b) {
    if (a == 0 || b == 0) return 0;
    if (a > kLimit / b) return -1;
    return a * b;
}

size_t elem_size(int dt) { return dt == kF32 ? 4 : 2; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

// Shared checks of the four calls.  Fills p and the element counts of the dense and band
// tensors; returns DIAGMM_OK, or the status to return.
diagmm_status_t check_common(const char* fn, int64_t b, int64_t n, int64_t h, int64_t d,
                             int64_t w, int64_t wu, int64_t dil, int in_dt, int out_dt,
                             Problem* p, int64_t* dense_elems, int64_t* band_elems) {
    if (b < 0 || n < 0 || h < 0 || w < 0 || wu < 0 || dil < 0)
        return fail(DIAGMM_ERR_SHAPE, "%s: negative size (b=%lld n=%lld h=%lld w=%lld "
                    "w_upper=%lld dilation=%lld)", fn, (long long)b, (long long)n, (long long)h,
                    (long long)w, (long long)wu, (long long)dil);
    if (d < 1) return fail(DIAGMM_ERR_SHAPE, "%s: d must be >= 1 (got %lld)", fn, (long long)d);
    if (w >= kLimit / 4 || wu >= kLimit / 4 || dil >= kLimit / 4)
        return fail(DIAGMM_ERR_SHAPE, "%s: window or dilation too large", fn);
    const int64_t s = dil > 1 ? dil : 1;
    if (mul_checked(w + 1, s) < 0 || mul_checked(wu + 1, s) < 0 || mul_checked(w + 1, s) > kLimit / 4 ||
        mul_checked(wu + 1, s) > kLimit / 4)
        return fail(DIAGMM_ERR_SHAPE, "%s: window times dilation overflows", fn);
    if (in_dt < kF32 || in_dt > kBF16 || out_dt < kF32 || out_dt > kBF16)
        return fail(DIAGMM_ERR_DTYPE, "%s: unknown dtype code (in=%d out=%d)", fn, in_dt, out_dt);
    if (!(out_dt == in_dt || out_dt == kF32))
        return fail(DIAGMM_ERR_DTYPE, "%s: output dtype must be the input dtype or f32", fn);
    const int64_t K = w + wu + 1;
    const int64_t rows = mul_checked(mul_checked(b, n), h);
    const int64_t de = rows < 0 ? -1 : mul_checked(rows, d);
    const int64_t be = rows < 0 ? -1 : mul_checked(rows, K);
    if (rows < 0 || de < 0 || be < 0 || be > kLimit / 8 || de > kLimit / 8)
        return fail(DIAGMM_ERR_SHAPE, "%s: element count overflows int64", fn);
    *p = Problem{b, n, h, d, w, wu, s, K};
    *dense_elems = de;
    *band_elems = be;
    return DIAGMM_OK;
}

diagmm_status_t launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(DIAGMM_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev >= 64) dev = 63;
    if (cached[dev] <= 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    // DIAGMM_MAX_WORKGROUPS=m caps the persistent grids at m workgroups (a testing switch:
    // on a small grid each workgroup walks many tiles, strip changes included).
    int cus = cached[dev];
    if (const char* e = std::getenv("DIAGMM_MAX_WORKGROUPS")) {
        const int m = std::atoi(e);
        if (m >= 1 && m < cus) cus = m;
    }
    return cus;
}

// Round-to-nearest-even of a float into the 16-bit types, on the host.
uint32_t pad_bits(float value, int out_dtype) {
    uint32_t u;
    std::memcpy(&u, &value, sizeof u);
    if (out_dtype == kF32) return u;
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t mag = u & 0x7fffffffu;
    if (out_dtype == kBF16) {
        if (mag > 0x7f800000u) return sign | 0x7fc0u;
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    }
    // binary16
    if (mag > 0x7f800000u) return sign | 0x7e00u;         // NaN
    if (mag >= 0x477ff000u) return sign | 0x7c00u;        // >= 65520 rounds to infinity
    if (mag < 0x33000000u) return sign;                   // < 2^-25 rounds to zero
    const int exp = static_cast<int>(mag >> 23) - 127;
    uint32_t mant = (mag & 0x7fffffu) | 0x800000u;        // 24-bit significand
    int shift;                                            // bits to drop
    uint32_t base;
    if (exp < -14) {                                      // half subnormal: quantum 2^-24
        shift = -exp - 1;                                 // value = mant * 2^(exp-23)
        base = 0;
    } else {
        shift = 13;
        base = static_cast<uint32_t>(exp + 15) << 10;
        mant &= 0x7fffffu;
        mant |= 0x800000u;
    }
    uint32_t kept = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u))) ++kept;
    if (exp < -14) return sign | kept;                    // may carry into 0x400: smallest normal
    return sign | (base + (kept - 0x400u));               // kept in [0x400, 0x800]: carry bumps exp
}

}  // namespace diagmm

using namespace diagmm;

extern "C" {

int diagmm_abi_version(void) { return DIAGMM_ABI_VERSION; }

const char* diagmm_last_error(void) { return g_last_error; }

const char* diagmm_status_string(diagmm_status_t st) {
    switch (st) {
    case DIAGMM_OK: return "ok";
    case DIAGMM_ERR_NULL: return "null pointer";
    case DIAGMM_ERR_SHAPE: return "invalid shape";
    case DIAGMM_ERR_DTYPE: return "unsupported dtype";
    case DIAGMM_ERR_ALIAS: return "output overlaps an input";
    case DIAGMM_ERR_UNSUPPORTED: return "unsupported arguments";
    case DIAGMM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

diagmm_status_t diagmm_qk(const void* q, const void* k, void* band, int64_t b, int64_t n,
                          int64_t h, int64_t d, int64_t w, int64_t w_upper, int64_t dilation,
                          float padding_value, diagmm_dtype_t in_dtype,
                          diagmm_dtype_t out_dtype, void* stream) {
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common("diagmm_qk", b, n, h, d, w, w_upper, dilation, in_dtype,
                                      out_dtype, &p, &de, &be);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (!q || !k || !band) return fail(DIAGMM_ERR_NULL, "diagmm_qk: null pointer");
    const int64_t dbytes = de * elem_size(in_dtype), bbytes = be * elem_size(out_dtype);
    if (overlaps(band, bbytes, q, dbytes) || overlaps(band, bbytes, k, dbytes))
        return fail(DIAGMM_ERR_ALIAS, "diagmm_qk: band overlaps q or k");
    const uint32_t pad = pad_bits(padding_value, out_dtype);
    const Plan plan = plan_qk(p, in_dtype, out_dtype);
    timing_set_op(kOpQk);
    return launched("diagmm_qk", run_qk(plan, q, k, band, p, in_dtype, out_dtype, pad,
                                        static_cast<hipStream_t>(stream)));
}

static diagmm_status_t pv_like(const char* fn, int mode, const void* band, const void* x,
                               void* out, int64_t b, int64_t n, int64_t h, int64_t d, int64_t w,
                               int64_t w_upper, int64_t dilation, int in_dtype, int out_dtype,
                               void* stream) {
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common(fn, b, n, h, d, w, w_upper, dilation, in_dtype, out_dtype,
                                      &p, &de, &be);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (!band || !x || !out) return fail(DIAGMM_ERR_NULL, "%s: null pointer", fn);
    const int64_t obytes = de * elem_size(out_dtype);
    if (overlaps(out, obytes, band, be * elem_size(in_dtype)) ||
        overlaps(out, obytes, x, de * elem_size(in_dtype)))
        return fail(DIAGMM_ERR_ALIAS, "%s: output overlaps an input", fn);
    const Plan plan = mode == 1 ? plan_pv(p, in_dtype, out_dtype) : plan_pvT(p, in_dtype, out_dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    timing_set_op(mode == 1 ? kOpPv : kOpPvT);
    return launched(fn, mode == 1 ? run_pv(plan, band, x, out, p, in_dtype, out_dtype, s)
                                  : run_pvT(plan, band, x, out, p, in_dtype, out_dtype, s));
}

diagmm_status_t diagmm_pv(const void* band, const void* v, void* out, int64_t b, int64_t n,
                          int64_t h, int64_t d, int64_t w, int64_t w_upper, int64_t dilation,
                          float padding_value, diagmm_dtype_t in_dtype,
                          diagmm_dtype_t out_dtype, void* stream) {
    (void)padding_value;
    return pv_like("diagmm_pv", 1, band, v, out, b, n, h, d, w, w_upper, dilation, in_dtype,
                   out_dtype, stream);
}

diagmm_status_t diagmm_pvT(const void* band, const void* x, void* out, int64_t b, int64_t n,
                           int64_t h, int64_t d, int64_t w, int64_t w_upper,
                           int64_t dilation, float padding_value, diagmm_dtype_t in_dtype,
                           diagmm_dtype_t out_dtype, void* stream) {
    (void)padding_value;
    return pv_like("diagmm_pvT", 2, band, x, out, b, n, h, d, w, w_upper, dilation, in_dtype,
                   out_dtype, stream);
}

diagmm_status_t diagmm_banded_softmax(const void* scores, void* probs, int64_t b, int64_t n,
                                      int64_t h, int64_t w, int64_t w_upper,
                                      int64_t dilation, float scale, diagmm_dtype_t in_dtype,
                                      diagmm_dtype_t out_dtype, void* stream) {
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common("diagmm_banded_softmax", b, n, h, 1, w, w_upper, dilation,
                                      in_dtype, out_dtype, &p, &de, &be);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (!scores || !probs) return fail(DIAGMM_ERR_NULL, "diagmm_banded_softmax: null pointer");
    const bool in_place = scores == probs && in_dtype == out_dtype;
    if (!in_place && overlaps(probs, be * elem_size(out_dtype), scores, be * elem_size(in_dtype)))
        return fail(DIAGMM_ERR_ALIAS, "diagmm_banded_softmax: probs overlaps scores (only "
                    "exact in-place with equal dtypes is allowed)");
    const Plan plan = plan_softmax(p, in_dtype, out_dtype);
    timing_set_op(kOpSoftmax);
    return launched("diagmm_banded_softmax",
                    run_softmax(plan, scores, probs, p, scale, in_dtype, out_dtype,
                                static_cast<hipStream_t>(stream)));
}

diagmm_status_t diagmm_banded_softmax_masked(const void* scores, void* probs,
                                             const float* key_mask, int64_t b, int64_t n,
                                             int64_t h, int64_t w, int64_t w_upper,
                                             int64_t dilation, float scale, float mask_value,
                                             diagmm_dtype_t in_dtype, diagmm_dtype_t out_dtype,
                                             void* stream) {
    const char* fn = "diagmm_banded_softmax_masked";
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common(fn, b, n, h, 1, w, w_upper, dilation, in_dtype, out_dtype,
                                      &p, &de, &be);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (!scores || !probs || !key_mask) return fail(DIAGMM_ERR_NULL, "%s: null pointer", fn);
    const bool in_place = scores == probs && in_dtype == out_dtype;
    const int64_t pb = be * static_cast<int64_t>(elem_size(out_dtype));
    if (!in_place && overlaps(probs, pb, scores, be * elem_size(in_dtype)))
        return fail(DIAGMM_ERR_ALIAS, "%s: probs overlaps scores (only exact in-place with "
                    "equal dtypes is allowed)", fn);
    if (overlaps(probs, pb, key_mask, p.rows() * 4))
        return fail(DIAGMM_ERR_ALIAS, "%s: probs overlaps key_mask", fn);
    if (!softmax_masked_supported(p))
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: more than 2^31 rows or 2^30 slots", fn);
    timing_set_op(kOpSoftmaxMasked);
    return launched(fn, launch_softmax_masked(scores, probs, key_mask, p, scale, mask_value,
                                              in_dtype, out_dtype,
                                              static_cast<hipStream_t>(stream)));
}

diagmm_status_t diagmm_banded_softmax_backward(const void* probs, const void* dprobs,
                                               void* dscores, int64_t b, int64_t n,
                                               int64_t h, int64_t w, int64_t w_upper,
                                               int64_t dilation, float scale,
                                               diagmm_dtype_t dtype, void* stream) {
    const char* fn = "diagmm_banded_softmax_backward";
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common(fn, b, n, h, 1, w, w_upper, dilation, dtype, dtype, &p,
                                      &de, &be);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (!probs || !dprobs || !dscores) return fail(DIAGMM_ERR_NULL, "%s: null pointer", fn);
    const int64_t bytes = be * static_cast<int64_t>(elem_size(dtype));
    for (const void* in : {probs, dprobs})
        if (dscores != in && overlaps(dscores, bytes, in, bytes))
            return fail(DIAGMM_ERR_ALIAS, "%s: dscores overlaps probs or dprobs (only the "
                        "exact same pointer, in place, is allowed)", fn);
    if (!softmax_bwd_supported(p))
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: more than 2^31 rows or 2^30 slots", fn);
    const bool fast = !force_simple() && softmax_bwd_fast(p, dtype, probs, dprobs, dscores);
    timing_set_op(kOpSoftmaxBwd);
    return launched(fn, launch_softmax_bwd(probs, dprobs, dscores, p, scale, dtype, fast,
                                           static_cast<hipStream_t>(stream)));
}

diagmm_status_t diagmm_banded_dropout(const void* probs, const float* rand, void* out,
                                      int64_t b, int64_t n, int64_t h, int64_t w,
                                      int64_t w_upper, int64_t dilation, float drop_p,
                                      diagmm_dtype_t dtype, void* stream) {
    const char* fn = "diagmm_banded_dropout";
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common(fn, b, n, h, 1, w, w_upper, dilation, dtype, dtype, &p,
                                      &de, &be);
    if (st != DIAGMM_OK) return st;
    if (!(drop_p >= 0.0f && drop_p < 1.0f))
        return fail(DIAGMM_ERR_SHAPE, "%s: p = %g is outside [0, 1)", fn, double(drop_p));
    if (p.rows() * p.h == 0) return ok();
    if (!probs || !rand || !out) return fail(DIAGMM_ERR_NULL, "%s: null pointer", fn);
    const int64_t bytes = be * static_cast<int64_t>(elem_size(dtype));
    if (out != probs && overlaps(out, bytes, probs, bytes))
        return fail(DIAGMM_ERR_ALIAS, "%s: out overlaps probs (only the exact same pointer, "
                    "in place, is allowed)", fn);
    if (overlaps(out, bytes, rand, be * 4))
        return fail(DIAGMM_ERR_ALIAS, "%s: out overlaps rand", fn);
    if (!dropout_supported(p))
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: more than 2^31 - 1 rows or 2^30 slots", fn);
    const bool wide = !force_simple() && dropout_wide(p, dtype, probs, rand, out);
    timing_set_op(kOpDropout);
    return launched(fn, launch_dropout(probs, rand, out, p, drop_p, dtype, wide,
                                       static_cast<hipStream_t>(stream)));
}

diagmm_status_t diagmm_banded_attention(const void* q, const void* k, const void* v, void* out,
                                        int64_t b, int64_t n, int64_t h, int64_t d, int64_t w,
                                        int64_t w_upper, int64_t dilation, float scale,
                                        diagmm_dtype_t dtype, void* stream) {
    const char* fn = "diagmm_banded_attention";
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common(fn, b, n, h, d, w, w_upper, dilation, dtype, dtype, &p,
                                      &de, &be);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (!q || !k || !v || !out) return fail(DIAGMM_ERR_NULL, "%s: null pointer", fn);
    const int64_t bytes = de * static_cast<int64_t>(elem_size(dtype));
    for (const void* in : {q, k, v})
        if (overlaps(out, bytes, in, bytes))
            return fail(DIAGMM_ERR_ALIAS, "%s: out overlaps q, k or v", fn);
    if (!attention_supported(p, dtype, q, k, v, out))
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: needs f16 or bf16, d in {32, 64, 128} and "
                    "16-byte aligned tensors", fn);
    timing_set_op(kOpAttention);
    return launched(fn, launch_attention(q, k, v, nullptr, nullptr, nullptr, out, nullptr, 0,
                                         nullptr, p, scale, dtype,
                                         static_cast<hipStream_t>(stream)));
}

// Shared checks of the global-token call and its workspace query: the common sizes, ng
// and the supported shapes; fills p, the dense element count and the workspace size.
static diagmm_status_t check_global(const char* fn, int64_t b, int64_t n, int64_t h, int64_t d,
                                    int64_t w, int64_t w_upper, int64_t dilation, int64_t ng,
                                    int dtype, Problem* p, int64_t* de, int64_t* ws_bytes) {
    int64_t be;
    diagmm_status_t st = check_common(fn, b, n, h, d, w, w_upper, dilation, dtype, dtype, p, de,
                                      &be);
    if (st != DIAGMM_OK) return st;
    if (ng < 0 || ng > n) return fail(DIAGMM_ERR_SHAPE, "%s: ng = %lld outside [0, n]", fn,
                                      static_cast<long long>(ng));
    if (mul_checked(b, ng) < 0 || mul_checked(b, ng) > kLimit / 8)
        return fail(DIAGMM_ERR_SHAPE, "%s: b * ng overflows", fn);
    *ws_bytes = p->rows() * p->h == 0 ? 0 : attention_global_workspace(*p, ng);
    return DIAGMM_OK;
}

diagmm_status_t diagmm_banded_attention_global_workspace(int64_t b, int64_t n, int64_t h,
                                                         int64_t d, int64_t w, int64_t w_upper,
                                                         int64_t dilation, int64_t ng,
                                                         int64_t* bytes) {
    const char* fn = "diagmm_banded_attention_global_workspace";
    if (!bytes) return fail(DIAGMM_ERR_NULL, "%s: null bytes pointer", fn);
    Problem p;
    int64_t de, ws;
    diagmm_status_t st = check_global(fn, b, n, h, d, w, w_upper, dilation, ng, kF16, &p, &de,
                                      &ws);
    if (st != DIAGMM_OK) return st;
    *bytes = ws;
    return ok();
}

// The global-token call on a given workspace (validated here).
static diagmm_status_t attention_global_impl(const char* fn, const void* q, const void* k,
                                             const void* v, const void* global_q,
                                             const void* global_k, const void* global_v,
                                             void* out, const int32_t* global_pos, int64_t ng,
                                             int64_t b, int64_t n, int64_t h, int64_t d,
                                             int64_t w, int64_t w_upper, int64_t dilation,
                                             float scale, diagmm_dtype_t dtype, void* workspace,
                                             int64_t workspace_bytes, void* stream) {
    Problem p;
    int64_t de, need;
    diagmm_status_t st = check_global(fn, b, n, h, d, w, w_upper, dilation, ng, dtype, &p, &de,
                                      &need);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    const int given = (global_q != nullptr) + (global_k != nullptr) + (global_v != nullptr);
    if (!q || !k || !v || !out || (ng > 0 && !global_pos) || (given != 0 && given != 3) ||
        (need > 0 && !workspace))
        return fail(DIAGMM_ERR_NULL, "%s: null pointer (or only some of global_q, global_k, "
                    "global_v)", fn);
    if (workspace_bytes < need)
        return fail(DIAGMM_ERR_SHAPE, "%s: workspace of %lld bytes, %lld needed", fn,
                    static_cast<long long>(workspace_bytes), static_cast<long long>(need));
    const int64_t bytes = de * static_cast<int64_t>(elem_size(dtype));
    for (const void* in : {q, k, v, global_q, global_k, global_v})
        if (in && overlaps(out, bytes, in, bytes))
            return fail(DIAGMM_ERR_ALIAS, "%s: out overlaps an input", fn);
    if (ng > 0 && overlaps(out, bytes, global_pos, b * ng * 4))
        return fail(DIAGMM_ERR_ALIAS, "%s: out overlaps global_pos", fn);
    if (need > 0) {
        if (overlaps(workspace, need, out, bytes) ||
            overlaps(workspace, need, global_pos, b * ng * 4))
            return fail(DIAGMM_ERR_ALIAS, "%s: workspace overlaps out or global_pos", fn);
        for (const void* in : {q, k, v, global_q, global_k, global_v})
            if (in && overlaps(workspace, need, in, bytes))
                return fail(DIAGMM_ERR_ALIAS, "%s: workspace overlaps an input", fn);
    }
    const bool aligned = (need == 0 || (reinterpret_cast<uintptr_t>(workspace) & 255) == 0) &&
                         (given == 0 || attention_supported(p, dtype, global_q, global_k,
                                                            global_v, out));
    if (!attention_supported(p, dtype, q, k, v, out) || !attention_global_supported(p, ng) ||
        !aligned)
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: needs f16 or bf16, d in {32, 64, 128}, "
                    "16-byte aligned tensors, a 256-byte aligned workspace, "
                    "64 + w + w_upper <= 16384 and n <= 65536", fn);
    timing_set_op(kOpAttention);
    return launched(fn, launch_attention(q, k, v, global_q, global_k, global_v, out, global_pos,
                                         ng, workspace, p, scale, dtype,
                                         static_cast<hipStream_t>(stream)));
}

diagmm_status_t diagmm_banded_attention_global(const void* q, const void* k, const void* v,
                                               const void* global_q, const void* global_k,
                                               const void* global_v, void* out,
                                               const int32_t* global_pos, int64_t ng,
                                               int64_t b, int64_t n, int64_t h, int64_t d,
                                               int64_t w, int64_t w_upper, int64_t dilation,
                                               float scale, diagmm_dtype_t dtype,
                                               void* workspace, int64_t workspace_bytes,
                                               void* stream) {
    return attention_global_impl("diagmm_banded_attention_global", q, k, v, global_q, global_k,
                                 global_v, out, global_pos, ng, b, n, h, d, w, w_upper,
                                 dilation, scale, dtype, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- allocation-free form
// A file-scope device array serves as the workspace of the global-token call for callers
// that cannot allocate.  Each GPU the library runs on holds its own copy for the life of
// the process; its address on a device is looked up once per device, with that device
// current, and only that address is handed to kernels (the array's name is a host-side
// stand-in).  Calls on one GPU share the array: calls that overlap in time race.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up on the first call there).
static diagmm_status_t scratch_address(const char* fn, void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DIAGMM_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", fn, dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t s = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (s != hipSuccess || !ptr)
            return fail(DIAGMM_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn,
                        dev, hipGetErrorString(s));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DIAGMM_OK;
}

diagmm_status_t diagmm_banded_attention_global_noalloc(
    const void* q, const void* k, const void* v, const void* global_q, const void* global_k,
    const void* global_v, void* out, const int32_t* global_pos, int64_t ng, int64_t b,
    int64_t n, int64_t h, int64_t d, int64_t w, int64_t w_upper, int64_t dilation, float scale,
    diagmm_dtype_t dtype, void* stream) {
    const char* fn = "diagmm_banded_attention_global_noalloc";
    Problem p;
    int64_t de, need;
    diagmm_status_t st = check_global(fn, b, n, h, d, w, w_upper, dilation, ng, dtype, &p, &de,
                                      &need);
    if (st != DIAGMM_OK) return st;
    if (p.rows() * p.h == 0) return ok();
    if (need > kScratchBytes)
        return fail(DIAGMM_ERR_UNSUPPORTED, "%s: needs %lld bytes of scratch, the static "
                    "scratch holds %lld (use diagmm_banded_attention_global with a workspace)",
                    fn, static_cast<long long>(need), static_cast<long long>(kScratchBytes));
    if (!q || !k || !v || !out || (ng > 0 && !global_pos))
        return fail(DIAGMM_ERR_NULL, "%s: null pointer", fn);
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_address(fn, &ws);
        if (st != DIAGMM_OK) return st;
    }
    return attention_global_impl(fn, q, k, v, global_q, global_k, global_v, out, global_pos, ng,
                                 b, n, h, d, w, w_upper, dilation, scale, dtype, ws,
                                 need > 0 ? kScratchBytes : 0, stream);
}

diagmm_status_t diagmm_plan(int mode, int64_t b, int64_t n, int64_t h, int64_t d, int64_t w,
                            int64_t w_upper, int64_t dilation, diagmm_dtype_t in_dtype,
                            diagmm_dtype_t out_dtype, diagmm_plan_t* out) {
    if (!out) return fail(DIAGMM_ERR_NULL, "diagmm_plan: null plan pointer");
    if (mode < 0 || mode > 7 || mode == 5)
        return fail(DIAGMM_ERR_UNSUPPORTED, "diagmm_plan: mode %d", mode);
    Problem p;
    int64_t de, be;
    diagmm_status_t st = check_common("diagmm_plan", b, n, h, (mode >= 3 && mode != 7) ? 1 : d, w, w_upper,
                                      dilation, in_dtype, out_dtype, &p, &de, &be);
    if (st != DIAGMM_OK) return st;
    if (mode == 7) {
        if (out_dtype != in_dtype)
            return fail(DIAGMM_ERR_DTYPE, "diagmm_plan: attention has one dtype");
        const void* al = reinterpret_cast<const void*>(uintptr_t(256));   // aligned tensors
        if (!attention_supported(p, in_dtype, al, al, al, al))
            return fail(DIAGMM_ERR_UNSUPPORTED, "diagmm_plan: attention needs f16 or bf16 and "
                        "d in {32, 64, 128}");
        std::memset(out, 0, sizeof *out);
        std::snprintf(out->kernel, sizeof out->kernel, "attn_fwd_%s_d%lld",
                      in_dtype == DIAGMM_F16 ? "f16" : "bf16", static_cast<long long>(d));
        out->rows_per_tile = 64;
        out->slots_per_tile = 64;
        out->workgroups = out->tiles = attention_workgroups(p);
        out->threads = 256;
        out->lds_bytes = 2 * 64 * 2 * d;
        out->residues = p.s;
        return ok();
    }
    if (mode == 6) {
        if (out_dtype != in_dtype)
            return fail(DIAGMM_ERR_DTYPE, "diagmm_plan: dropout has one dtype");
        const void* al = reinterpret_cast<const void*>(uintptr_t(256));   // aligned tensors
        const bool wide = !force_simple() && dropout_wide(p, in_dtype, al, al, al);
        std::memset(out, 0, sizeof *out);
        std::snprintf(out->kernel, sizeof out->kernel, "%s",
                      wide ? "dropout_wide" : "dropout_elems");
        out->workgroups = out->tiles = dropout_workgroups(p, in_dtype, wide);
        out->slots_per_tile = dropout_chunk(in_dtype, wide);
        out->threads = 256;
        out->residues = 1;
        return ok();
    }
    if (mode == 4) {
        if (out_dtype != in_dtype)
            return fail(DIAGMM_ERR_DTYPE, "diagmm_plan: the softmax backward has one dtype");
        const void* al = reinterpret_cast<const void*>(uintptr_t(256));   // aligned tensors
        const bool fast = !force_simple() && softmax_bwd_fast(p, in_dtype, al, al, al);
        std::memset(out, 0, sizeof *out);
        std::snprintf(out->kernel, sizeof out->kernel, "%s",
                      softmax_bwd_kernel_name(p, in_dtype, fast));
        out->rows_per_tile = 1;
        out->slots_per_tile = p.K;
        out->tiles = p.rows() * p.h;
        out->workgroups = softmax_bwd_workgroups(p, in_dtype, fast);
        out->threads = 256;
        out->residues = 1;
        return ok();
    }
    Plan plan = mode == 0 ? plan_qk(p, in_dtype, out_dtype)
              : mode == 1 ? plan_pv(p, in_dtype, out_dtype)
              : mode == 2 ? plan_pvT(p, in_dtype, out_dtype)
                          : plan_softmax(p, in_dtype, out_dtype);
    std::memset(out, 0, sizeof *out);
    std::snprintf(out->kernel, sizeof out->kernel, "%s", plan.kernel);
    out->rows_per_tile = plan.rows_per_tile;
    out->slots_per_tile = plan.slots_per_tile;
    out->tiles = plan.tiles;
    out->workgroups = plan.workgroups;
    out->threads = plan.threads;
    out->lds_bytes = plan.lds_bytes;
    out->residues = plan.residues;
    out->strip_workgroups = plan.strip_wgs;
    out->interleaved = plan.interleaved;
    return ok();
}

}  // extern "C"
