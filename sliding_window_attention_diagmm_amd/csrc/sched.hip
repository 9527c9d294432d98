// Band-tile scheduler (see sched.hpp).
#include <cstdlib>
#include <cstring>

#include "launch.hpp"
#include "sched.hpp"

namespace diagmm {

// DIAGMM_KERNEL=simple forces the element-per-thread kernels (a debugging and
// comparison switch; the default picks the tiled kernels where they apply).
bool force_simple() {
    const char* e = std::getenv("DIAGMM_KERNEL");
    return e && std::strcmp(e, "simple") == 0;
}

// DIAGMM_QK=tiles keeps qk on the persistent tile kernel where the streaming one would
// run (a comparison switch).
static bool qk_tiles_forced() {
    const char* e = std::getenv("DIAGMM_QK");
    return e && std::strcmp(e, "tiles") == 0;
}

// DIAGMM_TILE_ORDER=interleaved / contiguous overrides the choice of tile order of pv on
// the flat split and of pvT on either split (a testing and comparison switch): 1 and 2,
// else 0.
int tile_order_forced() {
    const char* e = std::getenv("DIAGMM_TILE_ORDER");
    if (!e) return 0;
    if (std::strcmp(e, "interleaved") == 0) return 1;
    return std::strcmp(e, "contiguous") == 0 ? 2 : 0;
}

namespace {

Plan simple_plan(const Problem& p, int64_t cols, const char* name) {
    Plan pl;
    pl.family = Family::kSimple;
    pl.kernel = name;
    pl.rows_per_tile = 1;
    pl.slots_per_tile = 1;
    pl.tiles = p.rows() * p.h * cols;
    const int64_t blocks = (pl.tiles + 255) / 256;
    pl.workgroups = blocks < (int64_t(1) << 20) ? blocks : (int64_t(1) << 20);
    pl.threads = 256;
    pl.lds_bytes = 0;
    pl.residues = 1;
    return pl;
}

bool mfma_dtype(int in_dt) { return in_dt == kF16 || in_dt == kBF16; }
bool mfma_depth(int64_t d) { return d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

Plan plan_qk(const Problem& p, int in_dt, int out_dt) {
    if (force_simple() || !mfma_dtype(in_dt) || !mfma_depth(p.d))
        return simple_plan(p, p.K, "qk_simple");
    const QkStreamPlan sp = plan_qk_stream(p, in_dt, out_dt);
    if (sp.ok && !qk_tiles_forced()) {
        Plan pl;
        pl.family = Family::kQkStream;
        pl.kernel = "qk_stream";
        pl.rows_per_tile = sp.rows_per_range;
        pl.slots_per_tile = p.K;
        pl.tiles = sp.ranges;
        pl.workgroups = sp.workgroups;
        pl.threads = 768;
        pl.lds_bytes = sp.lds_bytes;
        pl.residues = p.s < p.n ? p.s : (p.n > 0 ? p.n : 1);
        pl.strip_wgs = sp.g;
        return pl;
    }
    const QkTilePlan tp = plan_qk_mfma(p, out_dt);
    if (!tp.ok) return simple_plan(p, p.K, "qk_simple");
    Plan pl;
    pl.family = Family::kQkMfma;
    pl.kernel = "qk_mfma";
    pl.rows_per_tile = kQkRows;
    pl.slots_per_tile = tp.grid.kb;
    pl.tiles = tp.grid.tiles;
    pl.workgroups = tp.workgroups;
    pl.strip_wgs = tp.strip_wgs;
    pl.threads = 512;
    pl.lds_bytes = tp.lds_bytes;
    pl.residues = tp.grid.res;
    return pl;
}

Plan plan_pv(const Problem& p, int in_dt, int out_dt) {
    (void)out_dt;
    if (force_simple() || !mfma_dtype(in_dt) || !mfma_depth(p.d))
        return simple_plan(p, p.d, "pv_simple");
    const PvTilePlan tp = plan_pv_mfma(p);
    if (!tp.ok) return simple_plan(p, p.d, "pv_simple");
    Plan pl;
    pl.family = Family::kPvMfma;
    pl.kernel = "pv_mfma";
    pl.rows_per_tile = kPvRows;
    pl.slots_per_tile = tp.grid.kb;
    pl.tiles = tp.grid.tiles;
    pl.workgroups = tp.workgroups;
    pl.threads = 512;
    pl.lds_bytes = tp.lds_bytes;
    pl.residues = tp.grid.res;
    pl.strip_wgs = tp.strip_wgs;
    pl.interleaved = tp.interleave ? 1 : 0;
    return pl;
}

Plan plan_pvT(const Problem& p, int in_dt, int out_dt) {
    (void)out_dt;
    if (force_simple() || !mfma_dtype(in_dt) || !mfma_depth(p.d))
        return simple_plan(p, p.d, "pvT_simple");
    const PvTilePlan tp = plan_pvt_mfma(p);
    if (!tp.ok) return simple_plan(p, p.d, "pvT_simple");
    Plan pl;
    pl.family = Family::kPvTMfma;
    pl.kernel = "pvT_mfma";
    pl.rows_per_tile = kPvTRows;
    pl.slots_per_tile = tp.grid.kb;
    pl.tiles = tp.grid.tiles;
    pl.workgroups = tp.workgroups;
    pl.threads = 512;
    pl.lds_bytes = tp.lds_bytes;
    pl.residues = tp.grid.res;
    pl.strip_wgs = tp.strip_wgs;
    pl.interleaved = tp.interleave ? 1 : 0;
    return pl;
}

Plan plan_softmax(const Problem& p, int in_dt, int out_dt) {
    Plan pl;
    if (!force_simple() && softmax_wave_supported(p, in_dt, out_dt)) {
        pl.family = Family::kSoftmaxWave;
        pl.kernel = "softmax_wave";
        pl.rows_per_tile = 1;
        pl.slots_per_tile = p.K;
        pl.tiles = p.rows() * p.h;
        pl.workgroups = (pl.tiles + 3) / 4;
        pl.threads = 256;
        pl.lds_bytes = 0;
        return pl;
    }
    pl.family = Family::kSoftmaxRow;
    pl.kernel = "softmax_rows";
    pl.rows_per_tile = 1;
    pl.slots_per_tile = p.K;
    pl.tiles = p.rows() * p.h;
    pl.workgroups = pl.tiles < (int64_t(1) << 20) ? pl.tiles : (int64_t(1) << 20);
    pl.threads = 256;
    pl.lds_bytes = 16;
    return pl;
}

hipError_t run_qk(const Plan& plan, const void* q, const void* k, void* band, const Problem& p,
                  int in_dt, int out_dt, uint32_t pad, hipStream_t stream) {
    // The tiled kernels move 16-byte pieces; other pointers take the general path.
    if (plan.family == Family::kQkStream && aligned16(q) && aligned16(k) && aligned16(band))
        return launch_qk_stream(q, k, band, p, plan_qk_stream(p, in_dt, out_dt), in_dt, pad,
                                stream);
    if (plan.family == Family::kQkMfma && aligned16(q) && aligned16(k) && aligned16(band))
        return launch_qk_mfma(q, k, band, p, plan_qk_mfma(p, out_dt), in_dt, out_dt, pad, stream);
    return launch_qk_simple(q, k, band, p, in_dt, out_dt, pad, stream);
}

hipError_t run_pv(const Plan& plan, const void* band, const void* v, void* out, const Problem& p,
                  int in_dt, int out_dt, hipStream_t stream) {
    if (plan.family == Family::kPvMfma && aligned16(band) && aligned16(v) && aligned16(out))
        return launch_pv_mfma(band, v, out, p, plan_pv_mfma(p), in_dt, out_dt, stream);
    return launch_pv_simple(band, v, out, p, in_dt, out_dt, stream);
}

hipError_t run_pvT(const Plan& plan, const void* band, const void* x, void* out,
                   const Problem& p, int in_dt, int out_dt, hipStream_t stream) {
    if (plan.family == Family::kPvTMfma && aligned16(band) && aligned16(x) && aligned16(out))
        return launch_pvt_mfma(band, x, out, p, plan_pvt_mfma(p), in_dt, out_dt, stream);
    return launch_pvT_simple(band, x, out, p, in_dt, out_dt, stream);
}

hipError_t run_softmax(const Plan& plan, const void* scores, void* probs, const Problem& p,
                       float scale, int in_dt, int out_dt, hipStream_t stream) {
    if (plan.family == Family::kSoftmaxWave && aligned16(scores) && aligned16(probs))
        return launch_softmax_wave(scores, probs, p, scale, in_dt, stream);
    return launch_softmax_rows(scores, probs, p, scale, in_dt, out_dt, stream);
}

}  // namespace diagmm
