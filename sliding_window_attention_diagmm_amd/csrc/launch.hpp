// Internal launch interface between the C ABI (api.hip) and the kernel families.
// Every launcher enqueues on `stream` and returns the HIP error of the launch.
#pragma once

#include "common.hpp"
#include "tiles.hpp"
#include "timing.hpp"

namespace diagmm {

// Element-per-thread kernels: any shape, any supported dtype pair.  They are the
// general path (any d, any window) and the cross-check for the tiled kernels.
hipError_t launch_qk_simple(const void* q, const void* k, void* band, const Problem& p,
                            int in_dt, int out_dt, uint32_t pad, hipStream_t stream);
hipError_t launch_pv_simple(const void* band, const void* v, void* out, const Problem& p,
                            int in_dt, int out_dt, hipStream_t stream);
hipError_t launch_pvT_simple(const void* band, const void* x, void* out, const Problem& p,
                             int in_dt, int out_dt, hipStream_t stream);
hipError_t launch_softmax_rows(const void* scores, void* probs, const Problem& p, float scale,
                               int in_dt, int out_dt, hipStream_t stream);

// Banded softmax, one wavefront per row (equal in/out dtypes, rows up to ~8.7K slots,
// 16-byte aligned pointers).
bool softmax_wave_supported(const Problem& p, int in_dt, int out_dt);
hipError_t launch_softmax_wave(const void* scores, void* probs, const Problem& p, float scale,
                               int dt, hipStream_t stream);

// DIAGMM_KERNEL=simple: the general kernels only (debugging and comparison switch).
bool force_simple();
// DIAGMM_TILE_ORDER=interleaved / contiguous: the tile order of pv and pvT forced (1 / 2),
// else 0.
int tile_order_forced();

// Banded softmax backward (one dtype for probs, dprobs and dscores): the group / wave
// kernel when `fast` (softmax_bwd_fast), else one workgroup per row.
bool softmax_bwd_supported(const Problem& p);
int64_t softmax_bwd_workgroups(const Problem& p, int dt, bool fast);
bool softmax_bwd_fast(const Problem& p, int dt, const void* probs, const void* dprobs,
                      const void* dscores);
const char* softmax_bwd_kernel_name(const Problem& p, int dt, bool fast);
hipError_t launch_softmax_bwd(const void* probs, const void* dprobs, void* dscores,
                              const Problem& p, float scale, int dt, bool fast,
                              hipStream_t stream);

// Banded softmax with a per-key additive mask (float32 [b][n]).
bool softmax_masked_supported(const Problem& p);
hipError_t launch_softmax_masked(const void* scores, void* probs, const float* key_mask,
                                 const Problem& p, float scale, float mask_value, int in_dt,
                                 int out_dt, hipStream_t stream);

// Dropout on a band with caller-drawn uniforms (one dtype for probs and out): 16-byte
// pieces when `wide` (dropout_wide), else element by element.
bool dropout_supported(const Problem& p);
bool dropout_wide(const Problem& p, int dt, const void* probs, const void* rand,
                  const void* out);
int64_t dropout_chunk(int dt, bool wide);   // band elements per workgroup
int64_t dropout_workgroups(const Problem& p, int dt, bool wide);
hipError_t launch_dropout(const void* probs, const float* rand, void* out, const Problem& p,
                          float drop_p, int dt, bool wide, hipStream_t stream);

// Sliding-window attention in one pass (f16 / bf16, d in {32, 64, 128}, 16-byte aligned
// tensors): 256-thread workgroups of 64 class rows, keys staged 64 at a time.
bool attention_supported(const Problem& p, int dt, const void* q, const void* k, const void* v,
                         const void* out);
bool attention_global_supported(const Problem& p, int64_t ng);
// Workspace bytes of the global-token form (0 when ng == 0): the positions of the global
// rows and their partial softmax states.
int64_t attention_global_workspace(const Problem& p, int64_t ng);
int64_t attention_workgroups(const Problem& p);
// glob: ng int32 positions per batch on the device (ignored when ng == 0); gq, gk, gv:
// the global rows' matrices (NULL: q, k, v); workspace: attention_global_workspace bytes,
// 256-byte aligned, on the device (ignored when ng == 0).
hipError_t launch_attention(const void* q, const void* k, const void* v, const void* gq,
                            const void* gk, const void* gv, void* out, const int32_t* glob,
                            int64_t ng, void* workspace, const Problem& p, float scale,
                            int dt, hipStream_t stream);

// qk on MFMA (f16 / bf16 inputs, d in {32, 64, 128}, 16-byte aligned pointers).
constexpr int kQkRows = 128;                 // rows per tile
constexpr int64_t kQkLdsBytes = 160 * 1024;  // one workgroup per compute unit

struct QkTilePlan {
    TileGrid grid;
    int64_t rs = 0;         // staging row stride (elements)
    int64_t lds_bytes = 0;
    int64_t workgroups = 0; // persistent workgroups (at most one per compute unit)
    int64_t strip_wgs = 0;  // workgroups per strip with the strip split, 0 = flat split
    bool ok = false;        // the shape fits the kernel's 32-bit tile arithmetic
};

QkTilePlan plan_qk_mfma(const Problem& p, int out_dt);
hipError_t launch_qk_mfma(const void* q, const void* k, void* band, const Problem& p,
                          const QkTilePlan& tp, int in_dt, int out_dt, uint32_t pad,
                          hipStream_t stream);

// qk streaming (f16 / bf16 in and out, d = 64, 16-byte aligned pointers):
// strips cut into ranges of at most 208 class rows, one workgroup per compute unit.
struct QkStreamPlan {
    int64_t g = 0;              // ranges per strip
    int64_t ranges = 0;         // strips * g
    int64_t workgroups = 0;
    int64_t rows_per_range = 0; // longest range (class rows)
    int64_t lds_bytes = 0;
    bool lines = false;         // whole 128-byte lines per store (pieces held one step)
    bool stream_stores = false; // line-path stores non-temporal (bands larger than the MALL)
    int32_t order = 0;          // range order: 0 strip-major, 1 head-fastest
    bool interleave = false;    // each XCD's ranges dealt round-robin over its workgroups
    bool ok = false;
};
QkStreamPlan plan_qk_stream(const Problem& p, int in_dt, int out_dt);
hipError_t launch_qk_stream(const void* q, const void* k, void* band, const Problem& p,
                            const QkStreamPlan& sp, int in_dt, uint32_t pad,
                            hipStream_t stream);

// pv on MFMA (f16 / bf16 inputs, d in {32, 64, 128}, 16-byte aligned pointers).
constexpr int kPvRows = 64;
constexpr int64_t kPvLdsBytes = 160 * 1024;

struct PvTilePlan {
    TileGrid grid;          // nkb / kb: slot chunks per tile and slots per chunk
    int64_t lds_bytes = 0;
    int64_t workgroups = 0;
    int64_t strip_wgs = 0;  // workgroups per strip with the strip split, 0 = flat split
    bool interleave = false;  // units dealt round-robin over each XCD's workgroups
    bool ok = false;
};

PvTilePlan plan_pv_mfma(const Problem& p);

// pvT on MFMA (same dtypes, depths and alignment as pv); tiles of 64 output rows.
constexpr int kPvTRows = 64;
PvTilePlan plan_pvt_mfma(const Problem& p);
hipError_t launch_pvt_mfma(const void* band, const void* x, void* out, const Problem& p,
                           const PvTilePlan& tp, int in_dt, int out_dt, hipStream_t stream);
hipError_t launch_pv_mfma(const void* band, const void* v, void* out, const Problem& p,
                          const PvTilePlan& tp, int in_dt, int out_dt, hipStream_t stream);

}  // namespace diagmm
