// Internal launch interface between the C ABI (api.hip) and the kernel families.
// Every launcher enqueues on `stream` and returns the HIP error of the launch.
#pragma once

#include "common.hpp"

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

}  // namespace diagmm
