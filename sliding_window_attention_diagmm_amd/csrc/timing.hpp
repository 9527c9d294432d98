// Kernel timers, a measurement aid for benchmarks.  While a timing session is open
// (diagmm_timing_begin .. diagmm_timing_end), every kernel launch of the library goes
// through hipExtLaunchKernel with a pair of HIP events that the runtime records at the
// kernel's own start and end on its stream (no separate marker packets, so the interval
// is the kernel's execution, as a profiler's kernel trace reports it), tagged with the
// entry point that launched it.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace diagmm {

// Entry point tags (the modes of diagmm_plan).
constexpr int kOpQk = 0, kOpPv = 1, kOpPvT = 2, kOpSoftmax = 3, kOpSoftmaxBwd = 4,
              kOpSoftmaxMasked = 5, kOpDropout = 6, kOpAttention = 7;

// The entry point whose kernels are launched next (set by the C ABI before it launches).
void timing_set_op(int op);
// Events for the next launch when a session is open and has room; false otherwise.
bool timing_slot(hipEvent_t* start, hipEvent_t* stop);

// Launch a kernel, timed when a session is open.
template <class F, class... Args>
void launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                   Args... args) {
    hipEvent_t e0, e1;
    if (timing_slot(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), stream, e0, e1,
                              0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

}  // namespace diagmm
