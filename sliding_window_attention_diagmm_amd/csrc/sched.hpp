// Band-tile scheduler: picks the kernel family for a call and how its output is cut
// into tiles and workgroups.  plan_* are pure host functions (also reachable through
// diagmm_plan for inspection); run_* enqueue the chosen kernels.
#pragma once

#include "common.hpp"

namespace diagmm {

enum class Family {
    kSimple,      // element per thread (any shape)
    kQkMfma,      // qk: MFMA on dense 16x16 sub-tiles, LDS-staged band store
    kQkStream,    // qk: balanced row ranges, keys streamed, staged 256-byte row runs
    kPvMfma,      // pv: band tile un-skewed into MFMA operands
    kPvTMfma,     // pvT: transposed band tile into MFMA operands
    kSoftmaxRow,  // softmax: one workgroup per band row
    kSoftmaxWave, // softmax: one wavefront per band row, row held in registers
};

struct Plan {
    Family family = Family::kSimple;
    const char* kernel = "simple";
    int64_t rows_per_tile = 1;   // output rows per tile, within one residue class
    int64_t slots_per_tile = 1;  // band slots (qk, softmax) or dense columns (pv, pvT)
    int64_t tiles = 0;
    int64_t workgroups = 0;
    int64_t threads = 256;
    int64_t lds_bytes = 0;
    int64_t residues = 1;        // s: rows i = r (mod s) form independent problems
    int64_t strip_wgs = 0;       // workgroups per strip (strip split), 0 = flat split
    int64_t interleaved = 0;     // pv, pvT: tiles dealt round-robin over each XCD's workgroups
};

Plan plan_qk(const Problem& p, int in_dt, int out_dt);
Plan plan_pv(const Problem& p, int in_dt, int out_dt);
Plan plan_pvT(const Problem& p, int in_dt, int out_dt);
Plan plan_softmax(const Problem& p, int in_dt, int out_dt);

hipError_t run_qk(const Plan& plan, const void* q, const void* k, void* band, const Problem& p,
                  int in_dt, int out_dt, uint32_t pad, hipStream_t stream);
hipError_t run_pv(const Plan& plan, const void* band, const void* v, void* out, const Problem& p,
                  int in_dt, int out_dt, hipStream_t stream);
hipError_t run_pvT(const Plan& plan, const void* band, const void* x, void* out,
                   const Problem& p, int in_dt, int out_dt, hipStream_t stream);
hipError_t run_softmax(const Plan& plan, const void* scores, void* probs, const Problem& p,
                       float scale, int in_dt, int out_dt, hipStream_t stream);

}  // namespace diagmm
