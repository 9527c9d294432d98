// Kernel timers: the session state behind timing.hpp and the diagmm_timing_* calls.
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/diagmm.h"
#include "timing.hpp"

namespace diagmm {
namespace {

constexpr int64_t kMaxTimed = int64_t(1) << 20;

struct Rec {
    int op;
    hipEvent_t start, stop;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<hipEvent_t> g_pool;     // created on demand, kept for later sessions
std::vector<Rec> g_recs;
int64_t g_cap = 0;
thread_local int g_op = -1;

}  // namespace

void timing_set_op(int op) { g_op = op; }

bool timing_slot(hipEvent_t* start, hipEvent_t* stop) {
    if (!g_on.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on.load(std::memory_order_relaxed) ||
        static_cast<int64_t>(g_recs.size()) >= g_cap)
        return false;
    const size_t i = 2 * g_recs.size();
    *start = g_pool[i];
    *stop = g_pool[i + 1];
    g_recs.push_back(Rec{g_op, *start, *stop});
    return true;
}

}  // namespace diagmm

using namespace diagmm;

extern "C" {

diagmm_status_t diagmm_timing_begin(int64_t capacity) {
    if (capacity < 1 || capacity > kMaxTimed) return DIAGMM_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_mu);
    while (static_cast<int64_t>(g_pool.size()) < 2 * capacity) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return DIAGMM_ERR_HIP;
        g_pool.push_back(e);
    }
    g_recs.clear();
    g_cap = capacity;
    g_on.store(true);
    return DIAGMM_OK;
}

diagmm_status_t diagmm_timing_end(void) {
    g_on.store(false);
    return DIAGMM_OK;
}

diagmm_status_t diagmm_timing_read(int64_t max, int32_t* ops, double* ms, int64_t* count) {
    if (!count || (max > 0 && (!ops || !ms))) return DIAGMM_ERR_NULL;
    std::lock_guard<std::mutex> lk(g_mu);
    const int64_t n = static_cast<int64_t>(g_recs.size());
    *count = n;
    for (int64_t i = 0; i < n && i < max; ++i) {
        if (hipEventSynchronize(g_recs[i].stop) != hipSuccess) return DIAGMM_ERR_HIP;
        float t = 0.f;
        if (hipEventElapsedTime(&t, g_recs[i].start, g_recs[i].stop) != hipSuccess)
            return DIAGMM_ERR_HIP;
        ops[i] = g_recs[i].op;
        ms[i] = t;
    }
    return DIAGMM_OK;
}

}  // extern "C"
