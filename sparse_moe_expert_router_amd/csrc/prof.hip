// Opt-in per-kernel timing with HIP events (diagnostics).  When enabled, every kernel launch of
// the library is bracketed by hipEventRecord on the launch's stream; moe_profile_collect waits
// for those events and accumulates the elapsed time per kernel kind.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "moe_launch.hpp"

namespace moe {
namespace {

const char *const KERNEL_NAMES[K_COUNT] = {
    "router_logits", "topk", "select_permute", "gateup_int8", "down_int8", "combine_rows",
    "up_e2m1", "down_e2m1", "quantize_rows", "ggemm_gateup_i8", "ggemm_down_i8"};

struct Pending {
    int kind;
    hipEvent_t start, end;
};

struct Profiler {
    std::mutex mu;
    bool enabled = false;
    std::vector<hipEvent_t> pool;
    std::vector<Pending> pending;
    long long launches[K_COUNT] = {};
    double ms[K_COUNT] = {};

    hipEvent_t take()
    {
        if (pool.empty()) {
            // timing only: no system-scope fence when the event is recorded, so the interval holds
            // the kernel and not a writeback and invalidation of the caches around it (with the
            // fence the events read 1.4 - 1.8 us longer per launch than the kernel trace, and the
            // launch after an event starts with cold caches)
            hipEvent_t e = nullptr;
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
            return e;
        }
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
};

Profiler &prof()
{
    static Profiler p;
    return p;
}

}  // namespace

ProfScope::ProfScope(int kind, hipStream_t s) : kind_(kind), stream_(s), start_(nullptr)
{
    Profiler &p = prof();
    std::lock_guard<std::mutex> lock(p.mu);
    if (!p.enabled) return;
    start_ = p.take();
    if (start_ && hipEventRecord(static_cast<hipEvent_t>(start_), s) != hipSuccess) {
        p.pool.push_back(static_cast<hipEvent_t>(start_));
        start_ = nullptr;
    }
}

ProfScope::~ProfScope()
{
    if (!start_) return;
    Profiler &p = prof();
    std::lock_guard<std::mutex> lock(p.mu);
    hipEvent_t end = p.take();
    if (end && hipEventRecord(end, stream_) == hipSuccess) {
        p.pending.push_back(Pending{kind_, static_cast<hipEvent_t>(start_), end});
    } else {
        if (end) p.pool.push_back(end);
        p.pool.push_back(static_cast<hipEvent_t>(start_));
    }
}

}  // namespace moe

extern "C" {

moe_status moe_profile_enable(int32_t on)
{
    moe::Profiler &p = moe::prof();
    std::lock_guard<std::mutex> lock(p.mu);
    p.enabled = on != 0;
    return MOE_OK;
}

moe_status moe_profile_collect(void)
{
    moe::Profiler &p = moe::prof();
    std::lock_guard<std::mutex> lock(p.mu);
    moe_status st = MOE_OK;
    for (const moe::Pending &q : p.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(q.end) != hipSuccess || hipEventElapsedTime(&ms, q.start, q.end) != hipSuccess) {
            st = MOE_EHIP;
        } else {
            p.launches[q.kind] += 1;
            p.ms[q.kind] += ms;
        }
        p.pool.push_back(q.start);
        p.pool.push_back(q.end);
    }
    p.pending.clear();
    return st;
}

void moe_profile_reset(void)
{
    moe::Profiler &p = moe::prof();
    std::lock_guard<std::mutex> lock(p.mu);
    for (int i = 0; i < moe::K_COUNT; ++i) {
        p.launches[i] = 0;
        p.ms[i] = 0.0;
    }
}

int32_t moe_profile_kinds(void) { return moe::K_COUNT; }

moe_status moe_profile_get(int32_t kind, const char **name, int64_t *launches, double *total_ms)
{
    if (kind < 0 || kind >= moe::K_COUNT) return MOE_EINVAL;
    moe::Profiler &p = moe::prof();
    std::lock_guard<std::mutex> lock(p.mu);
    if (name) *name = moe::KERNEL_NAMES[kind];
    if (launches) *launches = p.launches[kind];
    if (total_ms) *total_ms = p.ms[kind];
    return MOE_OK;
}

}  // extern "C"
