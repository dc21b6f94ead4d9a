// Opt-in per-kernel timing.  When enabled, every kernel launch of the
// library is bracketed by two HIP events recorded on the launch's own
// stream; sp_timing_collect() waits for them and aggregates the elapsed
// times per kernel name.  Disabled (the default) it costs one atomic load
// per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/ulysses_sp.h"
#include "launch.h"

namespace {

struct Rec {
    const char *name;
    hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

KernelTimer::KernelTimer(const char *name, hipStream_t s) : name_(name), s_(s), a_(nullptr), b_(nullptr) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_mu);
    a_ = take_event();
    b_ = take_event();
    if (!a_ || !b_ || hipEventRecord(a_, s_) != hipSuccess) {
        if (a_) g_pool.push_back(a_);
        if (b_) g_pool.push_back(b_);
        a_ = b_ = nullptr;
    }
}

KernelTimer::~KernelTimer() {
    if (!a_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (hipEventRecord(b_, s_) == hipSuccess) {
        g_recs.push_back({name_, a_, b_});
    } else {
        g_pool.push_back(a_);
        g_pool.push_back(b_);
    }
}

#pragma GCC visibility push(default)
extern "C" {

int sp_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_mu);
    const int prev = g_on.load() ? 1 : 0;
    if (on && !prev) {
        for (auto &r : g_recs) {
            (void)hipEventSynchronize(r.b);
            g_pool.push_back(r.a);
            g_pool.push_back(r.b);
        }
        g_recs.clear();
    }
    g_on.store(on != 0);
    return prev;
}

int sp_timing_collect(sp_kernel_time *out, int max_entries) {
    std::lock_guard<std::mutex> lk(g_mu);
    std::vector<sp_kernel_time> agg;
    for (auto &r : g_recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            return -1;
        sp_kernel_time *slot = nullptr;
        for (auto &x : agg)
            if (std::strncmp(x.name, r.name, sizeof(x.name)) == 0) slot = &x;
        if (!slot) {
            sp_kernel_time z;
            std::memset(&z, 0, sizeof z);
            std::strncpy(z.name, r.name, sizeof(z.name) - 1);
            z.min_ms = 1e30;
            agg.push_back(z);
            slot = &agg.back();
        }
        slot->launches += 1;
        slot->total_ms += ms;
        if (ms < slot->min_ms) slot->min_ms = ms;
        if (ms > slot->max_ms) slot->max_ms = ms;
    }
    const int n = (int)agg.size();
    if (out == nullptr) return n;            // a count query keeps the records
    for (int i = 0; i < n && i < max_entries; ++i) out[i] = agg[i];
    for (auto &r : g_recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    return n;
}

}  // extern "C"
#pragma GCC visibility pop
