// timing.cpp -- per-kernel HIP-event timing behind csa_timing_enable / csa_timing_read.
#include "timing.hpp"

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "csa.h"

namespace csa {
namespace {

struct State {
    std::atomic<int> kernel{-1};
    std::mutex mu;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;   // recorded, not yet read
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;      // free for reuse
};

State& state()
{
    static State s;
    return s;
}

}  // namespace

TimedLaunch::TimedLaunch(int id, hipStream_t st) : st_(st)
{
    State& s = state();
    if (s.kernel.load(std::memory_order_relaxed) != id) return;
    std::lock_guard<std::mutex> lk(s.mu);
    if (!s.pool.empty()) {
        a_ = s.pool.back().first;
        b_ = s.pool.back().second;
        s.pool.pop_back();
    } else if (hipEventCreate(&a_) != hipSuccess || hipEventCreate(&b_) != hipSuccess) {
        a_ = b_ = nullptr;
        return;
    }
    if (hipEventRecord(a_, st_) != hipSuccess) {
        s.pool.emplace_back(a_, b_);
        a_ = b_ = nullptr;
    }
}

TimedLaunch::~TimedLaunch()
{
    if (!a_) return;
    State& s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    if (hipEventRecord(b_, st_) == hipSuccess) s.pending.emplace_back(a_, b_);
    else s.pool.emplace_back(a_, b_);
}

}  // namespace csa

extern "C" {

int csa_timing_enable(int kernel)
{
    if (kernel < -1 || kernel >= csa::K_COUNT) return CSA_ERR_ARG;
    csa::state().kernel.store(kernel, std::memory_order_relaxed);
    return CSA_OK;
}

int csa_timing_read(int* launches, double* total_ms)
{
    csa::State& s = csa::state();
    std::lock_guard<std::mutex> lk(s.mu);
    int n = 0;
    double sum = 0.0;
    int rc = CSA_OK;
    for (auto& ev : s.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(ev.second) != hipSuccess || hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess)
            rc = CSA_ERR_HIP;
        else {
            sum += ms;
            ++n;
        }
        s.pool.push_back(ev);
    }
    s.pending.clear();
    if (launches) *launches = n;
    if (total_ms) *total_ms = sum;
    return rc;
}

const char* csa_kernel_name(int kernel)
{
    static const char* names[csa::K_COUNT] = {"compress_fwd", "compress_bwd", "index_topk", "attn_query_fwd",
                                               "attn_query_dq", "attn_rows", "attn_reduce", "loss_query",
                                               "loss_keys", "loss_reduce", "compress_epilogue"};
    return (kernel >= 0 && kernel < csa::K_COUNT) ? names[kernel] : "";
}

}  // extern "C"
