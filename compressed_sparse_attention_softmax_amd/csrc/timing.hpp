// timing.hpp -- optional per-kernel timing with HIP events (internal).
//
// While timing is enabled for one kernel id, every launch of that kernel is
// bracketed by two events recorded on the stream it is launched on, so the
// elapsed time between them is that launch's duration on the device.
#pragma once
#include <hip/hip_runtime.h>

namespace csa {

enum KernelId {
    K_COMPRESS_FWD = 0,
    K_COMPRESS_BWD = 1,
    K_INDEX_TOPK = 2,
    K_ATTN_FWD = 3,
    K_ATTN_DQ = 4,
    K_ATTN_ROWS = 5,
    K_ATTN_REDUCE = 6,
    K_LOSS_QUERY = 7,
    K_LOSS_KEYS = 8,
    K_LOSS_REDUCE = 9,
    K_COMPRESS_EPI = 10,
    K_COUNT = 11,
};

// RAII bracket around one launch: records the start event at construction and
// the stop event at destruction when timing is enabled for `id`.
class TimedLaunch {
  public:
    TimedLaunch(int id, hipStream_t st);
    ~TimedLaunch();
    TimedLaunch(const TimedLaunch&) = delete;
    TimedLaunch& operator=(const TimedLaunch&) = delete;

  private:
    hipStream_t st_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};

}  // namespace csa
