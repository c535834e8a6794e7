// Kernel timer: optional instrumentation that brackets every launch of one chosen kernel with
// a pair of HIP events recorded on the launch's own stream, so a benchmark can read that
// kernel's device time over a region of ordinary calls. Disarmed (the default) it is a no-op.
#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "../../include/ls_replay.h"
#include "kernels.h"

namespace {

constexpr size_t kMaxLaunches = 1 << 16;

struct Timer {
  std::mutex mu;
  int kernel = -1;                                   // armed kernel id, -1 = disarmed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;  // created lazily, reused
  size_t used = 0;                                   // pairs recorded since arming
  bool open = false;                                 // a begin event is waiting for its end
  bool failed = false;                               // an event call failed or too many launches
};

Timer& timer() {
  static Timer t;
  return t;
}

}  // namespace

namespace lsr {

void timer_mark(int kernel, hipStream_t st, bool end) {
  Timer& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (t.kernel != kernel || t.failed) return;
  if (!end) {
    if (t.used >= kMaxLaunches) {
      t.failed = true;
      return;
    }
    if (t.used == t.ev.size()) {
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
        t.failed = true;
        return;
      }
      t.ev.emplace_back(a, b);
    }
    if (hipEventRecord(t.ev[t.used].first, st) != hipSuccess) t.failed = true;
    t.open = true;
  } else if (t.open) {
    if (hipEventRecord(t.ev[t.used].second, st) != hipSuccess) t.failed = true;
    ++t.used;
    t.open = false;
  }
}

}  // namespace lsr

extern "C" {

int ls_kernel_timer_start(int32_t kernel) {
  if (kernel < LS_KERNEL_ATTN_FWD || kernel > LS_KERNEL_GRPO_ROWS) return LS_ERR_INVALID_ARG;
  Timer& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  t.kernel = kernel;
  t.used = 0;
  t.open = false;
  t.failed = false;
  return LS_OK;
}

int ls_kernel_timer_stop(float* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return LS_ERR_INVALID_ARG;
  Timer& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  const bool was_armed = t.kernel >= 0;
  t.kernel = -1;
  *total_ms = 0.0f;
  *launches = 0;
  if (!was_armed) return LS_ERR_INVALID_ARG;
  if (t.failed) return LS_ERR_HIP;
  double sum = 0.0;
  for (size_t i = 0; i < t.used; ++i) {
    if (hipEventSynchronize(t.ev[i].second) != hipSuccess) return LS_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.ev[i].first, t.ev[i].second) != hipSuccess) return LS_ERR_HIP;
    sum += ms;
  }
  *total_ms = (float)sum;
  *launches = (int32_t)t.used;
  return LS_OK;
}

}  // extern "C"
