// Optional per-kernel device timing: HIP events recorded on the launch stream
// around each kernel of the entry points, read back on request.

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "ttt_internal.h"

namespace {

struct Record {
  int kernel;
  hipEvent_t start, stop;
};

struct Timer {
  std::mutex mu;
  bool on = false;
  bool event_error = false;
  std::vector<hipEvent_t> pool;  // created once, reused across enables
  size_t next = 0;               // first unused pool entry
  std::vector<Record> records;

  hipEvent_t take() {
    if (next == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[next++];
  }
};

Timer& timer() {
  static Timer* t = new Timer();  // never destroyed: events outlive static teardown
  return *t;
}

}  // namespace

namespace ttt {

KernelScope::KernelScope(ttt_kernel kernel, hipStream_t s) : s_(s) {
  Timer& t = timer();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.on) return;
  hipEvent_t a = t.take();
  hipEvent_t b = a ? t.take() : nullptr;
  if (!a || !b || hipEventRecord(a, s) != hipSuccess) {
    t.event_error = true;
    return;
  }
  t.records.push_back({static_cast<int>(kernel), a, b});
  stop_ = b;
}

KernelScope::~KernelScope() {
  if (!stop_) return;
  if (hipEventRecord(stop_, s_) != hipSuccess) {
    Timer& t = timer();
    std::lock_guard<std::mutex> lock(t.mu);
    t.event_error = true;
  }
}

}  // namespace ttt

extern "C" {

TTT_API int ttt_timing_enable(int on) {
  Timer& t = timer();
  std::lock_guard<std::mutex> lock(t.mu);
  if (on) {
    // Events of the old record may still be pending; wait so they can be reused.
    for (const Record& r : t.records) (void)hipEventSynchronize(r.stop);
    t.records.clear();
    t.next = 0;
    t.event_error = false;
  }
  t.on = on != 0;
  return TTT_OK;
}

TTT_API int ttt_timing_read(int kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= TTT_KERNEL_COUNT) return TTT_ERR_INVALID_ARG;
  Timer& t = timer();
  std::lock_guard<std::mutex> lock(t.mu);
  double sum = 0.0;
  int64_t n = 0;
  for (const Record& r : t.records) {
    if (r.kernel != kernel) continue;
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return TTT_ERR_HIP;
    sum += ms;
    ++n;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = n;
  return t.event_error ? TTT_ERR_HIP : TTT_OK;
}

}  // extern "C"
