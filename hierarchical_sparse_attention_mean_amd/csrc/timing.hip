// timing.hip -- opt-in per-kernel event timing for benchmarks (llsa_timing_enable / llsa_timing_read).
#include <atomic>
#include <mutex>
#include <vector>

#include "launch.hpp"
#include "llsa.h"

namespace llsa {

namespace {

struct Record {
  int family;
  hipEvent_t start, stop;
};

std::atomic<int> g_enabled{0};
std::mutex g_mu;
std::vector<Record> g_records;

void release_locked() {
  for (Record& r : g_records) {
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
  }
  g_records.clear();
}

}  // namespace

LaunchTimer::LaunchTimer(int family, hipStream_t stream) : family_(family), stream_(stream) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  if (hipEventCreate(&start_) != hipSuccess || hipEventCreate(&stop_) != hipSuccess) {
    start_ = stop_ = nullptr;
    return;
  }
  hipEventRecord(start_, stream_);
}

LaunchTimer::~LaunchTimer() {
  if (!start_) return;
  hipEventRecord(stop_, stream_);
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back({family_, start_, stop_});
}

}  // namespace llsa

extern "C" {

int llsa_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(llsa::g_mu);
  llsa::release_locked();
  llsa::g_enabled.store(on ? 1 : 0);
  return LLSA_OK;
}

int llsa_timing_read(int kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return LLSA_ERR_NULL;
  if (kernel < 0 || kernel >= LLSA_KERNEL_COUNT) return LLSA_ERR_PARAM;
  std::lock_guard<std::mutex> lk(llsa::g_mu);
  double t = 0.0;
  int64_t c = 0;
  for (const llsa::Record& r : llsa::g_records) {
    if (r.family != kernel) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return LLSA_ERR_LAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return LLSA_ERR_LAUNCH;
    t += ms;
    ++c;
  }
  *total_ms = t;
  *launches = c;
  return LLSA_OK;
}

}  // extern "C"
