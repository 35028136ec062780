// Optional per-kernel timing for benchmarks.  While enabled, every kernel the
// library launches is bracketed by two HIP events recorded on the launch
// stream; cla_timing_read() waits for them and reports the total time and the
// launch count per kernel name.  Disabled by default: then the hooks cost one
// branch per launch.  A start event waits in a per-stream slot until its stop
// event is recorded, so launches enqueued from several threads on different
// streams pair their own events.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/cla.h"
#include "internal.h"

namespace cla {
namespace timing {
namespace {

struct Rec {
  const char *name;
  hipEvent_t start, stop;
};

std::mutex mu;
std::atomic<bool> enabled{false};
std::vector<Rec> recs;
std::vector<hipEvent_t> pool;
// start events recorded by before() and not yet closed by after(), one per
// stream
std::vector<std::pair<hipStream_t, hipEvent_t>> pending;

hipEvent_t get_event() {
  if (!pool.empty()) {
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

// Removes and returns the open start event of `stream` (nullptr if none).
hipEvent_t take_pending(hipStream_t stream) {
  for (size_t i = 0; i < pending.size(); ++i) {
    if (pending[i].first == stream) {
      hipEvent_t e = pending[i].second;
      pending.erase(pending.begin() + (ptrdiff_t)i);
      return e;
    }
  }
  return nullptr;
}

void before(hipStream_t stream) {
  if (!enabled) return;
  std::lock_guard<std::mutex> g(mu);
  hipEvent_t stale = take_pending(stream);
  if (stale) pool.push_back(stale);
  hipEvent_t start = get_event();
  if (!start) return;
  if (hipEventRecord(start, stream) != hipSuccess) {
    pool.push_back(start);
    return;
  }
  pending.push_back({stream, start});
}

void after(hipStream_t stream, const char *name) {
  if (!enabled) return;
  std::lock_guard<std::mutex> g(mu);
  hipEvent_t start = take_pending(stream);
  if (!start) return;
  hipEvent_t stop = get_event();
  if (!stop || hipEventRecord(stop, stream) != hipSuccess) {
    pool.push_back(start);
    if (stop) pool.push_back(stop);
    return;
  }
  recs.push_back({name, start, stop});
}

void cancel(hipStream_t stream) {
  std::lock_guard<std::mutex> g(mu);
  hipEvent_t start = take_pending(stream);
  if (start) pool.push_back(start);
}

}  // namespace timing
}  // namespace cla

extern "C" {

int cla_timing_enable(int enable) {
  std::lock_guard<std::mutex> g(cla::timing::mu);
  cla::timing::enabled = enable != 0;
  return CLA_OK;
}

int cla_timing_read(const char **names, double *total_ms, int64_t *counts, int max) {
  using namespace cla::timing;
  std::lock_guard<std::mutex> g(mu);
  std::vector<const char *> keys;
  std::vector<double> tot;
  std::vector<int64_t> cnt;
  int status = CLA_OK;
  for (const Rec &r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = CLA_ERR_HIP;
    size_t k = 0;
    while (k < keys.size() && strcmp(keys[k], r.name) != 0) ++k;
    if (k == keys.size()) {
      keys.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[k] += ms;
    cnt[k] += 1;
    pool.push_back(r.start);
    pool.push_back(r.stop);
  }
  recs.clear();
  if (status != CLA_OK) return -status;
  const int n = (int)keys.size();
  for (int k = 0; k < n && k < max; ++k) {
    if (names) names[k] = keys[k];
    if (total_ms) total_ms[k] = tot[k];
    if (counts) counts[k] = cnt[k];
  }
  return n;
}

}  // extern "C"
