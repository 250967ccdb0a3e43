// av_prof.cpp — optional per-launch timing: when enabled, every kernel launch
// of the library is bracketed by HIP events recorded on the launch's stream.
// Used by the benchmark to time each kernel inside its timed region.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "av_launch.h"

namespace av {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};

constexpr size_t kMaxRecords = 1 << 16;

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Rec> g_recs;        // records of the current session
std::vector<hipEvent_t> g_pool;  // events reusable by the next session
thread_local int t_open = -1;    // index of the record opened by this thread

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

void prof_begin(const char* name, hipStream_t stream) {
  t_open = -1;
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_recs.size() >= kMaxRecords) return;
  Rec r{name, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  hipEventRecord(r.start, stream);
  g_recs.push_back(r);
  t_open = (int)g_recs.size() - 1;
}

void prof_end(hipStream_t stream) {
  if (t_open < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (t_open < (int)g_recs.size()) hipEventRecord(g_recs[t_open].stop, stream);
  t_open = -1;
}

int prof_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (enable) {
    for (auto& r : g_recs) {
      g_pool.push_back(r.start);
      g_pool.push_back(r.stop);
    }
    g_recs.clear();
  }
  g_enabled.store(enable != 0);
  return 0;
}

int prof_count() {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int)g_recs.size();
}

int prof_get(int i, char* name, int cap, float* ms) {
  Rec r;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (i < 0 || i >= (int)g_recs.size()) return -1;
    r = g_recs[i];
  }
  if (name && cap > 0) {
    std::strncpy(name, r.name, (size_t)cap - 1);
    name[cap - 1] = '\0';
  }
  if (hipEventSynchronize(r.stop) != hipSuccess) return -2;
  float t = 0.f;
  if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return -2;
  if (ms) *ms = t;
  return 0;
}

}  // namespace av
