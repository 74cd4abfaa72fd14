// Per-kernel timing diagnostics.  When enabled, every kernel the library
// enqueues is bracketed by a pair of HIP events recorded on the launch stream;
// rmm_timing_collect() waits for the recorded pairs and folds the elapsed
// times into per-"tag/kernel" totals.  Disabled (the default) it costs one
// relaxed atomic load per launch.
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "rmm_internal.h"
#include "timing.h"

namespace rmm {
namespace {

struct Pending {
  std::string key;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::map<std::string, std::pair<double, int64_t>> g_totals;
thread_local std::string g_tag;

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

bool timing_on() { return g_on.load(std::memory_order_relaxed); }

KernelTimer::KernelTimer(const char *kernel, hipStream_t s) : stream_(s) {
  if (!timing_on()) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = take_event();
  b_ = take_event();
  if (!a_ || !b_) {   // out of events: give back the one that was taken, time nothing
    if (a_) g_pool.push_back(static_cast<hipEvent_t>(a_));
    if (b_) g_pool.push_back(static_cast<hipEvent_t>(b_));
    a_ = b_ = nullptr;
    return;
  }
  key_ = g_tag.empty() ? std::string(kernel) : g_tag + "/" + kernel;
  if (hipEventRecord(static_cast<hipEvent_t>(a_), s) != hipSuccess) {   // e.g. a stream under capture
    g_pool.push_back(static_cast<hipEvent_t>(a_));
    g_pool.push_back(static_cast<hipEvent_t>(b_));
    a_ = b_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!a_) return;
  const bool ok = hipEventRecord(static_cast<hipEvent_t>(b_), stream_) == hipSuccess;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!ok) {   // this launch goes untimed; the events return to the pool
    g_pool.push_back(static_cast<hipEvent_t>(a_));
    g_pool.push_back(static_cast<hipEvent_t>(b_));
    return;
  }
  g_pending.push_back({key_, static_cast<hipEvent_t>(a_), static_cast<hipEvent_t>(b_)});
}

}  // namespace rmm

#define RMM_API extern "C" __attribute__((visibility("default")))

RMM_API rmm_status_t rmm_timing_enable(int on) {
  rmm::g_on.store(on != 0, std::memory_order_relaxed);
  return RMM_OK;
}

RMM_API rmm_status_t rmm_timing_set_tag(const char *tag) {
  rmm::g_tag = tag ? tag : "";
  return RMM_OK;
}

RMM_API rmm_status_t rmm_timing_collect(void) {
  std::lock_guard<std::mutex> lk(rmm::g_mu);
  rmm_status_t st = RMM_OK;
  for (auto &p : rmm::g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
      st = RMM_ERR_HIP;
    } else {
      auto &t = rmm::g_totals[p.key];
      t.first += ms;
      t.second += 1;
    }
    rmm::g_pool.push_back(p.a);
    rmm::g_pool.push_back(p.b);
  }
  rmm::g_pending.clear();
  return st;
}

RMM_API int rmm_timing_count(void) {
  std::lock_guard<std::mutex> lk(rmm::g_mu);
  return (int)rmm::g_totals.size();
}

RMM_API rmm_status_t rmm_timing_entry(int i, char *name, size_t name_len, double *total_ms,
                                      int64_t *launches) {
  std::lock_guard<std::mutex> lk(rmm::g_mu);
  if (i < 0 || i >= (int)rmm::g_totals.size() || !name || name_len == 0 || !total_ms || !launches)
    return RMM_ERR_INVALID_ARG;
  auto it = rmm::g_totals.begin();
  std::advance(it, i);
  snprintf(name, name_len, "%s", it->first.c_str());
  *total_ms = it->second.first;
  *launches = it->second.second;
  return RMM_OK;
}

RMM_API rmm_status_t rmm_timing_reset(void) {
  std::lock_guard<std::mutex> lk(rmm::g_mu);
  rmm::g_totals.clear();
  return RMM_OK;
}
