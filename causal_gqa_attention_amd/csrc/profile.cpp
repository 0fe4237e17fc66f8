// Opt-in per-kernel timing: while enabled, every kernel the library launches is
// bracketed by two hipEvents recorded on its launch stream.  Disabled (the default),
// the only cost per launch is one relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "xattn_internal.h"

namespace xattn {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<int> g_on{0};
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

ProfScope::ProfScope(const char* name, hipStream_t stream) : stream_(stream) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  stop_ = take_event();
  name_ = name;
  if (start_ && stop_ && hipEventRecord(start_, stream_) == hipSuccess) return;
  if (start_) g_pool.push_back(start_);
  if (stop_) g_pool.push_back(stop_);
  start_ = stop_ = nullptr;
}

ProfScope::~ProfScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    g_recs.push_back({name_, start_, stop_});
  } else {
    g_pool.push_back(start_);
    g_pool.push_back(stop_);
  }
}

void profile_start() {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  g_on.store(1);
}

int profile_stop(char (*names)[48], long long* launches, double* total_ms, int max_entries,
                 hipError_t* err) {
  g_on.store(0);
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<long long, double>> agg;
  std::vector<std::string> order;
  *err = hipSuccess;
  for (auto& r : g_recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) *err = e;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {1, (double)ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  int n = 0;
  for (const auto& name : order) {
    if (n >= max_entries) break;
    std::strncpy(names[n], name.c_str(), 47);
    names[n][47] = '\0';
    launches[n] = agg[name].first;
    total_ms[n] = agg[name].second;
    ++n;
  }
  return (int)order.size();
}

}  // namespace xattn
