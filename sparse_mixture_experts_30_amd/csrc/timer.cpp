// Per-kernel timing with HIP events, for measurement.  While the timer is on,
// every kernel launch of the library is bracketed by two events recorded on
// the stream the kernel is launched on; reading waits for them and sums the
// elapsed time per kernel name.  Off (the default) it costs one relaxed load
// per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_internal.hpp"

namespace moe {
namespace {

struct Mark {
  const char* name;
  hipEvent_t begin, end;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::string g_only;               // empty: every kernel
std::vector<hipEvent_t> g_pool;   // free events
std::vector<Mark> g_marks;        // recorded pairs, oldest first
std::map<std::string, std::pair<double, int64_t>> g_sum;  // read results
std::vector<std::string> g_names; // storage behind the names handed out

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

bool wanted(const char* name) { return g_only.empty() || g_only == name; }

}  // namespace

KernelTimerScope::KernelTimerScope(hipStream_t s, const char* name) : s_(s), name_(name) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!wanted(name)) return;
  begin_ = take_event();
  if (begin_ && hipEventRecord((hipEvent_t)begin_, s) != hipSuccess) {
    g_pool.push_back((hipEvent_t)begin_);
    begin_ = nullptr;
  }
}

KernelTimerScope::~KernelTimerScope() {
  if (!begin_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t end = take_event();
  if (!end || hipEventRecord(end, s_) != hipSuccess) {
    g_pool.push_back((hipEvent_t)begin_);
    if (end) g_pool.push_back(end);
    return;
  }
  g_marks.push_back({name_, (hipEvent_t)begin_, end});
}

}  // namespace moe

extern "C" {

moe_status moe_kernel_timer_enable(int on, const char* only) {
  std::lock_guard<std::mutex> lk(moe::g_mu);
  moe::g_only = (on && only) ? only : "";
  moe::g_on.store(on ? 1 : 0);
  return MOE_OK;
}

int moe_kernel_timer_read(int cap, const char** names, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(moe::g_mu);
  moe::g_sum.clear();
  for (const moe::Mark& m : moe::g_marks) {
    float ms = 0.f;
    if (hipEventSynchronize(m.end) == hipSuccess &&
        hipEventElapsedTime(&ms, m.begin, m.end) == hipSuccess) {
      auto& v = moe::g_sum[m.name];
      v.first += ms;
      v.second += 1;
    }
    moe::g_pool.push_back(m.begin);
    moe::g_pool.push_back(m.end);
  }
  moe::g_marks.clear();
  moe::g_names.clear();
  int n = 0;
  for (const auto& kv : moe::g_sum) {
    moe::g_names.push_back(kv.first);
    if (n < cap) {
      if (total_ms) total_ms[n] = kv.second.first;
      if (launches) launches[n] = kv.second.second;
    }
    ++n;
  }
  for (int i = 0; i < n && i < cap; ++i)
    if (names) names[i] = moe::g_names[i].c_str();
  return n;
}

}  // extern "C"
