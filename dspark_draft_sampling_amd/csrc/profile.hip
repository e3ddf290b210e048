// profile.hip — opt-in per-kernel timing with HIP events, and the Markov
// launch-plan switch (the library's only process-wide settings).
//
// When enabled, every kernel launch of the library records two events at the
// kernel's own start and end (hipExtLaunchKernelGGL); dspark_profile_summary
// synchronises them and
// reports, per kernel name, the launch count and the summed duration.  This is
// the only process-wide state of the library and it is off by default.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "dspark.h"
#include "internal.hpp"

namespace dspark {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<int> g_on{0};
std::atomic<int> g_markov_plan{DSPARK_MARKOV_AUTO};
std::mutex g_mu;
std::vector<Rec> g_recs;

}  // namespace

int markov_plan_mode() { return g_markov_plan.load(std::memory_order_relaxed); }

ProfScope::ProfScope(const char* name) : name_(name), a_(nullptr), b_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  if (hipEventCreate(&a_) != hipSuccess) {
    a_ = nullptr;
    return;
  }
  if (hipEventCreate(&b_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    a_ = nullptr;
    b_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back(Rec{name_, a_, b_});
}

}  // namespace dspark

extern "C" {

int dspark_markov_plan(int plan) {
  if (plan != DSPARK_MARKOV_AUTO && plan != DSPARK_MARKOV_PER_STEP && plan != DSPARK_MARKOV_COOPERATIVE &&
      plan != DSPARK_MARKOV_REQUEST_GROUPS)
    return -1;
  return dspark::g_markov_plan.exchange(plan);
}

int dspark_profile_enable(int on) {
  dspark::g_on.store(on ? 1 : 0);
  return 0;
}

int dspark_release(void) {
  std::vector<dspark::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(dspark::g_mu);
    recs.swap(dspark::g_recs);
  }
  for (const auto& r : recs) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  dspark::release_markov_chain();
  return 0;
}

int dspark_profile_summary(char* buf, size_t n) {
  std::vector<dspark::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(dspark::g_mu);
    recs.swap(dspark::g_recs);
  }
  std::map<std::string, std::pair<long, double>> acc;
  int rc = 0;
  for (const auto& r : recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      rc = DSPARK_EDEVICE;
    auto& e = acc[r.name];
    e.first += 1;
    e.second += ms;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  std::string out;
  for (const auto& kv : acc) {
    char line[256];
    std::snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first,
                  kv.second.second);
    out += line;
  }
  if (buf && n > 0) {
    const size_t m = out.size() < n - 1 ? out.size() : n - 1;
    std::memcpy(buf, out.data(), m);
    buf[m] = '\0';
  }
  return rc;
}

}  // extern "C"
