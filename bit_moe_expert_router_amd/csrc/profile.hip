// profile.hip -- optional per-kernel timing with HIP events.
//
// When enabled (moe_profile_enable), every kernel the library launches carries a
// pair of HIP events that the launch itself timestamps at the kernel's start and
// end (hipExtLaunchKernelGGL), so the elapsed time is the kernel's own duration,
// not the dispatch latency around it; the times are accumulated per kernel name
// when moe_profile_read is called.  Off by default; when off, the launch path
// checks one flag.  Not for use under stream capture.
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

namespace moe {

namespace {

const char* const kNames[KID_COUNT] = {"route_logits", "route_topk", "route_permute", "plan",
                                       "gateup",       "down",       "shared_gateup", "shared_down",
                                       "combine",      "rmsnorm",    "zero",          "xprep",        "swiglu",
                                       "route",        "set_table",     "cache"};

struct Rec {
  int kid;
  hipEvent_t b, e;
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  Rec open{-1, nullptr, nullptr};

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t ev = pool.back();
      pool.pop_back();
      return ev;
    }
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) return nullptr;
    return ev;
  }
};

Profiler& prof() {
  static Profiler p;
  return p;
}

}  // namespace

bool prof_on() { return prof().on; }

bool prof_events(int kid, hipEvent_t* b, hipEvent_t* e) {
  Profiler& p = prof();
  if (!p.on) return false;
  std::lock_guard<std::mutex> g(p.mu);
  hipEvent_t eb = p.get();
  if (!eb) return false;
  hipEvent_t ee = p.get();
  if (!ee) {
    p.pool.push_back(eb);
    return false;
  }
  p.recs.push_back(Rec{kid, eb, ee});
  *b = eb;
  *e = ee;
  return true;
}

}  // namespace moe

extern "C" {

moe_status moe_profile_enable(int32_t on) {
  moe::Profiler& p = moe::prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return MOE_OK;
}

int32_t moe_profile_read(int32_t max_kernels, char* names, double* total_ms, int64_t* launches) {
  moe::Profiler& p = moe::prof();
  std::lock_guard<std::mutex> g(p.mu);
  double ms[moe::KID_COUNT] = {0};
  int64_t n[moe::KID_COUNT] = {0};
  for (const moe::Rec& r : p.recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.e) == hipSuccess && hipEventElapsedTime(&t, r.b, r.e) == hipSuccess) {
      ms[r.kid] += t;
      n[r.kid] += 1;
    }
    p.pool.push_back(r.b);
    p.pool.push_back(r.e);
  }
  p.recs.clear();
  int32_t out = 0;
  for (int k = 0; k < moe::KID_COUNT && out < max_kernels; ++k) {
    if (!n[k]) continue;
    if (names) {
      strncpy(names + 32 * out, moe::kNames[k], 31);
      names[32 * out + 31] = 0;
    }
    if (total_ms) total_ms[out] = ms[k];
    if (launches) launches[out] = n[k];
    ++out;
  }
  return out;
}

}  // extern "C"
