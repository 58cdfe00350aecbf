// profile.hip -- optional per-kernel timing with HIP events.
//
// When enabled (moe_profile_enable), every kernel the library launches is
// bracketed by a pair of HIP events recorded on the launch stream; the elapsed
// times are accumulated per kernel name when moe_profile_read is called.  Off by
// default; when off, the launch path checks one flag.  Not for use under stream
// capture.
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

namespace moe {

namespace {

const char* const kNames[KID_COUNT] = {"route_logits", "route_topk", "route_permute", "plan",
                                       "gateup",       "down",       "shared_gateup", "shared_down",
                                       "combine",      "rmsnorm",    "zero",          "xprep",        "swiglu"};

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

void prof_begin(int kid, hipStream_t s) {
  Profiler& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> g(p.mu);
  hipEvent_t b = p.get();
  if (!b) return;
  (void)hipEventRecord(b, s);
  p.open = Rec{kid, b, nullptr};
}

void prof_end(int kid, hipStream_t s) {
  Profiler& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (p.open.kid != kid || !p.open.b) return;
  hipEvent_t e = p.get();
  if (!e) return;
  (void)hipEventRecord(e, s);
  p.open.e = e;
  p.recs.push_back(p.open);
  p.open = Rec{-1, nullptr, nullptr};
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
