// profile.hip -- optional per-kernel timing with HIP events.
//
// When enabled (moe_profile_enable), every kernel the library launches carries a
// pair of HIP events that the launch itself timestamps at the kernel's start and
// end (hipExtLaunchKernelGGL), so the elapsed time is the kernel's own duration,
// not the dispatch latency around it; the times are accumulated per kernel name
// when moe_profile_read is called.  Off by default; when off, the launch path
// checks one flag.  Not for use under stream capture.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "common.h"

namespace moe {

namespace {

const char* const kNames[KID_COUNT] = {"route_logits", "route_topk", "route_permute", "plan",
                                       "gateup",       "down",       "shared_gateup", "shared_down",
                                       "combine",      "rmsnorm",    "zero",          "xprep",        "swiglu",
                                       "route",        "set_table",     "cache",         "stream_read"};

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

// Streaming-read probe: 16-byte loads, eight in flight per thread, each wave
// instruction reading 1,024 contiguous bytes, a grid-stride walk over the buffer.
// The loaded words are XOR-folded per thread; a thread stores its fold only if it
// equals a value no input here produces, so the loads cannot be dropped and the
// writes are nil.
constexpr int kStreamUnroll = 8;
constexpr int64_t kStreamMaxBlocks = 4096;  // 16 blocks of four waves per compute unit
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256 * kStreamUnroll;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kStreamUnroll + threadIdx.x; base < n16;
       base += stride) {
    uint4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t i = base + 256 * u;
      v[u] = i < n16 ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace moe

extern "C" {

moe_status moe_stream_read(const void* src, size_t bytes, void* sink, moe_stream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)src & 15))
    return MOE_E_ARG;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per_block = 256 * moe::kStreamUnroll;
  const int grid = (int)std::min<int64_t>((n16 + per_block - 1) / per_block, moe::kStreamMaxBlocks);
  hipStream_t s = (hipStream_t)stream;
  MOE_LAUNCH(moe::KID_STREAM, moe::k_stream_read, dim3(grid), dim3(256), 0, s, (const uint4*)src,
             n16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

moe_status moe_profile_enable(int32_t on) {
  moe::Profiler& p = moe::prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return MOE_OK;
}

int32_t moe_profile_read_stats(int32_t max_kernels, char* names, double* total_ms,
                               double* median_ms, double* typical_mean_ms, int64_t* launches) {
  moe::Profiler& p = moe::prof();
  std::lock_guard<std::mutex> g(p.mu);
  std::vector<double> t_of[moe::KID_COUNT];
  for (const moe::Rec& r : p.recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.e) == hipSuccess && hipEventElapsedTime(&t, r.b, r.e) == hipSuccess)
      t_of[r.kid].push_back(t);
    p.pool.push_back(r.b);
    p.pool.push_back(r.e);
  }
  p.recs.clear();
  int32_t out = 0;
  for (int k = 0; k < moe::KID_COUNT && out < max_kernels; ++k) {
    std::vector<double>& v = t_of[k];
    if (v.empty()) continue;
    if (names) {
      strncpy(names + 32 * out, moe::kNames[k], 31);
      names[32 * out + 31] = 0;
    }
    double sum = 0.0;
    for (double x : v) sum += x;
    if (total_ms) total_ms[out] = sum;
    std::sort(v.begin(), v.end());
    const size_t m = v.size();
    const double med = m % 2 ? v[m / 2] : 0.5 * (v[m / 2 - 1] + v[m / 2]);
    if (median_ms) median_ms[out] = med;
    if (typical_mean_ms) {  // the mean of the launches within twice the median
      double s2 = 0.0;
      int64_t c = 0;
      for (double x : v)
        if (x <= 2.0 * med) {
          s2 += x;
          ++c;
        }
      typical_mean_ms[out] = s2 / (double)c;
    }
    if (launches) launches[out] = (int64_t)v.size();
    ++out;
  }
  return out;
}

int32_t moe_profile_read(int32_t max_kernels, char* names, double* total_ms, int64_t* launches) {
  return moe_profile_read_stats(max_kernels, names, total_ms, nullptr, nullptr, launches);
}

}  // extern "C"
