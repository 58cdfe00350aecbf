// cache.hip -- a device-side expert cache over a layer's pointer table.
//
// Every expert has a home copy (device memory, or pinned host memory read
// zero-copy) and the layer's table points at it; a slot arena in device memory
// holds copies of the experts the cache admits.  After routing, one block per
// layer marks the step's experts (those owning a pair: the grouping has already
// deduplicated the picks), counts hits, picks a victim slot for each miss, and
// rewrites the table in place: an admitted expert's entry points at its slot, an
// evicted one's back at its home copy.  A gather kernel then copies the admitted
// experts into their slots.  Both kernels read the step's counts from device
// memory, so nothing waits for the host (page "GLM-5.3-Flash EXL3 3.05bpw on 1x
// RTX PRO 6000 - GPU expert cache, host-RAM streaming", field
// config.expert_cache.mechanism: LFU scores decaying by 0.995, each miss taking
// the lowest-scoring slot the step does not use, tables rewritten in place, then
// a copy kernel; page "0xSero/glm53-flash-offload", paragraph "Elastic CLOCK
// expert cache": CLOCK victims and a gather kernel).  The bytes an expert's
// kernels read are the same wherever they live, so the layer's results do not
// change.
//
// Policy semantics are those of host/cachesim.c (the host replay the tests check
// this manager against): misses are admitted in ascending expert id; a free slot
// is taken first (lowest index); LFU keeps a score for every expert (times decay
// each step, plus one per step that uses it) and evicts the lowest score, ties
// to the least recently used, then the lower id; CLOCK sweeps the slots from its
// hand, clearing set reference bits, and takes the first clear slot whose expert
// the step does not need.  A miss finds no slot when every resident expert is
// needed; it is then read from its home copy.
#include "common.h"

namespace moe {

constexpr int kCacheThreads = 1024;  // one block per layer: E, S <= 1024

// state header (the first 256 bytes of the state buffer); the arrays follow at
// 256-byte boundaries in the order of cache_layout
struct CacheHdr {
  int64_t step, hits, misses;            // steps managed, totals
  int32_t step_hits, step_misses;        // the last step's counts
  int32_t n_jobs, hand;                  // admissions of the last step, CLOCK hand
  int32_t slots, policy, E, n_filled;
  double decay;
  uint64_t arena;                        // slot arena base address
  int64_t slot_bytes, off_up, off_down;  // slot stride, offsets of up and down
  int64_t bytes_gu, bytes_dn;            // bytes of a gate (or up) and a down matrix
};
static_assert(sizeof(CacheHdr) <= 256, "cache header");

struct CacheLayout {
  int64_t home, slot_of, expert_of, ref, score, last, jobs, total;
};
__host__ __device__ inline CacheLayout cache_layout(int E, int S) {
  CacheLayout c{};
  int64_t o = 256;
  auto take = [&](int64_t b) {
    const int64_t r = o;
    o += align256(b > 0 ? b : 0);
    return r;
  };
  c.home = take((int64_t)E * (int64_t)sizeof(moe_expert_ref));
  c.slot_of = take((int64_t)E * 4);
  c.expert_of = take((int64_t)S * 4);
  c.ref = take((int64_t)S * 4);
  c.score = take((int64_t)E * 8);
  c.last = take((int64_t)E * 8);
  c.jobs = take((int64_t)2 * S * 4);
  c.total = o;
  return c;
}

int64_t cache_state_bytes(int E, int S) { return cache_layout(E, S).total; }

template <typename T>
__device__ __forceinline__ T* at(uint8_t* st, int64_t off) {
  return reinterpret_cast<T*>(st + off);
}

// ---------------------------------------------------------------- init
__global__ __launch_bounds__(kCacheThreads) void k_cache_init(uint8_t* __restrict__ st,
                                                              CacheHdr h) {
  const CacheLayout L = cache_layout(h.E, h.slots);
  if (threadIdx.x == 0) *reinterpret_cast<CacheHdr*>(st) = h;
  for (int e = threadIdx.x; e < h.E; e += kCacheThreads) {
    at<int32_t>(st, L.slot_of)[e] = -1;
    at<double>(st, L.score)[e] = 0.0;
    at<int64_t>(st, L.last)[e] = -1;
  }
  for (int q = threadIdx.x; q < h.slots; q += kCacheThreads) {
    at<int32_t>(st, L.expert_of)[q] = -1;
    at<int32_t>(st, L.ref)[q] = 0;
  }
}

// ---------------------------------------------------------------- manage
// LFU victim order: (score, last use, id) ascending
struct Cand {
  double score;
  int64_t last;
  int32_t id, slot;
};
__device__ __forceinline__ bool before(const Cand& a, const Cand& b) {
  if (a.slot < 0) return false;
  if (b.slot < 0) return true;
  if (a.score != b.score) return a.score < b.score;
  if (a.last != b.last) return a.last < b.last;
  return a.id < b.id;
}
__device__ __forceinline__ Cand shfl_cand(const Cand& c, int src) {
  Cand r;
  r.score = __shfl(c.score, src);
  r.last = __shfl(c.last, src);
  r.id = __shfl(c.id, src);
  r.slot = __shfl(c.slot, src);
  return r;
}

__global__ __launch_bounds__(kCacheThreads) void k_cache_manage(
    const int32_t* __restrict__ offsets, moe_expert_ref* __restrict__ table,
    uint8_t* __restrict__ st) {
  __shared__ CacheHdr h;
  __shared__ uint8_t need[kCacheThreads];
  __shared__ int32_t miss[kCacheThreads];
  __shared__ int wcount[16];
  __shared__ Cand wbest[16];
  __shared__ int s_victim;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) h = *reinterpret_cast<const CacheHdr*>(st);
  __syncthreads();
  const int E = h.E, S = h.slots;
  const CacheLayout L = cache_layout(E, S);
  moe_expert_ref* home = at<moe_expert_ref>(st, L.home);
  int32_t* slot_of = at<int32_t>(st, L.slot_of);
  int32_t* expert_of = at<int32_t>(st, L.expert_of);
  int32_t* ref = at<int32_t>(st, L.ref);
  double* score = at<double>(st, L.score);
  int64_t* last = at<int64_t>(st, L.last);
  int32_t* jobs = at<int32_t>(st, L.jobs);
  const int64_t step = h.step;

  // the step's experts, hits, scores; misses listed in ascending id
  const int e = tid;
  const bool nd = e < E && offsets[e + 1] > offsets[e];
  if (e < kCacheThreads) need[e] = nd;
  int so = e < E ? slot_of[e] : -1;
  if (e < E && h.policy == 0) {  // LFU: decay every score, one more for a use
    double v = __dmul_rn(score[e], h.decay);
    if (nd) v = __dadd_rn(v, 1.0);
    score[e] = v;
  }
  const bool hit = nd && so >= 0, mis = nd && so < 0;
  if (nd) last[e] = step;
  if (hit && h.policy == 1) ref[so] = 1;
  const uint64_t bm = __ballot(mis);
  const int below = __popcll(bm & ((1ull << lane) - 1ull));
  if (lane == 0) wcount[wv] = __popcll(bm);
  const int n_hit = __syncthreads_count(hit);
  int base = 0, n_miss = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wv) base += wcount[w];
    n_miss += wcount[w];
  }
  if (mis) miss[base + below] = e;
  __syncthreads();

  // admissions, one miss at a time (each may evict the victim the next one sees)
  int n_jobs = 0, n_filled = h.n_filled, hand = h.hand;
  for (int i = 0; i < n_miss && S > 0; ++i) {
    const int em = miss[i];
    int k = -1;
    if (n_filled < S) {
      k = n_filled++;
    } else if (h.policy == 1) {  // CLOCK: one thread sweeps from the hand
      if (tid == 0) {
        int found = -1;
        for (int n = 0; n < 2 * S && found < 0; ++n) {
          const int q = hand;
          hand = hand + 1 == S ? 0 : hand + 1;
          if (need[expert_of[q]]) continue;
          if (ref[q]) {
            ref[q] = 0;
            continue;
          }
          found = q;
        }
        s_victim = found;
        wcount[0] = hand;
      }
      __syncthreads();
      k = s_victim;
      hand = wcount[0];
    } else {  // LFU: the lowest (score, last use, id) among slots the step does not need
      Cand c{0.0, 0, 0, -1};
      if (tid < S) {
        const int v = expert_of[tid];
        if (!need[v]) c = Cand{score[v], last[v], v, tid};
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const Cand x = shfl_cand(c, lane ^ o);
        if (before(x, c)) c = x;
      }
      if (lane == 0) wbest[wv] = c;
      __syncthreads();
      if (tid == 0) {
        Cand b = wbest[0];
        for (int w = 1; w < 16; ++w)
          if (before(wbest[w], b)) b = wbest[w];
        s_victim = b.slot;
      }
      __syncthreads();
      k = s_victim;
    }
    if (k >= 0 && tid == 0) {
      const int v = expert_of[k];
      if (v >= 0) {  // evicted: back to its home copy
        slot_of[v] = -1;
        table[v] = home[v];
      }
      slot_of[em] = k;
      expert_of[k] = em;
      ref[k] = 1;
      const uint64_t sb = h.arena + (uint64_t)k * (uint64_t)h.slot_bytes;
      table[em] = moe_expert_ref{(const void*)sb, (const void*)(sb + h.off_up),
                                 (const void*)(sb + h.off_down)};
      jobs[2 * n_jobs] = em;
      jobs[2 * n_jobs + 1] = k;
    }
    if (k >= 0) ++n_jobs;
    __syncthreads();  // expert_of, need and the victim before the next miss
  }
  if (tid == 0) {
    CacheHdr* g = reinterpret_cast<CacheHdr*>(st);
    g->step = step + 1;
    g->hits = h.hits + n_hit;
    g->misses = h.misses + n_miss;
    g->step_hits = n_hit;
    g->step_misses = n_miss;
    g->n_jobs = n_jobs;
    g->hand = hand;
    g->n_filled = n_filled;
  }
}

// ---------------------------------------------------------------- gather copy
// Item (job j, piece c): 16 KB of one of the admitted expert's three matrices,
// 16-byte loads and stores; blocks stride over the items of the step's jobs.
constexpr int kPiece = 16384;

__global__ __launch_bounds__(256) void k_cache_copy(const uint8_t* __restrict__ st) {
  const CacheHdr* h = reinterpret_cast<const CacheHdr*>(st);
  const int n_jobs = h->n_jobs;
  if (n_jobs == 0) return;
  const CacheLayout L = cache_layout(h->E, h->slots);
  const moe_expert_ref* home = reinterpret_cast<const moe_expert_ref*>(st + L.home);
  const int32_t* jobs = reinterpret_cast<const int32_t*>(st + L.jobs);
  const int64_t pg = (h->bytes_gu + kPiece - 1) / kPiece, pd = (h->bytes_dn + kPiece - 1) / kPiece;
  const int64_t per_job = 2 * pg + pd;
  const int64_t items = (int64_t)n_jobs * per_job;
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int j = (int)(it / per_job);
    int64_t c = it - (int64_t)j * per_job;
    const int e = jobs[2 * j], k = jobs[2 * j + 1];
    const uint8_t* src;
    uint8_t* dst = reinterpret_cast<uint8_t*>(h->arena + (uint64_t)k * (uint64_t)h->slot_bytes);
    int64_t bytes;
    if (c < pg) {
      src = (const uint8_t*)home[e].gate;
      bytes = h->bytes_gu;
    } else if (c < 2 * pg) {
      c -= pg;
      src = (const uint8_t*)home[e].up;
      dst += h->off_up;
      bytes = h->bytes_gu;
    } else {
      c -= 2 * pg;
      src = (const uint8_t*)home[e].down;
      dst += h->off_down;
      bytes = h->bytes_dn;
    }
    const int64_t b0 = c * kPiece, b1 = b0 + kPiece < bytes ? b0 + kPiece : bytes;
    u4 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t o = b0 + (int64_t)(threadIdx.x + 256 * r) * 16;
      if (o < b1) v[r] = *reinterpret_cast<const u4*>(src + o);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t o = b0 + (int64_t)(threadIdx.x + 256 * r) * 16;
      if (o < b1) *reinterpret_cast<u4*>(dst + o) = v[r];
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_cache_init(uint8_t* state, int E, int S, int policy, double decay,
                             uint64_t arena, int64_t slot_bytes, int64_t bytes_gu,
                             int64_t bytes_dn, const moe_expert_ref* host_home,
                             moe_expert_ref* table, hipStream_t s) {
  CacheHdr h{};
  h.slots = S;
  h.policy = policy;
  h.E = E;
  h.decay = decay;
  h.arena = arena;
  h.slot_bytes = slot_bytes;
  h.off_up = bytes_gu;
  h.off_down = 2 * bytes_gu;
  h.bytes_gu = bytes_gu;
  h.bytes_dn = bytes_dn;
  MOE_LAUNCH(KID_CACHE, k_cache_init, dim3(1), dim3(kCacheThreads), 0, s, state, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the home copies, and the table pointing at them
  const CacheLayout L = cache_layout(E, S);
  e = launch_set_table(reinterpret_cast<moe_expert_ref*>(state + L.home), host_home, E, s);
  if (e != hipSuccess) return e;
  return launch_set_table(table, host_home, E, s);
}

hipError_t launch_cache_step(const int32_t* offsets, moe_expert_ref* table, uint8_t* state,
                             hipStream_t s) {
  MOE_LAUNCH(KID_CACHE, k_cache_manage, dim3(1), dim3(kCacheThreads), 0, s, offsets, table, state);
  MOE_LAUNCH(KID_CACHE, k_cache_copy, dim3(1024), dim3(256), 0, s, state);
  return hipGetLastError();
}

}  // namespace moe
