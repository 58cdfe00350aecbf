// route.hip -- router logits, top-k with renormalised softmax weights, and the
// bit-exact grouping of (token, pick) pairs by expert.
//
// Routing picks the top-8 of 288 experts per token per MoE layer (page
// "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX 3090 -- RAM/NVMe expert tiering", field
// summary); the picks are then deduplicated into a per-layer expert union with
// each expert's token list (page "0xSero/glm53-flash-offload", paragraphs
// "Elastic CLOCK expert cache" and "Batched decode").  The router function itself
// is not printed on the pages; it is the softmax over logits x.Wr^T + bias with
// the top-k weights renormalised.
//
// Logits are accumulated in fp64: a bf16 x fp32 product is exact in fp64, so the
// selection equals the exact-arithmetic one up to the rounding of a 5120-term
// fp64 sum (relative 1e-15), far below the smallest 8th/9th-logit margins the
// workloads produce.  Every reduction has a fixed order (no float atomics).
#include <type_traits>

#include "common.h"

namespace moe {

// ---------------------------------------------------------------- logits, small T
// Block = one expert x up to 4 tokens; 256 threads stride over H in float4 steps,
// each thread issuing all its loads of a batch (8 float4 of the router row and
// the matching activations of every token) before using any, so a 5120-wide row
// costs one memory round trip.  Items past the row end load the last item and
// use a zero router value.
constexpr int kLogitTok = 4;
constexpr int kLogitBatch = 8;

__global__ __launch_bounds__(256) void k_logits_small(const uint16_t* __restrict__ x, int T,
                                                      int H, int E,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias,
                                                      double* __restrict__ logits) {
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kLogitTok;
  const int nt = min(kLogitTok, T - t0);
  const int H4 = H / 4;
  const float4* w4 = reinterpret_cast<const float4*>(wr + (int64_t)e * H);
  double acc[kLogitTok];
#pragma unroll
  for (int j = 0; j < kLogitTok; ++j) acc[j] = 0.0;
  for (int b = 0; b < H4; b += 256 * kLogitBatch) {
    float4 w[kLogitBatch];
    uint2 xv[kLogitTok][kLogitBatch];
#pragma unroll
    for (int r = 0; r < kLogitBatch; ++r) {
      const int i = min(b + (int)threadIdx.x + 256 * r, H4 - 1);
      w[r] = w4[i];
#pragma unroll
      for (int j = 0; j < kLogitTok; ++j)
        xv[j][r] = reinterpret_cast<const uint2*>(x + (int64_t)(t0 + min(j, nt - 1)) * H)[i];
    }
#pragma unroll
    for (int r = 0; r < kLogitBatch; ++r) {
      if (b + (int)threadIdx.x + 256 * r >= H4) w[r] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < kLogitTok; ++j) {
        acc[j] = fma((double)bf16_to_f32((uint16_t)xv[j][r].x), (double)w[r].x, acc[j]);
        acc[j] = fma((double)bf16_to_f32((uint16_t)(xv[j][r].x >> 16)), (double)w[r].y, acc[j]);
        acc[j] = fma((double)bf16_to_f32((uint16_t)xv[j][r].y), (double)w[r].z, acc[j]);
        acc[j] = fma((double)bf16_to_f32((uint16_t)(xv[j][r].y >> 16)), (double)w[r].w, acc[j]);
      }
    }
  }
  __shared__ double red[4][kLogitTok];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kLogitTok; ++j) {
    if (j < nt) {
      double v = acc[j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) red[wv][j] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int j = threadIdx.x;
    double v = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
    if (bias) v += (double)bias[e];
    logits[(int64_t)(t0 + j) * E + e] = v;
  }
}

// ---------------------------------------------------------------- logits, large T
// Tiled fp64 product: block = 32 tokens x 32 experts, 256 threads with 2x2
// outputs each, reduction dim staged through LDS in steps of 32.
constexpr int kLT = 32, kLE = 32, kLK = 32;

__global__ __launch_bounds__(256) void k_logits_tiled(const uint16_t* __restrict__ x, int T,
                                                      int H, int E,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias,
                                                      double* __restrict__ logits) {
  __shared__ double xs[kLK][kLT + 1];
  __shared__ double ws[kLK][kLE + 1];
  const int t0 = blockIdx.y * kLT, e0 = blockIdx.x * kLE;
  const int tid = threadIdx.x;
  const int ti = (tid % 16) * 2, ei = (tid / 16) * 2;
  double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  for (int k0 = 0; k0 < H; k0 += kLK) {
    for (int i = tid; i < kLT * kLK; i += 256) {
      int r = i / kLK, c = i % kLK;
      int t = t0 + r, e = e0 + r;
      xs[c][r] = t < T ? (double)bf16_to_f32(x[(int64_t)t * H + k0 + c]) : 0.0;
      ws[c][r] = e < E ? (double)wr[(int64_t)e * H + k0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kLK; ++c) {
      double a0 = xs[c][ti], a1 = xs[c][ti + 1];
      double b0 = ws[c][ei], b1 = ws[c][ei + 1];
      acc[0][0] = fma(a0, b0, acc[0][0]);
      acc[0][1] = fma(a0, b1, acc[0][1]);
      acc[1][0] = fma(a1, b0, acc[1][0]);
      acc[1][1] = fma(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int t = t0 + ti + i, e = e0 + ei + j;
      if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i][j] + (bias ? (double)bias[e] : 0.0);
    }
}

// ---------------------------------------------------------------- top-k + weights
// One wave per token.  Each lane keeps the logits of experts lane + 64*i.  Each
// of the K rounds takes the wave maximum of the remaining logits (DPP row
// shifts, then the row totals), then the lowest id among the lanes that hold it
// (same reduction on ids): the picks come out in output order (descending logit,
// ties to the lower id).  Lane k keeps pick k.  Weights: lane k < K computes
// exp(l_k - l_0) in fp64; every lane adds the K terms in k order.
constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / 64;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v, int fill) {
  return __builtin_amdgcn_update_dpp(fill, v, CTRL, 0xF, 0xF, false);
}
// 64-bit max over the wave (every lane gets the result)
__device__ __forceinline__ double wave_max_f64(double v) {
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    const int lo = __double2loint(v), hi = __double2hiint(v);
    const double o = __hiloint2double(dpp_i<C>(hi, 0xFFF00000), dpp_i<C>(lo, 0));  // fill = -inf
    v = fmax(v, o);
  };
  step(std::integral_constant<int, 0x111>{});
  step(std::integral_constant<int, 0x112>{});
  step(std::integral_constant<int, 0x114>{});
  step(std::integral_constant<int, 0x118>{});
  step(std::integral_constant<int, 0x142>{});
  step(std::integral_constant<int, 0x143>{});
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_i<0x111>(v, 0x7FFFFFFF));
  v = min(v, dpp_i<0x112>(v, 0x7FFFFFFF));
  v = min(v, dpp_i<0x114>(v, 0x7FFFFFFF));
  v = min(v, dpp_i<0x118>(v, 0x7FFFFFFF));
  v = min(v, dpp_i<0x142>(v, 0x7FFFFFFF));
  v = min(v, dpp_i<0x143>(v, 0x7FFFFFFF));
  return __builtin_amdgcn_readlane(v, 63);
}

// this lane's pick (lane < K) and its weight; -1 for other lanes
__device__ __forceinline__ int wave_topk(const double* __restrict__ l, int E, int K, float* wk) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  double v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < per && e < E) ? l[e] : -INFINITY;
  }
  double my_l = -INFINITY;
  int my_id = -1;
  for (int k = 0; k < K; ++k) {
    // local best: highest value, lowest id among equals (ids grow with i)
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per && e < E && v[i] > bv) {
        bv = v[i];
        bi = e;
      }
    }
    const double m = wave_max_f64(bv);
    const int id = wave_min_i32(bv == m ? bi : 0x7FFFFFFF);
    if ((id & 63) == lane) {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i)
        if (i == (id >> 6)) v[i] = -INFINITY;  // taken
    }
    if (lane == k) {
      my_l = m;
      my_id = id;
    }
  }
  const double l0 = __shfl(my_l, 0);
  const double term = lane < K ? exp(my_l - l0) : 0.0;
  double den = 0.0;
  for (int k = 0; k < K; ++k) den += __shfl(term, k);
  *wk = (float)(term / den);
  return lane < K ? my_id : -1;
}

__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int T, int E,
                                              int K, int32_t* __restrict__ ids,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float wk;
  const int id = wave_topk(logits + (int64_t)t * E, E, K, &wk);
  if (lane < K) {
    ids[t * K + lane] = id;
    wout[t * K + lane] = wk;
  }
}

// ---------------------------------------------------------------- grouping
// One wave.  Pairs are taken 64 at a time in pair order; lanes holding the same
// expert id are matched with one ballot per id bit, which gives each pair its
// rank among equal ids in the chunk and the chunk's count per id.  Pass 1 counts,
// an exclusive scan gives the offsets, pass 2 scatters (stable by pair index).
// Ids outside [0, E) are left out (pair_pos = -1).  Integer only: bit-exact.
__device__ __forceinline__ uint64_t match_mask(int e, int nbits) {
  uint64_t m = __ballot(1);
  for (int b = 0; b < nbits; ++b) {
    uint64_t bal = __ballot((e >> b) & 1);
    m &= ((e >> b) & 1) ? bal : ~bal;
  }
  return m;
}

// exclusive scan of cnt[0..E) in LDS by one wave (E <= 1024), total in cnt[E]
__device__ __forceinline__ void wave_exclusive_scan(int* cnt, int E) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int b = lane * per;
  int loc = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < E) loc += cnt[b + i];
  int inc = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  int run = inc - loc;
  for (int i = 0; i < per; ++i)
    if (b + i < E) {
      const int c = cnt[b + i];
      cnt[b + i] = run;
      run += c;
    }
  if (lane == 63) cnt[E] = inc;
}

// stable grouping of P pairs by one wave; ids read through `ids` (global or LDS)
__device__ void wave_group(const int32_t* ids, int P, int E, int* cnt, int* run,
                           int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
                           int32_t* __restrict__ pair_pos) {
  const int lane = threadIdx.x & 63;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;  // keys in [0, E]; E marks an invalid id
  for (int e = lane; e < E; e += 64) {
    cnt[e] = 0;
    run[e] = 0;
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < P; c0 += 64) {
    const int p = c0 + lane;
    const int e = p < P ? ids[p] : -1;
    const bool ok = p < P && e >= 0 && e < E;
    const uint64_t m = match_mask(ok ? e : E, nbits);
    if (ok && (m & lt) == 0) cnt[e] += __popcll(m);
  }
  wave_exclusive_scan(cnt, E);
  for (int e = lane; e <= E; e += 64) offsets[e] = cnt[e];
  for (int c0 = 0; c0 < P; c0 += 64) {
    const int p = c0 + lane;
    const int e = p < P ? ids[p] : -1;
    const bool ok = p < P && e >= 0 && e < E;
    const uint64_t m = match_mask(ok ? e : E, nbits);
    int pos = -1;
    if (ok) {
      pos = cnt[e] + run[e] + __popcll(m & lt);
      sorted_pairs[pos] = p;
    }
    if (p < P) pair_pos[p] = pos;
    if (ok && (m & lt) == 0) run[e] += __popcll(m);
  }
}

__global__ __launch_bounds__(64) void k_permute(const int32_t* __restrict__ ids, int P, int E,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ sorted_pairs,
                                                int32_t* __restrict__ pair_pos) {
  __shared__ int cnt[kMaxE + 1];
  __shared__ int run[kMaxE];
  wave_group(ids, P, E, cnt, run, offsets, sorted_pairs, pair_pos);
}

// ---------------------------------------------------------------- top-k + grouping, small T
// Decode batches (T <= 16, T * K <= 64): wave t picks the top-k of token t, then
// the first wave groups the T*K pairs; one launch instead of two.
__global__ __launch_bounds__(1024) void k_topk_group_small(
    const double* __restrict__ logits, int T, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos) {
  __shared__ int32_t s_ids[64];
  __shared__ int cnt[kMaxE + 1];
  __shared__ int run[kMaxE];
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (t < T) {
    float wk;
    const int id = wave_topk(logits + (int64_t)t * E, E, K, &wk);
    if (lane < K) {
      ids[t * K + lane] = id;
      wout[t * K + lane] = wk;
      s_ids[t * K + lane] = id;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) wave_group(s_ids, T * K, E, cnt, run, offsets, sorted_pairs, pair_pos);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_route(const moe_cfg& c, const uint16_t* x, int T, const float* wr,
                        const float* bias, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_pairs, int32_t* pair_pos, double* logits,
                        int32_t* counter, hipStream_t s) {
  const int H = c.hidden, E = c.n_experts, K = c.top_k;
  (void)counter;
  if (T <= 32) {
    MOE_LAUNCH(KID_LOGITS, k_logits_small, dim3(E, (T + kLogitTok - 1) / kLogitTok), dim3(256), 0, s,
               x, T, H, E, wr, bias, logits);
  } else {
    MOE_LAUNCH(KID_LOGITS, k_logits_tiled, dim3((E + kLE - 1) / kLE, (T + kLT - 1) / kLT), dim3(256),
               0, s, x, T, H, E, wr, bias, logits);
  }
  if (T <= 16 && T * K <= 64) {
    MOE_LAUNCH(KID_TOPK, k_topk_group_small, dim3(1), dim3(64 * T), 0, s, logits, T, E, K,
               ids, w, offsets, sorted_pairs, pair_pos);
    return hipGetLastError();
  }
  MOE_LAUNCH(KID_TOPK, k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, K, ids, w);
  MOE_LAUNCH(KID_PERMUTE, k_permute, dim3(1), dim3(64), 0, s, ids, T * K, E, offsets, sorted_pairs,
             pair_pos);
  return hipGetLastError();
}

}  // namespace moe
