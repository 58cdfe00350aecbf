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

MOE_TRACE_DECL

// Sum of a double over the wave in a fixed order, returned to every lane: row
// prefix sums by DPP shifts (1, 2, 4, 8), then the row totals carried by
// row_bcast 15 and 31 into lane 63 (no LDS round trips, unlike a shuffle
// butterfly).
template <int CTRL>
__device__ __forceinline__ double dpp_shift_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_shift_f64<0x111>(v);  // row_shr:1
  v += dpp_shift_f64<0x112>(v);  // row_shr:2
  v += dpp_shift_f64<0x114>(v);  // row_shr:4
  v += dpp_shift_f64<0x118>(v);  // row_shr:8
  v += dpp_shift_f64<0x142>(v);  // row_bcast:15
  v += dpp_shift_f64<0x143>(v);  // row_bcast:31
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
  return __hiloint2double(hi, lo);
}

// ---------------------------------------------------------------- logits, small T
// Block (b, c) = experts b*EPB .. b*EPB+EPB-1 x tokens c*NT .. c*NT+NT-1; 256
// threads stride over H in float4 steps (items tid + 256*r of the row, r
// ascending), each thread issuing all its loads of a batch (the router rows'
// float4 and the matching activations of every token) before using any, so a
// 5120-wide row costs one memory round trip; items past the row end load the
// last item and add nothing.  Each thread's fp64 sum, then the wave sum (DPP)
// and the fixed-order sum of the four waves: the logits do not depend on EPB or
// NT.  Several experts per block read the activation rows once per EPB experts
// (the one-launch routing kernel takes one expert per block: its two-level
// ticket keeps the arrivals serialised on any one counter few).
constexpr int kLogitTok = 4;  // tokens per block, 3 to 32 tokens
constexpr int kLogitEPB = 2;  // experts per block, 3 to 32 tokens
constexpr int kRowBatch = 5;  // float4 items of a row per thread per round trip
template <int NT, int EPB>
__device__ __forceinline__ void logits_multi_block(const uint16_t* __restrict__ x, int T, int H,
                                                   int E, const float* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   double* __restrict__ logits) {
  const int e0 = blockIdx.x * EPB, t0 = blockIdx.y * NT;
  const int H4 = H / 4;
  const int tid = threadIdx.x;
  double acc[EPB][NT];
#pragma unroll
  for (int j = 0; j < EPB; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = 0.0;
  for (int b = 0; b < H4; b += 256 * kRowBatch) {
    float4 w[EPB][kRowBatch];
    uint2 xv[NT][kRowBatch];
#pragma unroll
    for (int r = 0; r < kRowBatch; ++r) {
      const int i = min(b + tid + 256 * r, H4 - 1);
#pragma unroll
      for (int j = 0; j < EPB; ++j)
        w[j][r] = reinterpret_cast<const float4*>(wr + (int64_t)min(e0 + j, E - 1) * H)[i];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        xv[t][r] = reinterpret_cast<const uint2*>(x + (int64_t)min(t0 + t, T - 1) * H)[i];
    }
#pragma unroll
    for (int r = 0; r < kRowBatch; ++r) {
      if (b + tid + 256 * r < H4) {
#pragma unroll
        for (int j = 0; j < EPB; ++j)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            double a = acc[j][t];
            a = fma((double)bf16_to_f32((uint16_t)xv[t][r].x), (double)w[j][r].x, a);
            a = fma((double)bf16_to_f32((uint16_t)(xv[t][r].x >> 16)), (double)w[j][r].y, a);
            a = fma((double)bf16_to_f32((uint16_t)xv[t][r].y), (double)w[j][r].z, a);
            a = fma((double)bf16_to_f32((uint16_t)(xv[t][r].y >> 16)), (double)w[j][r].w, a);
            acc[j][t] = a;
          }
      }
    }
  }
  __shared__ double red[4][EPB * NT];
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int j = 0; j < EPB; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const double v = wave_sum_f64(acc[j][t]);
      if (lane == 0) red[wv][j * NT + t] = v;
    }
  __syncthreads();
  if (tid < EPB * NT) {
    const int j = tid / NT, t = tid % NT, e = e0 + j;
    if (e < E && t0 + t < T) {
      double v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      if (bias) v += (double)bias[e];
      st_coherent(logits + (int64_t)(t0 + t) * E + e, v);
    }
  }
}

// ---------------------------------------------------------------- logits of normalised rows
// The logits of experts e0 .. e0+EPB-1 for tokens t0 .. t0+NT-1 of x =
// bf16(RMSNorm(resid)), the normalisation done in the block: thread tid holds the
// float4 items tid + 256*j of each token's fp32 row, which are also the items it
// takes in the logit sums; the squares are summed exactly as the normalisation
// kernel sums them (rms_wave_sum, rms_inv), and the bf16 values it forms enter the
// same logit arithmetic, in the same order, as the block above.  So the
// logits equal those of the plain kernels on the normalisation kernel's output,
// bit for bit.  Blocks of the first expert chunk also store the bf16 rows to xn
// (the experts' input).  H <= 8192.
template <int NT, int EPB>
__device__ __forceinline__ void logits_norm_block(const float* __restrict__ resid, float eps,
                                                  uint16_t* __restrict__ xn, int T, int H, int E,
                                                  const float* __restrict__ wr,
                                                  const float* __restrict__ bias,
                                                  double* __restrict__ logits, int e0, int t0) {
  const int H4 = H / 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // router items first: they do not depend on the normalisation
  float4 w[EPB][kRnPieces];
#pragma unroll
  for (int i = 0; i < kRnPieces; ++i) {
    const int q = min(tid + 256 * i, H4 - 1);
#pragma unroll
    for (int j = 0; j < EPB; ++j)
      w[j][i] = reinterpret_cast<const float4*>(wr + (int64_t)min(e0 + j, E - 1) * H)[q];
  }
  rn_f4 rv[NT][kRnPieces];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < kRnPieces; ++i)
      rv[t][i] = reinterpret_cast<const rn_f4*>(resid + (int64_t)min(t0 + t, T - 1) * H)
          [min(tid + 256 * i, H4 - 1)];
  __shared__ float s_part[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float ss = rms_wave_sum(rv[t], H4);
    if (lane == 0) s_part[t][wv] = ss;
  }
  __syncthreads();
  float inv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) inv[t] = rms_inv(s_part[t], H, eps);
  double acc[EPB][NT];
#pragma unroll
  for (int j = 0; j < EPB; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = 0.0;
#pragma unroll
  for (int i = 0; i < kRnPieces; ++i) {
    const int q = tid + 256 * i;
    if (q < H4) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint2 xv = make_uint2(rms_bf16x2(rv[t][i].x, rv[t][i].y, inv[t]),
                                    rms_bf16x2(rv[t][i].z, rv[t][i].w, inv[t]));
        if (e0 == 0 && t0 + t < T) reinterpret_cast<uint2*>(xn + (int64_t)(t0 + t) * H)[q] = xv;
#pragma unroll
        for (int j = 0; j < EPB; ++j) {
          double a = acc[j][t];
          a = fma((double)bf16_to_f32((uint16_t)xv.x), (double)w[j][i].x, a);
          a = fma((double)bf16_to_f32((uint16_t)(xv.x >> 16)), (double)w[j][i].y, a);
          a = fma((double)bf16_to_f32((uint16_t)xv.y), (double)w[j][i].z, a);
          a = fma((double)bf16_to_f32((uint16_t)(xv.y >> 16)), (double)w[j][i].w, a);
          acc[j][t] = a;
        }
      }
    }
  }
  __shared__ double red[4][EPB * NT];
#pragma unroll
  for (int j = 0; j < EPB; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const double v = wave_sum_f64(acc[j][t]);
      if (lane == 0) red[wv][j * NT + t] = v;
    }
  __syncthreads();
  if (tid < EPB * NT) {
    const int j = tid / NT, t = tid % NT, e = e0 + j;
    if (e < E && t0 + t < T) {
      double v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      if (bias) v += (double)bias[e];
      st_coherent(logits + (int64_t)(t0 + t) * E + e, v);
    }
  }
}

// batches of 3 to 32 tokens (block (b, c) as above)
template <int NT, int EPB>
__global__ __launch_bounds__(256) void k_logits_multi(const uint16_t* __restrict__ x, int T, int H,
                                                      int E, const float* __restrict__ wr,
                                                      const float* __restrict__ bias,
                                                      double* __restrict__ logits) {
  logits_multi_block<NT, EPB>(x, T, H, E, wr, bias, logits);
}
template <int NT, int EPB>
__global__ __launch_bounds__(256) void k_logits_multi_norm(const float* __restrict__ resid,
                                                           float eps, uint16_t* __restrict__ xn,
                                                           int T, int H, int E,
                                                           const float* __restrict__ wr,
                                                           const float* __restrict__ bias,
                                                           double* __restrict__ logits) {
  logits_norm_block<NT, EPB>(resid, eps, xn, T, H, E, wr, bias, logits, blockIdx.x * EPB,
                             blockIdx.y * NT);
}

// ---------------------------------------------------------------- logits, large T
// fp64 matrix cores (v_mfma_f64_16x16x4_f64): block = 32 tokens x 96 experts, four
// waves of 16 x 48; the reduction dim in steps of 32 staged through LDS as fp64
// (bf16 and fp32 inputs widen exactly), the next step's global loads in flight
// during the current step's products.  Every product is exact; the sums are fp64.
// 96 experts per block divide the 288 experts of the pages' model without padding,
// and 8,192 tokens give 768 blocks, three per CU.
constexpr int kLT = 32, kLE = 96, kLK = 32;
constexpr int kLRow = kLK + 4;  // doubles per LDS row (2-way bank conflicts at most)
typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_logits_mfma(const uint16_t* __restrict__ x, int T, int H,
                                                     int E, const float* __restrict__ wr,
                                                     const float* __restrict__ bias,
                                                     double* __restrict__ logits) {
  __shared__ __align__(16) double xs[kLT * kLRow];
  __shared__ __align__(16) double ws[kLE * kLRow];
  const int t0 = blockIdx.y * kLT, e0 = blockIdx.x * kLE;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // loader: thread (row, 8 consecutive k): token rows lr < 32 (threads 0..127)
  // and expert rows lr and 64 + lr (the second for lr < 32)
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const bool xl = lr < kLT, w2 = lr + 64 < kLE;
  const bool xok = xl && t0 + lr < T, wok = e0 + lr < E, wok2 = w2 && e0 + 64 + lr < E;
  const uint16_t* xp = x + (int64_t)min(t0 + min(lr, kLT - 1), T - 1) * H + lk;
  const float* wp = wr + (int64_t)min(e0 + lr, E - 1) * H + lk;
  const float* wp2 = wr + (int64_t)min(e0 + 64 + min(lr, kLE - 65), E - 1) * H + lk;
  uint4 xv;
  float4 wv0, wv1, wv2, wv3;
  auto load = [&](int k0) {
    xv = *reinterpret_cast<const uint4*>(xp + k0);
    wv0 = *reinterpret_cast<const float4*>(wp + k0);
    wv1 = *reinterpret_cast<const float4*>(wp + k0 + 4);
    wv2 = *reinterpret_cast<const float4*>(wp2 + k0);
    wv3 = *reinterpret_cast<const float4*>(wp2 + k0 + 4);
  };
  auto stage = [&]() {
    if (xl) {
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      double* xd = xs + lr * kLRow + lk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xd[2 * j] = xok ? (double)bf16_to_f32((uint16_t)xw[j]) : 0.0;
        xd[2 * j + 1] = xok ? (double)bf16_to_f32((uint16_t)(xw[j] >> 16)) : 0.0;
      }
    }
    const float wf[8] = {wv0.x, wv0.y, wv0.z, wv0.w, wv1.x, wv1.y, wv1.z, wv1.w};
    double* wd = ws + lr * kLRow + lk;
#pragma unroll
    for (int j = 0; j < 8; ++j) wd[j] = wok ? (double)wf[j] : 0.0;
    if (w2) {
      const float wg[8] = {wv2.x, wv2.y, wv2.z, wv2.w, wv3.x, wv3.y, wv3.z, wv3.w};
      double* wd2 = ws + (64 + lr) * kLRow + lk;
#pragma unroll
      for (int j = 0; j < 8; ++j) wd2[j] = wok2 ? (double)wg[j] : 0.0;
    }
  };
  const int wm = wv >> 1, wn = wv & 1;  // wave tile: tokens 16wm.., experts 48wn..
  const int fr = lane & 15, fk = lane >> 4;
  f64x4 acc[1][3];
#pragma unroll
  for (int j = 0; j < 3; ++j) acc[0][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  load(0);
  for (int k0 = 0; k0 < H; k0 += kLK) {
    stage();
    __syncthreads();
    if (k0 + kLK < H) load(k0 + kLK);
#pragma unroll
    for (int kk = 0; kk < kLK; kk += 4) {
      double a, b[3];
      a = xs[(16 * wm + fr) * kLRow + kk + fk];
#pragma unroll
      for (int j = 0; j < 3; ++j) b[j] = ws[(48 * wn + 16 * j + fr) * kLRow + kk + fk];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        acc[0][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b[j], acc[0][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds expert column fr, token rows fk + 4q of each 16 x 16 tile
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int e = e0 + 48 * wn + 16 * j + fr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + 16 * wm + fk + 4 * q;
      if (t < T && e < E) logits[(int64_t)t * E + e] = acc[0][j][q] + (bias ? (double)bias[e] : 0.0);
    }
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

__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_i<0x111>(v, INT_MIN));
  v = max(v, dpp_i<0x112>(v, INT_MIN));
  v = max(v, dpp_i<0x114>(v, INT_MIN));
  v = max(v, dpp_i<0x118>(v, INT_MIN));
  v = max(v, dpp_i<0x142>(v, INT_MIN));
  v = max(v, dpp_i<0x143>(v, INT_MIN));
  return __builtin_amdgcn_readlane(v, 63);
}
// a lane's double, read by every lane
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
  return __hiloint2double(hi, lo);
}
// Order-preserving 32-bit key of a double: its nearest float, as an integer
// that compares like the float (both zeros map to 0).  Rounding to float never
// reverses an order, so a strictly larger key means a strictly larger value;
// only equal keys need the exact comparison.
__device__ __forceinline__ int coarse_key(double v) {
  const float f = (float)v;
  const int b = __float_as_int(f);
  return f == 0.f ? 0 : (b ^ ((b >> 31) & 0x7FFFFFFF));
}

// this lane's pick (lane < K; -1 for other lanes) and its logit (*lk).
// Each lane first sorts its PER candidates (experts lane + 64i) by descending
// logit with an odd-even transposition network (swaps only on a strictly larger
// value, so equal logits keep ascending id order).  Round k then finds the wave
// maximum of the lane heads: first on their 32-bit keys (one DPP max), and only
// when several lanes share the largest key, exactly in fp64 among those lanes,
// the lowest id winning on equal logits.  The winning lane pops its head.
template <int PER>
__device__ __forceinline__ int wave_topk_pick(const double* __restrict__ l, int E, int K,
                                              double* lk, int trace = -1) {
  const int lane = threadIdx.x & 63;
  double v[PER];
  int id[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? ld_coherent(l + e) : -INFINITY;
    id[i] = e < E ? e : 0x7FFFFFFF;
  }
#pragma unroll
  for (int r = 0; r < PER; ++r)
#pragma unroll
    for (int i = r & 1; i + 1 < PER; i += 2) {
      const bool sw = v[i + 1] > v[i];
      const double a = v[i], b2 = v[i + 1];
      const int ia = id[i], ib = id[i + 1];
      v[i] = sw ? b2 : a;
      v[i + 1] = sw ? a : b2;
      id[i] = sw ? ib : ia;
      id[i + 1] = sw ? ia : ib;
    }
  if (trace >= 0) MOE_TR(trace);
  double my_l = -INFINITY;
  int my_id = -1;
  int key = id[0] != 0x7FFFFFFF ? coarse_key(v[0]) : INT_MIN;
  for (int k = 0; k < K; ++k) {
    const int mk = wave_max_i32(key);
    const uint64_t cand = __ballot(key == mk && id[0] != 0x7FFFFFFF);
    int win;
    if (__popcll(cand) == 1) {
      win = __ffsll((unsigned long long)cand) - 1;
    } else {  // several lanes share the largest key: exact maximum, then the lowest id
      const bool c = (cand >> lane) & 1;
      const double m = wave_max_f64(c ? v[0] : -INFINITY);
      const int best = wave_min_i32(c && v[0] == m ? id[0] : 0x7FFFFFFF);
      win = __ffsll((unsigned long long)__ballot(c && v[0] == m && id[0] == best)) - 1;
    }
    const int pick = __builtin_amdgcn_readlane(id[0], win);
    const double pl = readlane_f64(v[0], win);
    if (lane == win) {
#pragma unroll
      for (int i = 0; i + 1 < PER; ++i) {
        v[i] = v[i + 1];
        id[i] = id[i + 1];
      }
      v[PER - 1] = -INFINITY;
      id[PER - 1] = 0x7FFFFFFF;
      key = id[0] != 0x7FFFFFFF ? coarse_key(v[0]) : INT_MIN;
    }
    if (lane == k) {
      my_l = pl;
      my_id = pick;
    }
  }
  if (trace >= 0) MOE_TR(trace + 1);
  *lk = my_l;
  return lane < K ? my_id : -1;
}

// the weight of this lane's pick (lane < K) from the picks' logits lk (lane k
// holds the k-th largest): exp(l_k - l_0) / sum_j exp(l_j - l_0), the sum in pick
// order
__device__ __forceinline__ float topk_weight(double lk, int K) {
  const int lane = threadIdx.x & 63;
  const double l0 = readlane_f64(lk, 0);
  const double term = lane < K ? exp(lk - l0) : 0.0;
  double den = 0.0;
  for (int k = 0; k < K; ++k) den += readlane_f64(term, k);
  return (float)(term / den);
}

template <int PER>
__device__ __forceinline__ int wave_topk(const double* __restrict__ l, int E, int K, float* wk) {
  double lk;
  const int id = wave_topk_pick<PER>(l, E, K, &lk);
  *wk = topk_weight(lk, K);
  return id;
}

template <int PER>
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int T, int E,
                                              int K, int32_t* __restrict__ ids,
                                              float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float wk;
  const int id = wave_topk<PER>(logits + (int64_t)t * E, E, K, &wk);
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

// ---------------------------------------------------------------- grouping, many pairs
// Chunks of kGChunk pairs, one wave each.  Count: per-chunk histograms by the same
// ballot matching.  Scan (one block): per expert, the exclusive prefix over the
// chunks, then the exclusive prefix over the experts, giving each (chunk, expert)
// its first sorted position.  Scatter: each chunk again in pair order from its
// bases.  The same stable order as the single-wave grouping; integer only.
constexpr int kGChunk = 1024;

__global__ __launch_bounds__(64) void k_group_count(const int32_t* __restrict__ ids, int P, int E,
                                                    int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxE];
  const int lane = threadIdx.x;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int c0 = blockIdx.x * kGChunk, c1 = min(P, c0 + kGChunk);
  for (int b = c0; b < c1; b += 64) {
    const int p = b + lane;
    const int e = p < c1 ? ids[p] : -1;
    const bool ok = p < c1 && e >= 0 && e < E;
    const uint64_t m = match_mask(ok ? e : E, nbits);
    if (ok && (m & lt) == 0) cnt[e] += __popcll(m);
  }
  for (int e = lane; e < E; e += 64) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void k_group_scan(int32_t* __restrict__ hist, int nb, int E,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
  int run = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nb; b0 += 16) {
      int c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = b0 + j < nb ? hist[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < nb) hist[(int64_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
  }
  int inc = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int base = inc - run, total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wv) base += wsum[w];
    total += wsum[w];
  }
  if (e < E) {
    offsets[e] = base;
    for (int b = 0; b < nb; ++b) hist[(int64_t)b * E + e] += base;
  }
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(64) void k_group_scatter(const int32_t* __restrict__ ids, int P, int E,
                                                      const int32_t* __restrict__ hist,
                                                      int32_t* __restrict__ sorted_pairs,
                                                      int32_t* __restrict__ pair_pos) {
  __shared__ int run[kMaxE];
  const int lane = threadIdx.x;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;
  for (int e = lane; e < E; e += 64) run[e] = hist[(int64_t)blockIdx.x * E + e];
  const uint64_t lt = (1ull << lane) - 1ull;
  const int c0 = blockIdx.x * kGChunk, c1 = min(P, c0 + kGChunk);
  for (int b = c0; b < c1; b += 64) {
    const int p = b + lane;
    const int e = p < c1 ? ids[p] : -1;
    const bool ok = p < c1 && e >= 0 && e < E;
    const uint64_t m = match_mask(ok ? e : E, nbits);
    int pos = -1;
    if (ok) {
      pos = run[e] + __popcll(m & lt);
      sorted_pairs[pos] = p;
    }
    if (p < c1) pair_pos[p] = pos;
    if (ok && (m & lt) == 0) run[e] += __popcll(m);
  }
}

// ---------------------------------------------------------------- grouping, small T
// Among the live lanes: how many hold a key smaller than this lane's, and (eq) the
// lanes that hold the same key, by one ballot per key bit from the top (keys in
// [0, 2^nbits)).  Integer only.
__device__ __forceinline__ int wave_rank(int key, bool live, int nbits, uint64_t& eq) {
  eq = __ballot(live);
  int less = 0;
  for (int b = nbits - 1; b >= 0; --b) {
    const uint64_t bal = __ballot(live && ((key >> b) & 1));
    if ((key >> b) & 1) {
      less += __popcll(eq & ~bal);
      eq &= bal;
    } else {
      eq &= ~bal;
    }
  }
  return less;
}

// Grouping of at most 64 pairs by one wave.  Lane p (pair p < P) has key id_p
// (E for an id outside [0, E)).  Its sorted position is the number of pairs with
// a smaller (key, pair index), counted from the top key bit down with one ballot
// per bit.  With the valid keys placed in sorted order in s_key[128] (LDS),
// offsets[e] is the number of them below e, found by a branch-free binary search
// (lane l takes e = l + 64*i).  The result is the stable counting sort; pairs with an invalid
// id are left out (pair_pos = -1).  Integer only: bit-exact.
template <int NOFF>  // NOFF * 64 > E
__device__ __forceinline__ void wave_group_small(int id, int P, int E, int* s_key,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ sorted_pairs,
                                                 int32_t* __restrict__ pair_pos) {
  const int lane = threadIdx.x & 63;
  int nbits = 0;
  while ((1 << nbits) < E + 1) ++nbits;
  const bool live = lane < P;
  const bool ok = live && id >= 0 && id < E;
  const int key = ok ? id : E;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint64_t eq = __ballot(live);
  int less = 0;
  for (int b = nbits - 1; b >= 0; --b) {
    const uint64_t bal = __ballot(live && ((key >> b) & 1));
    if ((key >> b) & 1) {
      less += __popcll(eq & ~bal);
      eq &= bal;
    } else {
      eq &= ~bal;
    }
  }
  const int pos = less + __popcll(eq & lt);
  // sorted keys in s_key[0 .. nvalid), INT_MAX above (LDS operations of one wave
  // take effect in order, so the keys overwrite the fill)
  s_key[lane] = INT_MAX;
  s_key[64 + lane] = INT_MAX;
  if (ok) {
    sorted_pairs[pos] = lane;
    s_key[pos] = key;
  }
  if (live) pair_pos[lane] = ok ? pos : -1;
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes have landed
  int below[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) below[i] = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1) {
    int kj[NOFF];
#pragma unroll
    for (int i = 0; i < NOFF; ++i) kj[i] = s_key[below[i] + step - 1];
#pragma unroll
    for (int i = 0; i < NOFF; ++i) below[i] = kj[i] < lane + 64 * i ? below[i] + step : below[i];
  }
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    const int e = lane + 64 * i;
    if (e <= E) offsets[e] = below[i];
  }
}

// The same grouping for at most 16 pairs, without LDS: every lane reads the P
// keys as wave-uniform values and counts, for its own pair, the pairs with a
// smaller (key, pair index), and for its experts e = lane + 64*i, the valid pairs
// with an id below e.  Integer only: bit-exact, and the same stable order.
constexpr int kTinyPairs = 16;
template <int NOFF>  // NOFF * 64 > E
__device__ __forceinline__ void wave_group_tiny(int id, int P, int E,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ sorted_pairs,
                                                int32_t* __restrict__ pair_pos) {
  const int lane = threadIdx.x & 63;
  const bool live = lane < P;
  const bool ok = live && id >= 0 && id < E;
  const int key = ok ? id : E;
  int pos = 0;
  int below[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) below[i] = 0;
#pragma unroll
  for (int q = 0; q < kTinyPairs; ++q) {
    if (q < P) {  // uniform
      const int kq = __builtin_amdgcn_readlane(key, q);
      pos += (kq < key) || (kq == key && q < lane);
#pragma unroll
      for (int i = 0; i < NOFF; ++i) below[i] += kq < lane + 64 * i;
    }
  }
  if (ok) sorted_pairs[pos] = lane;
  if (live) pair_pos[lane] = ok ? pos : -1;
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    const int e = lane + 64 * i;
    if (e <= E) offsets[e] = below[i];
  }
}

// Decode batches of 3 to 16 tokens: wave t picks the top-k of token t; once every
// token's picks are in LDS, wave T (wave 0 at 16 tokens) groups the pairs while
// the picking waves form their weights.
// PLAN (a layer call of 3 to 8 tokens, whose routing is consistent by
// construction): the launch also does the decode plan's work, so that the plan
// launch is skipped.  Blocks 1.. form the gate/up codec's offset sums osx[t][g]
// (one wave per (t, g), the same arithmetic as the plan kernel); block 0's wave
// 15, beside the grouping wave, lists the active experts in the plan's order
// (more pairs first, then lower id) with their table entries, stores U and
// records the routing as consistent.
template <int PER, bool PLAN>
__global__ __launch_bounds__(1024) void k_topk_group_small(
    const double* __restrict__ logits, int T, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, PlanIn pl) {
  __shared__ int32_t s_ids[64];
  __shared__ int s_key[128];
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (PLAN && blockIdx.x > 0) {  // the offset sums
    const int ngx = pl.H / pl.G, it = (blockIdx.x - 1) * 16 + t;
    if (it < T * ngx) {
      const int tt = it / ngx, g = it - tt * ngx;
      const uint32_t* x32 = reinterpret_cast<const uint32_t*>(pl.x);
      const float off = lane < pl.pairs ? pl.off[lane] : 0.f;
      const uint32_t pr = lane < pl.pairs ? x32[((int64_t)tt * pl.H + g * pl.G) / 2 + lane] : 0u;
      const float v = wave_sum_uniform<kQ3G128>(off * (bf16_to_f32((uint16_t)pr) +
                                                       bf16_to_f32((uint16_t)(pr >> 16))));
      if (lane == 0) pl.osx[it] = v;
    }
    return;
  }
  double lk = 0.0;
  if (t < T) {
    const int id = wave_topk_pick<PER>(logits + (int64_t)t * E, E, K, &lk);
    if (lane < K) {
      ids[t * K + lane] = id;
      s_ids[t * K + lane] = id;
    }
  }
  // (an LDS-only barrier: __syncthreads() would also wait for the stores above)
  lds_barrier();
  if (t == (T < 16 ? T : 0)) {
    const int P = T * K;
    if (P <= kTinyPairs)
      wave_group_tiny<PER + 1>(lane < P ? s_ids[lane] : -1, P, E, offsets, sorted_pairs, pair_pos);
    else
      wave_group_small<PER + 1>(lane < P ? s_ids[lane] : -1, P, E, s_key, offsets, sorted_pairs,
                                pair_pos);
  }
  if (PLAN && t == 15) {  // the active list (P <= 64; picked ids are in [0, E <= 1024))
    const int P = T * K;
    const bool live = lane < P;
    const int key = live ? s_ids[lane] : 0;
    moe_expert_ref r{nullptr, nullptr, nullptr};
    if (live) r = pl.table[key];  // requested first
    uint64_t eq;
    const int less = wave_rank(key, live, 10, eq);  // pairs with a smaller id; same id: eq
    const int cnt = __popcll(eq);
    const bool first = live && (eq & ((1ull << lane) - 1ull)) == 0;
    // the plan's order: more pairs first, then the lower id
    const int key2 = ((63 - min(cnt, 63)) << 10) | key;
    uint64_t eq2;
    const int a = wave_rank(key2, first, 16, eq2);
    const uint64_t F = __ballot(first);
    if (first) {
      ActEntry v;
      v.e = key;
      v.seg0 = less;
      v.n = cnt;
      v.pad = 0;
      v.ptr[0] = r.gate;
      v.ptr[1] = r.up;
      v.ptr[2] = r.down;
      pl.act[a] = v;
    }
    if (lane == 0) {
      pl.act_hdr[0] = __popcll(F);
      record_routing(pl.ctr0, true);
    }
  }
  if (t < T) {
    const float wk = topk_weight(lk, K);
    if (lane < K) wout[t * K + lane] = wk;
  }
}

// ---------------------------------------------------------------- one launch, small T
// Logits, top-k and grouping of a batch of one or two tokens in one kernel: the
// logit blocks above, one expert each (logits stored written-through), then the
// block that takes the last ticket, whose loads see every block's logits: wave t
// picks the top-k of token t and wave 2 groups the pairs.  The ticket has two
// levels (a block counts in its group's counter, the last of a group in the
// kernel's), so that no counter takes more than a few dozen arrivals; each
// counter is reset by the block that finds it complete.  Larger
// batches pick their tokens faster in a kernel of their own with one wave per
// token (here the last block's four waves would take their tokens in turn:
// 17.7 us at eight tokens against 14.8 us for the two launches).
constexpr int kRouteMaxT = 2;
// ENT (a layer call): the last block's fourth wave, beside the grouping wave,
// stores the active experts' entries for the expert kernels of the same call (entry a: the a-th active expert in
// ascending id, its first sorted position, pair count, U and table entry; the
// entries a in [U, min(E, P)) say "none"), so that those kernels need no lookup
// of their own.  The routing here is consistent by construction.
template <int NT, int PER, int EPB, bool NORM, bool ENT>
__global__ __launch_bounds__(256) void k_route_small(
    const uint16_t* __restrict__ x, const float* __restrict__ resid, float eps,
    uint16_t* __restrict__ xn, int T, int H, int E, const float* __restrict__ wr,
    const float* __restrict__ bias, double* logits, int K, int32_t* __restrict__ ids,
    float* __restrict__ wout, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ ctr,
    const moe_expert_ref* __restrict__ table, ActEntry* __restrict__ ent) {
  const int bid = blockIdx.x + gridDim.x * blockIdx.y;
  MOE_TR(4 * bid);
  if (NORM)
    logits_norm_block<NT, EPB>(resid, eps, xn, T, H, E, wr, bias, logits, blockIdx.x * EPB,
                               blockIdx.y * NT);
  else
    logits_multi_block<NT, EPB>(x, T, H, E, wr, bias, logits);
  MOE_TR(4 * bid + 1);
  __shared__ int s_last;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nb = gridDim.x * gridDim.y;
    // two levels: the last block of each group counts in the kernel's counter
    // (each block's logits were stored and acknowledged before its group ticket)
    const int g = bid % kRouteGroups, gsize = nb / kRouteGroups + (g < nb % kRouteGroups);
    int32_t* cg = ctr + kCtrRouteGrp + g * kCtrStride;
    bool last = false;
    if (take_ticket(cg) == gsize - 1) {
      st_coherent(cg, 0);  // every block of the group has counted
      last = take_ticket(ctr) == min(kRouteGroups, nb) - 1;
    }
    s_last = last;
  }
  MOE_TR(4 * bid + 2);
  lds_barrier();
  if (!s_last) return;
  __shared__ int32_t s_ids[64];
  __shared__ int s_key[128];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // waves 0 and 1 pick (one token each); once the picks are in LDS, wave 2 groups
  // the pairs while the picking waves form their weights
  double lk = 0.0;
  if (wv < T) {
    const int id = wave_topk_pick<PER>(logits + (int64_t)wv * E, E, K, &lk, wv == 0 ? 2002 : -1);
    if (lane < K) {
      ids[wv * K + lane] = id;
      s_ids[wv * K + lane] = id;
    }
  }
  MOE_TR(2000);
  lds_barrier();  // s_ids only; the stores above need not have completed
  if (wv == kRouteMaxT) {
    const int P = T * K;
    const int key = lane < P ? s_ids[lane] : -1;
    if (P <= kTinyPairs)
      wave_group_tiny<PER + 1>(key, P, E, offsets, sorted_pairs, pair_pos);
    else
      wave_group_small<PER + 1>(key, P, E, s_key, offsets, sorted_pairs, pair_pos);
    if (lane == 0) st_coherent(ctr, 0);
    MOE_TR(2001);
  }
  if (ENT && wv == kRouteMaxT + 1) {  // beside the grouping: the expert entries
    const int P = T * K;
    const int key = lane < P ? s_ids[lane] : -1;  // (picked ids are in [0, E); P <= 64)
    moe_expert_ref r{nullptr, nullptr, nullptr};
    if (lane < P) r = table[key];  // requested first
    int cnt = 0, less = 0, a = 0;
    bool first = lane < P;
    for (int q = 0; q < P; ++q) {
      const int kq = __builtin_amdgcn_readlane(key, q);
      cnt += kq == key;
      less += kq < key;
      first = first && !(kq == key && q < lane);
    }
    const uint64_t F = __ballot(first);
    for (int q = 0; q < P; ++q)
      if ((F >> q) & 1) a += __builtin_amdgcn_readlane(key, q) < key;
    const int U = __popcll(F), maxU = min(E, P);
    if (first) {
      ActEntry v;
      v.e = key;
      v.seg0 = less;
      v.n = cnt;
      v.pad = U;
      v.ptr[0] = r.gate;
      v.ptr[1] = r.up;
      v.ptr[2] = r.down;
      ent[a] = v;
    }
    if (lane >= U && lane < maxU) {
      ActEntry v;
      v.e = -1;
      v.seg0 = 0;
      v.n = 0;
      v.pad = U;
      v.ptr[0] = v.ptr[1] = v.ptr[2] = nullptr;
      ent[lane] = v;
    }
  }
  if (wv < T) {
    const float wk = topk_weight(lk, K);
    if (lane < K) wout[wv * K + lane] = wk;
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_route(const moe_cfg& c, const RouteIn& in, int T, const float* wr,
                        const float* bias, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_pairs, int32_t* pair_pos, double* logits,
                        int32_t* ghist, int32_t* counters, hipStream_t s) {
  const int H = c.hidden, E = c.n_experts, K = c.top_k, P = T * K;
  const int per = (E + 63) / 64;
  bool norm = in.resid != nullptr;
  const uint16_t* x = norm ? in.xn : in.x;
  if (norm && T > 32) {  // the matrix-core logits take the normalisation kernel's output
    const hipError_t e = launch_rmsnorm(const_cast<float*>(in.resid), nullptr, T, H, in.eps,
                                        in.xn, s);
    if (e != hipSuccess) return e;
    norm = false;
  }
#define MOE_PER_SWITCH(X)                                                    \
  switch (per <= 8 ? per : 16) {                                             \
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(16)                            \
    default: return hipErrorInvalidValue;                                    \
  }
  if (T <= kRouteMaxT && P <= 64) {  // one launch
    int32_t* ctr = counters + kCtrRoute;
    const dim3 g1(E);  // one expert per logit block
    const bool ent = in.table != nullptr && in.entries != nullptr;
#define MOE_RS2(NT, N, NORM, ENT)                                                               \
  MOE_LAUNCH(KID_ROUTE, (k_route_small<NT, N, 1, NORM, ENT>), g1, dim3(256), 0, s, x, in.resid,  \
             in.eps, in.xn, T, H, E, wr, bias, logits, K, ids, w, offsets, sorted_pairs, pair_pos, \
             ctr, in.table, in.entries)
#define MOE_RS1(NT, N, NORM)                                                                    \
  if (ent) MOE_RS2(NT, N, NORM, true); else MOE_RS2(NT, N, NORM, false);
#define MOE_RS(N)                                                                               \
  case N:                                                                                       \
    if (T == 1) {                                                                               \
      if (norm) { MOE_RS1(1, N, true) } else { MOE_RS1(1, N, false) }                           \
    } else {                                                                                    \
      if (norm) { MOE_RS1(2, N, true) } else { MOE_RS1(2, N, false) }                           \
    }                                                                                           \
    break;
    MOE_PER_SWITCH(MOE_RS)
#undef MOE_RS
#undef MOE_RS1
#undef MOE_RS2
    if (ent && in.wrote_entries) *in.wrote_entries = 1;
    return hipGetLastError();
  }
  if (T <= 32) {
    const dim3 g((E + kLogitEPB - 1) / kLogitEPB, (T + kLogitTok - 1) / kLogitTok);
    if (norm)
      MOE_LAUNCH(KID_LOGITS, (k_logits_multi_norm<kLogitTok, kLogitEPB>), g, dim3(256), 0, s,
                 in.resid, in.eps, in.xn, T, H, E, wr, bias, logits);
    else
      MOE_LAUNCH(KID_LOGITS, (k_logits_multi<kLogitTok, kLogitEPB>), g, dim3(256), 0, s, x, T, H,
                 E, wr, bias, logits);
  } else {
    MOE_LAUNCH(KID_LOGITS, k_logits_mfma, dim3((E + kLE - 1) / kLE, (T + kLT - 1) / kLT), dim3(256),
               0, s, x, T, H, E, wr, bias, logits);
  }
  if (T <= 16 && P <= 64) {
    PlanIn pl{};
    const int ngx = c.group > 0 ? H / c.group : 0;
    const bool plan = in.table && in.entries && in.act_hdr && in.osx && in.ctr0 && T <= 8 &&
                      (pl.pairs = codec_pair_offsets(in.codec, pl.off)) > 0;
    if (plan) {
      pl.table = in.table;
      pl.act_hdr = in.act_hdr;
      pl.act = in.entries;
      pl.x = norm ? in.xn : in.x;
      pl.osx = in.osx;
      pl.ctr0 = in.ctr0;
      pl.H = H;
      pl.G = c.group;
    }
#define MOE_TGS(N)                                                                             \
  case N:                                                                                      \
    if (plan)                                                                                  \
      MOE_LAUNCH(KID_TOPK, (k_topk_group_small<N, true>), dim3(1 + (T * ngx + 15) / 16),       \
                 dim3(1024), 0, s, logits, T, E, K, ids, w, offsets, sorted_pairs, pair_pos, pl); \
    else                                                                                       \
      MOE_LAUNCH(KID_TOPK, (k_topk_group_small<N, false>), dim3(1),                            \
                 dim3(64 * std::min(T + 1, 16)), 0, s, logits, T, E, K, ids, w, offsets,        \
                 sorted_pairs, pair_pos, pl);                                                  \
    break;
    MOE_PER_SWITCH(MOE_TGS)
#undef MOE_TGS
    if (plan && in.wrote_entries) *in.wrote_entries = 1;
    return hipGetLastError();
  }
#define MOE_TK(N)                                                                              \
  case N:                                                                                      \
    MOE_LAUNCH(KID_TOPK, k_topk<N>, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, K, ids, w); \
    break;
  MOE_PER_SWITCH(MOE_TK)
#undef MOE_TK
#undef MOE_PER_SWITCH
  if (P <= 4 * kGChunk) {
    MOE_LAUNCH(KID_PERMUTE, k_permute, dim3(1), dim3(64), 0, s, ids, P, E, offsets, sorted_pairs,
               pair_pos);
  } else {
    const int nb = (P + kGChunk - 1) / kGChunk;
    MOE_LAUNCH(KID_PERMUTE, k_group_count, dim3(nb), dim3(64), 0, s, ids, P, E, ghist);
    MOE_LAUNCH(KID_PERMUTE, k_group_scan, dim3(1), dim3(1024), 0, s, ghist, nb, E, offsets);
    MOE_LAUNCH(KID_PERMUTE, k_group_scatter, dim3(nb), dim3(64), 0, s, ids, P, E, ghist,
               sorted_pairs, pair_pos);
  }
  return hipGetLastError();
}

MOE_TRACE_EXPORT(route)

}  // namespace moe
