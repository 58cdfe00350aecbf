// expert.hip -- the routed experts' SwiGLU FFNs on packed low-bit weights, the
// shared expert, the weighted combine and the stack's RMSNorm glue.
//
// Each picked expert runs gate, up and down matrices reached through the layer's
// pointer table (page "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX PRO 6000 - GPU expert
// cache, host-RAM streaming", field config.expert_cache.mechanism: three tables of
// per-expert pointers, rewritten in place); results depend only on the logical
// expert id, never on where its bytes live (page "0xSero/glm53-flash-offload",
// paragraph "Elastic CLOCK expert cache").  The combine sums the experts of a
// token in fixed pick order with no atomics, so a run is bit-reproducible (the
// 2x RTX 5090 page, field config.serving.exactness, notes that unordered MoE
// reductions are not).
//
// Decode GEMV layout (weights are read once per step, so HBM bandwidth bounds it):
// one lane owns one output row of a 64-row tile; a wave64 16-byte load of chunk
// j of a tile reads 1024 contiguous bytes, three chunks give every lane its
// row's 128 codes of one group.  Codes are expanded two at a time into bf16 pairs
// (see UnitCodec) and multiplied with the activations by v_dot2_f32_bf16, whose
// second operand is a pair of activations read by scalar loads (identical for
// all lanes).  The group scale is applied to each group's fp32 partial sum.
#include "common.h"

namespace moe {

// ---------------------------------------------------------------- plan
// active[0..U-1] = experts with at least one pair, ascending; active[E] = U.
// xcorr[t][g] = sum_k off_k * x[t][g*G + k] (k ascending), the offset sum that
// the unit codec's dot products carry.
template <int BITS>
__global__ __launch_bounds__(256) void k_plan(const int32_t* __restrict__ offsets, int E,
                                              const uint16_t* __restrict__ x, int T, int H,
                                              int32_t* __restrict__ active,
                                              float* __restrict__ xcorr) {
  using C = UnitCodec<BITS>;
  const int ng = H / C::G;
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item < T * ng) {
    const int t = item / ng, g = item % ng;
    const uint32_t* xp = reinterpret_cast<const uint32_t*>(x + (int64_t)t * H + g * C::G);
    float acc = 0.f;
    for (int P = 0; P < C::PAIRS; ++P) {
      uint32_t v = xp[P];
      acc = fmaf(C::pair_off(P), bf16_to_f32((uint16_t)v), acc);
      acc = fmaf(C::pair_off(P), bf16_to_f32((uint16_t)(v >> 16)), acc);
    }
    xcorr[item] = acc;
  }
  if (blockIdx.x == 0) {
    __shared__ int wsum[4];
    // E <= 1024: four passes of 256 experts
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 256) {
      const int e = e0 + threadIdx.x;
      const bool on = e < E && offsets[e + 1] > offsets[e];
      const uint64_t bal = __ballot(on);
      const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
      if (lane == 0) wsum[wv] = __popcll(bal);
      __syncthreads();
      int pre = base;
      for (int i = 0; i < wv; ++i) pre += wsum[i];
      pre += __popcll(bal & ((1ull << lane) - 1ull));
      if (on) active[pre] = e;
      base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
      __syncthreads();
    }
    if (threadIdx.x == 0) active[E] = base;
  }
}

// ---------------------------------------------------------------- gate/up
// Block (a, strip): active expert a, rows [64*strip, 64*strip+64) of gate and up,
// all groups; 8 waves take groups g = wave, wave+8, ...; tokens in batches of
// kNT.  Per (row, token): g = sum_groups s * (dot - xcorr), same for u; then
// h = silu(g) * u, stored as bf16 hi + bf16 remainder (h to ~2^-16 relative) at
// the pair's sorted position, plus the offset sums of h per segment of
// min(G, 64) rows for the down matrix.
constexpr int kNT = 8;
constexpr int kGUWaves = 8;

struct TokRef {
  int pos;  // sorted position of the pair
  int tok;  // token index
};

template <int BITS>
__device__ __forceinline__ void load_unit(const uint8_t* codes, int64_t tile, int lane,
                                          uint32_t (&w)[UnitCodec<BITS>::WORDS]) {
  using C = UnitCodec<BITS>;
#pragma unroll
  for (int j = 0; j < C::CHUNKS; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(codes + (tile * C::CHUNKS + j) * 1024 + 16 * lane);
    w[4 * j + 0] = v.x;
    w[4 * j + 1] = v.y;
    w[4 * j + 2] = v.z;
    w[4 * j + 3] = v.w;
  }
}

template <int BITS>
__global__ __launch_bounds__(512) void k_gateup(
    const moe_expert_ref* __restrict__ table, const int32_t* __restrict__ active, int E,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs, int K,
    const uint16_t* __restrict__ x, int H, int I, int scale_f16, const float* __restrict__ xcorr,
    uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo, float* __restrict__ hcorr) {
  using C = UnitCodec<BITS>;
  const int a = blockIdx.x;
  const int U = active[E];
  if (a >= U) return;
  const int e = active[a];
  const int seg0 = offsets[e], n_e = offsets[e + 1] - seg0;
  const int strip = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ng = H / C::G;
  const MatGeom gm{I, H, BITS, C::G};
  const uint8_t* gate = reinterpret_cast<const uint8_t*>(table[e].gate);
  const uint8_t* up = reinterpret_cast<const uint8_t*>(table[e].up);
  const uint16_t* gsc = reinterpret_cast<const uint16_t*>(gate + gm.scales_off());
  const uint16_t* usc = reinterpret_cast<const uint16_t*>(up + gm.scales_off());
  const int row = strip * 64 + lane;
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  const int hseg = C::G < 64 ? C::G : 64;

  __shared__ float red[kGUWaves][2][kNT][64];
  __shared__ float hc[kNT][64];

  for (int b0 = 0; b0 < n_e; b0 += kNT) {
    const int nt = min(kNT, n_e - b0);
    int tok[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) tok[j] = j < nt ? sorted_pairs[seg0 + b0 + j] / K : 0;
    float ag[kNT], au[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) ag[j] = au[j] = 0.f;
    for (int g = wv; g < ng; g += kGUWaves) {
      const int64_t tile = (int64_t)strip * ng + g;
      uint32_t wg[C::WORDS], wu[C::WORDS];
      load_unit<BITS>(gate, tile, lane, wg);
      load_unit<BITS>(up, tile, lane, wu);
      const float sg = scale_to_f32(gsc[(int64_t)row * ng + g], scale_f16);
      const float su = scale_to_f32(usc[(int64_t)row * ng + g], scale_f16);
      uint32_t p[C::PAIRS];
      C::decode(wg, p);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        if (j < nt) {
          const uint32_t* xr = x32 + ((int64_t)tok[j] * H + g * C::G) / 2;
          float d = -xcorr[(int64_t)tok[j] * ng + g];
#pragma unroll
          for (int P = 0; P < C::PAIRS; ++P) d = dot2_bf16(p[P], xr[P], d);
          ag[j] = fmaf(sg, d, ag[j]);
        }
      }
      C::decode(wu, p);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        if (j < nt) {
          const uint32_t* xr = x32 + ((int64_t)tok[j] * H + g * C::G) / 2;
          float d = -xcorr[(int64_t)tok[j] * ng + g];
#pragma unroll
          for (int P = 0; P < C::PAIRS; ++P) d = dot2_bf16(p[P], xr[P], d);
          au[j] = fmaf(su, d, au[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      red[wv][0][j][lane] = ag[j];
      red[wv][1][j][lane] = au[j];
    }
    __syncthreads();
    // wave j (< nt) finishes token j: lane = row
    if (wv < nt) {
      const int j = wv;
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < kGUWaves; ++w) {
        gs += red[w][0][j][lane];
        us += red[w][1][j][lane];
      }
      const float h = gs / (1.f + __expf(-gs)) * us;
      const uint16_t hi = f32_to_bf16_rne(h);
      const uint16_t lo = f32_to_bf16_rne(h - bf16_to_f32(hi));
      const int64_t pos = seg0 + b0 + j;
      h_hi[pos * I + row] = hi;
      h_lo[pos * I + row] = lo;
      // offset of this row as a reduction index of the down matrix
      const float off = UnitCodec<BITS>::pair_off((row % C::G) / 2);
      hc[j][lane] = off * bf16_to_f32(hi) + off * bf16_to_f32(lo);
    }
    __syncthreads();
    if (threadIdx.x < nt * (64 / hseg)) {
      const int j = threadIdx.x / (64 / hseg), s = threadIdx.x % (64 / hseg);
      float acc = 0.f;
      for (int r = 0; r < hseg; ++r) acc += hc[j][s * hseg + r];
      const int64_t pos = seg0 + b0 + j;
      hcorr[pos * (I / hseg) + (strip * 64) / hseg + s] = acc;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down
// Block (a, strip): rows [64*strip, +64) of the down matrix of active expert a,
// 4 waves take groups g = wave, wave+4, ...; each token's h (hi and lo pairs)
// comes through scalar loads.  y goes to pair_out at the pair's sorted position.
constexpr int kDNWaves = 4;

template <int BITS>
__global__ __launch_bounds__(256) void k_down(
    const moe_expert_ref* __restrict__ table, const int32_t* __restrict__ active, int E,
    const int32_t* __restrict__ offsets, int H, int I, int scale_f16,
    const uint16_t* __restrict__ h_hi, const uint16_t* __restrict__ h_lo,
    const float* __restrict__ hcorr, float* __restrict__ pair_out) {
  using C = UnitCodec<BITS>;
  const int a = blockIdx.x;
  const int U = active[E];
  if (a >= U) return;
  const int e = active[a];
  const int seg0 = offsets[e], n_e = offsets[e + 1] - seg0;
  const int strip = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ng = I / C::G;
  const int hseg = C::G < 64 ? C::G : 64;
  const int nseg = I / hseg, seg_per_g = C::G / hseg;
  const MatGeom gm{H, I, BITS, C::G};
  const uint8_t* down = reinterpret_cast<const uint8_t*>(table[e].down);
  const uint16_t* dsc = reinterpret_cast<const uint16_t*>(down + gm.scales_off());
  const int row = strip * 64 + lane;
  __shared__ float red[kDNWaves][kNT][64];

  for (int b0 = 0; b0 < n_e; b0 += kNT) {
    const int nt = min(kNT, n_e - b0);
    float acc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[j] = 0.f;
    for (int g = wv; g < ng; g += kDNWaves) {
      const int64_t tile = (int64_t)strip * ng + g;
      uint32_t w[C::WORDS];
      load_unit<BITS>(down, tile, lane, w);
      const float s = scale_to_f32(dsc[(int64_t)row * ng + g], scale_f16);
      uint32_t p[C::PAIRS];
      C::decode(w, p);
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        if (j < nt) {
          const int64_t pos = seg0 + b0 + j;
          const uint32_t* hh = reinterpret_cast<const uint32_t*>(h_hi + pos * I + g * C::G);
          const uint32_t* hl = reinterpret_cast<const uint32_t*>(h_lo + pos * I + g * C::G);
          float corr = 0.f;
          for (int q = 0; q < seg_per_g; ++q) corr += hcorr[pos * nseg + g * seg_per_g + q];
          float d = -corr;
#pragma unroll
          for (int P = 0; P < C::PAIRS; ++P) d = dot2_bf16(p[P], hh[P], d);
#pragma unroll
          for (int P = 0; P < C::PAIRS; ++P) d = dot2_bf16(p[P], hl[P], d);
          acc[j] = fmaf(s, d, acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) red[wv][j][lane] = acc[j];
    __syncthreads();
    if (wv == 0) {
      for (int j = 0; j < nt; ++j) {
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < kDNWaves; ++w) y += red[w][j][lane];
        pair_out[(int64_t)(seg0 + b0 + j) * H + row] = y;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- combine
// out[t][n] = sum_k w[t][k] * pair_out[pair_pos[t*K+k]][n] (k ascending; pairs
// left out of the grouping are skipped) + shared[t][n].
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ pair_out,
                                                 const int32_t* __restrict__ pair_pos,
                                                 const float* __restrict__ w, int K, int H,
                                                 const float* __restrict__ shared,
                                                 float* __restrict__ out) {
  const int t = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= H) return;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) {
    const int pos = pair_pos[t * K + k];
    if (pos >= 0) acc = fmaf(w[t * K + k], pair_out[(int64_t)pos * H + n], acc);
  }
  if (shared) acc += shared[(int64_t)t * H + n];
  out[(int64_t)t * H + n] = acc;
}

// ---------------------------------------------------------------- shared expert
// Row-major bf16 weights.  Block = 8 rows x 32 lanes per row (each lane reads 8
// consecutive bf16 per step, a half-wave covers 256 of a row); fp32 FMAs.
constexpr int kShRows = 8;

__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void k_shared_gateup(const uint16_t* __restrict__ wg,
                                                       const uint16_t* __restrict__ wu,
                                                       const uint16_t* __restrict__ x, int T,
                                                       int H, int Is, float* __restrict__ hs) {
  const int r = blockIdx.x * kShRows + (threadIdx.x >> 5);
  const int sub = threadIdx.x & 31;
  for (int t0 = 0; t0 < T; t0 += kNT) {
    const int nt = min(kNT, T - t0);
    float ag[kNT], au[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) ag[j] = au[j] = 0.f;
    for (int k0 = sub * 8; k0 < H; k0 += 256) {
      const uint4 g4 = *reinterpret_cast<const uint4*>(wg + (int64_t)r * H + k0);
      const uint4 u4 = *reinterpret_cast<const uint4*>(wu + (int64_t)r * H + k0);
      const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w}, uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        if (j < nt) {
          const uint4 x4 = *reinterpret_cast<const uint4*>(x + (int64_t)(t0 + j) * H + k0);
          const uint32_t xw[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float xl = bf16_to_f32((uint16_t)xw[q]), xh = bf16_to_f32((uint16_t)(xw[q] >> 16));
            ag[j] = fmaf(bf16_to_f32((uint16_t)gw[q]), xl, ag[j]);
            ag[j] = fmaf(bf16_to_f32((uint16_t)(gw[q] >> 16)), xh, ag[j]);
            au[j] = fmaf(bf16_to_f32((uint16_t)uw[q]), xl, au[j]);
            au[j] = fmaf(bf16_to_f32((uint16_t)(uw[q] >> 16)), xh, au[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const float gs = half_wave_sum(ag[j]), us = half_wave_sum(au[j]);
      if (sub == 0 && j < nt) hs[(int64_t)(t0 + j) * Is + r] = gs / (1.f + __expf(-gs)) * us;
    }
  }
}

__global__ __launch_bounds__(256) void k_shared_down(const uint16_t* __restrict__ wd,
                                                     const float* __restrict__ hs, int T, int H,
                                                     int Is, float* __restrict__ ys) {
  const int r = blockIdx.x * kShRows + (threadIdx.x >> 5);
  const int sub = threadIdx.x & 31;
  for (int t0 = 0; t0 < T; t0 += kNT) {
    const int nt = min(kNT, T - t0);
    float acc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) acc[j] = 0.f;
    for (int k0 = sub * 8; k0 < Is; k0 += 256) {
      const uint4 d4 = *reinterpret_cast<const uint4*>(wd + (int64_t)r * Is + k0);
      const uint32_t dw[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int j = 0; j < kNT; ++j) {
        if (j < nt) {
          const float4 h0 = *reinterpret_cast<const float4*>(hs + (int64_t)(t0 + j) * Is + k0);
          const float4 h1 = *reinterpret_cast<const float4*>(hs + (int64_t)(t0 + j) * Is + k0 + 4);
          const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[j] = fmaf(bf16_to_f32((uint16_t)dw[q]), hv[2 * q], acc[j]);
            acc[j] = fmaf(bf16_to_f32((uint16_t)(dw[q] >> 16)), hv[2 * q + 1], acc[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const float y = half_wave_sum(acc[j]);
      if (sub == 0 && j < nt) ys[(int64_t)(t0 + j) * H + r] = y;
    }
  }
}

// ---------------------------------------------------------------- rmsnorm glue
// resid += add (if given); y = bf16(resid / sqrt(mean(resid^2) + eps)), one block
// per token, fixed-order reduction.
__global__ __launch_bounds__(256) void k_rmsnorm(float* __restrict__ resid,
                                                 const float* __restrict__ add, int H, float eps,
                                                 uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  float* r = resid + (int64_t)t * H;
  float ss = 0.f;
  for (int h = threadIdx.x; h < H; h += 256) {
    float v = r[h];
    if (add) {
      v += add[(int64_t)t * H + h];
      r[h] = v;
    }
    ss = fmaf(v, v, ss);
  }
  __shared__ float part[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float inv = 1.f / sqrtf(tot / (float)H + eps);
  for (int h = threadIdx.x; h < H; h += 256) y[(int64_t)t * H + h] = f32_to_bf16_rne(r[h] * inv);
}

// ---------------------------------------------------------------- counters init
__global__ void k_zero_i32(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------- launchers

template <int BITS>
hipError_t launch_forward_t(const FwdArgs& f, hipStream_t s) {
  using C = UnitCodec<BITS>;
  const moe_cfg& c = *f.c;
  const int H = c.hidden, I = c.inter, E = c.n_experts, K = c.top_k, T = f.T;
  const WsLayout L = ws_layout(c, T);
  int32_t* active = reinterpret_cast<int32_t*>(f.ws + L.active);
  float* xcorr = reinterpret_cast<float*>(f.ws + L.xcorr);
  uint16_t* h_hi = reinterpret_cast<uint16_t*>(f.ws + L.h_hi);
  uint16_t* h_lo = reinterpret_cast<uint16_t*>(f.ws + L.h_lo);
  float* hcorr = reinterpret_cast<float*>(f.ws + L.hcorr);
  float* pair_out = f.pair_out ? f.pair_out : reinterpret_cast<float*>(f.ws + L.pair_out);
  float* sh_h = reinterpret_cast<float*>(f.ws + L.sh_h);
  float* sh_out = reinterpret_cast<float*>(f.ws + L.sh_out);
  const int ngx = H / C::G;
  const int plan_blocks = (T * ngx + 255) / 256;
  MOE_LAUNCH(KID_PLAN, k_plan<BITS>, dim3(plan_blocks > 0 ? plan_blocks : 1), dim3(256), 0, s,
                     f.offsets, E, f.x, T, H, active, xcorr);
  const int maxU = min(E, T * K);
  MOE_LAUNCH(KID_GATEUP, k_gateup<BITS>, dim3(maxU, I / 64), dim3(64 * kGUWaves), 0, s, f.table,
                     active, E, f.offsets, f.sorted_pairs, K, f.x, H, I, c.scale_f16, xcorr, h_hi,
                     h_lo, hcorr);
  MOE_LAUNCH(KID_DOWN, k_down<BITS>, dim3(maxU, H / 64), dim3(64 * kDNWaves), 0, s, f.table, active,
                     E, f.offsets, H, I, c.scale_f16, h_hi, h_lo, hcorr, pair_out);
  const bool has_shared = c.shared_inter > 0 && f.sg && f.su && f.sd;
  if (has_shared) {
    const int Is = c.shared_inter;
    MOE_LAUNCH(KID_SH_GATEUP, k_shared_gateup, dim3(Is / kShRows), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(f.sg),
                       reinterpret_cast<const uint16_t*>(f.su), f.x, T, H, Is, sh_h);
    MOE_LAUNCH(KID_SH_DOWN, k_shared_down, dim3(H / kShRows), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(f.sd), sh_h, T, H, Is, sh_out);
  }
  MOE_LAUNCH(KID_COMBINE, k_combine, dim3((H + 255) / 256, T), dim3(256), 0, s, pair_out, f.pair_pos,
                     f.w, K, H, has_shared ? sh_out : nullptr, f.out);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& f, hipStream_t s) {
  return f.c->bits == 3 ? launch_forward_t<3>(f, s) : launch_forward_t<4>(f, s);
}

hipError_t launch_rmsnorm(float* resid, const float* add, int T, int H, float eps, uint16_t* y,
                          hipStream_t s) {
  MOE_LAUNCH(KID_RMSNORM, k_rmsnorm, dim3(T), dim3(256), 0, s, resid, add, H, eps, y);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  MOE_LAUNCH(KID_ZERO, k_zero_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moe
