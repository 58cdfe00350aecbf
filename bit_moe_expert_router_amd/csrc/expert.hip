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
// The routed experts themselves run in decode.hip (GEMV kernels, batches of at
// most 64 tokens) and prefill.hip (matrix-core kernels); this file holds what
// both share: the bf16 shared expert, the combine of the prefill path and the
// RMSNorm glue.
#include "common.h"

namespace moe {

// ---------------------------------------------------------------- combine
// out[t][n] = sum_k w[t][k] * pair_out[t*K + k][n] (k ascending; pairs whose id is
// outside [0, E) were left out of the grouping and are skipped) + the shared
// expert's output (nsh slices shared[q][t][n], added in order).
// All KM rows are requested at once (k >= K repeats row K-1 and is dropped), so
// the combine costs one memory round trip.
template <int KM>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ pair_out,
                                                 const int32_t* __restrict__ ids,
                                                 const float* __restrict__ w, int K, int E, int H,
                                                 const float* __restrict__ shared, int nsh, int T,
                                                 const int32_t* __restrict__ call_bad,
                                                 float* __restrict__ out,
                                                 float* __restrict__ resid) {
  const int t = blockIdx.y;
  const int n = min((int)(blockIdx.x * 256 + threadIdx.x), H - 1);
  float y[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) y[k] = pair_out[((int64_t)t * K + min(k, K - 1)) * H + n];
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int id = ids[t * K + min(k, K - 1)];
    if (k < K && id >= 0 && id < E) acc = fmaf(w[t * K + min(k, K - 1)], y[k], acc);
  }
  if (shared) {  // the shared expert's slices, in slice order
    float sh = 0.f;
    for (int q = 0; q < nsh; ++q) sh += shared[((int64_t)q * T + t) * H + n];
    acc += sh;
  }
  // inconsistent caller routing: the output is left untouched
  if (blockIdx.x * 256 + threadIdx.x < H && !call_bad[0]) {
    out[(int64_t)t * H + n] = acc;
    if (resid) resid[(int64_t)t * H + n] += acc;  // a stack layer: the residual update
  }
}

// ---------------------------------------------------------------- shared expert
// Row-major bf16 weights.  Block = 8 rows x 32 lanes per row, over one slice of
// the reduction dimension (the slices' partial sums are added in slice order
// later), each lane reading 16-byte pieces 256 elements apart.  A block first
// stages its slice of the activations (up to 8 tokens per pass) in LDS, then
// requests all of its weights at once, so a launch is one memory round trip
// deep.  Gate/up take bf16 pair products (v_dot2_f32_bf16, exact products, fp32
// sums); h = silu(g) * u stays fp32 and the down products are fp32 FMAs.
typedef float f32x4s __attribute__((ext_vector_type(4)));
constexpr int kShRows = 8;
constexpr int kNT = 8;       // tokens per pass
constexpr int kShSteps = 8;  // 256-element steps per slice, at most
constexpr int kShareSlicesGU = 4;
constexpr int kShareSlicesDN = 2;
static_assert(kShareSlicesDN <= kMaxShared, "the decode combine reads at most kMaxShared slices");

__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// part[(ks*2 + m)][t][r]: slice ks of gate (m = 0) and up (m = 1) for row r.
template <int S>
__global__ __launch_bounds__(256) void k_shared_gateup(const uint16_t* __restrict__ wg,
                                                       const uint16_t* __restrict__ wu,
                                                       const uint16_t* __restrict__ x, int T,
                                                       int H, int Is, float* __restrict__ part) {
  __shared__ __align__(16) uint32_t xs[kNT * S * 128];  // [token][slice element pair]
  const int r = blockIdx.x * kShRows + (threadIdx.x >> 5);
  const int sub = threadIdx.x & 31;
  const int ks = blockIdx.y, kb = ks * S * 256;
  for (int t0 = 0; t0 < T; t0 += kNT) {
    const int nt = min(kNT, T - t0);
    // activation slice: piece q (16 bytes) = token q / (S*32), elements 8*(q % (S*32))
    constexpr int NQ = kNT * S * 32, IT = (NQ + 255) / 256;
    u32x4 xv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = min(it * 256 + (int)threadIdx.x, NQ - 1);
      const int j = min(q / (S * 32), nt - 1), e = 8 * (q % (S * 32));
      xv[it] = *reinterpret_cast<const u32x4*>(x + (int64_t)(t0 + j) * H + kb + e);
    }
    asm volatile("" ::: "memory");
    u32x4 g4[S], u4[S];
#pragma unroll
    for (int st = 0; st < S; ++st) {
      g4[st] = *reinterpret_cast<const u32x4*>(wg + (int64_t)r * H + kb + 256 * st + 8 * sub);
      u4[st] = *reinterpret_cast<const u32x4*>(wu + (int64_t)r * H + kb + 256 * st + 8 * sub);
    }
    asm volatile("" ::: "memory");
    lds_barrier();  // the previous pass is done with xs
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = it * 256 + threadIdx.x;
      if (q < NQ) *reinterpret_cast<u32x4*>(xs + 4 * q) = xv[it];
    }
    lds_barrier();
    float ag[kNT], au[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      ag[j] = au[j] = 0.f;
      if (j < nt) {
#pragma unroll
        for (int st = 0; st < S; ++st) {
          const u32x4 xq = *reinterpret_cast<const u32x4*>(xs + (j * S * 32 + st * 32 + sub) * 4);
          ag[j] = dot2_bf16(g4[st].x, xq.x, ag[j]);
          ag[j] = dot2_bf16(g4[st].y, xq.y, ag[j]);
          ag[j] = dot2_bf16(g4[st].z, xq.z, ag[j]);
          ag[j] = dot2_bf16(g4[st].w, xq.w, ag[j]);
          au[j] = dot2_bf16(u4[st].x, xq.x, au[j]);
          au[j] = dot2_bf16(u4[st].y, xq.y, au[j]);
          au[j] = dot2_bf16(u4[st].z, xq.z, au[j]);
          au[j] = dot2_bf16(u4[st].w, xq.w, au[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const float g = half_wave_sum(ag[j]), u = half_wave_sum(au[j]);
      if (sub == 0 && j < nt) {
        part[((int64_t)(ks * 2 + 0) * T + t0 + j) * Is + r] = g;
        part[((int64_t)(ks * 2 + 1) * T + t0 + j) * Is + r] = u;
      }
    }
  }
}

// hs[t][k] = silu(sum_ks g) * (sum_ks u), slices added in order.
__global__ __launch_bounds__(256) void k_shared_h(const float* __restrict__ part, int KS, int T,
                                                  int Is, float* __restrict__ hs) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * Is) return;
  float g = 0.f, u = 0.f;
  for (int ks = 0; ks < KS; ++ks) {
    g += part[(int64_t)(ks * 2 + 0) * T * Is + i];
    u += part[(int64_t)(ks * 2 + 1) * T * Is + i];
  }
  hs[i] = g / (1.f + __expf(-g)) * u;
}

// ys[kd][t][r]: slice kd of the down product for row r.
template <int S>
__global__ __launch_bounds__(256) void k_shared_down(const uint16_t* __restrict__ wd,
                                                     const float* __restrict__ hs, int T, int H,
                                                     int Is, float* __restrict__ ys) {
  __shared__ __align__(16) float hsl[kNT * S * 256];
  const int r = blockIdx.x * kShRows + (threadIdx.x >> 5);
  const int sub = threadIdx.x & 31;
  const int kd = blockIdx.y, kb = kd * S * 256;
  for (int t0 = 0; t0 < T; t0 += kNT) {
    const int nt = min(kNT, T - t0);
    constexpr int NQ = kNT * S * 64, IT = (NQ + 255) / 256;  // float4 pieces
    f32x4s hv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = min(it * 256 + (int)threadIdx.x, NQ - 1);
      const int j = min(q / (S * 64), nt - 1), e = 4 * (q % (S * 64));
      hv[it] = *reinterpret_cast<const f32x4s*>(hs + (int64_t)(t0 + j) * Is + kb + e);
    }
    asm volatile("" ::: "memory");
    u32x4 d4[S];
#pragma unroll
    for (int st = 0; st < S; ++st)
      d4[st] = *reinterpret_cast<const u32x4*>(wd + (int64_t)r * Is + kb + 256 * st + 8 * sub);
    asm volatile("" ::: "memory");
    lds_barrier();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = it * 256 + threadIdx.x;
      if (q < NQ) *reinterpret_cast<f32x4s*>(hsl + 4 * q) = hv[it];
    }
    lds_barrier();
    float acc[kNT];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      acc[j] = 0.f;
      if (j < nt) {
#pragma unroll
        for (int st = 0; st < S; ++st) {
          const float* hp = hsl + j * S * 256 + st * 256 + 8 * sub;
          const f32x4s h0 = *reinterpret_cast<const f32x4s*>(hp);
          const f32x4s h1 = *reinterpret_cast<const f32x4s*>(hp + 4);
          const uint32_t dw[4] = {d4[st].x, d4[st].y, d4[st].z, d4[st].w};
          const float hf[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[j] = fmaf(bf16_to_f32((uint16_t)dw[q]), hf[2 * q], acc[j]);
            acc[j] = fmaf(bf16_to_f32((uint16_t)(dw[q] >> 16)), hf[2 * q + 1], acc[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const float y = half_wave_sum(acc[j]);
      if (sub == 0 && j < nt) ys[((int64_t)kd * T + t0 + j) * H + r] = y;
    }
  }
}

// Slices: the reduction dimension D (a multiple of 256) is cut into the largest
// number of slices <= `want` whose length is a whole number of 256-element steps
// and at most kShSteps of them.
__host__ inline int shared_slices(int D, int want) {
  const int steps = D / 256;
  for (int n = want; n >= 1; --n)
    if (steps % n == 0 && steps / n <= kShSteps) return n;
  return 0;
}

hipError_t launch_shared(const FwdArgs& f, const WsLayout& L, hipStream_t s, float** out,
                         int* nslices) {
  const moe_cfg& c = *f.c;
  const int H = c.hidden, Is = c.shared_inter, T = f.T;
  float* part = reinterpret_cast<float*>(f.ws + L.sh_part);
  float* hs = reinterpret_cast<float*>(f.ws + L.sh_h);
  float* ys = reinterpret_cast<float*>(f.ws + L.sh_out);
  const int KS = shared_slices(H, kShareSlicesGU), KD = shared_slices(Is, kShareSlicesDN);
  if (!KS || !KD) return hipErrorInvalidValue;
#define MOE_SGU(N)                                                                               \
  case N:                                                                                        \
    MOE_LAUNCH(KID_SH_GATEUP, k_shared_gateup<N>, dim3(Is / kShRows, KS), dim3(256), 0, s,       \
               reinterpret_cast<const uint16_t*>(f.sg), reinterpret_cast<const uint16_t*>(f.su), \
               f.x, T, H, Is, part);                                                             \
    break;
  switch (H / 256 / KS) {
    MOE_SGU(1) MOE_SGU(2) MOE_SGU(3) MOE_SGU(4) MOE_SGU(5) MOE_SGU(6) MOE_SGU(7) MOE_SGU(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_SGU
  MOE_LAUNCH(KID_SH_GATEUP, k_shared_h, dim3((T * Is + 255) / 256), dim3(256), 0, s, part, KS, T,
             Is, hs);
#define MOE_SDN(N)                                                                               \
  case N:                                                                                        \
    MOE_LAUNCH(KID_SH_DOWN, k_shared_down<N>, dim3(H / kShRows, KD), dim3(256), 0, s,            \
               reinterpret_cast<const uint16_t*>(f.sd), hs, T, H, Is, ys);                       \
    break;
  switch (Is / 256 / KD) {
    MOE_SDN(1) MOE_SDN(2) MOE_SDN(3) MOE_SDN(4) MOE_SDN(5) MOE_SDN(6) MOE_SDN(7) MOE_SDN(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_SDN
  *out = ys;
  *nslices = KD;
  return hipGetLastError();
}

// ---------------------------------------------------------------- rmsnorm glue
// resid += add (if given); y = bf16(resid / sqrt(mean(resid^2) + eps)), fixed-
// order reduction.  One block per token; each thread requests all of its 16-byte pieces of the
// residual (and of the addend) at once, so the kernel is one memory round trip
// deep: H/4 pieces over 256 threads, at most kRnPieces per thread (H <= 8192).
__global__ __launch_bounds__(256) void k_rmsnorm(float* __restrict__ resid,
                                                 const float* __restrict__ add, int H, float eps,
                                                 uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  const int H4 = H / 4;
  rn_f4* r = reinterpret_cast<rn_f4*>(resid + (int64_t)t * H);
  const rn_f4* ad = add ? reinterpret_cast<const rn_f4*>(add + (int64_t)t * H) : nullptr;
  rn_f4 v[kRnPieces];
#pragma unroll
  for (int i = 0; i < kRnPieces; ++i) {
    const int q = min((int)threadIdx.x + 256 * i, H4 - 1);
    v[i] = r[q];
  }
  if (ad) {
    rn_f4 a[kRnPieces];
#pragma unroll
    for (int i = 0; i < kRnPieces; ++i) a[i] = ad[min((int)threadIdx.x + 256 * i, H4 - 1)];
#pragma unroll
    for (int i = 0; i < kRnPieces; ++i) {
      v[i] += a[i];
      const int q = threadIdx.x + 256 * i;
      if (q < H4) r[q] = v[i];
    }
  }
  const float ss = rms_wave_sum(v, H4);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = rms_inv(part, H, eps);
  uint2* yo = reinterpret_cast<uint2*>(y + (int64_t)t * H);
#pragma unroll
  for (int i = 0; i < kRnPieces; ++i) {
    const int q = threadIdx.x + 256 * i;
    if (q < H4) yo[q] = make_uint2(rms_bf16x2(v[i].x, v[i].y, inv), rms_bf16x2(v[i].z, v[i].w, inv));
  }
}

// ---------------------------------------------------------------- pointer table
// A layer's table entries travel as a kernel argument (by value, kTableChunk
// entries per launch), so setting a table needs no host staging buffer, returns
// without waiting, and a captured graph keeps its own copy of the entries.
constexpr int kTableChunk = 128;  // 3 KB of kernel arguments
struct TableChunk {
  moe_expert_ref e[kTableChunk];
};

__global__ __launch_bounds__(kTableChunk) void k_set_table(moe_expert_ref* __restrict__ dst,
                                                           TableChunk src, int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = src.e[i];
}

hipError_t launch_set_table(moe_expert_ref* dst, const moe_expert_ref* host, int n,
                            hipStream_t s) {
  for (int b = 0; b < n; b += kTableChunk) {
    TableChunk c;
    const int m = std::min(kTableChunk, n - b);
    for (int i = 0; i < kTableChunk; ++i) c.e[i] = host[b + std::min(i, m - 1)];
    MOE_LAUNCH(KID_TABLE, k_set_table, dim3(1), dim3(kTableChunk), 0, s, dst + b, c, m);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- counters init
__global__ void k_zero_i32(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_forward(const FwdArgs& f, hipStream_t s) {
  const moe_cfg& c = *f.c;
  const int H = c.hidden, E = c.n_experts, K = c.top_k, T = f.T;
  const WsLayout L = ws_layout(c, T);
  const bool has_shared = c.shared_inter > 0 && f.sg && f.su && f.sd;
  float* sh_out = nullptr;
  int nsh = 0;
  hipEvent_t join = nullptr;
  if (has_shared) {
    // the shared expert needs only x: it runs on the side stream while the
    // routed experts run on s; the combine waits for it
    const bool fork = f.side && f.ev_fork && f.ev_join;
    hipStream_t ss = fork ? f.side : s;
    if (fork) {
      hipError_t e = hipEventRecord(f.ev_fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(f.side, f.ev_fork, 0);
      if (e != hipSuccess) return e;
    }
    const hipError_t err = launch_shared(f, L, ss, &sh_out, &nsh);
    if (err != hipSuccess) return err;
    if (fork) {
      const hipError_t e = hipEventRecord(f.ev_join, f.side);
      if (e != hipSuccess) return e;
      join = f.ev_join;
    }
  }
  if (!prefill_eligible(c, T)) return launch_decode(f, L, sh_out, nsh, join, s);
  float* pair_out = f.pair_out ? f.pair_out : reinterpret_cast<float*>(f.ws + L.pair_out);
  hipError_t err = launch_prefill(f, L, pair_out, s);
  if (err == hipSuccess && join) err = hipStreamWaitEvent(s, join, 0);
  if (err != hipSuccess) return err;
  const int32_t* call_bad = reinterpret_cast<const int32_t*>(f.ws + L.counters) + kCtrCallBad;
  if (K <= 8) {
    MOE_LAUNCH(KID_COMBINE, k_combine<8>, dim3((H + 255) / 256, T), dim3(256), 0, s, pair_out,
               f.ids, f.w, K, E, H, sh_out, nsh, T, call_bad, f.out, f.resid);
  } else {
    MOE_LAUNCH(KID_COMBINE, k_combine<16>, dim3((H + 255) / 256, T), dim3(256), 0, s, pair_out,
               f.ids, f.w, K, E, H, sh_out, nsh, T, call_bad, f.out, f.resid);
  }
  return hipGetLastError();
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
