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

// ---------------------------------------------------------------- active experts
// The a-th expert (ascending logical id) that owns at least one pair, the number
// U of such experts, its segment of the grouping and its table entry.
// Wave-cooperative (every lane returns the same values).  Each lane loads the
// offsets and the table entries of its candidate experts lane + 64*i in the same
// round trip, so the expert's weight addresses are known after one memory
// latency instead of two.  E <= 1024.
struct Active {
  int e;     // -1 if a >= U
  int U;
  int seg0;  // first sorted position of the expert's pairs
  int n;     // number of pairs
  const void* ptr[3];  // gate, up, down
};

__device__ __forceinline__ Active find_active(const int32_t* __restrict__ offsets,
                                              const moe_expert_ref* __restrict__ table, int E,
                                              int a) {
  const int lane = threadIdx.x & 63;
  constexpr int kSpec = 5;  // candidates per lane whose table entry is fetched up front
  const int nch = (E + 63) / 64;
  int lo[16], hi[16];
  moe_expert_ref ref[kSpec];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < nch) {  // uniform
      const int e = lane + 64 * i;
      lo[i] = (e < E) ? offsets[e] : 0;
      hi[i] = (e < E) ? offsets[e + 1] : 0;
      if (i < kSpec) ref[i] = e < E ? table[e] : moe_expert_ref{nullptr, nullptr, nullptr};
    }
  }
  Active r{-1, 0, 0, 0, {nullptr, nullptr, nullptr}};
  int U = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < nch) {
      const bool nz = hi[i] > lo[i];
      const uint64_t bal = __ballot(nz);
      const int cnt = __popcll(bal);
      if (r.e < 0 && a < U + cnt) {  // uniform: the a-th active expert is in this chunk
        // lane holding it: the (a-U)-th set bit of bal
        uint64_t m = bal;
        for (int k = 0; k < a - U; ++k) m &= m - 1;
        const int src = __ffsll((unsigned long long)m) - 1;
        r.e = 64 * i + src;
        r.seg0 = __shfl(lo[i], src);
        r.n = __shfl(hi[i], src) - r.seg0;
        if (i < kSpec) {
          r.ptr[0] = (const void*)__shfl((long long)ref[i].gate, src);
          r.ptr[1] = (const void*)__shfl((long long)ref[i].up, src);
          r.ptr[2] = (const void*)__shfl((long long)ref[i].down, src);
        } else {
          const moe_expert_ref t = table[r.e];
          r.ptr[0] = t.gate;
          r.ptr[1] = t.up;
          r.ptr[2] = t.down;
        }
      }
      U += cnt;
    }
  }
  r.U = U;
  return r;
}

// ---------------------------------------------------------------- unit loads
// A 16-bit scale is fetched as the aligned dword that contains it (the scales
// region is 256-byte aligned, so the dword lies inside it) and selected at use.
__device__ __forceinline__ uint32_t load_scale_dword(gu16_t sc, int64_t idx) {
  typedef const uint32_t __attribute__((address_space(1)))* gu32_t;
  return *(gu32_t)(sc + (idx & ~(int64_t)1));
}
__device__ __forceinline__ uint16_t scale_from_dword(uint32_t w, int64_t idx) {
  return (uint16_t)(w >> ((idx & 1) * 16));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BITS>
__device__ __forceinline__ void load_unit4(gbytes_t codes, int64_t tile, int lane,
                                           u32x4 (&w)[UnitCodec<BITS>::CHUNKS]) {
  using C = UnitCodec<BITS>;
  typedef const u32x4 __attribute__((address_space(1)))* gu4_t;
#pragma unroll
  for (int j = 0; j < C::CHUNKS; ++j)
    w[j] = *(gu4_t)(codes + (tile * C::CHUNKS + j) * 1024 + 16 * lane);
}

// The unit's words, passed through an empty asm so that the decode that follows
// stays inside the token loop (hoisting every group's decoded pairs out of it
// would need GPW * 128 registers).
template <int BITS>
__device__ __forceinline__ void unit_words(const u32x4 (&c)[UnitCodec<BITS>::CHUNKS],
                                           uint32_t (&w)[UnitCodec<BITS>::WORDS]) {
#pragma unroll
  for (int j = 0; j < UnitCodec<BITS>::CHUNKS; ++j) {
    w[4 * j + 0] = c[j].x;
    w[4 * j + 1] = c[j].y;
    w[4 * j + 2] = c[j].z;
    w[4 * j + 3] = c[j].w;
  }
#pragma unroll
  for (int k = 0; k < UnitCodec<BITS>::WORDS; ++k) asm volatile("" : "+v"(w[k]));
}

// ---------------------------------------------------------------- gate / up
// Block (a, strip, m*KP + kp): matrix m (0 gate, 1 up) of the a-th active
// expert, rows [64*strip, 64*strip+64), part kp of the reduction dimension (a
// contiguous range of groups); 4 waves take groups g0 + wave + 4*i, i < GPW.
//
// Memory schedule.  Each wave first requests the activations of its groups for
// up to kXTok of the expert's tokens (they go to the wave's own LDS region), then
// all of its groups' codes and scales, so the whole weight stream is in flight
// after one memory latency and stays in registers.  The token passes then read
// the activations from LDS (one broadcast 16-byte read gives four pairs), so no
// pass waits on memory; experts with more than kXTok tokens stage the next
// tokens when the first ones are done.  The per-group offset sums of the
// activations (what the unit codec's dot products carry) come from the same LDS
// copy.
//
// Tokens run two at a time against the resident weights; each code pair is
// expanded right before its dot products.  The partial product (fp32) goes to
// gu[m*KP + kp][pos][row] at the pair's sorted position; the parts are added in
// kp order, with SwiGLU, where the down matrix reads them.
constexpr int kGUWaves = 4;
constexpr int kTokPerPass = 2;
// tokens whose activations a wave stages at a time: XT (2 for batches of at most
// two tokens, else 8)

// Sum over the 64 lanes in a fixed order (row prefix sums by DPP, then the row
// totals), returned to every lane; deterministic, no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_shift(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int BITS>
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += dpp_shift<0x111>(v);  // row_shr:1
  v += dpp_shift<0x112>(v);  // row_shr:2
  v += dpp_shift<0x114>(v);  // row_shr:4
  v += dpp_shift<0x118>(v);  // row_shr:8
  v += dpp_shift<0x142>(v);  // row_bcast:15
  v += dpp_shift<0x143>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Stage the activations of tokens c0 .. c0+nt-1 of the expert (token index of
// position j held by lane j in `tok`) for the wave's groups g_i = gbase + 4i
// (clamped to glast) into xs[j][i][pair] (bf16 pairs).  16-byte pieces: piece q
// covers token q / (GPW*PC), group (q / PC) % GPW, pairs 4*(q % PC) .. +3.
template <int BITS, int GPW, int XT>
struct XStage {
  using C = UnitCodec<BITS>;
  static constexpr int PC = C::G / 8;                    // 16-byte pieces per group
  static constexpr int NQ = XT * GPW * PC;               // pieces of a full chunk
  static constexpr int IT = (NQ + 63) / 64;              // pieces per lane
  u32x4 v[IT];
  __device__ __forceinline__ void load(const uint16_t* x, int H, int tok, int c0, int nt,
                                       int gbase, int glast, int lane) {
    typedef const u32x4 __attribute__((address_space(1)))* g4;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = min(it * 64 + lane, NQ - 1);
      const int j = q / (GPW * PC), i = (q / PC) % GPW, pc = q % PC;
      const int tj = __shfl(tok, c0 + min(j, nt - 1));
      const int g = min(gbase + kGUWaves * i, glast);
      v[it] = *(g4)(as_global(x + (int64_t)tj * H + g * C::G + 8 * pc));
    }
  }
  __device__ __forceinline__ void store(uint32_t* xs, int lane) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = it * 64 + lane;
      if (q < NQ) *reinterpret_cast<u32x4*>(xs + 4 * q) = v[it];
    }
  }
};

template <int BITS, int GPW, int XT>
__global__ __launch_bounds__(256, 2) void k_gateup(
    const moe_expert_ref* __restrict__ table, int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, int K, const uint16_t* __restrict__ x, int H, int I,
    int P, int KP, int scale_f16, float* __restrict__ gu) {
  using C = UnitCodec<BITS>;
  using XS = XStage<BITS, GPW, XT>;
  constexpr int XW = XT * GPW * C::PAIRS;  // bf16 pairs per wave
  __shared__ float red[kGUWaves][kTokPerPass][64];
  __shared__ __align__(16) uint32_t xs_all[kGUWaves * XW];
  const int ng = H / C::G;

  const Active act = find_active(offsets, table, E, blockIdx.x);
  if (act.e < 0) return;
  const int seg0 = __builtin_amdgcn_readfirstlane(act.seg0);
  const int n_e = __builtin_amdgcn_readfirstlane(act.n);
  const int strip = blockIdx.y, m = blockIdx.z / KP, kp = blockIdx.z % KP;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const MatGeom gm{I, H, BITS, C::G};
  const gbytes_t mat = as_global(m ? act.ptr[1] : act.ptr[0]);
  const gu16_t msc = (gu16_t)(mat + gm.scales_off());
  const int row = strip * 64 + lane;
  const int gpb = (ng + KP - 1) / KP, g0 = kp * gpb, g1 = min(ng, g0 + gpb);
  uint32_t* xs = xs_all + wv * XW;

  // token of each of the expert's positions (lane = position; n_e <= 64 at decode)
  int tok = sorted_pairs[seg0 + min(lane, n_e - 1)] / K;
  XS xst;
  int nt = min(n_e, XT);
  xst.load(x, H, tok, 0, nt, g0 + wv, g1 - 1, lane);
  asm volatile("" ::: "memory");

  // weights: all groups of this wave at once (group index clamped, not branched
  // on, so that the waits the compiler places stay exact)
  u32x4 cw[GPW][C::CHUNKS];
  uint32_t sr[GPW];  // the aligned dword holding the scale (any 16-bit handling here would wait)
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int g = min(g0 + wv + kGUWaves * i, g1 - 1);
    load_unit4<BITS>(mat, (int64_t)strip * ng + g, lane, cw[i]);
    sr[i] = load_scale_dword(msc, (int64_t)row * ng + g);
  }
  asm volatile("" ::: "memory");

  const float off = lane < C::PAIRS ? C::pair_off(lane) : 0.f;
  xst.store(xs, lane);  // the first tokens (waits for them only, not for the weights)
  for (int c0 = 0; c0 < n_e; c0 += XT) {
    if (c0 > 0) {  // next tokens; positions come 64 per lane window
      nt = min(n_e - c0, XT);
      if (c0 % 64 == 0) tok = sorted_pairs[seg0 + c0 + min(lane, n_e - c0 - 1)] / K;
      xst.load(x, H, tok, c0 % 64, nt, g0 + wv, g1 - 1, lane);
      xst.store(xs, lane);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
    for (int b0 = 0; b0 < nt; b0 += kTokPerPass) {
      const bool two = b0 + 1 < nt;
      const int j1 = two ? b0 + 1 : b0;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int g = g0 + wv + kGUWaves * i;
        if (g < g1) {
          const uint32_t* x0 = xs + (b0 * GPW + i) * C::PAIRS;
          const uint32_t* x1 = xs + (j1 * GPW + i) * C::PAIRS;
          uint32_t sraw = sr[i];
          asm volatile("" : "+v"(sraw));  // convert here, not hoisted ahead of the loads
          const float sc = scale_to_f32(scale_from_dword(sraw, (int64_t)row * ng + g), scale_f16);
          // offset sums of the two tokens' activations over the group
          const uint32_t p0 = lane < C::PAIRS ? x0[lane] : 0u;
          const uint32_t p1 = lane < C::PAIRS ? x1[lane] : 0u;
          const float c0s = wave_sum_uniform<BITS>(off * bf16_to_f32((uint16_t)p0) +
                                                   off * bf16_to_f32((uint16_t)(p0 >> 16)));
          uint32_t w[C::WORDS];
          float d0 = 0.f, d1 = 0.f;
          unit_words<BITS>(cw[i], w);
          if (two) {
            const float c1s = wave_sum_uniform<BITS>(off * bf16_to_f32((uint16_t)p1) +
                                                     off * bf16_to_f32((uint16_t)(p1 >> 16)));
            C::for_each_pair(w, [&](int Pp, uint32_t pr) {
              d0 = dot2_bf16(pr, x0[Pp], d0);
              d1 = dot2_bf16(pr, x1[Pp], d1);
            });
            a1 = fmaf(sc, d1 - c1s, a1);
          } else {
            C::for_each_pair(w, [&](int Pp, uint32_t pr) { d0 = dot2_bf16(pr, x0[Pp], d0); });
          }
          a0 = fmaf(sc, d0 - c0s, a0);
        }
      }
      red[wv][0][lane] = a0;
      red[wv][1][lane] = a1;
      lds_barrier();
      if (wv < (two ? 2 : 1)) {
        const int j = wv;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < kGUWaves; ++w) y += red[w][j][lane];
        gu[((int64_t)blockIdx.z * P + seg0 + c0 + b0 + j) * I + row] = y;
      }
      lds_barrier();
    }
  }
}

// Batches of one or two tokens (a single pass): the activations take the scalar
// path instead (s_load into SGPRs, the second operand of v_dot2_f32_bf16), which
// keeps the kernel at three waves per SIMD so the whole weight stream of a
// decode step is in flight at once; the offset sums come from vector loads that
// are requested before the weights.
template <int BITS, int GPW>
__global__ __launch_bounds__(256, 2) void k_gateup_smem(
    const moe_expert_ref* __restrict__ table, int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, int K,
    const uint16_t* __restrict__ x,  // read-only: dot operands through scalar loads
    const uint16_t* x_vec,           // the same activations; not restrict, so that its vector
                                     // loads stay ahead of the weight loads
    int H, int I,
    int P, int KP, int scale_f16, float* __restrict__ gu) {
  using C = UnitCodec<BITS>;
  __shared__ float red[kGUWaves][kTokPerPass][64];
  const int ng = H / C::G;

  const Active act = find_active(offsets, table, E, blockIdx.x);
  if (act.e < 0) return;
  const int seg0 = __builtin_amdgcn_readfirstlane(act.seg0);
  const int n_e = __builtin_amdgcn_readfirstlane(act.n);
  const int strip = blockIdx.y, m = blockIdx.z / KP, kp = blockIdx.z % KP;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const MatGeom gm{I, H, BITS, C::G};
  const gbytes_t mat = as_global(m ? act.ptr[1] : act.ptr[0]);
  const gu16_t msc = (gu16_t)(mat + gm.scales_off());
  const int row = strip * 64 + lane;
  const int gpb = (ng + KP - 1) / KP, g0 = kp * gpb, g1 = min(ng, g0 + gpb);
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  const uint32_t* xv32 = reinterpret_cast<const uint32_t*>(x_vec);

  // activation pairs of this wave's groups for the offset sums (lane = pair),
  // requested before the weights so that their waits never wait for the weights
  auto load_xo = [&](int t, uint32_t (&xo)[GPW]) {
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = min(g0 + wv + kGUWaves * i, g1 - 1);
      const int pl = lane < C::PAIRS ? lane : 0;
      xo[i] = xv32[((int64_t)t * H + g * C::G) / 2 + pl];
    }
  };
  int t0 = sorted_pairs[seg0] / K;
  int t1 = n_e > 1 ? sorted_pairs[seg0 + 1] / K : t0;
  uint32_t xo0[GPW], xo1[GPW];
  load_xo(t0, xo0);
  load_xo(t1, xo1);
  asm volatile("" ::: "memory");

  // weights: all groups of this wave at once (group index clamped, not branched
  // on, so that the waits the compiler places stay exact)
  u32x4 cw[GPW][C::CHUNKS];
  uint32_t sr[GPW];  // the aligned dword holding the scale (any 16-bit handling here would wait)
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int g = min(g0 + wv + kGUWaves * i, g1 - 1);
    load_unit4<BITS>(mat, (int64_t)strip * ng + g, lane, cw[i]);
    sr[i] = load_scale_dword(msc, (int64_t)row * ng + g);
  }
  asm volatile("" ::: "memory");

  for (int b0 = 0; b0 < n_e; b0 += kTokPerPass) {
    const bool two = b0 + 1 < n_e;
    if (b0 > 0) {
      t0 = sorted_pairs[seg0 + b0] / K;
      t1 = two ? sorted_pairs[seg0 + b0 + 1] / K : t0;
      load_xo(t0, xo0);
      load_xo(t1, xo1);
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = g0 + wv + kGUWaves * i;
      if (g < g1) {
        const uint32_t* x0 = x32 + ((int64_t)t0 * H + g * C::G) / 2;
        const uint32_t* x1 = x32 + ((int64_t)t1 * H + g * C::G) / 2;
        uint32_t sraw = sr[i];
        asm volatile("" : "+v"(sraw));  // convert here, not hoisted ahead of the loads
        const float sc = scale_to_f32(scale_from_dword(sraw, (int64_t)row * ng + g), scale_f16);
        uint32_t w[C::WORDS];
        float d0 = 0.f, d1 = 0.f;
        unit_words<BITS>(cw[i], w);
        if (two) {
          C::for_each_pair(w, [&](int Pp, uint32_t pr) {
            d0 = dot2_bf16(pr, x0[Pp], d0);
            d1 = dot2_bf16(pr, x1[Pp], d1);
          });
          a1 = fmaf(sc, d1, a1);
        } else {
          C::for_each_pair(w, [&](int Pp, uint32_t pr) { d0 = dot2_bf16(pr, x0[Pp], d0); });
        }
        a0 = fmaf(sc, d0, a0);
      }
    }
    // subtract sum_g s_g * (offset sum of group g)
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = g0 + wv + kGUWaves * i;
      if (g < g1) {
        uint32_t sraw = sr[i];
        asm volatile("" : "+v"(sraw));
        const float sc = scale_to_f32(scale_from_dword(sraw, (int64_t)row * ng + g), scale_f16);
        const float off = lane < C::PAIRS ? C::pair_off(lane) : 0.f;
        const float c0 = wave_sum_uniform<BITS>(
            off * bf16_to_f32((uint16_t)xo0[i]) + off * bf16_to_f32((uint16_t)(xo0[i] >> 16)));
        a0 = fmaf(-sc, c0, a0);
        if (two) {
          const float c1 = wave_sum_uniform<BITS>(
              off * bf16_to_f32((uint16_t)xo1[i]) + off * bf16_to_f32((uint16_t)(xo1[i] >> 16)));
          a1 = fmaf(-sc, c1, a1);
        }
      }
    }
    red[wv][0][lane] = a0;
    red[wv][1][lane] = a1;
    lds_barrier();
    if (wv < (two ? 2 : 1)) {
      const int j = wv;
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < kGUWaves; ++w) y += red[w][j][lane];
      gu[((int64_t)blockIdx.z * P + seg0 + b0 + j) * I + row] = y;
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------- SwiGLU
// h of every grouped pair position: h = silu(sum_q g_q) * (sum_q u_q), parts
// added in kp order, kept as bf16 hi + bf16 remainder (h to ~2^-16 relative):
// hh[pos][k], hl[pos][k].  One block per position; positions past the grouped
// pairs (ids left out) are skipped.
__global__ __launch_bounds__(256) void k_swiglu(const float* __restrict__ gu,
                                                const int32_t* __restrict__ offsets, int E, int P,
                                                int I, int KP, uint16_t* __restrict__ hh,
                                                uint16_t* __restrict__ hl) {
  const int pos = blockIdx.x;
  if (pos >= offsets[E]) return;
  const int I4 = I / 4;
  const float4* g4 = reinterpret_cast<const float4*>(gu);
  for (int k4 = threadIdx.x; k4 < I4; k4 += 256) {
    float4 pg[kMaxKParts], pu[kMaxKParts];
#pragma unroll
    for (int q = 0; q < kMaxKParts; ++q) {
      const int qq = min(q, KP - 1);
      pg[q] = g4[((int64_t)qq * P + pos) * I4 + k4];
      pu[q] = g4[((int64_t)(KP + qq) * P + pos) * I4 + k4];
    }
    float4 g = pg[0], u = pu[0];
#pragma unroll
    for (int q = 1; q < kMaxKParts; ++q)
      if (q < KP) {
        g.x += pg[q].x; g.y += pg[q].y; g.z += pg[q].z; g.w += pg[q].w;
        u.x += pu[q].x; u.y += pu[q].y; u.z += pu[q].z; u.w += pu[q].w;
      }
    const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float h = gv[e] * __builtin_amdgcn_rcpf(1.f + __expf(-gv[e])) * uv[e];
      hi[e] = f32_to_bf16_rne(h);
      lo[e] = f32_to_bf16_rne(h - bf16_to_f32(hi[e]));
    }
    const int64_t o = (int64_t)pos * I + 4 * k4;
    *reinterpret_cast<uint2*>(hh + o) = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
    *reinterpret_cast<uint2*>(hl + o) = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
  }
}

// ---------------------------------------------------------------- down
// Block (a, strip): rows [64*strip, +64) of the down matrix of the a-th active
// expert; 4 waves take groups g = wave + 4*i, i < GPW.  The same schedule as the
// gate/up kernel: each wave requests h (hi and lo rows) of up to XT of the
// expert's positions for its groups into its own LDS region, then its weights;
// the token passes run from LDS with two dot products per code pair (hi, lo).
// y goes to row p = t*K + k of pair_out.
constexpr int kDNWaves = 4;

template <int BITS, int GPW, int XT>
struct HStage {
  using C = UnitCodec<BITS>;
  static constexpr int PC = C::G / 8;             // 16-byte pieces per group row
  static constexpr int NQ = XT * GPW * 2 * PC;    // pieces of a full chunk (hi and lo)
  static constexpr int IT = (NQ + 63) / 64;
  u32x4 v[IT];
  __device__ __forceinline__ void load(const uint16_t* hh, const uint16_t* hl, int I, int pos0,
                                       int nt, int gbase, int glast, int lane) {
    typedef const u32x4 __attribute__((address_space(1)))* g4;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = min(it * 64 + lane, NQ - 1);
      const int j = q / (GPW * 2 * PC), i = (q / (2 * PC)) % GPW, sel = (q / PC) % 2, pc = q % PC;
      const int g = min(gbase + kDNWaves * i, glast);
      const uint16_t* src = (sel ? hl : hh) + (int64_t)(pos0 + min(j, nt - 1)) * I + g * C::G + 8 * pc;
      v[it] = *(g4)(as_global(src));
    }
  }
  __device__ __forceinline__ void store(uint32_t* xs, int lane) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = it * 64 + lane;
      if (q < NQ) *reinterpret_cast<u32x4*>(xs + 4 * q) = v[it];
    }
  }
};

template <int BITS, int GPW, int XT>
__global__ __launch_bounds__(256, 2) void k_down(
    const moe_expert_ref* __restrict__ table, int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, int H, int I, int scale_f16,
    const uint16_t* __restrict__ hh, const uint16_t* __restrict__ hl, float* __restrict__ pair_out) {
  using C = UnitCodec<BITS>;
  using HS = HStage<BITS, GPW, XT>;
  constexpr int XW = XT * GPW * 2 * C::PAIRS;  // uint32 per wave: [token][group][hi|lo][pair]
  __shared__ float red[kDNWaves][kTokPerPass][64];
  __shared__ __align__(16) uint32_t xs_all[kDNWaves * XW];
  const int ng = I / C::G;

  const Active act = find_active(offsets, table, E, blockIdx.x);
  if (act.e < 0) return;
  const int seg0 = __builtin_amdgcn_readfirstlane(act.seg0);
  const int n_e = __builtin_amdgcn_readfirstlane(act.n);
  const int strip = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const MatGeom gm{H, I, BITS, C::G};
  const gbytes_t down = as_global(act.ptr[2]);
  const gu16_t dsc = (gu16_t)(down + gm.scales_off());
  const int row = strip * 64 + lane;
  uint32_t* xs = xs_all + wv * XW;

  // pair ids of the expert's first 64 positions (lane = position), then h of the
  // first positions, all ahead of the weights
  int pids = sorted_pairs[seg0 + min(lane, n_e - 1)];
  HS hst;
  int nt = min(n_e, XT);
  hst.load(hh, hl, I, seg0, nt, wv, ng - 1, lane);
  asm volatile("" ::: "memory");

  u32x4 cw[GPW][C::CHUNKS];
  uint32_t sr[GPW];  // the aligned dword holding the scale (any 16-bit handling here would wait)
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int g = min(wv + kDNWaves * i, ng - 1);
    load_unit4<BITS>(down, (int64_t)strip * ng + g, lane, cw[i]);
    sr[i] = load_scale_dword(dsc, (int64_t)row * ng + g);
  }
  asm volatile("" ::: "memory");

  const float off = lane < C::PAIRS ? C::pair_off(lane) : 0.f;
  auto osum = [&](const uint32_t* hhp, const uint32_t* hlp) {
    const uint32_t a = lane < C::PAIRS ? hhp[lane] : 0u, b = lane < C::PAIRS ? hlp[lane] : 0u;
    return wave_sum_uniform<BITS>(off * ((bf16_to_f32((uint16_t)a) + bf16_to_f32((uint16_t)(a >> 16))) +
                                         (bf16_to_f32((uint16_t)b) + bf16_to_f32((uint16_t)(b >> 16)))));
  };
  hst.store(xs, lane);
  for (int c0 = 0; c0 < n_e; c0 += XT) {
    if (c0 > 0) {
      nt = min(n_e - c0, XT);
      hst.load(hh, hl, I, seg0 + c0, nt, wv, ng - 1, lane);
      hst.store(xs, lane);
      if (c0 % 64 == 0) pids = sorted_pairs[seg0 + c0 + min(lane, n_e - c0 - 1)];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
    for (int jp = 0; jp < nt; jp += kTokPerPass) {
      const bool two = jp + 1 < nt;
      const int j1 = two ? jp + 1 : jp;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int g = wv + kDNWaves * i;
        if (g < ng) {
          const uint32_t* hh0 = xs + ((jp * GPW + i) * 2 + 0) * C::PAIRS;
          const uint32_t* hl0 = xs + ((jp * GPW + i) * 2 + 1) * C::PAIRS;
          const uint32_t* hh1 = xs + ((j1 * GPW + i) * 2 + 0) * C::PAIRS;
          const uint32_t* hl1 = xs + ((j1 * GPW + i) * 2 + 1) * C::PAIRS;
          uint32_t wd[C::WORDS];
          unit_words<BITS>(cw[i], wd);
          uint32_t sraw = sr[i];
          asm volatile("" : "+v"(sraw));
          const float sc = scale_to_f32(scale_from_dword(sraw, (int64_t)row * ng + g), scale_f16);
          const float k0 = osum(hh0, hl0);
          float d0 = 0.f, d1 = 0.f;
          if (two) {
            const float k1 = osum(hh1, hl1);
            C::for_each_pair(wd, [&](int Pp, uint32_t pr) {
              d0 = dot2_bf16(pr, hl0[Pp], dot2_bf16(pr, hh0[Pp], d0));
              d1 = dot2_bf16(pr, hl1[Pp], dot2_bf16(pr, hh1[Pp], d1));
            });
            a1 = fmaf(sc, d1 - k1, a1);
          } else {
            C::for_each_pair(wd, [&](int Pp, uint32_t pr) {
              d0 = dot2_bf16(pr, hl0[Pp], dot2_bf16(pr, hh0[Pp], d0));
            });
          }
          a0 = fmaf(sc, d0 - k0, a0);
        }
      }
      red[wv][0][lane] = a0;
      red[wv][1][lane] = a1;
      lds_barrier();
      if (wv < (two ? 2 : 1)) {
        const int j = wv;
        float y = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDNWaves; ++ww) y += red[ww][j][lane];
        const int idx = (c0 + jp + j) % 64;  // wave-uniform
        const int p = __builtin_amdgcn_readlane(pids, idx);
        pair_out[(int64_t)p * H + row] = y;
      }
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------- combine
// out[t][n] = sum_k w[t][k] * pair_out[t*K + k][n] (k ascending; pairs whose id is
// outside [0, E) were left out of the grouping and are skipped) + shared[t][n].
// All KM rows are requested at once (k >= K repeats row K-1 and is dropped), so
// the combine costs one memory round trip.
template <int KM>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ pair_out,
                                                 const int32_t* __restrict__ ids,
                                                 const float* __restrict__ w, int K, int E, int H,
                                                 const float* __restrict__ shared,
                                                 float* __restrict__ out) {
  const int t = blockIdx.y;
  const int n = min((int)(blockIdx.x * 256 + threadIdx.x), H - 1);
  float y[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) y[k] = pair_out[((int64_t)t * K + min(k, K - 1)) * H + n];
  const float sh = shared ? shared[(int64_t)t * H + n] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int id = ids[t * K + min(k, K - 1)];
    if (k < K && id >= 0 && id < E) acc = fmaf(w[t * K + min(k, K - 1)], y[k], acc);
  }
  if (shared) acc += sh;
  if (blockIdx.x * 256 + threadIdx.x < H) out[(int64_t)t * H + n] = acc;
}

// ---------------------------------------------------------------- shared expert
// Row-major bf16 weights.  Block = 8 rows x 32 lanes per row (each lane reads 8
// consecutive bf16 per step, a half-wave covers 256 of a row); fp32 FMAs.
constexpr int kShRows = 8;
constexpr int kNT = 8;  // tokens per pass of the shared-expert kernels

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
  float* gu = reinterpret_cast<float*>(f.ws + L.gu);
  float* pair_out = f.pair_out ? f.pair_out : reinterpret_cast<float*>(f.ws + L.pair_out);
  float* sh_h = reinterpret_cast<float*>(f.ws + L.sh_h);
  float* sh_out = reinterpret_cast<float*>(f.ws + L.sh_out);
  if (prefill_eligible(c, T)) {
    const hipError_t err = launch_prefill(f, L, pair_out, s);
    if (err != hipSuccess) return err;
  } else {
    const int maxU = min(E, T * K);
    // gate/up: reduction dim split over KP blocks of at most 4 waves x 5 groups
    const int ngh = H / C::G;
    const int KP = (ngh + 5 * kGUWaves - 1) / (5 * kGUWaves);  // <= kMaxKParts for H/G <= 64
    const int gpw_gu = ((ngh + KP - 1) / KP + kGUWaves - 1) / kGUWaves;
    const int gpw_dn = (I / C::G + kDNWaves - 1) / kDNWaves;
  #define MOE_GU(N)                                                                               \
    case N:                                                                                       \
      if (T <= 2) {                                                                               \
        MOE_LAUNCH(KID_GATEUP, (k_gateup_smem<BITS, N>), dim3(maxU, I / 64, 2 * KP),              \
                   dim3(64 * kGUWaves), 0, s, f.table, E, f.offsets, f.sorted_pairs, K, f.x, f.x, \
                   H, I, T * K, KP, c.scale_f16, gu);                                             \
      } else {                                                                                    \
        MOE_LAUNCH(KID_GATEUP, (k_gateup<BITS, N, 8>), dim3(maxU, I / 64, 2 * KP),                \
                   dim3(64 * kGUWaves), 0, s, f.table, E, f.offsets, f.sorted_pairs, K, f.x, H,   \
                   I, T * K, KP, c.scale_f16, gu);                                                \
      }                                                                                           \
      break;
    switch (gpw_gu) {
      MOE_GU(1) MOE_GU(2) MOE_GU(3) MOE_GU(4) MOE_GU(5)
      default: return hipErrorInvalidValue;
    }
  #undef MOE_GU
    float* hbuf = reinterpret_cast<float*>(f.ws + L.hdec);
    uint16_t* hh = reinterpret_cast<uint16_t*>(hbuf);
    uint16_t* hl = hh + (int64_t)T * K * I;
    MOE_LAUNCH(KID_SWIGLU, k_swiglu, dim3(T * K), dim3(256), 0, s, gu, f.offsets, E, T * K, I, KP,
               hh, hl);
  #define MOE_DN(N)                                                                               \
    case N:                                                                                       \
      if (T <= 2) {                                                                               \
        MOE_LAUNCH(KID_DOWN, (k_down<BITS, N, 2>), dim3(maxU, H / 64), dim3(64 * kDNWaves), 0, s, \
                   f.table, E, f.offsets, f.sorted_pairs, H, I, c.scale_f16, hh, hl, pair_out);   \
      } else {                                                                                    \
        MOE_LAUNCH(KID_DOWN, (k_down<BITS, N, 8>), dim3(maxU, H / 64), dim3(64 * kDNWaves), 0, s, \
                   f.table, E, f.offsets, f.sorted_pairs, H, I, c.scale_f16, hh, hl, pair_out);   \
      }                                                                                           \
      break;
    switch (gpw_dn) {
      MOE_DN(1) MOE_DN(2) MOE_DN(3) MOE_DN(4) MOE_DN(5) MOE_DN(6) MOE_DN(7) MOE_DN(8)
      default: return hipErrorInvalidValue;
    }
  #undef MOE_DN
  }
  const bool has_shared = c.shared_inter > 0 && f.sg && f.su && f.sd;
  if (has_shared) {
    const int Is = c.shared_inter;
    MOE_LAUNCH(KID_SH_GATEUP, k_shared_gateup, dim3(Is / kShRows), dim3(256), 0, s,
               reinterpret_cast<const uint16_t*>(f.sg), reinterpret_cast<const uint16_t*>(f.su),
               f.x, T, H, Is, sh_h);
    MOE_LAUNCH(KID_SH_DOWN, k_shared_down, dim3(H / kShRows), dim3(256), 0, s,
               reinterpret_cast<const uint16_t*>(f.sd), sh_h, T, H, Is, sh_out);
  }
  if (K <= 8) {
    MOE_LAUNCH(KID_COMBINE, k_combine<8>, dim3((H + 255) / 256, T), dim3(256), 0, s, pair_out,
               f.ids, f.w, K, E, H, has_shared ? sh_out : nullptr, f.out);
  } else {
    MOE_LAUNCH(KID_COMBINE, k_combine<16>, dim3((H + 255) / 256, T), dim3(256), 0, s, pair_out,
               f.ids, f.w, K, E, H, has_shared ? sh_out : nullptr, f.out);
  }
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
