// decode_impl.h -- the routed experts of a decode batch (at most 64 tokens) as
// persistent, wave-level GEMVs over packed low-bit weights.  The kernels and the
// per-codec launcher are templates; decode.hip, decode_q2.hip and decode_q4.hip
// instantiate them, one codec family per source, so the builds run in parallel.
//
// Each picked expert runs gate, up and down matrices reached through the layer's
// pointer table (page "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX PRO 6000 - GPU expert
// cache, host-RAM streaming", field config.expert_cache.mechanism); a decode step
// reads every picked expert's bytes once, so HBM bandwidth bounds it.
//
// Work decomposition, three or more tokens.  A plan kernel lists the active
// experts (those owning at least one pair) with their pair segment and blob
// pointers.  The GEMV kernels then run a fixed grid of waves that take work items
// in a zig-zag order: an item is (active expert, 64-row strip, matrix, chunk of
// GPW reduction groups).  A wave requests the item's codes and scales first (one
// 16-byte load per chunk of a 64-row tile: 1,024 contiguous bytes per wave), then
// forms the partial products of its 64 rows for the expert's tokens and writes
// them to a partial buffer, one slice per chunk.  The codec's offset sums of each
// activation row and group come precomputed (the plan launch for gate/up, the
// SwiGLU pass for down).  The gate/up GEMV takes the activations through scalar
// loads into v_dot2_f32_bf16 (one load of 8 pairs serves all 64 lanes; a
// broadcast through LDS or a vector load would move every byte 64 times); the
// down GEMV stages its positions' h rows in the wave's LDS region and runs on the
// matrix cores.  No item waits on another: there are no block barriers and no
// cross-wave reductions, and a wave that finishes an item starts the next one at
// once, so the weight stream stays in flight.  The slices are added in chunk
// order by the SwiGLU pass (gate/up) and by the combine (down): results are
// deterministic.
//
// One or two tokens.  Block-level kernels without the plan launch: each gate/up
// block finds its expert itself (one round trip for the offsets and the table)
// and one block per expert hands that entry to the down kernel; gate/up splits
// the reduction over the block's waves and two blocks, and the down kernel forms
// h from the gate/up parts while staging it and adds its weighted outputs into
// the combine's integer words, whose last add writes the combined output.  Both
// run their products on the matrix cores.
//
// Arithmetic (as in the unit codec): codes are expanded two at a time into bf16
// (B + c) and multiplied with bf16 activations in fp32 (v_dot2_f32_bf16, or
// 4 x 4 x 4 bf16 matrix-core blocks); the per-group constant sum_k (B_k + z) x_k is
// subtracted, then the group scale applied.  The down matrix takes h as bf16 hi +
// bf16 remainder (two products per code pair, or two rows of the matrix-core
// operand).
#pragma once
#include <algorithm>

#include "common.h"

namespace moe {

MOE_TRACE_DECL

typedef uint32_t u32x4d __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));


// ---------------------------------------------------------------- plan
// act_hdr[0] = U, the number of experts owning at least one pair; act[a] for
// a < U lists them by descending pair count (count clamped at 63), ties by
// ascending expert id, so that the GEMVs' zig-zag item order gives every wave a
// similar mix of heavy and light items.  The order only schedules work: where
// an item's results land depends on the item alone.
constexpr int kPlanKeys = 65;  // 0..63: 63 - min(n, 63) for active experts; 64: inactive

// Blocks 1.. of the same launch form, for every token t and reduction group g of
// the gate/up matrices, the codec's offset sum osx[t][g] = sum_P off_P (x_2P +
// x_2P+1) (one wave per (t, g), lane = pair, the fixed-order wave sum), which the
// gate/up GEMV subtracts per group instead of reducing it in every work item;
// block 0 checks the routing (thread i: expert i and grouped position i; P, E <=
// 1024) and builds the list, or, for inconsistent routing, an empty one.
template <int CODEC>
__global__ __launch_bounds__(1024) void k_plan_decode(const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ sorted_pairs,
                                                      int P, int32_t* __restrict__ ctr,
                                                      const moe_expert_ref* __restrict__ table,
                                                      int E, int32_t* __restrict__ act_hdr,
                                                      ActEntry* __restrict__ act,
                                                      const uint16_t* __restrict__ x, int T, int H,
                                                      float* __restrict__ osx) {
  using C = UnitCodec<CODEC>;
  __shared__ int cntw[16][kPlanKeys];  // per wave and key: experts (then the exclusive prefix over waves)
  __shared__ int base[kPlanKeys];      // exclusive prefix over keys of the totals
  __shared__ int s_off[1025];
  __shared__ int s_id[1024];
  const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
  if (blockIdx.x > 0) {  // blocks 1.. : one (t, g) item per wave
    const int ngx = H / C::G;
    const int it = (blockIdx.x - 1) * 16 + wv;
    if (it < T * ngx) {
      const int t = it / ngx, g = it - t * ngx;
      const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
      const float off = lane < C::PAIRS ? C::pair_off(lane) : 0.f;
      const uint32_t pr = lane < C::PAIRS ? x32[((int64_t)t * H + g * C::G) / 2 + lane] : 0u;
      const float v = wave_sum_uniform<CODEC>(off * (bf16_to_f32((uint16_t)pr) +
                                                    bf16_to_f32((uint16_t)(pr >> 16))));
      if (lane == 0) osx[it] = v;
    }
    return;
  }
  for (int i = e; i < 16 * kPlanKeys; i += 1024) (&cntw[0][0])[i] = 0;
  // expert e's table entry with its offsets (one round trip; used if it is active)
  moe_expert_ref r{nullptr, nullptr, nullptr};
  if (e < E) r = table[e];
  const int lo = e < E ? offsets[e] : 0;
  const int hi = e < E ? offsets[e + 1] : 0;
  // the routing check (as routing_ok_wave, one thread per expert and position)
  const int idv = e < P ? ids[e] : -1;
  const int sp_i = e < P ? sorted_pairs[e] : 0;
  const int sp_prev = (e > 0 && e < P) ? sorted_pairs[e - 1] : -1;
  if (e < E) s_off[e] = lo;
  if (e == E - 1) s_off[E] = hi;
  if (e < P) s_id[e] = idv;
  const int nvalid = __syncthreads_count(idv >= 0 && idv < E);
  const int oE = s_off[E];
  bool bad = (e < E && hi < lo) || (e == 0 && (lo != 0 || oE != nvalid));
  if (e < oE && oE <= P) {
    const bool pin = sp_i >= 0 && sp_i < P;
    const int ep = pin ? s_id[sp_i] : -1;
    const bool ein = ep >= 0 && ep < E;
    const int elo = ein ? s_off[ep] : 0, ehi = ein ? s_off[ep + 1] : 0;
    bad |= !ein || e < elo || e >= ehi || (e > elo && sp_prev >= sp_i);
  }
  if (__syncthreads_or(bad)) {  // nothing runs, the outputs are left untouched
    if (e == 0) {
      act_hdr[0] = 0;
      record_routing(ctr, false);
    }
    return;
  }
  if (e == 0) record_routing(ctr, true);
  const int n = hi - lo;
  const int key = n > 0 ? 63 - min(n, 63) : 64;
  // lanes of this wave with the same key (one ballot per key bit)
  uint64_t eq = __ballot(1);
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const uint64_t bal = __ballot((key >> b) & 1);
    eq &= ((key >> b) & 1) ? bal : ~bal;
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  const int below = __popcll(eq & lt);
  __syncthreads();
  if (below == 0) cntw[wv][key] = __popcll(eq);
  __syncthreads();
  if (e < kPlanKeys) {  // thread k: prefix of key k over the waves, and its total
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int c = cntw[w][e];
      cntw[w][e] = run;
      run += c;
    }
    base[e] = run;
  }
  __syncthreads();
  if (e == 0) {  // exclusive prefix over the keys (65 entries)
    int run = 0;
    for (int k = 0; k < kPlanKeys; ++k) {
      const int c = base[k];
      base[k] = run;
      run += c;
    }
  }
  __syncthreads();
  if (n > 0) {
    const int a = base[key] + cntw[wv][key] + below;
    ActEntry ent;
    ent.e = e;
    ent.seg0 = lo;
    ent.n = n;
    ent.pad = 0;
    ent.ptr[0] = r.gate;
    ent.ptr[1] = r.up;
    ent.ptr[2] = r.down;
    act[a] = ent;
  }
  if (e == 0) act_hdr[0] = base[64];
}

// ---------------------------------------------------------------- GEMV, dot products
// (the gate/up GEMV; the down GEMV is k_gemv_mma below: on the matrix cores the
// down products, two per code pair and position here, cost less, while for
// gate/up the staging of the activations the matrix cores need costs as much as
// it saves on this kernel's batches of mostly one or two tokens per expert)
// MODE 0: gate and up (R = I rows, reduction D = H); activations are the bf16
// token rows xa[T][H]; out[(m*NCH + ch)*P + pos][row] (pos = sorted position).
// MODE 1: down (R = H, D = I); activations are h hi rows xa[P][I] and lo rows
// xb[P][I] by sorted position; out[ch*P + p][row] (p = pair id t*K + k).
template <int CODEC, int GPW, int XT, int MODE, int WPS>
__global__ __launch_bounds__(256, WPS) void k_gemv(
    const int32_t* __restrict__ act_hdr, const ActEntry* __restrict__ act,
    const int32_t* __restrict__ sorted_pairs, int K, const uint16_t* __restrict__ xa,
    const uint16_t* __restrict__ xb, int R, int D, int P, int scale_f16, float* __restrict__ out,
    const float* __restrict__ osx) {
  using C = UnitCodec<CODEC>;
  constexpr int NM = MODE == 0 ? 2 : 1;        // matrices per expert
  constexpr int NS = MODE == 0 ? 1 : 2;        // activation rows per token (x; or h hi, lo)
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ng = D / C::G, NCH = (ng + GPW - 1) / GPW, nstrips = R / 64;
  const int per_a = nstrips * NM * NCH;
  const int total = act_hdr[0] * per_a;
  const int nw = gridDim.x * 4;
  const MatGeom gm{R, D, C::BITS, C::G};

  // zig-zag over the waves: round r takes items r*nw .. r*nw + nw-1, forwards
  // on even rounds and backwards on odd ones
  const int w_id = blockIdx.x * 4 + wv;
  for (int r = 0; r * nw < total; ++r) {
    const int item = r * nw + ((r & 1) ? nw - 1 - w_id : w_id);
    if (item >= total) continue;
    const int a = item / per_a, r0 = item - a * per_a;
    const int strip = r0 / (NM * NCH), r1 = r0 - strip * (NM * NCH);
    const int m = r1 / NCH, ch = r1 - m * NCH;
    const int seg0 = act[a].seg0, n_e = act[a].n;
    const gbytes_t mat = as_global(act[a].ptr[MODE == 0 ? m : 2]);
    const gu16_t msc = (gu16_t)(mat + gm.scales_off());
    const int row = strip * 64 + lane;
    const int g0 = ch * GPW, g1 = min(ng, g0 + GPW);
#ifdef MOE_TRACE
    // sampled waves (every 16th), first 8 rounds: item start, weights in, item done
    const bool trs = (w_id & 15) == 0 && r < 8;
    const int tslot = (MODE == 0 ? 8192 : 20480) + ((w_id >> 4) * 8 + r) * 4;
    if (trs) {
      MOE_TRW(tslot);
      if ((threadIdx.x & 63) == 0) g_moe_trace[tslot + 3] = (unsigned long long)n_e;
    }
#endif

    // the item's codes and scales first: they need only the expert's address
    // (group index clamped, not branched on)
    u32x4 cw[GPW][C::CHUNKS];
    uint32_t sr[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = min(g0 + i, g1 - 1);
      load_unit4<CODEC>(mat, (int64_t)strip * ng + g, lane, cw[i]);
      sr[i] = load_scale_dword(msc, scale_idx((int64_t)strip * ng + g, lane));
    }
    asm volatile("" ::: "memory");
#ifdef MOE_TRACE
    if (trs) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the weights are in (trace builds only)
      MOE_TRW(tslot + 1);
    }
#endif
    for (int c0 = 0; c0 < n_e; c0 += XT) {
      const int nt = min(n_e - c0, XT);
      // pair ids of positions c0 .. c0+XT-1 (clamped to the expert's last):
      // uniform, so scalar loads, which the activation loads need not wait for
      // behind the weights
      int pid[XT];
      if constexpr (MODE == 1) {
#pragma unroll
        for (int j = 0; j < XT; ++j) {
          pid[j] = sorted_pairs[seg0 + c0 + min(j, nt - 1)];
          asm volatile("" : "+s"(pid[j]));  // each a scalar load of its own
        }
      }
      // the dot products read the activation rows through scalar loads; the
      // offset sums of each row and group come precomputed (osx)
      for (int jp = 0; jp < nt; jp += 2) {
        const bool two = jp + 1 < nt;
        const int j1 = two ? jp + 1 : jp;
        // the two tokens' activation rows in global memory (uniform addresses:
        // the dot products take them through scalar loads, one load per 8 or 16
        // pairs for the whole wave)
        const uint32_t *r0a, *r0b, *r1a, *r1b;
        int tk0 = 0, tk1 = 0;
        if (MODE == 0) {
          tk0 = sorted_pairs[seg0 + c0 + jp] / K;
          tk1 = sorted_pairs[seg0 + c0 + j1] / K;
          r0a = r0b = reinterpret_cast<const uint32_t*>(xa + (int64_t)tk0 * D);
          r1a = r1b = reinterpret_cast<const uint32_t*>(xa + (int64_t)tk1 * D);
        } else {
          r0a = reinterpret_cast<const uint32_t*>(xa + (int64_t)(seg0 + c0 + jp) * D);
          r0b = reinterpret_cast<const uint32_t*>(xb + (int64_t)(seg0 + c0 + jp) * D);
          r1a = reinterpret_cast<const uint32_t*>(xa + (int64_t)(seg0 + c0 + j1) * D);
          r1b = reinterpret_cast<const uint32_t*>(xb + (int64_t)(seg0 + c0 + j1) * D);
        }
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
          if (g0 + i < g1) {
            const int go = (g0 + i) * C::G / 2;
            const uint32_t *s0a = r0a + go, *s0b = r0b + go, *s1a = r1a + go, *s1b = r1b + go;
            uint32_t sraw = sr[i];
            asm volatile("" : "+v"(sraw));  // convert here, not hoisted ahead of the loads
            const float sc =
                scale_to_f32(scale_from_dword(sraw, lane), scale_f16);
            uint32_t w[C::WORDS];
            unit_words<CODEC>(cw[i], w);
            float d0 = 0.f, d1 = 0.f;
            // offset sums: per token (gate/up) or per sorted position (down) and group
            const int64_t o0 = MODE == 0 ? tk0 : seg0 + c0 + jp;
            const int64_t o1 = MODE == 0 ? tk1 : seg0 + c0 + j1;
            const float k0 = osx[o0 * ng + g0 + i];
            if (two) {
              const float k1 = osx[o1 * ng + g0 + i];
              C::for_each_pair(w, [&](int Pp, uint32_t pr) {
                if (NS == 2) {
                  d0 = dot2_bf16(pr, s0b[Pp], dot2_bf16(pr, s0a[Pp], d0));
                  d1 = dot2_bf16(pr, s1b[Pp], dot2_bf16(pr, s1a[Pp], d1));
                } else {
                  d0 = dot2_bf16(pr, s0a[Pp], d0);
                  d1 = dot2_bf16(pr, s1a[Pp], d1);
                }
              });
              a1 = fmaf(sc, d1 - k1, a1);
            } else {
              C::for_each_pair(w, [&](int Pp, uint32_t pr) {
                if (NS == 2) d0 = dot2_bf16(pr, s0b[Pp], dot2_bf16(pr, s0a[Pp], d0));
                else d0 = dot2_bf16(pr, s0a[Pp], d0);
              });
            }
            a0 = fmaf(sc, d0 - k0, a0);
          }
        }
        if (MODE == 0) {
          float* o = out + ((int64_t)(m * NCH + ch) * P + seg0 + c0 + jp) * R + row;
          o[0] = a0;
          if (two) o[R] = a1;
        } else {
          out[((int64_t)ch * P + pid[jp]) * R + row] = a0;
          if (two) out[((int64_t)ch * P + pid[jp + 1]) * R + row] = a1;
        }
      }
    }
#ifdef MOE_TRACE
    if (trs) MOE_TRW(tslot + 2);
#endif
  }
}

// ---------------------------------------------------------------- GEMV, matrix cores
// MODE 0: gate and up (R = I rows, reduction D = H); activations are the bf16
// token rows xa[T][H]; out[(m*NCH + ch)*P + pos][row] (pos = sorted position).
// MODE 1: down (R = H, D = I); activations are h hi rows xa[P][I] and lo rows
// xb[P][I] by sorted position; out[ch*P + p][row] (p = pair id t*K + k).
//
// The products run on the matrix cores: v_mfma_f32_4x4x4bf16_1k computes 16
// independent 4 x 4 x 4 blocks, lanes 4b..4b+3 forming block b.  The B operand
// is the wave's own expanded weights (lane = output row; one step = 4 reduction
// elements = two code pairs); the A operand of lane l is 4 elements of
// activation row l % 4 of a quad of rows, and the result's register i in lane l
// is output row l's dot product with row i of the quad (D[b][i][j] sits in lane
// 4b + j, register i).  A quad is four tokens (gate/up) or two positions' h hi
// and lo rows (down).  A pass takes NQ = 2 quads: both share each expanded
// weight step, so a code pair is expanded once per pass whatever the number of
// tokens.  The pass's activation rows (the item's reduction range) are staged in
// the wave's own LDS region first (16-byte pieces; no block barriers), and read
// back 8 bytes per lane per step.
template <int CODEC, int GPW, int MODE, int WPS>
__global__ __launch_bounds__(256, WPS) void k_gemv_mma(
    const int32_t* __restrict__ act_hdr, const ActEntry* __restrict__ act,
    const int32_t* __restrict__ sorted_pairs, int K, const uint16_t* __restrict__ xa,
    const uint16_t* __restrict__ xb, int R, int D, int P, int scale_f16, float* __restrict__ out,
    const float* __restrict__ osx) {
  using C = UnitCodec<CODEC>;
  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef float f4v __attribute__((ext_vector_type(4)));
  constexpr int NM = MODE == 0 ? 2 : 1;        // matrices per expert
  constexpr int NQ = 2;                        // quads per pass
  constexpr int NR = 4 * NQ;                   // staged activation rows per pass
  constexpr int XT = MODE == 0 ? NR : NR / 2;  // positions per pass
  constexpr int KC = GPW * C::G;               // reduction elements of an item
  constexpr int PC = KC / 8;                   // 16-byte pieces of a staged row
  __shared__ __align__(16) uint16_t xs_all[4][NR][KC];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint16_t (*xs)[KC] = xs_all[wv];
  const int ng = D / C::G, NCH = (ng + GPW - 1) / GPW, nstrips = R / 64;
  const int per_a = nstrips * NM * NCH;
  const int total = act_hdr[0] * per_a;
  const int nw = gridDim.x * 4;
  const MatGeom gm{R, D, C::BITS, C::G};

  // zig-zag over the waves: round r takes items r*nw .. r*nw + nw-1, forwards
  // on even rounds and backwards on odd ones
  const int w_id = blockIdx.x * 4 + wv;
  for (int r = 0; r * nw < total; ++r) {
    const int item = r * nw + ((r & 1) ? nw - 1 - w_id : w_id);
    if (item >= total) continue;
    const int a = item / per_a, r0 = item - a * per_a;
    const int strip = r0 / (NM * NCH), r1 = r0 - strip * (NM * NCH);
    const int m = r1 / NCH, ch = r1 - m * NCH;
    const int seg0 = act[a].seg0, n_e = act[a].n;
    const gbytes_t mat = as_global(act[a].ptr[MODE == 0 ? m : 2]);
    const gu16_t msc = (gu16_t)(mat + gm.scales_off());
    const int row = strip * 64 + lane;
    const int g0 = ch * GPW, g1 = min(ng, g0 + GPW);

    // the item's codes and scales first: they need only the expert's address
    // (group index clamped, not branched on)
    u32x4 cw[GPW][C::CHUNKS];
    uint32_t sr[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = min(g0 + i, g1 - 1);
      load_unit4<CODEC>(mat, (int64_t)strip * ng + g, lane, cw[i]);
      sr[i] = load_scale_dword(msc, scale_idx((int64_t)strip * ng + g, lane));
    }
    asm volatile("" ::: "memory");
    for (int c0 = 0; c0 < n_e; c0 += XT) {
      const int nt = min(n_e - c0, XT);
      // positions c0 .. c0+XT-1 (clamped to the expert's last); uniform
      int pid[XT], orow[XT];
#pragma unroll
      for (int j = 0; j < XT; ++j) {
        pid[j] = sorted_pairs[seg0 + c0 + min(j, nt - 1)];
        orow[j] = MODE == 0 ? pid[j] / K : seg0 + c0 + min(j, nt - 1);  // osx row
      }
      // stage the pass's activation rows (row slot q: gate/up token q; down:
      // position q/2, h hi for even q, lo for odd q), elements g0*G .. +KC
      // (clamped inside the row); only the rows of the nt positions: a quad's
      // other rows hold stale data, whose products land only in results that are
      // not stored
      constexpr int QP = MODE == 0 ? 4 : 2;       // positions per quad
      const int nq = (nt + QP - 1) / QP;          // quads this pass
      const int nrow = MODE == 0 ? nt : 2 * nt;   // rows staged
#pragma unroll
      for (int it = 0; it < (NR * PC + 63) / 64; ++it) {
        const int pc = it * 64 + lane;
        if (pc < nrow * PC) {
          const int q = pc / PC, col = pc - q * PC;
          const uint16_t* src;
          if (MODE == 0) {
            int tk = orow[0];
#pragma unroll
            for (int j = 1; j < XT; ++j)
              if (q == j) tk = orow[j];
            src = xa + (int64_t)tk * D;
          } else {
            const int pos = seg0 + c0 + min(q >> 1, nt - 1);
            src = ((q & 1) ? xb : xa) + (int64_t)pos * D;
          }
          const int k = min(g0 * C::G + col * 8, D - 8);
          *reinterpret_cast<u32x4*>(&xs[q][col * 8]) = *reinterpret_cast<const u32x4*>(src + k);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
      f4v acc[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) acc[q] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        if (g0 + i < g1) {
          uint32_t sraw = sr[i];
          asm volatile("" : "+v"(sraw));  // convert here, not hoisted ahead of the loads
          const float sc =
              scale_to_f32(scale_from_dword(sraw, lane), scale_f16);
          uint32_t w[C::WORDS];
          unit_words<CODEC>(cw[i], w);
          f4v d[NQ];
#pragma unroll
          for (int q = 0; q < NQ; ++q) d[q] = f4v{0.f, 0.f, 0.f, 0.f};
          uint32_t even = 0;
          C::for_each_pair(w, [&](int Pp, uint32_t pr) {
            if ((Pp & 1) == 0) {
              even = pr;
              return;
            }
            const s4v b = __builtin_bit_cast(s4v, u32x2v{even, pr});
            const int k = i * C::G + 2 * (Pp - 1);  // step of pairs Pp-1, Pp
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              if (q < nq) {  // uniform
                const s4v av = *reinterpret_cast<const s4v*>(&xs[4 * q + (lane & 3)][k]);
                d[q] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(av, b, d[q], 0, 0, 0);
              }
            }
          });
          // subtract the codec's offset sums, apply the group scale
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            if (MODE == 0) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[q][e] = fmaf(sc, d[q][e] - osx[(int64_t)orow[4 * q + e] * ng + g0 + i], acc[q][e]);
            } else {
#pragma unroll
              for (int e = 0; e < 2; ++e)
                acc[q][2 * e] = fmaf(sc, (d[q][2 * e] + d[q][2 * e + 1]) -
                                             osx[(int64_t)orow[2 * q + e] * ng + g0 + i],
                                     acc[q][2 * e]);
            }
          }
        }
      }
      // results: gate/up by sorted position, down by pair
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (MODE == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q + e < nt)
              out[((int64_t)(m * NCH + ch) * P + seg0 + c0 + 4 * q + e) * R + row] = acc[q][e];
        } else {
#pragma unroll
          for (int e = 0; e < 2; ++e)
            if (2 * q + e < nt) out[((int64_t)ch * P + pid[2 * q + e]) * R + row] = acc[q][2 * e];
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // the pass's LDS reads, before the next staging
    }
  }
}

// ---------------------------------------------------------------- one or two tokens
// Batches of one or two tokens have a single token pass per expert, and the
// latency chain of the step dominates; they keep a block-level schedule with one
// kernel launch fewer: block (a, strip, m*KP + kp) finds the a-th active expert
// itself (one round trip for the offsets and the table entries together; block
// (a, 0, 0) stores the result for the down kernel), its four waves take groups
// g0 + wave + 4*i of part kp of the reduction, and the waves' sums meet in LDS.
constexpr int kGUWaves = 4;
constexpr int kTokPerPass = 2;
#ifndef MOE_GU_AHEAD
#define MOE_GU_AHEAD 2
#endif
constexpr int kGUAhead = MOE_GU_AHEAD;  // weight groups a gate/up wave has in flight
constexpr int kMaxKParts = 4;

// ---------------------------------------------------------------- active experts
// The a-th expert (ascending logical id) that owns at least one pair, the number
// U of such experts, its segment of the grouping and its table entry.
// Wave-cooperative (every lane returns the same values); positions clamped into
// [0, P).  Each lane loads the
// offsets and the table entries of its candidate experts lane + 64*i in the same
// round trip, so the expert's weight addresses are known after one memory
// latency instead of two.  E <= 1024.
struct Active {
  int e;     // -1 if a >= U
  int U;
  int seg0;  // first sorted position of the expert's pairs
  int n;     // number of pairs
  const void* ptr[3];  // gate, up, down
  bool ok;   // CHECK: the routing is consistent (routing_ok_regs)
};

// The lookup in two halves, so that a kernel can request other data between the
// lookup's loads and their use: issue() requests the offsets and table entries
// (and with CHECK the routing check's inputs, P <= 64), resolve() finds the a-th
// active expert from them.
template <bool CHECK>
struct ActiveLookup {
  static constexpr int kSpec = 5;  // candidates per lane whose table entry is fetched up front
  int nch;
  int lo[16], hi[16];
  moe_expert_ref ref[kSpec];
  int cid, cs, csp;
  __device__ __forceinline__ void issue(const int32_t* __restrict__ offsets,
                                        const moe_expert_ref* __restrict__ table, int E, int P,
                                        const int32_t* __restrict__ ids = nullptr,
                                        const int32_t* __restrict__ sp = nullptr) {
    const int lane = threadIdx.x & 63;
    nch = (E + 63) / 64;
    cid = -1, cs = 0, csp = -1;
    if (CHECK) {
      cid = lane < P ? ids[lane] : -1;
      cs = lane < P ? sp[lane] : 0;
      csp = (lane > 0 && lane < P) ? sp[lane - 1] : -1;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nch) {  // uniform
        const int e = lane + 64 * i;
        lo[i] = (e < E) ? offsets[e] : 0;
        hi[i] = (e < E) ? offsets[e + 1] : 0;
        if (i < kSpec) ref[i] = e < E ? table[e] : moe_expert_ref{nullptr, nullptr, nullptr};
      }
    }
  }
  __device__ __forceinline__ Active resolve(const moe_expert_ref* __restrict__ table, int E,
                                            int P, int a) {
    Active r{-1, 0, 0, 0, {nullptr, nullptr, nullptr}, true};
    if (CHECK) r.ok = routing_ok_regs(lo, hi, cid, cs, csp, P, E);
    // segments clamped into [0, P]: every position read stays inside the grouping
    // buffers even when caller-supplied offsets are wrong (such a call writes no
    // output)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nch) {
        lo[i] = min(max(lo[i], 0), P);
        hi[i] = min(max(hi[i], lo[i]), P);
      }
    }
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
};

// CHECK: also check the routing (P <= 64), its loads in the same round trip
template <bool CHECK>
__device__ __forceinline__ Active find_active(const int32_t* __restrict__ offsets,
                                              const moe_expert_ref* __restrict__ table, int E,
                                              int P, int a, const int32_t* __restrict__ ids = nullptr,
                                              const int32_t* __restrict__ sp = nullptr) {
  ActiveLookup<CHECK> l;
  l.issue(offsets, table, E, P, ids, sp);
  return l.resolve(table, E, P, a);
}

// Batches of one or two tokens (a single pass).  Each wave first requests the
// slices of the tokens' activation rows that its groups reduce over (cache
// hits), then its weights, and stages the slices in its own LDS region; the
// products run on the matrix cores: v_mfma_f32_4x4x4bf16_1k with the token rows
// as A (lane l supplies row l & 3, which holds token l & 1) and the lane's two
// expanded code pairs as column l of B, one instruction per two code pairs for
// both tokens.  Three waves per SIMD keep the whole weight stream of a decode
// step in flight at once.
template <int CODEC, int GPW, bool PRE>
__global__ __launch_bounds__(256, 3) void k_gateup_smem(
    const moe_expert_ref* __restrict__ table, int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, int K, const uint16_t* __restrict__ x, int H, int I,
    int P, int KP, int scale_f16, float* __restrict__ gu, const int32_t* __restrict__ ids,
    int32_t* __restrict__ ctr0, ActEntry* __restrict__ dact) {
  using C = UnitCodec<CODEC>;
  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef float f4v __attribute__((ext_vector_type(4)));
  constexpr int PC = C::G / 8;                    // 16-byte pieces of a group's row slice
  constexpr int NPC = kTokPerPass * GPW * PC;     // pieces a wave stages
  constexpr int NIT = (NPC + 63) / 64;
  __shared__ float red[kGUWaves][kTokPerPass][64];
  __shared__ __align__(16) uint16_t xs_all[kGUWaves][kTokPerPass * GPW * C::G];
  const int ng = H / C::G;
  const int tb = 4 * (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  MOE_TR(tb);

  // block (0, 0, 0) also checks the caller's routing, with its lookup (same round
  // trip), and records the verdict for the down kernel, which writes the outputs;
  // every read here stays inside the buffers whatever the routing holds
  const bool first = (blockIdx.x | blockIdx.y | blockIdx.z) == 0;  // uniform
  Active act;
  if (PRE) {  // the routing kernel of the same call stored the entries (scalar loads)
    const ActEntry* ae = dact + blockIdx.x;
    act = Active{ae->e, ae->pad, ae->seg0, ae->n, {ae->ptr[0], ae->ptr[1], ae->ptr[2]}, true};
    if (first && threadIdx.x == 0) record_routing(ctr0, true);
  } else if (first) {
    act = find_active<true>(offsets, table, E, P, blockIdx.x, ids, sorted_pairs);
    if (threadIdx.x == 0) record_routing(ctr0, act.ok);
  } else {
    act = find_active<false>(offsets, table, E, P, blockIdx.x);
  }
  MOE_TR(tb + 1);
  // block (a, 0, 0) hands its lookup to the down kernel's blocks of expert a
  if (!PRE && (blockIdx.y | blockIdx.z) == 0 && threadIdx.x == 0) {
    ActEntry ent;
    ent.e = act.e;
    ent.seg0 = act.seg0;
    ent.n = act.n;
    ent.pad = act.U;
    ent.ptr[0] = nullptr;
    ent.ptr[1] = nullptr;
    ent.ptr[2] = act.ptr[2];
    dact[blockIdx.x] = ent;
  }
  if (act.e < 0) return;
  const int seg0 = __builtin_amdgcn_readfirstlane(act.seg0);
  const int n_e = __builtin_amdgcn_readfirstlane(act.n);
  const int strip = blockIdx.y, m = blockIdx.z / KP, kp = blockIdx.z % KP;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const MatGeom gm{I, H, C::BITS, C::G};
  const gbytes_t mat = as_global(m ? act.ptr[1] : act.ptr[0]);
  const gu16_t msc = (gu16_t)(mat + gm.scales_off());
  const int row = strip * 64 + lane;
  const int gpb = (ng + KP - 1) / KP, g0 = kp * gpb, g1 = min(ng, g0 + gpb);
  uint16_t* xs = xs_all[wv];  // [token slot][group i][G]
  const uint32_t* xs32 = reinterpret_cast<const uint32_t*>(xs);

  // weights: the first kGUAhead groups of this wave are requested up front
  // (group index clamped, not branched on, so that the waits the compiler places
  // stay exact); each later group right after the products of the group
  // kGUAhead before it, so that the requests of the whole grid complete in
  // waves and every wave's products run while its later groups still stream
  // (with every group requested at once, all of a wave's data lands near the
  // end of the stream and the products follow it).
  auto issue = [&](int i, u32x4 (&cw)[GPW][C::CHUNKS], uint32_t (&sr)[GPW]) {
    const int g = min(g0 + wv + kGUWaves * i, g1 - 1);
    load_unit4<CODEC>(mat, (int64_t)strip * ng + g, lane, cw[i]);
    sr[i] = load_scale_dword(msc, scale_idx((int64_t)strip * ng + g, lane));
  };
  // the row slices of tokens t0 (slot 0) and t1 (slot 1): piece q = (slot, group
  // i, 16-byte column), loaded ahead of the weights (vector loads complete in
  // order, so these cache hits do not queue behind the weight stream) and
  // written to LDS once they are in
  auto load_x = [&](int t0, int t1, u32x4 (&xr)[NIT]) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int q = min(it * 64 + lane, NPC - 1);
      const int j = q / (GPW * PC), r = q - j * (GPW * PC), i = r / PC, col = r - i * PC;
      const int g = min(g0 + wv + kGUWaves * i, g1 - 1);
      xr[it] = *reinterpret_cast<const u32x4*>(x + (int64_t)(j ? t1 : t0) * H + g * C::G + col * 8);
    }
  };
  auto store_x = [&](const u32x4 (&xr)[NIT]) {
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      if (it * 64 + lane < NPC) *reinterpret_cast<u32x4*>(xs + (it * 64 + lane) * 8) = xr[it];
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
  };
  // pair ids clamped into [0, P): token rows stay inside x for any routing
  auto pair_at = [&](int pos) { return min(max(sorted_pairs[pos], 0), P - 1); };
  auto tokens = [&](int b0, int& t0, int& t1) {
    t0 = pair_at(seg0 + b0) / K;
    t1 = b0 + 1 < n_e ? pair_at(seg0 + b0 + 1) / K : t0;
  };
  int t0, t1;
  tokens(0, t0, t1);
  u32x4 xr[NIT];
  load_x(t0, t1, xr);
  asm volatile("" ::: "memory");
  u32x4 cw[GPW][C::CHUNKS];
  uint32_t sr[GPW];  // the aligned dword holding the scale (any 16-bit handling here would wait)
#pragma unroll
  for (int i = 0; i < GPW; ++i)
    if (i < kGUAhead) issue(i, cw, sr);
  asm volatile("" ::: "memory");
  store_x(xr);

  // one pass over positions b0, b0+1 of the expert (their row slices staged; the
  // first kGUAhead groups already requested, the later ones requested as the
  // pass goes)
  auto pass = [&](int b0) {
    const bool two = b0 + 1 < n_e;
    const uint16_t* arow = xs + (lane & 1) * (GPW * C::G);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = g0 + wv + kGUWaves * i;
      if (g < g1) {
        uint32_t sraw = sr[i];
        asm volatile("" : "+v"(sraw));  // convert here, not hoisted ahead of the loads
        const float sc = scale_to_f32(scale_from_dword(sraw, lane), scale_f16);
        uint32_t w[C::WORDS];
        unit_words<CODEC>(cw[i], w);
        const uint16_t* ar = arow + i * C::G;
        f4v d = f4v{0.f, 0.f, 0.f, 0.f};
        uint32_t even = 0;
        C::for_each_pair(w, [&](int Pp, uint32_t pr) {
          if ((Pp & 1) == 0) {
            even = pr;
            return;
          }
          const s4v b = __builtin_bit_cast(s4v, u32x2v{even, pr});
          const s4v av = *reinterpret_cast<const s4v*>(ar + 2 * (Pp - 1));
          d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(av, b, d, 0, 0, 0);
        });
        a0 = fmaf(sc, d[0], a0);
        a1 = fmaf(sc, d[1], a1);  // (one position: slot 1 holds the same token)
      }
      if (i + kGUAhead < GPW) {
        asm volatile("" ::: "memory");
        issue(i + kGUAhead, cw, sr);
        asm volatile("" ::: "memory");
      }
    }
    // subtract sum_g s_g * (offset sum of group g), the pairs read from the slices
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int g = g0 + wv + kGUWaves * i;
      if (g < g1) {
        uint32_t sraw = sr[i];
        asm volatile("" : "+v"(sraw));
        const float sc = scale_to_f32(scale_from_dword(sraw, lane), scale_f16);
        const float off = lane < C::PAIRS ? C::pair_off(lane) : 0.f;
        const int pl = lane < C::PAIRS ? lane : 0;
        const uint32_t xa = xs32[i * C::PAIRS + pl], xb = xs32[(GPW + i) * C::PAIRS + pl];
        const float c0 = wave_sum_uniform<CODEC>(
            off * bf16_to_f32((uint16_t)xa) + off * bf16_to_f32((uint16_t)(xa >> 16)));
        a0 = fmaf(-sc, c0, a0);
        if (two) {
          const float c1 = wave_sum_uniform<CODEC>(
              off * bf16_to_f32((uint16_t)xb) + off * bf16_to_f32((uint16_t)(xb >> 16)));
          a1 = fmaf(-sc, c1, a1);
        }
      }
    }
    MOE_TR(tb + 2);
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
  };
  pass(0);
  // more than two positions (a token that lists the expert twice): later passes
  // stage their rows and request the groups again, in the same way
  for (int b0 = kTokPerPass; b0 < n_e; b0 += kTokPerPass) {
    tokens(b0, t0, t1);
    load_x(t0, t1, xr);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < GPW; ++i)
      if (i < kGUAhead) issue(i, cw, sr);
    asm volatile("" ::: "memory");
    store_x(xr);
    pass(b0);
  }
  MOE_TR(tb + 3);
}

// down of the one/two-token path
// Block (a, strip): rows [64*strip, +64) of the down matrix of the a-th active
// expert (looked up by the gate/up kernel); 4 waves take groups g = wave + 4*i,
// i < GPW.  The same schedule as the
// gate/up kernel: each wave requests h (hi and lo rows) of up to XT of the
// expert's positions for its groups into its own LDS region, then its weights;
// the products run on the matrix cores (4 x 4 x 4 bf16 blocks: the rows of A are
// the positions' h hi and lo from LDS, B the lanes' expanded code pairs), one
// instruction per two code pairs for both positions and both halves of h.
// y goes to row p = t*K + k of pair_out when the caller asks for the pair
// outputs (or the combine kernel reads them).  When `out` is given, the blocks
// also form out[t] = sum_k w[t][k] y(t,k) (pairs with an id outside [0, E)
// skipped) + the shared expert's slices through the fixed-point accumulator
// words below: one launch fewer than a combine kernel, and no hand-off of the
// pair outputs through memory.
constexpr int kDNWaves = 4;
constexpr int kCombineMaxK = 16;
static_assert(kCombineMaxK < 32, "a combine word counts at most 31 pairs");

// The fixed-point combine of the one/two-token down kernel.  Every block adds,
// per token t and output column n, its pairs' terms w*y (each exact in fp64,
// rounded once to a multiple of 2^-28) into one 64-bit word of the workspace
// with a single agent-scope atomic add: bits 0-4 count the pairs added, bits
// 5-9 the pairs whose term was out of range (|w*y| >= 2^21 or not finite, added
// as 0), bits 10-63 the signed sum (|sum| < 16 * 2^49 units).  Integer sums do
// not depend on the order of the adds, so the result is the same on every run;
// the lane whose add brings the count to the token's number of valid pairs holds
// the complete sum in the add's return value, writes out[t][n] and zeroes the
// word for the next call.  No data hand-off through memory, no ticket.
__device__ __forceinline__ uint64_t fx_term(float w, float y) {
  const double term = (double)w * (double)y;  // exact: 24 x 24 significant bits
  const bool ok = fabs(term) < 0x1p21;        // false for NaN
  const int64_t q = ok ? (int64_t)__builtin_rint(term * 0x1p28) : 0;
  return ((uint64_t)q << 10) + (ok ? 1u : 33u);
}
__device__ __forceinline__ float fx_value(uint64_t tot) {
  if ((tot >> 5) & 31) return __builtin_nanf("");
  return (float)((double)((int64_t)tot >> 10) * 0x1p-28);  // |sum| < 2^53: exact in fp64
}
// out[t][n] = v + the shared expert's slices (added in slice order); a stack
// layer also adds it to the residual
__device__ __forceinline__ void fx_finish(float v, const float* shared, int nsh, int T, int t,
                                          int n, int H, float* __restrict__ out,
                                          float* __restrict__ resid) {
  if (shared) {
    float sh = 0.f;
    for (int q = 0; q < nsh; ++q) sh += shared[((int64_t)q * T + t) * H + n];
    v += sh;
  }
  out[(int64_t)t * H + n] = v;
  if (resid) resid[(int64_t)t * H + n] += v;
}

// h of the wave's groups for up to XT positions, formed from the KP gate and up
// partial products (added in part order, as the SwiGLU pass of the larger
// batches does): item q = (token j, group i, pair p) of the wave; lane-strided.
template <int CODEC, int GPW, int XT, int KP>
struct HFromParts {
  using C = UnitCodec<CODEC>;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  static constexpr int NI = XT * GPW * C::PAIRS;
  static constexpr int IT = (NI + 63) / 64;
  f32x2 g[IT][KP], u[IT][KP];
  __device__ __forceinline__ void load(const float* part, int P, int I, int pos0, int nt,
                                       int gbase, int glast, int lane) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = min(it * 64 + lane, NI - 1);
      const int j = q / (GPW * C::PAIRS), i = (q / C::PAIRS) % GPW, pp = q % C::PAIRS;
      const int gg = min(gbase + kDNWaves * i, glast);
      const int64_t pos = pos0 + min(j, nt - 1);
      const int k = gg * C::G + 2 * pp;
#pragma unroll
      for (int r = 0; r < KP; ++r) {
        g[it][r] = *reinterpret_cast<const f32x2*>(part + ((int64_t)r * P + pos) * I + k);
        u[it][r] = *reinterpret_cast<const f32x2*>(part + ((int64_t)(KP + r) * P + pos) * I + k);
      }
    }
  }
  __device__ __forceinline__ void store(uint32_t* xs, int lane) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int q = it * 64 + lane;
      if (q < NI) {
        f32x2 gs = g[it][0], us = u[it][0];
#pragma unroll
        for (int r = 1; r < KP; ++r) {
          gs += g[it][r];
          us += u[it][r];
        }
        uint32_t hi = 0, lo = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float gv = e ? gs.y : gs.x, uv = e ? us.y : us.x;
          const float h = gv * __builtin_amdgcn_rcpf(1.f + __expf(-gv)) * uv;
          const uint16_t bh = f32_to_bf16_rne(h);
          hi |= (uint32_t)bh << (16 * e);
          lo |= (uint32_t)f32_to_bf16_rne(h - bf16_to_f32(bh)) << (16 * e);
        }
        const int j = q / (GPW * C::PAIRS), i = (q / C::PAIRS) % GPW, pp = q % C::PAIRS;
        xs[((j * GPW + i) * 2 + 0) * C::PAIRS + pp] = hi;
        xs[((j * GPW + i) * 2 + 1) * C::PAIRS + pp] = lo;
      }
    }
  }
};

template <int CODEC, int GPW, int XT, int KP, bool SPEC>
__global__ __launch_bounds__(256, 2) void k_down_blk(
    int E, const int32_t* __restrict__ sorted_pairs, int H, int I, int P, int scale_f16,
    const float* __restrict__ part, float* pair_out, const int32_t* __restrict__ ids,
    const float* __restrict__ wts, int K, int T, const float* shared, int nsh,
    int32_t* __restrict__ ctr0, float* __restrict__ out, float* __restrict__ resid,
    uint64_t* __restrict__ fxw, int store_y, const ActEntry* __restrict__ dact) {
  using C = UnitCodec<CODEC>;
  using HS = HFromParts<CODEC, GPW, XT, KP>;
  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef float f4v __attribute__((ext_vector_type(4)));
  constexpr int XW = XT * GPW * 2 * C::PAIRS;  // uint32 per wave: [token][group][hi|lo][pair]
  __shared__ float red[kDNWaves][kTokPerPass][64];
  __shared__ __align__(16) uint32_t xs_all[kDNWaves * XW];
  const int ng = I / C::G;
  const int tb = 4096 + 8 * (blockIdx.x + gridDim.x * blockIdx.y);
  MOE_TR(tb);

  // The a-th active expert as block (a, 0, 0) of the gate/up kernel found it
  // (its entry in dact: expert, segment, U in the pad field, the down matrix):
  // scalar loads, one round trip, no lookup of its own.  SPEC (one token): when
  // the routing is consistent and the token lists each expert once, the a-th
  // active expert's pair sits at sorted position a, so the block requests the h
  // parts of position a in the same round trip, and uses them only if the entry
  // confirms that position (otherwise it requests them again).
  const ActEntry* ae = dact + blockIdx.x;
  const int ae_e = ae->e, ae_seg0 = ae->seg0, ae_n = ae->n, ae_u = ae->pad;
  const void* ae_down = ae->ptr[2];
  const int call_bad = ctr0[kCtrCallBad];
  asm volatile("" ::: "memory");
  HS hsp;
  if (SPEC) hsp.load(part, P, I, min((int)blockIdx.x, P - 1), 1, wv_of_thread(), ng - 1,
                     threadIdx.x & 63);
  asm volatile("" ::: "memory");
  const Active act{ae_e, ae_u, ae_seg0, ae_n, {nullptr, nullptr, ae_down}, true};
  MOE_TR(tb + 1);
  const int strip = blockIdx.y;
  if (call_bad) return;  // inconsistent caller routing: the outputs are left untouched
  // each token's number of valid pairs: the count that completes its words
  int nval0 = 0, nval1 = 0;
  if (out) {
    for (int k = 0; k < K; ++k) {
      const int i0 = ids[k];
      nval0 += i0 >= 0 && i0 < E;
      if (T > 1) {
        const int i1 = ids[K + k];
        nval1 += i1 >= 0 && i1 < E;
      }
    }
  }
  if (act.e < 0) {  // no expert for this block
    // block 0 writes the tokens without a valid pair (the shared expert only)
    const int t = threadIdx.x >> 6;
    if (out && blockIdx.x == 0 && t < T && (t ? nval1 : nval0) == 0)
      fx_finish(0.f, shared, nsh, T, t, strip * 64 + (threadIdx.x & 63), H, out, resid);
    return;
  }
  const int seg0 = __builtin_amdgcn_readfirstlane(act.seg0);
  const int n_e = __builtin_amdgcn_readfirstlane(act.n);
  const int lane = threadIdx.x & 63;
  const int wv = wv_of_thread();
  const MatGeom gm{H, I, C::BITS, C::G};
  const gbytes_t down = as_global(act.ptr[2]);
  const gu16_t dsc = (gu16_t)(down + gm.scales_off());
  const int row = strip * 64 + lane;
  uint32_t* xs = xs_all + wv * XW;

  // pair ids of the expert's first 64 positions (lane = position), then h of the
  // first positions, all ahead of the weights
  int pids = sorted_pairs[seg0 + min(lane, n_e - 1)];  // (a checked routing: in [0, P))
  float wpos = out ? wts[min(max(pids, 0), P - 1)] : 0.f;  // the pair's weight
  uint64_t fa0 = 0, fa1 = 0;  // this wave's combine words, tokens 0 and 1
  const bool spec = SPEC && seg0 == (int)blockIdx.x && n_e == 1;  // uniform
  HS hst;
  int nt = min(n_e, XT);
  if (!spec) hst.load(part, P, I, seg0, nt, wv, ng - 1, lane);
  asm volatile("" ::: "memory");

  u32x4 cw[GPW][C::CHUNKS];
  uint32_t sr[GPW];  // the aligned dword holding the scale (any 16-bit handling here would wait)
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int g = min(wv + kDNWaves * i, ng - 1);
    load_unit4<CODEC>(down, (int64_t)strip * ng + g, lane, cw[i]);
    sr[i] = load_scale_dword(dsc, scale_idx((int64_t)strip * ng + g, lane));
  }
  asm volatile("" ::: "memory");

  const float off = lane < C::PAIRS ? C::pair_off(lane) : 0.f;
  auto osum = [&](const uint32_t* hhp, const uint32_t* hlp) {
    const uint32_t a = lane < C::PAIRS ? hhp[lane] : 0u, b = lane < C::PAIRS ? hlp[lane] : 0u;
    return wave_sum_uniform<CODEC>(off * ((bf16_to_f32((uint16_t)a) + bf16_to_f32((uint16_t)(a >> 16))) +
                                         (bf16_to_f32((uint16_t)b) + bf16_to_f32((uint16_t)(b >> 16)))));
  };
  // (each path stores its own registers: a merged store would wait for the
  // whole weight stream before the first products)
  if (spec) {
    hsp.store(xs, lane);
    asm volatile("" ::: "memory");
  } else {
    hst.store(xs, lane);
    asm volatile("" ::: "memory");
  }
  MOE_TR(tb + 2);
  for (int c0 = 0; c0 < n_e; c0 += XT) {
    if (c0 > 0) {
      nt = min(n_e - c0, XT);
      hst.load(part, P, I, seg0 + c0, nt, wv, ng - 1, lane);
      hst.store(xs, lane);
      if (c0 % 64 == 0) {
        pids = sorted_pairs[seg0 + c0 + min(lane, n_e - c0 - 1)];
        if (out) wpos = wts[min(max(pids, 0), P - 1)];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
    for (int jp = 0; jp < nt; jp += kTokPerPass) {
      const bool two = jp + 1 < nt;
      const int j1 = two ? jp + 1 : jp;
      float a0 = 0.f, a1 = 0.f;
      // the matrix-core operand A holds four h rows: (position jp, hi), (jp, lo),
      // (j1, hi), (j1, lo); lane l supplies row l & 3 (every 4 x 4 block the same
      // rows), and the weights' code pairs 2s, 2s+1 of lane l are column l of B
      const int jr = (lane & 2) ? j1 : jp;
      const uint32_t* arow = xs + (jr * GPW * 2 + (lane & 1)) * C::PAIRS;
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int g = wv + kDNWaves * i;
        if (g < ng) {
          const uint32_t* hh0 = xs + ((jp * GPW + i) * 2 + 0) * C::PAIRS;
          const uint32_t* hl0 = xs + ((jp * GPW + i) * 2 + 1) * C::PAIRS;
          const uint32_t* hh1 = xs + ((j1 * GPW + i) * 2 + 0) * C::PAIRS;
          const uint32_t* hl1 = xs + ((j1 * GPW + i) * 2 + 1) * C::PAIRS;
          const uint32_t* ar = arow + i * 2 * C::PAIRS;
          uint32_t wd[C::WORDS];
          unit_words<CODEC>(cw[i], wd);
          uint32_t sraw = sr[i];
          asm volatile("" : "+v"(sraw));
          const float sc = scale_to_f32(scale_from_dword(sraw, lane), scale_f16);
          const float k0 = osum(hh0, hl0);
          f4v d = f4v{0.f, 0.f, 0.f, 0.f};
          uint32_t even = 0;
          C::for_each_pair(wd, [&](int Pp, uint32_t pr) {
            if ((Pp & 1) == 0) {
              even = pr;
              return;
            }
            const s4v b = __builtin_bit_cast(s4v, u32x2v{even, pr});
            const s4v av = *reinterpret_cast<const s4v*>(ar + Pp - 1);
            d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(av, b, d, 0, 0, 0);
          });
          a0 = fmaf(sc, (d[0] + d[1]) - k0, a0);
          if (two) a1 = fmaf(sc, (d[2] + d[3]) - osum(hh1, hl1), a1);
        }
      }
      MOE_TR(tb + 3);
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
        if (store_y) pair_out[(int64_t)p * H + row] = y;
        if (out) {
          const float wk = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wpos), idx));
          const uint64_t d = fx_term(wk, y);
          if (p >= K) fa1 += d; else fa0 += d;  // token p / K (T <= 2)
        }
      }
      lds_barrier();
    }
  }
  if (out) {  // the block's words, then one atomic add per token and column
    __shared__ uint64_t fxs[kDNWaves][2][64];
    fxs[wv][0][lane] = fa0;
    fxs[wv][1][lane] = fa1;
    __syncthreads();
    if (wv < T) {
      const int t = wv;
      uint64_t mine = 0;
#pragma unroll
      for (int ww = 0; ww < kDNWaves; ++ww) mine += fxs[ww][t][lane];
      if (mine != 0) {  // the block holds pairs of token t (count >= 1)
        uint64_t* wp = fxw + (int64_t)t * H + row;
        const uint64_t tot =
            __hip_atomic_fetch_add(wp, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + mine;
        MOE_TR(tb + 4);
        if ((int)(tot & 31) == (t ? nval1 : nval0)) {  // every pair of token t is in
          st_coherent(wp, (uint64_t)0);
          if ((tot >> 5) & 31) atomicOr(ctr0 + kCtrError, kErrCombine);
          fx_finish(fx_value(tot), shared, nsh, T, t, row, H, out, resid);
          MOE_TR(tb + 5);
        }
      } else if (blockIdx.x == 0 && (t ? nval1 : nval0) == 0) {
        fx_finish(0.f, shared, nsh, T, t, row, H, out, resid);
      }
    }
  }
}

// ---------------------------------------------------------------- SwiGLU
// h[pos][k] = silu(sum_ch g_ch) * (sum_ch u_ch), slices added in chunk order,
// as bf16 hi + bf16 remainder (h to ~2^-16 relative).  Positions past the
// grouped pairs are skipped.  MC >= NCH bounds the chunk slices read per element.
// Wave = reduction group g of the down matrix, lane = code pair P of the group
// (elements k = g*G + 2P, 2P+1).  The same wave also forms the down codec's
// offset sum osh[pos][g] = sum_P off_P (hi_2P + hi_2P+1 + lo_2P + lo_2P+1) (the
// fixed-order wave sum), which the down GEMV subtracts per group.
template <int CODEC, int MC>
__global__ __launch_bounds__(256) void k_swiglu_sum(const float* __restrict__ part,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int P, int I, int NCH,
                                                    uint16_t* __restrict__ hh,
                                                    uint16_t* __restrict__ hl,
                                                    float* __restrict__ osh) {
  using C = UnitCodec<CODEC>;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int pos = blockIdx.y;
  const int ngd = I / C::G;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ngd) return;  // wave-uniform
  const bool live = lane < C::PAIRS;
  const int k = g * C::G + 2 * (live ? lane : 0);
  // the number of grouped positions and the partial sums in one round trip (every
  // position < P has its rows in the buffer; positions past the grouped pairs
  // store nothing)
  const int n_grouped = offsets[E];
  f32x2 pg[MC], pu[MC];
#pragma unroll
  for (int c = 0; c < MC; ++c) {
    const int cc = min(c, NCH - 1);
    pg[c] = *reinterpret_cast<const f32x2*>(part + ((int64_t)cc * P + pos) * I + k);
    pu[c] = *reinterpret_cast<const f32x2*>(part + ((int64_t)(NCH + cc) * P + pos) * I + k);
  }
  asm volatile("" ::: "memory");
  if (pos >= n_grouped) return;
  uint32_t hp = 0, lp = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float gs = e ? pg[0].y : pg[0].x, us = e ? pu[0].y : pu[0].x;
#pragma unroll
    for (int c = 1; c < MC; ++c)
      if (c < NCH) {
        gs += e ? pg[c].y : pg[c].x;
        us += e ? pu[c].y : pu[c].x;
      }
    const float h = gs * __builtin_amdgcn_rcpf(1.f + __expf(-gs)) * us;
    const uint16_t hi = f32_to_bf16_rne(h);
    hp |= (uint32_t)hi << (16 * e);
    lp |= (uint32_t)f32_to_bf16_rne(h - bf16_to_f32(hi)) << (16 * e);
  }
  if (live) {
    reinterpret_cast<uint32_t*>(hh)[((int64_t)pos * I + k) / 2] = hp;
    reinterpret_cast<uint32_t*>(hl)[((int64_t)pos * I + k) / 2] = lp;
  }
  const float t = live ? (bf16_to_f32((uint16_t)hp) + bf16_to_f32((uint16_t)(hp >> 16))) +
                             (bf16_to_f32((uint16_t)lp) + bf16_to_f32((uint16_t)(lp >> 16)))
                       : 0.f;
  const float off = live ? C::pair_off(lane) : 0.f;
  const float v = wave_sum_uniform<CODEC>(off * t);
  if (lane == 0) osh[(int64_t)pos * ngd + g] = v;
}

// ---------------------------------------------------------------- combine
// y(t,k) = sum_ch part[ch][t*K+k] (chunk order); out[t] = sum_k w[t][k] y(t,k)
// (k ascending; pairs whose id is outside [0, E) are skipped) + the shared
// expert's nsh slices shared[q][t] (added in order);
// pair_out[t*K+k] = y(t,k) when requested.
template <int KM, int MC>
__global__ __launch_bounds__(256) void k_combine_parts(const float* __restrict__ part, int NCH,
                                                       int P, const int32_t* __restrict__ ids,
                                                       const float* __restrict__ w, int K, int E,
                                                       int H, const float* __restrict__ shared,
                                                       int nsh, int T,
                                                       const int32_t* __restrict__ call_bad,
                                                       float* __restrict__ out,
                                                       float* __restrict__ pair_out,
                                                       float* __restrict__ resid) {
  const int t = blockIdx.y;
  const int n = min((int)(blockIdx.x * 256 + threadIdx.x), H - 1);
  float y[KM][MC];
#pragma unroll
  for (int k = 0; k < KM; ++k)
#pragma unroll
    for (int c = 0; c < MC; ++c)
      y[k][c] = part[((int64_t)min(c, NCH - 1) * P + (int64_t)t * K + min(k, K - 1)) * H + n];
  // the shared expert's slices (at most kMaxShared) and the residual, in the same
  // round trip as the partial sums
  float shv[kMaxShared];
#pragma unroll
  for (int q = 0; q < kMaxShared; ++q)
    shv[q] = shared ? shared[((int64_t)min(q, nsh - 1) * T + t) * H + n] : 0.f;
  const float rv = resid ? resid[(int64_t)t * H + n] : 0.f;
  float acc = 0.f;
  const bool in = blockIdx.x * 256 + threadIdx.x < H;
  const int bad = call_bad[0];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int id = ids[t * K + min(k, K - 1)];
    if (k < K && id >= 0 && id < E) {
      float v = y[k][0];
#pragma unroll
      for (int c = 1; c < MC; ++c)
        if (c < NCH) v += y[k][c];
      acc = fmaf(w[t * K + min(k, K - 1)], v, acc);
      if (pair_out && in && !bad) pair_out[((int64_t)t * K + k) * H + n] = v;
    }
  }
  if (shared) {  // the shared expert's slices, in slice order
    float sh = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxShared; ++q)
      if (q < nsh) sh += shv[q];
    acc += sh;
  }
  if (in && !bad) {
    out[(int64_t)t * H + n] = acc;
    if (resid) resid[(int64_t)t * H + n] = rv + acc;  // a stack layer: the residual update
  }
}

// ---------------------------------------------------------------- launcher
static int compute_units() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}


template <int CODEC>
hipError_t launch_decode_t(const FwdArgs& f, const WsLayout& L, float* shared_out, int nsh,
                                  hipEvent_t join, hipStream_t s) {
  using C = UnitCodec<CODEC>;
  const moe_cfg& c = *f.c;
  const int H = c.hidden, I = c.inter, E = c.n_experts, K = c.top_k, T = f.T, P = T * K;
  int32_t* act_hdr = reinterpret_cast<int32_t*>(f.ws + L.act);
  ActEntry* act = act_entries(f.ws, L);
  float* gpart = reinterpret_cast<float*>(f.ws + L.gpart);
  float* dpart = reinterpret_cast<float*>(f.ws + L.dpart);
  uint16_t* hh = reinterpret_cast<uint16_t*>(f.ws + L.hdec);
  uint16_t* hl = hh + (int64_t)P * I;
  const int maxU = min(E, P);
  const int nch_gu = (H / C::G + kDecGPW - 1) / kDecGPW;
  const int nch_dn = (I / C::G + kDecGPWd - 1) / kDecGPWd;
  // blocks of four waves (one per SIMD), wps waves per SIMD resident
  auto grid_for = [&](int64_t items, int wps) {
    return (int)std::min<int64_t>((items + 3) / 4, (int64_t)compute_units() * wps);
  };
  const int64_t items_gu = (int64_t)maxU * (I / 64) * 2 * nch_gu;
  const int64_t items_dn = (int64_t)maxU * (H / 64) * nch_dn;
  int32_t* ctr0 = reinterpret_cast<int32_t*>(f.ws + L.counters);
  const int32_t* call_bad = ctr0 + kCtrCallBad;

  if (T <= 2) {  // block-level path: no plan kernel
    const int ngh = H / C::G;
    const int KP = (ngh + 5 * kGUWaves - 1) / (5 * kGUWaves);  // <= kMaxKParts for H/G <= 64
    const int gpw_gu = ((ngh + KP - 1) / KP + kGUWaves - 1) / kGUWaves;
    const int gpw_dn = (I / C::G + kDNWaves - 1) / kDNWaves;
    float* y = f.pair_out ? f.pair_out : dpart;  // pair-order expert outputs
#define MOE_GU1(N, PRE)                                                                          \
    MOE_LAUNCH(KID_GATEUP, (k_gateup_smem<CODEC, N, PRE>), dim3(maxU, I / 64, 2 * KP),            \
               dim3(64 * kGUWaves), 0, s, f.table, E, f.offsets, f.sorted_pairs, K, f.x, H, I, P,    \
               KP, c.scale_f16, gpart, f.ids, ctr0, act)
#define MOE_GU(N)                                                                                \
  case N:                                                                                        \
    if (f.pre_entries) MOE_GU1(N, true); else MOE_GU1(N, false);                                 \
    break;
    switch (gpw_gu) {
      MOE_GU(1) MOE_GU(2) MOE_GU(3) MOE_GU(4) MOE_GU(5)
      default: return hipErrorInvalidValue;
    }
#undef MOE_GU
#undef MOE_GU1
    // down: h formed from the KP gate and up parts while staging (no SwiGLU
    // launch); the blocks combine through the accumulator words (no combine
    // launch)
    const bool fuse = K <= kCombineMaxK && H / 64 <= kMaxStrips;
    float* cout = fuse ? f.out : nullptr;
    // pair outputs are stored when the caller asks for them or the combine
    // kernel reads them
    const int store_y = f.pair_out != nullptr || !fuse;
    if (join) {  // the combine adds the shared expert's output
      const hipError_t e = hipStreamWaitEvent(s, join, 0);
      if (e != hipSuccess) return e;
    }
#define MOE_DN1(N, KPT, SPEC)                                                                     \
  MOE_LAUNCH(KID_DOWN, (k_down_blk<CODEC, N, 2, KPT, SPEC>), dim3(maxU, H / 64),                   \
             dim3(64 * kDNWaves), 0, s, E, f.sorted_pairs, H, I, P, c.scale_f16,                   \
             gpart, y, f.ids, f.w, K, T, shared_out, nsh, ctr0, cout, f.resid,                \
             reinterpret_cast<uint64_t*>(ctr0 + kFxAcc), store_y, act)
#define MOE_DN(N, KPT)                                                                           \
  case N:                                                                                        \
    if (T == 1) MOE_DN1(N, KPT, true); else MOE_DN1(N, KPT, false);                             \
    break;
#define MOE_DN_KP(KPT)                                                                           \
    switch (gpw_dn) {                                                                            \
      MOE_DN(1, KPT) MOE_DN(2, KPT) MOE_DN(3, KPT) MOE_DN(4, KPT)                                \
      MOE_DN(5, KPT) MOE_DN(6, KPT) MOE_DN(7, KPT) MOE_DN(8, KPT)                                \
      default: return hipErrorInvalidValue;                                                      \
    }
    switch (KP) {
      case 1: MOE_DN_KP(1) break;
      case 2: MOE_DN_KP(2) break;
      case 3: MOE_DN_KP(3) break;
      case 4: MOE_DN_KP(4) break;
      default: return hipErrorInvalidValue;
    }
#undef MOE_DN_KP
#undef MOE_DN
#undef MOE_DN1
    if (fuse) return hipGetLastError();
    // y holds every pair's output in pair order: a single "chunk"
    if (K <= 8) {
      MOE_LAUNCH(KID_COMBINE, (k_combine_parts<8, 1>), dim3((H + 255) / 256, T), dim3(256), 0, s, y,
                 1, P, f.ids, f.w, K, E, H, shared_out, nsh, T, call_bad, f.out, nullptr, f.resid);
    } else {
      MOE_LAUNCH(KID_COMBINE, (k_combine_parts<16, 1>), dim3((H + 255) / 256, T), dim3(256), 0, s,
                 y, 1, P, f.ids, f.w, K, E, H, shared_out, nsh, T, call_bad, f.out, nullptr, f.resid);
    }
    return hipGetLastError();
  }

  float* osx = reinterpret_cast<float*>(f.ws + L.osx);
  if (!f.pre_entries)  // (in a layer call of up to 8 tokens the routing launch did the plan)
    MOE_LAUNCH(KID_PLAN, k_plan_decode<CODEC>, dim3(1 + (T * (H / C::G) + 15) / 16), dim3(1024),
               0, s, f.offsets, f.ids, f.sorted_pairs, P, ctr0, f.table, E, act_hdr, act, f.x, T,
               H, osx);
  // four waves per SIMD: without the activation staging the GEMVs fit in 128
  // registers; three for 4-bit codes in groups of 128 (four 16-byte loads per unit)
  constexpr int kWps = C::CHUNKS > 3 ? 3 : 4;
  MOE_LAUNCH(KID_GATEUP, (k_gemv<CODEC, kDecGPW, 8, 0, kWps>), dim3(grid_for(items_gu, kWps)),
             dim3(256), 0, s, act_hdr, act, f.sorted_pairs, K, f.x, nullptr, I, H, P, c.scale_f16,
             gpart, osx);
  float* osh = reinterpret_cast<float*>(f.ws + L.osh);
#define MOE_SW(MC)                                                                              \
  MOE_LAUNCH(KID_SWIGLU, (k_swiglu_sum<CODEC, MC>), dim3((I / C::G + 3) / 4, P), dim3(256), 0, s, \
             gpart, f.offsets, E, P, I, nch_gu, hh, hl, osh)
  if (nch_gu <= 8) MOE_SW(8); else if (nch_gu <= 16) MOE_SW(16); else MOE_SW(24);
#undef MOE_SW
  constexpr int kWpsD = C::CHUNKS > 3 ? 3 : 4;
  MOE_LAUNCH(KID_DOWN, (k_gemv_mma<CODEC, kDecGPWd, 1, kWpsD>), dim3(grid_for(items_dn, kWpsD)), dim3(256),
             0, s, act_hdr, act, f.sorted_pairs, K, hh, hl, H, I, P, c.scale_f16, dpart, osh);
  if (join) {
    const hipError_t e = hipStreamWaitEvent(s, join, 0);
    if (e != hipSuccess) return e;
  }
  // MC: chunks of the down reduction read per pair (I/G <= 32 groups, 3 per chunk)
#define MOE_CMB(KM, MC)                                                                        \
  MOE_LAUNCH(KID_COMBINE, (k_combine_parts<KM, MC>), dim3((H + 255) / 256, T), dim3(256), 0, s, \
             dpart, nch_dn, P, f.ids, f.w, K, E, H, shared_out, nsh, T, call_bad, f.out, f.pair_out, f.resid)
  if (K <= 8) {
    if (nch_dn <= 4) MOE_CMB(8, 4); else MOE_CMB(8, 12);
  } else {
    if (nch_dn <= 4) MOE_CMB(16, 4); else MOE_CMB(16, 12);
  }
#undef MOE_CMB
  return hipGetLastError();
}



}  // namespace moe
