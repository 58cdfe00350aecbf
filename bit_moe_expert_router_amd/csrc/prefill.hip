// prefill.hip -- the routed experts of a prefill chunk as grouped matrix products
// on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// A prefill chunk routes thousands of tokens (8,192 per chunk on the pages' model:
// page "0xSero/glm53-flash-offload", paragraph on prefill staging of chunks of at
// least 8,192 picks per layer), so each picked expert sees many rows and its
// gate/up/down products are dense contractions: [n_e x H] . [H x I] and
// [n_e x I] . [I x H] per expert.
//
// Operands.  A packed weight W[n][k] = q[n][k] * s[n][k/G] with q = c - 2^(bits-1)
// a small integer and s a bf16 scale: the product q*s has at most 3 + 8
// significant bits, so it is exact in fp16 (fp16 scales: rounded to nearest).
// The weights are expanded in LDS to fp16 W16 = q*s, one code pair per 32-bit
// word: shift and mask the two codes into the mantissas of 1024.0 (1024 + c),
// then one packed fp16 add of -(1024 + 2^(bits-1)) and one packed multiply by s;
// and the activations are fp16 copies of the bf16 tokens scaled
// by a per-token power of two (exact for every normal fp16 value, so the fp16
// range never clips a token).  Accumulation is fp32 throughout the reduction.
//
// Gate/up: tile = 128 sorted pair positions of one expert x 64 rows of both the
// gate and the up matrix, so the epilogue forms h = silu(g) * u directly and
// stores it once (fp16).  Down: tile = 128 positions x 128 rows of H; y goes to
// pair_out row p = t*K + k.  Both walk the reduction in steps of 128 elements
// (one 3-bit group or four 4-bit groups): global loads of steps s+1 and s+2 are
// in flight (two register stages) while the matrix cores work on step s out of LDS.
#include "common.h"

namespace moe {

constexpr int kPM = 128;           // sorted pair positions per tile
constexpr int kPK = 128;           // reduction elements per step
constexpr int kLdsRow = kPK + 16;  // fp16 per LDS row (a 32-byte pad: measured fewer bank conflicts than 16)
constexpr int kGuN = 64;           // gate/up rows per block, of each matrix
constexpr int kDnN = 128;          // down rows per block

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- activations to fp16
// x16[t] = fp16(x[t] * 2^-s_t) with s_t the smallest shift >= 0 that keeps the
// token's largest magnitude below 2^15; xshift[t] = s_t.
__global__ __launch_bounds__(256) void k_xprep(const uint16_t* __restrict__ x, int H,
                                               uint16_t* __restrict__ x16,
                                               int32_t* __restrict__ xshift) {
  const int t = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
  const int n8 = H / 8;
  int m = 0;
  for (int i = threadIdx.x; i < n8; i += 256) {
    const uint4 v = xr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, (int)max((w[j] >> 7) & 0xFF, (w[j] >> 23) & 0xFF));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  __shared__ int red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  // biased exponent m: magnitude < 2^(m - 126); keep it below 2^15
  const int s = max(0, m - 126 - 15);
  if (threadIdx.x == 0) xshift[t] = s;
  uint4* yr = reinterpret_cast<uint4*>(x16 + (int64_t)t * H);
  for (int i = threadIdx.x; i < n8; i += 256) {
    const uint4 v = xr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)ldexpf(bf16_to_f32((uint16_t)w[j]), -s);
      const _Float16 hi = (_Float16)ldexpf(bf16_to_f32((uint16_t)(w[j] >> 16)), -s);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    yr[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------- routing check
// The conditions of routing_ok_wave (common.h) for any number of pairs: thread i
// checks expert i's offsets, the id of pair i and grouped position i; block b
// writes its count of pairs with an id in [0, E) to vchk[2b] and whether any
// check failed to vchk[2b + 1].  The tile plan combines the blocks.
__global__ __launch_bounds__(256) void k_check_routing(const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ sp, int P,
                                                       int E, int32_t* __restrict__ vchk) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int oE = offsets[E];
  bool bad = false;
  if (i < E) {
    const int a = offsets[i], b = offsets[i + 1];
    bad |= b < a || (i == 0 && a != 0);
  }
  const int idv = i < P ? ids[i] : -1;
  if (i < oE && oE <= P) {
    const int p = sp[i];
    const bool pin = p >= 0 && p < P;
    const int ep = pin ? ids[p] : -1;
    const bool ein = ep >= 0 && ep < E;
    const int elo = ein ? offsets[ep] : 0, ehi = ein ? offsets[ep + 1] : 0;
    bad |= !ein || i < elo || i >= ehi || (i > elo && sp[i - 1] >= p);
  }
  const int cnt = __syncthreads_count(idv >= 0 && idv < E);
  const int anyb = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    vchk[2 * blockIdx.x] = cnt;
    vchk[2 * blockIdx.x + 1] = anyb;
  }
}

// ---------------------------------------------------------------- tile plan
// tiles[0] = number of tiles; tiles[1 + 2j] = expert, tiles[2 + 2j] = first sorted
// position of tile j.  Experts in ascending order, ceil(n_e / 128) tiles each.
// First the routing check's verdict (nb blocks of k_check_routing, plus offsets[E]
// against the count of valid pairs): for inconsistent routing there are no
// tiles, and the combine writes nothing.
__global__ __launch_bounds__(1024) void k_plan(const int32_t* __restrict__ offsets, int E,
                                               const int32_t* __restrict__ vchk, int nb,
                                               int32_t* __restrict__ ctr,
                                               int32_t* __restrict__ tiles) {
  __shared__ int wsum[16];
  __shared__ int wbad[16];
  const int e = threadIdx.x, lane = e & 63, wv = e >> 6;
  {
    int cnt = 0, b = 0;
    for (int j = e; j < nb; j += 1024) {
      cnt += vchk[2 * j];
      b |= vchk[2 * j + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      cnt += __shfl_xor(cnt, o);
      b |= __shfl_xor(b, o);
    }
    if (lane == 0) {
      wsum[wv] = cnt;
      wbad[wv] = b;
    }
    __syncthreads();
    int total = 0, anyb = 0;
    for (int w = 0; w < 16; ++w) {
      total += wsum[w];
      anyb |= wbad[w];
    }
    const bool ok = !anyb && offsets[E] == total;
    __syncthreads();  // wsum is reused below
    if (!ok) {
      if (e == 0) {
        tiles[0] = 0;
        record_routing(ctr, false);
      }
      return;
    }
    if (e == 0) record_routing(ctr, true);
  }
  const int lo = e < E ? offsets[e] : 0;
  const int n = e < E ? offsets[e + 1] - lo : 0;
  const int nt = (n + kPM - 1) / kPM;
  int inc = nt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int base = inc - nt, total = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wv) base += wsum[w];
    total += wsum[w];
  }
  for (int j = 0; j < nt; ++j) {
    tiles[1 + 2 * (base + j)] = e;
    tiles[2 + 2 * (base + j)] = lo + j * kPM;
  }
  if (e == 0) tiles[0] = total;
}

// ---------------------------------------------------------------- weight expansion
// Expand the code pairs a thread owns in one 128-element step into fp16 q*s pairs
// in its LDS row `wr` (fp16 elements, k = 0 at wr[0]).
//
// 3-bit, G = 128: pair P < 60 sits at field offset {1,4,7,10,13}[P%5] of both
// halves of word P/5; spare pair 60 + m has bit b of its code at bit 0 / 16 of
// word 3m + b.  4-bit, G = 32: the thread owns units 2hw, 2hw+1 of the step's
// four groups (4 words, pair P at word P/4, field offset 4(P%4)).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(b));
  return r;
}
// a code at bits 0..2 (3-bit) or 0..3 (4-bit) of each 16-bit half of `shifted`
__device__ __forceinline__ uint32_t q_times_s(uint32_t shifted, uint32_t mask, uint32_t magic,
                                              half2v bias, half2v s2) {
  const half2v v = __builtin_bit_cast(half2v, and_or(shifted, mask, magic));  // 1024 + c
  return __builtin_bit_cast(uint32_t, (v + bias) * s2);                       // (c - z) * s
}

// A group scale whose products q*s (|q| <= 8) are not all exact in fp16: zero
// is fine, magnitudes below 2^-14 (fp16 subnormals) or above 65504/8 are not.
__device__ __forceinline__ bool scale_inexact(float s) {
  const float a = fabsf(s);
  return !(a == 0.f || (a >= 6.103515625e-05f && a <= 8188.f));
}

template <int CODEC>
struct StepLoad;

// 3-bit, G = 128: half hw = 0 owns pairs 0..31 and spare pairs 60, 61 (words 0..6),
// half 1 owns pairs 32..59 and spare pairs 62, 63 (words 6..11); each half writes
// whole 16-byte chunks (4 pairs) of its LDS row.
template <>
struct StepLoad<kQ3G128> {
  uint32_t w[8];  // hw 0: words 0..7; hw 1: words 4..11
  uint32_t sraw;
  __device__ __forceinline__ void load(gbytes_t mat, int64_t tile, int lane, int hw, gu16_t sc) {
    typedef const u32x4p __attribute__((address_space(1)))* g4;
    const gbytes_t base = mat + tile * 3 * 1024 + 16 * lane + 1024 * hw;
    const u32x4p a = *(g4)(base);
    const u32x4p b = *(g4)(base + 1024);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    typedef const uint16_t __attribute__((address_space(1)))* g16;
    sraw = *(g16)(sc + scale_idx(tile, lane));
  }
  // returns whether the scale is outside the range where q*s is exact in fp16
  __device__ __forceinline__ bool expand(int hw, int scale_f16, _Float16* wr) const {
    const float sf = scale_f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)sraw)
                               : bf16_to_f32((uint16_t)sraw);
    const _Float16 s = (_Float16)sf;
    const half2v s2 = {s, s};
    const half2v z = {(_Float16)-1028.f, (_Float16)-1028.f};
    const uint32_t mask = 0x00070007u, magic = 0x64006400u;
    constexpr int off[5] = {1, 4, 7, 10, 13};
    u32x4p* out = reinterpret_cast<u32x4p*>(wr);  // chunk q = pairs 4q .. 4q+3
    // word W of the unit sits at w[W - wb] (wb = 0 for half 0, 4 for half 1)
    auto pair = [&](int P, int wb) {  // field pair P < 60
      return q_times_s(w[P / 5 - wb] >> off[P % 5], mask, magic, z, s2);
    };
    auto spare = [&](int m, int wb) {  // spare pair 60 + m: words 3m .. 3m+2
      const int b0 = 3 * m - wb;
      const uint32_t c = (w[b0] & 0x00010001u) | ((w[b0 + 1] & 0x00010001u) << 1) |
                         ((w[b0 + 2] & 0x00010001u) << 2);
      return q_times_s(c, mask, magic, z, s2);
    };
    if (hw == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        out[q] = u32x4p{pair(4 * q, 0), pair(4 * q + 1, 0), pair(4 * q + 2, 0), pair(4 * q + 3, 0)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint32_t*>(wr) + 60) = u32x2{spare(0, 0), spare(1, 0)};
    } else {
#pragma unroll
      for (int q = 8; q < 15; ++q)
        out[q] = u32x4p{pair(4 * q, 4), pair(4 * q + 1, 4), pair(4 * q + 2, 4), pair(4 * q + 3, 4)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint32_t*>(wr) + 62) = u32x2{spare(2, 4), spare(3, 4)};
    }
    return scale_inexact(sf);
  }
};

template <>
struct StepLoad<kQ4G32> {
  uint32_t w[8];
  uint32_t sraw;  // scales of the two groups
  __device__ __forceinline__ void load(gbytes_t mat, int64_t tile, int lane, int hw, gu16_t sc) {
    typedef const u32x4p __attribute__((address_space(1)))* g4;
    // tile = index of the step's first group's tile; units 2hw, 2hw+1 follow it
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4p a = *(g4)(mat + (tile + 2 * hw + u) * 1024 + 16 * lane);
      w[4 * u] = a.x; w[4 * u + 1] = a.y; w[4 * u + 2] = a.z; w[4 * u + 3] = a.w;
    }
    // the scales of the half's two groups (tiles tile + 2hw + u), low half first
    typedef const uint16_t __attribute__((address_space(1)))* g16;
    sraw = (uint32_t)*(g16)(sc + scale_idx(tile + 2 * hw, lane)) |
           ((uint32_t)*(g16)(sc + scale_idx(tile + 2 * hw + 1, lane)) << 16);
  }
  // returns whether a scale is outside the range where q*s is exact in fp16
  __device__ __forceinline__ bool expand(int hw, int scale_f16, _Float16* wr) const {
    const half2v z = {(_Float16)-1032.f, (_Float16)-1032.f};
    const uint32_t mask = 0x000F000Fu, magic = 0x64006400u;
    u32x4p* out = reinterpret_cast<u32x4p*>(wr) + 8 * hw;
    bool bad = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t sb = (uint16_t)(sraw >> (16 * u));
      const float sf = scale_f16 ? (float)__builtin_bit_cast(_Float16, sb) : bf16_to_f32(sb);
      bad |= scale_inexact(sf);
      const _Float16 s = (_Float16)sf;
      const half2v s2 = {s, s};
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // word d of the unit holds pairs 4d .. 4d+3
        const uint32_t x = w[4 * u + d];
        out[4 * u + d] = u32x4p{q_times_s(x, mask, magic, z, s2), q_times_s(x >> 4, mask, magic, z, s2),
                                q_times_s(x >> 8, mask, magic, z, s2), q_times_s(x >> 12, mask, magic, z, s2)};
      }
    }
    return bad;
  }
};

// 4-bit, G = 128 (16 words, 4 chunks): half hw owns chunks 2hw, 2hw+1 (words
// 8hw .. 8hw+7, pairs 32hw .. 32hw+31); word d holds pairs 4d .. 4d+3 at offsets
// 0, 4, 8, 12; one scale per step.
template <>
struct StepLoad<kQ4G128> {
  uint32_t w[8];
  uint32_t sraw;
  __device__ __forceinline__ void load(gbytes_t mat, int64_t tile, int lane, int hw, gu16_t sc) {
    typedef const u32x4p __attribute__((address_space(1)))* g4;
    const gbytes_t base = mat + tile * 4 * 1024 + 16 * lane + 2048 * hw;
    const u32x4p a = *(g4)(base);
    const u32x4p b = *(g4)(base + 1024);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    typedef const uint16_t __attribute__((address_space(1)))* g16;
    sraw = *(g16)(sc + scale_idx(tile, lane));
  }
  // returns whether the scale is outside the range where q*s is exact in fp16
  __device__ __forceinline__ bool expand(int hw, int scale_f16, _Float16* wr) const {
    const float sf = scale_f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)sraw)
                               : bf16_to_f32((uint16_t)sraw);
    const _Float16 s = (_Float16)sf;
    const half2v s2 = {s, s};
    const half2v z = {(_Float16)-1032.f, (_Float16)-1032.f};
    const uint32_t mask = 0x000F000Fu, magic = 0x64006400u;
    u32x4p* out = reinterpret_cast<u32x4p*>(wr) + 8 * hw;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t x = w[d];
      out[d] = u32x4p{q_times_s(x, mask, magic, z, s2), q_times_s(x >> 4, mask, magic, z, s2),
                      q_times_s(x >> 8, mask, magic, z, s2), q_times_s(x >> 12, mask, magic, z, s2)};
    }
    return scale_inexact(sf);
  }
};

// 2-bit, G = 128 (8 words, 2 chunks): half hw owns chunk hw (words 4hw .. 4hw+3,
// pairs 32hw .. 32hw+31); word d holds pairs 8d .. 8d+7 at offsets 0, 2, .., 14.
template <>
struct StepLoad<kQ2G128> {
  uint32_t w[4];
  uint32_t sraw;
  __device__ __forceinline__ void load(gbytes_t mat, int64_t tile, int lane, int hw, gu16_t sc) {
    typedef const u32x4p __attribute__((address_space(1)))* g4;
    const u32x4p a = *(g4)(mat + tile * 2 * 1024 + 16 * lane + 1024 * hw);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    typedef const uint16_t __attribute__((address_space(1)))* g16;
    sraw = *(g16)(sc + scale_idx(tile, lane));
  }
  // returns whether the scale is outside the range where q*s is exact in fp16
  __device__ __forceinline__ bool expand(int hw, int scale_f16, _Float16* wr) const {
    const float sf = scale_f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)sraw)
                               : bf16_to_f32((uint16_t)sraw);
    const _Float16 s = (_Float16)sf;
    const half2v s2 = {s, s};
    const half2v z = {(_Float16)-1026.f, (_Float16)-1026.f};
    const uint32_t mask = 0x00030003u, magic = 0x64006400u;
    u32x4p* out = reinterpret_cast<u32x4p*>(wr) + 8 * hw;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = w[d];
      out[2 * d] = u32x4p{q_times_s(x, mask, magic, z, s2), q_times_s(x >> 2, mask, magic, z, s2),
                          q_times_s(x >> 4, mask, magic, z, s2), q_times_s(x >> 6, mask, magic, z, s2)};
      out[2 * d + 1] = u32x4p{q_times_s(x >> 8, mask, magic, z, s2), q_times_s(x >> 10, mask, magic, z, s2),
                              q_times_s(x >> 12, mask, magic, z, s2), q_times_s(x >> 14, mask, magic, z, s2)};
    }
    return scale_inexact(sf);
  }
};

// Work item of block b when the grid (a multiple of 8 blocks) is split into
// eight contiguous ranges, one per XCD (blocks are dealt to the XCDs in turn):
// neighbouring items, which share activations and weights, share an L2.
__device__ __forceinline__ int xcd_item(int b, int nb) { return (b % 8) * (nb / 8) + b / 8; }

// 16-byte global loads of one step (128 elements, 256 bytes) of activation rows:
// lane l of wave w reads chunk l % 16 of rows 32w + 4c + l / 16, c < 8, so each
// load instruction covers four whole 256-byte row segments.  roff[c] is row c's
// element offset (+ the lane's chunk) from the array base.
struct RowLoad {
  u32x4p v[8];
  __device__ __forceinline__ void load(const uint16_t* base, const uint32_t (&roff)[8], int koff) {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = *reinterpret_cast<const u32x4p*>(base + roff[c] + koff);
  }
  __device__ __forceinline__ void store(_Float16* xs, int row0, int chunk) const {
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4p*>(xs + (row0 + 4 * c) * kLdsRow + 8 * chunk) = v[c];
  }
};

__device__ __forceinline__ half8 lds_frag(const _Float16* base) {
  return *reinterpret_cast<const half8*>(base);
}

// ---------------------------------------------------------------- gate / up
// Block: tile (expert e, positions m0 .. m0+127) x rows [64 nt, 64 nt + 64) of the
// gate and the up matrix.  Waves 2 x 2: wave (wm, wn) owns positions
// [64wm, 64wm+64) and rows [32wn, 32wn+32) of both matrices (16 accumulator tiles
// of 16 x 16).  h16[pos][row] = fp16(silu(g) * u), g and u rescaled by 2^s_t.
template <int CODEC>
__global__ __launch_bounds__(256, 2) void k_gateup_mfma(
    const moe_expert_ref* __restrict__ table, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ sorted_pairs, int K,
    const uint16_t* __restrict__ x16, const int32_t* __restrict__ xshift, int H, int I,
    int scale_f16, uint16_t* __restrict__ h16, int32_t* __restrict__ err) {
  using C = UnitCodec<CODEC>;
  __shared__ __align__(16) _Float16 xs[kPM * kLdsRow];
  __shared__ __align__(16) _Float16 wsm[2 * kGuN * kLdsRow];
  __shared__ int s_shift[kPM];
  const int nI = I / kGuN;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int tile = item / nI, nt = item % nI;
  if (tile >= tiles[0]) return;
  const int e = tiles[1 + 2 * tile], m0 = tiles[2 + 2 * tile];
  const int rows = min(kPM, offsets[e + 1] - m0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // activation rows: lane chunk of rows row0 + 4c
  const int chunk = lane & 15, row0 = 32 * wv + (lane >> 4);
  uint32_t roff[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int row = row0 + 4 * c;
    const int tok = sorted_pairs[m0 + min(row, rows - 1)] / K;
    roff[c] = (uint32_t)tok * (uint32_t)H + 8 * chunk;
    if (chunk == 0) s_shift[row] = xshift[tok];
  }
  // weights: thread (m, hw, row)
  const int m = tid >> 7, hw = (tid >> 6) & 1, wrow = lane;
  const moe_expert_ref ref = table[e];
  const gbytes_t mat = as_global(m ? ref.up : ref.gate);
  const MatGeom gm{I, H, C::BITS, C::G};
  const gu16_t msc = (gu16_t)(mat + gm.scales_off());
  const int ng = H / C::G;
  const int gps = kPK / C::G;  // groups per step
  const int64_t tile0 = (int64_t)nt * ng;
  _Float16* wr = wsm + (m * kGuN + wrow) * kLdsRow;

  const int wm = wv >> 1, wn = wv & 1;
  const int fr = lane & 15, fk = 8 * (lane >> 4);
  // 16-row sub-tiles of this wave that hold valid positions (the rest are skipped)
  const int ni = min(4, max(0, (rows - 64 * wm + 15) / 16));
  f32x4 acc[2][4][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[a][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = H / kPK;
  // two register stages: the loads of steps s+1 and s+2 are in flight while the
  // matrix cores work on step s
  RowLoad xl[2];
  StepLoad<CODEC> wl[2];
  auto issue = [&](int st, int b) {
    const int g = st * gps;
    xl[b].load(x16, roff, st * kPK);
    wl[b].load(mat, tile0 + g, wrow, hw, msc);
  };
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < kPK / 32; ++kk) {
      half8 a[4], bg[2], bu[2];
      if (ni == 0) break;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bg[j] = lds_frag(wsm + (32 * wn + 16 * j + fr) * kLdsRow + 32 * kk + fk);
        bu[j] = lds_frag(wsm + (kGuN + 32 * wn + 16 * j + fr) * kLdsRow + 32 * kk + fk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < ni) {
          a[i] = lds_frag(xs + (64 * wm + 16 * i + fr) * kLdsRow + 32 * kk + fk);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[0][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bg[j], acc[0][i][j], 0, 0, 0);
            acc[1][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bu[j], acc[1][i][j], 0, 0, 0);
          }
        }
      }
    }
  };
  // every issue is unconditional (past the end it repeats the last step), so the
  // waits before a stage's use count only the loads of the other stage
  bool inexact = false;  // a scale or an h value outside fp16's exact range
  auto run_stage = [&](int b, int next) {
    xl[b].store(xs, row0, chunk);
    inexact |= wl[b].expand(hw, scale_f16, wr);
    lds_barrier();
    issue(min(next, nsteps - 1), b);
    compute();
    lds_barrier();
  };
  issue(0, 0);
  issue(min(1, nsteps - 1), 1);
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    run_stage(0, s + 2);
    run_stage(1, s + 3);
  }
  if (s < nsteps) run_stage(0, s + 2);
  // epilogue: lane holds column fr of each 16 x 16 tile, rows 4*(lane/16) + q
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pr = 64 * wm + 16 * i + 4 * (lane >> 4) + q;
      const int sh = s_shift[pr];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float g = ldexpf(acc[0][i][j][q], sh), u = ldexpf(acc[1][i][j][q], sh);
        const float h = g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
        const int col = nt * kGuN + 32 * wn + 16 * j + fr;
        if (pr < rows) {
          h16[(int64_t)(m0 + pr) * I + col] = __builtin_bit_cast(uint16_t, (_Float16)h);
          inexact |= !(fabsf(h) < 65504.f);
        }
      }
    }
  if (__any(inexact) && lane == 0) atomicOr(err, kErrRange);
}

// ---------------------------------------------------------------- down
// Block: tile (expert e, positions m0 .. m0+127) x rows [128 nt, 128 nt + 128) of
// the down matrix.  Waves 2 x 2: wave (wm, wn) owns positions [64wm, 64wm+64) and
// rows [64wn, 64wn+64) (16 tiles).  pair_out[sorted_pairs[pos]][row] = y.
template <int CODEC>
__global__ __launch_bounds__(256, 2) void k_down_mfma(
    const moe_expert_ref* __restrict__ table, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ sorted_pairs, int P,
    const uint16_t* __restrict__ h16, int H, int I, int scale_f16, float* __restrict__ pair_out,
    int32_t* __restrict__ err) {
  using C = UnitCodec<CODEC>;
  __shared__ __align__(16) _Float16 xs[kPM * kLdsRow];
  __shared__ __align__(16) _Float16 wsm[kDnN * kLdsRow];
  __shared__ int s_pair[kPM];
  const int nH = H / kDnN;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int tile = item / nH, nt = item % nH;
  if (tile >= tiles[0]) return;
  const int e = tiles[1 + 2 * tile], m0 = tiles[2 + 2 * tile];
  const int rows = min(kPM, offsets[e + 1] - m0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  const int chunk = lane & 15, row0 = 32 * wv + (lane >> 4);
  uint32_t roff[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int row = row0 + 4 * c;
    const int pos = min(m0 + row, P - 1);
    roff[c] = (uint32_t)pos * (uint32_t)I + 8 * chunk;
    if (chunk == 0) s_pair[row] = sorted_pairs[pos];
  }
  // weights: thread (hw, tl, row): 64-row tile tl of the block's two
  const int hw = tid >> 7, tl = (tid >> 6) & 1, wrow = lane;
  const gbytes_t mat = as_global(table[e].down);
  const MatGeom gm{H, I, C::BITS, C::G};
  const gu16_t msc = (gu16_t)(mat + gm.scales_off());
  const int ng = I / C::G;
  const int gps = kPK / C::G;
  const int trow = nt * 2 + tl;  // 64-row tile index of the matrix
  const int64_t tile0 = (int64_t)trow * ng;
  _Float16* wr = wsm + (tl * 64 + wrow) * kLdsRow;

  const int wm = wv >> 1, wn = wv & 1;
  const int fr = lane & 15, fk = 8 * (lane >> 4);
  const int ni = min(4, max(0, (rows - 64 * wm + 15) / 16));
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = I / kPK;
  RowLoad xl[2];
  StepLoad<CODEC> wl[2];
  auto issue = [&](int st, int b) {
    const int g = st * gps;
    xl[b].load(h16, roff, st * kPK);
    wl[b].load(mat, tile0 + g, wrow, hw, msc);
  };
  auto compute = [&]() {
#pragma unroll
    for (int kk = 0; kk < kPK / 32; ++kk) {
      half8 a[4], b[4];
      if (ni == 0) break;
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lds_frag(wsm + (64 * wn + 16 * j + fr) * kLdsRow + 32 * kk + fk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < ni) {
          a[i] = lds_frag(xs + (64 * wm + 16 * i + fr) * kLdsRow + 32 * kk + fk);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };
  // every issue is unconditional (past the end it repeats the last step), so the
  // waits before a stage's use count only the loads of the other stage
  bool inexact = false;  // a scale or an h value outside fp16's exact range
  auto run_stage = [&](int b, int next) {
    xl[b].store(xs, row0, chunk);
    inexact |= wl[b].expand(hw, scale_f16, wr);
    lds_barrier();
    issue(min(next, nsteps - 1), b);
    compute();
    lds_barrier();
  };
  issue(0, 0);
  issue(min(1, nsteps - 1), 1);
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    run_stage(0, s + 2);
    run_stage(1, s + 3);
  }
  if (s < nsteps) run_stage(0, s + 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pr = 64 * wm + 16 * i + 4 * (lane >> 4) + q;
      if (pr < rows) {
        const int p = s_pair[pr];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pair_out[(int64_t)p * H + nt * kDnN + 64 * wn + 16 * j + fr] = acc[i][j][q];
      }
    }
  if (__any(inexact) && lane == 0) atomicOr(err, kErrRange);
}

// ---------------------------------------------------------------- launcher
static_assert(kPM == kPrefillTileRows, "tile rows");
static_assert(kPK == 128 && kDnN == 128 && kGuN == 64, "prefill_eligible assumes these");

template <int CODEC>
static hipError_t launch_prefill_t(const FwdArgs& f, const WsLayout& L, float* pair_out,
                                   hipStream_t s) {
  const moe_cfg& c = *f.c;
  const int H = c.hidden, I = c.inter, E = c.n_experts, K = c.top_k, T = f.T, P = T * K;
  uint16_t* x16 = reinterpret_cast<uint16_t*>(f.ws + L.x16);
  int32_t* xshift = reinterpret_cast<int32_t*>(f.ws + L.xshift);
  uint16_t* h16 = reinterpret_cast<uint16_t*>(f.ws + L.h16);
  int32_t* tiles = reinterpret_cast<int32_t*>(f.ws + L.tiles);
  int32_t* err = reinterpret_cast<int32_t*>(f.ws + L.counters) + kCtrError;
  const int64_t max_tiles = prefill_max_tiles(P, E);
  auto round8 = [](int64_t n) { return (int)((n + 7) / 8 * 8); };
  MOE_LAUNCH(KID_XPREP, k_xprep, dim3(T), dim3(256), 0, s, f.x, H, x16, xshift);
  int32_t* vchk = reinterpret_cast<int32_t*>(f.ws + L.vchk);
  const int nbc = (std::max(P, E) + 255) / 256;
  MOE_LAUNCH(KID_PLAN, k_check_routing, dim3(nbc), dim3(256), 0, s, f.ids, f.offsets,
             f.sorted_pairs, P, E, vchk);
  MOE_LAUNCH(KID_PLAN, k_plan, dim3(1), dim3(1024), 0, s, f.offsets, E, vchk, nbc,
             reinterpret_cast<int32_t*>(f.ws + L.counters), tiles);
  MOE_LAUNCH(KID_GATEUP, k_gateup_mfma<CODEC>, dim3(round8(max_tiles * (I / kGuN))),
             dim3(256), 0, s, f.table, f.offsets, tiles, f.sorted_pairs, K, x16, xshift, H, I,
             c.scale_f16, h16, err);
  MOE_LAUNCH(KID_DOWN, k_down_mfma<CODEC>, dim3(round8(max_tiles * (H / kDnN))),
             dim3(256), 0, s, f.table, f.offsets, tiles, f.sorted_pairs, P, h16, H, I,
             c.scale_f16, pair_out, err);
  return hipGetLastError();
}

hipError_t launch_prefill(const FwdArgs& f, const WsLayout& L, float* pair_out, hipStream_t s) {
  switch (codec_of(f.c->bits, f.c->group)) {
    case kQ3G128: return launch_prefill_t<kQ3G128>(f, L, pair_out, s);
    case kQ4G32: return launch_prefill_t<kQ4G32>(f, L, pair_out, s);
    case kQ2G128: return launch_prefill_t<kQ2G128>(f, L, pair_out, s);
    case kQ4G128: return launch_prefill_t<kQ4G128>(f, L, pair_out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
