// common.h -- internal definitions shared by the HIP sources of libmoe.so.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

__host__ __device__ constexpr int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

// Byte geometry of one packed matrix [rows][cols] (format v1 in moe.h).
struct MatGeom {
  int rows, cols, bits, group;
  __host__ __device__ int n_groups() const { return cols / group; }
  __host__ __device__ int unit_bytes() const { return bits * group / 8; }
  __host__ __device__ int chunks() const { return bits * group / 128; }
  __host__ __device__ int64_t codes_bytes() const {
    return (int64_t)(rows / 64) * n_groups() * 64 * unit_bytes();
  }
  __host__ __device__ int64_t scales_off() const { return align256(codes_bytes()); }
  __host__ __device__ int64_t bytes() const {
    return scales_off() + align256((int64_t)rows * n_groups() * 2);
  }
};

// Pointers read from the expert table are generic; loads through them would
// compile to flat loads, which also count against the scalar-load counter.  The
// blobs are device global memory, so they are cast to the global address space.
typedef const uint8_t __attribute__((address_space(1)))* gbytes_t;
typedef const uint16_t __attribute__((address_space(1)))* gu16_t;
__device__ __forceinline__ gbytes_t as_global(const void* p) { return (gbytes_t)p; }

// bfloat16 / fp16 helpers (bit patterns carried as uint16_t)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float scale_to_f32(uint16_t s, bool f16) {
  return f16 ? f16_to_f32(s) : bf16_to_f32(s);
}

// Force a uniform constant into a VGPR so that the bit-select below compiles to
// v_and_or_b32 (mask from an SGPR, magic from this VGPR) instead of two
// literal-operand instructions.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also orders global
// memory, which on gfx950 waits for every outstanding vector load (vmcnt(0)),
// including weight loads issued ahead on purpose; here only this wave's LDS
// operations are waited for.
// the wave's index in its block, as a wave-uniform (scalar) value
__device__ __forceinline__ int wv_of_thread() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- codecs
// The kernels are instantiated per codec (the template argument CODEC): 3-bit
// codes in groups of 128, 4-bit in groups of 32, 2-bit in groups of 128 and 4-bit
// in groups of 128.
constexpr int kQ3G128 = 3, kQ4G32 = 4, kQ2G128 = 2, kQ4G128 = 5;
__host__ inline int codec_of(int bits, int group) {
  if (bits == 3 && group == 128) return kQ3G128;
  if (bits == 4 && group == 32) return kQ4G32;
  if (bits == 2 && group == 128) return kQ2G128;
  if (bits == 4 && group == 128) return kQ4G128;
  return -1;
}

// ---------------------------------------------------------------- unit decode
// A unit (one row, one group of G codes) is decoded into G/2 registers, each a
// pair of bfloat16 values (B + c_{2P}, B + c_{2P+1}) for a per-pair constant B:
// the 3-bit code sits in the top mantissa bits of a bf16 whose exponent makes
// one code step equal 1.0, so OR-ing an exponent pattern onto the masked field
// yields B + c exactly.  B depends only on the field position:
//   field at bits 1..3 of a half -> pattern 0x4280 (64 + c)
//   field at bits 4..6           -> pattern 0x4100 (8 + c)
//   field at bits 0..2           -> pattern 0x4300 (128 + c)
// The dot product of these pairs with activations x therefore equals
//   sum_k (q_k + off_k) x_k,  off_k = B_k + 2^(bits-1),
// and the kernels subtract the per-group constant sum_k off_k x_k, computed once
// per activation vector and group.
template <int CODEC>
struct UnitCodec;

template <>
struct UnitCodec<kQ3G128> {
  static constexpr int BITS = 3, G = 128, WORDS = 12, CHUNKS = 3, PAIRS = 64;
  // offset of pair P: fields 0 and 2 of a word use B = 64, fields 1, 3, 4 use
  // B = 8, pairs 60..63 (the spare bits) use B = 128; zero point 4.
  __host__ __device__ static constexpr float pair_off(int P) {
    return P >= 60 ? 132.f : ((P % 5 == 0 || P % 5 == 2) ? 68.f : 12.f);
  }
  // visit (P, pair) in order, expanding each pair right before its use
  template <class F>
  __device__ __forceinline__ static void for_each_pair(const uint32_t (&w)[WORDS], F&& f) {
    const uint32_t m64 = in_vgpr(0x42804280u), m8 = in_vgpr(0x41004100u),
                   m128 = in_vgpr(0x43004300u);
#pragma unroll
    for (int d = 0; d < 12; ++d) {
      const uint32_t v = w[d];
      const uint32_t t = v >> 6;
      f(5 * d + 0, (v & 0x000E000Eu) | m64);
      f(5 * d + 1, (v & 0x00700070u) | m8);
      f(5 * d + 2, (t & 0x000E000Eu) | m64);
      f(5 * d + 3, (t & 0x00700070u) | m8);
      f(5 * d + 4, ((v >> 9) & 0x00700070u) | m8);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = w[3 * m], b = w[3 * m + 1], c = w[3 * m + 2];
      uint32_t v = (a & 0x00010001u) | m128;
      v |= (b << 1) & 0x00020002u;
      v |= (c << 2) & 0x00040004u;
      f(60 + m, v);
    }
  }
  __device__ __forceinline__ static void decode(const uint32_t (&w)[WORDS], uint32_t (&p)[PAIRS]) {
    const uint32_t m64 = in_vgpr(0x42804280u), m8 = in_vgpr(0x41004100u),
                   m128 = in_vgpr(0x43004300u);
#pragma unroll
    for (int d = 0; d < 12; ++d) {
      uint32_t v = w[d];
      uint32_t t = v >> 6;
      p[5 * d + 0] = (v & 0x000E000Eu) | m64;          // bits 1..3
      p[5 * d + 1] = (v & 0x00700070u) | m8;           // bits 4..6
      p[5 * d + 2] = (t & 0x000E000Eu) | m64;          // bits 7..9
      p[5 * d + 3] = (t & 0x00700070u) | m8;           // bits 10..12
      p[5 * d + 4] = ((v >> 9) & 0x00700070u) | m8;    // bits 13..15
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t a = w[3 * m], b = w[3 * m + 1], c = w[3 * m + 2];
      uint32_t v = (a & 0x00010001u) | m128;
      v |= (b << 1) & 0x00020002u;
      v |= (c << 2) & 0x00040004u;
      p[60 + m] = v;
    }
  }
};

// 4-bit codes, groups of G4 (32 or 128): word d holds pairs 4d .. 4d+3 at bit
// offsets 0, 4, 8, 12 of both halves; B = 128 (0x4300), zero point 8.
template <int G4>
struct UnitCodec4 {
  static constexpr int BITS = 4, G = G4, WORDS = G4 / 8, CHUNKS = G4 / 32, PAIRS = G4 / 2;
  __host__ __device__ static constexpr float pair_off(int) { return 136.f; }  // B 128, zero 8
  template <class F>
  __device__ __forceinline__ static void for_each_pair(const uint32_t (&w)[WORDS], F&& f) {
    const uint32_t m128 = in_vgpr(0x43004300u);
#pragma unroll
    for (int d = 0; d < WORDS; ++d) {
#pragma unroll
      for (int k = 0; k < 4; ++k) f(4 * d + k, ((w[d] >> (4 * k)) & 0x000F000Fu) | m128);
    }
  }
  __device__ __forceinline__ static void decode(const uint32_t (&w)[WORDS], uint32_t (&p)[PAIRS]) {
    const uint32_t m128 = in_vgpr(0x43004300u);
#pragma unroll
    for (int d = 0; d < WORDS; ++d) {
#pragma unroll
      for (int f = 0; f < 4; ++f) p[4 * d + f] = ((w[d] >> (4 * f)) & 0x000F000Fu) | m128;
    }
  }
};
template <>
struct UnitCodec<kQ4G32> : UnitCodec4<32> {};
template <>
struct UnitCodec<kQ4G128> : UnitCodec4<128> {};

// 2-bit codes, groups of 128: word d holds pairs 8d .. 8d+7 at bit offsets 2k of
// both halves.  Fields at bits 0-1, 2-3, 4-5 of a half take the exponent
// patterns 0x4300 (128 + c), 0x4200 (32 + c), 0x4100 (8 + c); the word shifted by
// 6 and by 12 brings the other fields to those positions.  Zero point 2.
template <>
struct UnitCodec<kQ2G128> {
  static constexpr int BITS = 2, G = 128, WORDS = 8, CHUNKS = 2, PAIRS = 64;
  __host__ __device__ static constexpr float pair_off(int P) {
    return (P % 8) % 3 == 0 ? 130.f : ((P % 8) % 3 == 1 ? 34.f : 10.f);
  }
  template <class F>
  __device__ __forceinline__ static void for_each_pair(const uint32_t (&w)[WORDS], F&& f) {
    const uint32_t m128 = in_vgpr(0x43004300u), m32 = in_vgpr(0x42004200u),
                   m8 = in_vgpr(0x41004100u);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t v = w[d], t = v >> 6, u = v >> 12;
      f(8 * d + 0, (v & 0x00030003u) | m128);
      f(8 * d + 1, (v & 0x000C000Cu) | m32);
      f(8 * d + 2, (v & 0x00300030u) | m8);
      f(8 * d + 3, (t & 0x00030003u) | m128);
      f(8 * d + 4, (t & 0x000C000Cu) | m32);
      f(8 * d + 5, (t & 0x00300030u) | m8);
      f(8 * d + 6, (u & 0x00030003u) | m128);
      f(8 * d + 7, (u & 0x000C000Cu) | m32);
    }
  }
  __device__ __forceinline__ static void decode(const uint32_t (&w)[WORDS], uint32_t (&p)[PAIRS]) {
    for_each_pair(w, [&](int P, uint32_t v) { p[P] = v; });
  }
};

// ---------------------------------------------------------------- unit loads (decode)
// Scales are stored in the codes' tile order: the scale of row 64*(tile's row
// block) + lane and the tile's group sits at index tile*64 + lane, so a wave's
// scales of one tile are 128 contiguous bytes.
// a codec's pair offsets (the pairs per group returned), for kernels that are
// not templated on the codec
template <class C>
__host__ inline int fill_pair_offsets(float* off) {
  for (int P = 0; P < C::PAIRS; ++P) off[P] = C::pair_off(P);
  return C::PAIRS;
}
__host__ inline int codec_pair_offsets(int codec, float* off) {
  switch (codec) {
    case kQ3G128: return fill_pair_offsets<UnitCodec<kQ3G128>>(off);
    case kQ4G32: return fill_pair_offsets<UnitCodec<kQ4G32>>(off);
    case kQ2G128: return fill_pair_offsets<UnitCodec<kQ2G128>>(off);
    case kQ4G128: return fill_pair_offsets<UnitCodec<kQ4G128>>(off);
    default: return 0;
  }
}

__device__ __forceinline__ int64_t scale_idx(int64_t tile, int lane) { return tile * 64 + lane; }
// A 16-bit scale is fetched as the aligned dword that contains it (the scales
// region is 256-byte aligned, so the dword lies inside it; lanes 2i and 2i+1 load
// the same dword) and selected at use by the index's parity (the lane's).
__device__ __forceinline__ uint32_t load_scale_dword(gu16_t sc, int64_t idx) {
  typedef const uint32_t __attribute__((address_space(1)))* gu32_t;
  return *(gu32_t)(sc + (idx & ~(int64_t)1));
}
__device__ __forceinline__ uint16_t scale_from_dword(uint32_t w, int64_t idx) {
  return (uint16_t)(w >> ((idx & 1) * 16));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CODEC>
__device__ __forceinline__ void load_unit4(gbytes_t codes, int64_t tile, int lane,
                                           u32x4 (&w)[UnitCodec<CODEC>::CHUNKS]) {
  using C = UnitCodec<CODEC>;
  typedef const u32x4 __attribute__((address_space(1)))* gu4_t;
#pragma unroll
  for (int j = 0; j < C::CHUNKS; ++j)
    w[j] = *(gu4_t)(codes + (tile * C::CHUNKS + j) * 1024 + 16 * lane);
}

// The unit's words, passed through an empty asm so that the decode that follows
// stays inside the token loop (hoisting every group's decoded pairs out of it
// would need GPW * 128 registers).
template <int CODEC>
__device__ __forceinline__ void unit_words(const u32x4 (&c)[UnitCodec<CODEC>::CHUNKS],
                                           uint32_t (&w)[UnitCodec<CODEC>::WORDS]) {
#pragma unroll
  for (int j = 0; j < UnitCodec<CODEC>::CHUNKS; ++j) {
    w[4 * j + 0] = c[j].x;
    w[4 * j + 1] = c[j].y;
    w[4 * j + 2] = c[j].z;
    w[4 * j + 3] = c[j].w;
  }
#pragma unroll
  for (int k = 0; k < UnitCodec<CODEC>::WORDS; ++k) asm volatile("" : "+v"(w[k]));
}

// Sum over the 64 lanes in a fixed order (row prefix sums by DPP, then the row
// totals), returned to every lane; deterministic, no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_shift(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CODEC>
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += dpp_shift<0x111>(v);  // row_shr:1
  v += dpp_shift<0x112>(v);  // row_shr:2
  v += dpp_shift<0x114>(v);  // row_shr:4
  v += dpp_shift<0x118>(v);  // row_shr:8
  v += dpp_shift<0x142>(v);  // row_bcast:15
  v += dpp_shift<0x143>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---------------------------------------------------------------- RMSNorm (unit gain)
// y = bf16(x / sqrt(mean(x^2) + eps)) of a row of H fp32 (H % 4 == 0, H <= 8192)
// by a block of 256 threads: thread i holds float4 items i + 256*j (j ascending)
// and sums their squares by fused multiply-adds in component order; the wave
// sums are fixed-order DPP reductions, and the four waves' sums are added in wave
// order.  The normalisation kernel and the routing kernels that normalise their
// own input all use these functions, so they produce the same bf16 rows.
constexpr int kRnPieces = 8;
typedef float rn_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float rms_wave_sum(const rn_f4 (&v)[kRnPieces], int H4) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kRnPieces; ++i)
    if ((int)threadIdx.x + 256 * i < H4) {
      ss = fmaf(v[i].x, v[i].x, ss);
      ss = fmaf(v[i].y, v[i].y, ss);
      ss = fmaf(v[i].z, v[i].z, ss);
      ss = fmaf(v[i].w, v[i].w, ss);
    }
  // the wave sum by DPP row prefixes and row totals (no LDS round trips)
  ss += dpp_shift<0x111>(ss);
  ss += dpp_shift<0x112>(ss);
  ss += dpp_shift<0x114>(ss);
  ss += dpp_shift<0x118>(ss);
  ss += dpp_shift<0x142>(ss);
  ss += dpp_shift<0x143>(ss);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss), 63));
}
// part[w] = wave w's sum
__device__ __forceinline__ float rms_inv(const float* part, int H, float eps) {
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  return 1.f / sqrtf(tot / (float)H + eps);
}
__device__ __forceinline__ uint32_t rms_bf16x2(float a, float b, float inv) {
  return f32_to_bf16_rne(a * inv) | ((uint32_t)f32_to_bf16_rne(b * inv) << 16);
}

// ---------------------------------------------------------------- cross-block hand-off
// Kernels whose last-arriving block finishes the work.  The ordering argument:
// (1) the blocks' results go out as agent-scope relaxed atomic stores, emitted
// with the agent-scope cache policy, i.e. written through the XCD's L2 to the
// memory side that every XCD shares; (2) each wave waits until its own stores
// have completed (vmcnt(0): a write-through store retires when the coherence
// point acknowledges it), and a block barrier orders all four waves before
// thread 0 (3) takes its ticket, an agent-scope atomic add performed at that
// same coherence point, whose total order puts every other block's completed
// stores before the last ticket (a two-level ticket chains this: a group's
// last block counts at the next level only after its group ticket returned);
// (4) the last block reads the results with
// agent-scope atomic loads, which are not served from its own L2 and so cannot
// see a stale line; (5) the signal fences around the wait and the branch on the
// ticket (read back through LDS after a barrier) keep the compiler from moving
// the stores after, or the loads before, these points.  There is no cache-wide
// fence: a device-scope __threadfence() (or an acq_rel ticket) writes back and
// invalidates the block's whole L2, microseconds per block when hundreds of
// blocks do it, and orders nothing more here since every datum the hand-off
// carries is itself written and read at agent scope.
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coherent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// ticket of a block (called by one thread after every wave's wait_stores and a
// block barrier): the arrival count before this block
__device__ __forceinline__ int take_ticket(int32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- workspace
// The workspace's leading region (MOE_WS_COUNTER_BYTES, kept zero between calls
// apart from the error word).  Counters for cross-block signalling: the block
// that finds itself last to arrive does a kernel's final step and resets the
// counter.  [kCtrRoute]: the routing kernel of small batches, whose blocks first
// count in kRouteGroups group counters at [kCtrRouteGrp + g*kCtrStride].  Each
// counter has a 128-byte line of its own: agent-scope atomics on one line are
// performed one after another at the memory side (about 11 ns each here), so
// 144 arrivals on one counter spread over 1.6 us.  From int32 index kFxAcc: the
// one/two-token combine's accumulator words, uint64[2][kMaxStrips * 64] (token,
// output column), each zeroed again by the lane that completes it.
constexpr int kCtrStride = 32;
constexpr int kCtrRoute = 0;
constexpr int kCtrRouteGrp = kCtrStride;
constexpr int kRouteGroups = 16;
constexpr int kMaxStrips = 160;  // H <= 10240 for the fused combine
constexpr int kFxAcc = 1024;
constexpr int kCounters = MOE_WS_COUNTER_BYTES / 4;
static_assert(kCtrRouteGrp + kRouteGroups * kCtrStride <= kFxAcc, "counter region");
static_assert(kFxAcc * 4 + 2 * kMaxStrips * 64 * 8 == MOE_WS_COUNTER_BYTES, "accumulator region");
// Two words of the same region are not counters.  [kCtrError] is the
// workspace's error word (byte offset 4, MOE_WS_ERROR_OFFSET in moe.h): bit 0 is
// set, and stays set, when moe_forward finds caller-supplied routing
// inconsistent; only moe_workspace_init or the caller clears it.  [kCtrCallBad]
// is the current call's verdict on its routing: written once per moe_forward by
// the kernel that checks the routing, read by the kernels that write the
// caller's outputs, which then write nothing.
constexpr int kCtrError = 1;
constexpr int kCtrCallBad = 2;
static_assert(kCtrError * 4 == MOE_WS_ERROR_OFFSET, "error word offset");
// the error word's bit for a matrix-core (prefill) call that met a value fp16
// cannot hold exactly (a group scale, or h = silu(g)*u)
constexpr int kErrRange = 4;
static_assert(kErrRange == MOE_ERR_RANGE, "error bit");
constexpr int kErrCombine = 8;
static_assert(kErrCombine == MOE_ERR_COMBINE, "error bit");

// ---------------------------------------------------------------- routing check
// Caller-supplied routing is consistent when offsets[0] == 0, the offsets never
// decrease, offsets[E] equals the number of pairs whose id lies in [0, E), and
// every grouped position i < offsets[E] holds a pair p in [0, P) whose id e has
// offsets[e] <= i < offsets[e+1], the pairs of one expert ascending.  Then
// sorted_pairs[0 .. offsets[E]) lists exactly the pairs with a valid id, grouped
// by expert and stable by pair index, as moe_route writes them.
//
// One wave checks P <= 64 pairs (every lane returns the verdict); E <= 1024.
// routing_ok_regs takes the raw offsets already in registers (lo[c] =
// offsets[lane + 64c], hi[c] = offsets[lane + 64c + 1] for lane + 64c < E) and the
// lane's id = ids[lane], s = sorted_pairs[lane], sprev = sorted_pairs[lane - 1]
// (-1, 0, -1 for lanes at or past P; sprev -1 for lane 0).
__device__ __forceinline__ bool routing_ok_regs(const int (&lo)[16], const int (&hi)[16], int id,
                                                int s, int sprev, int P, int E) {
  const int lane = threadIdx.x & 63;
  const int nch = (E + 63) / 64;
  bool bad = false;
  int oE = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    if (c < nch) {
      bad |= lane + 64 * c < E && hi[c] < lo[c];
      const int last = __shfl(hi[c], (E - 1) & 63);  // offsets[E] sits in chunk (E-1)/64
      if (c == (E - 1) >> 6) oE = last;
    }
  }
  bad |= lane == 0 && lo[0] != 0;
  const int nvalid = __popcll(__ballot(id >= 0 && id < E));
  bad |= oE != nvalid;
  // the expert of the pair at position `lane` and its segment (shuffles: every lane)
  const int e = __shfl(id, min(max(s, 0), 63));
  const int ec = min(max(e, 0), E - 1);
  int elo = 0, ehi = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    if (c < nch) {
      const int a = __shfl(lo[c], ec & 63), b = __shfl(hi[c], ec & 63);
      if ((ec >> 6) == c) {
        elo = a;
        ehi = b;
      }
    }
  }
  if (lane < oE && oE <= P)
    bad |= s < 0 || s >= P || e < 0 || e >= E || lane < elo || lane >= ehi ||
           (lane > elo && sprev >= s);
  return __ballot(bad) == 0;
}

// Record a call's verdict (one writer per call) and, for a bad one, set the
// sticky error bit.
__device__ __forceinline__ void record_routing(int32_t* ctr, bool ok) {
  ctr[kCtrCallBad] = ok ? 0 : 1;
  if (!ok) atomicOr(ctr + kCtrError, 1);
}


// Batches up to this many tokens run the GEMV (decode) kernels; larger ones the
// matrix-core (prefill) kernels when the shape allows them.
constexpr int kDecodeMaxTokens = 64;
// slices of the shared expert's output that a combine reads (its down kernel's split)
constexpr int kMaxShared = 2;
constexpr int kPrefillTileRows = 128;  // sorted pair positions per prefill tile
__host__ __device__ inline bool prefill_eligible(const moe_cfg& c, int T) {
  return T > kDecodeMaxTokens && c.hidden % 128 == 0 && c.inter % 128 == 0;
}
// upper bound of the prefill tile count: ceil(n_e / 128) summed over the experts
__host__ __device__ inline int64_t prefill_max_tiles(int64_t P, int64_t E) {
  return (P + kPrefillTileRows - 1) / kPrefillTileRows + (E < P ? E : P);
}

// Reduction groups per decode GEMV work item (gate/up, down): three each, which
// keeps the kernels free of register spills at three waves per SIMD.
constexpr int kDecGPW = 3;
constexpr int kDecGPWd = 3;

// Layout of the caller's workspace for T tokens (byte offsets, 256-aligned).
// Regions a mode does not use have size 0.
// an active expert as the decode kernels use it: logical id (-1: none), its
// first sorted position and pair count, and its table entry; pad holds U, the
// number of active experts, where the one/two-token kernels store it
struct ActEntry {
  int32_t e, seg0, n, pad;
  const void* ptr[3];  // gate, up, down
};

constexpr int kActHdrBytes = 64;  // the decode plan's header (U), then the entries
struct WsLayout {
  int64_t counters;   // int32[kCounters]: zero between calls
  int64_t logits;     // double[T][E]
  int64_t ghist;      // int32[ceil(P/1024)][E]: per-chunk expert counts, then bases (grouping)
  int64_t act;        // decode: int32 U (64-byte header), then the active-expert list (40 B each)
  int64_t osx;        // decode: float[T][H/G]: per token and reduction group, the offset sum
                      //   sum_P off_P (x_2P + x_2P+1) of the gate/up codec
  int64_t osh;        // decode: float[P][I/G]: the same for the down codec, per sorted
                      //   position and group, over h hi + lo
  int64_t gpart;      // decode: float[2*NCH][P][I]: gate then up partial products per
                      //   chunk of reduction groups, rows by sorted position
  int64_t hdec;       // decode: bf16[2][P][I]: h hi rows, then h lo rows, by sorted position
  int64_t dpart;      // decode: float[NCHd][P][H]: down partial products per chunk, rows by pair
  int64_t x16;        // prefill: fp16[T][H] activations scaled by 2^-xshift[t]
  int64_t xshift;     // prefill: int32[T]
  int64_t h16;        // prefill: fp16[P][I] h rows by sorted position
  int64_t tiles;      // prefill: int32[1 + 2*max_tiles] tile plan
  int64_t vchk;       // prefill: int32[2][ceil(max(P, E) / 256)]: per block of the routing
                      //   check, the valid-id pair count and an error flag
  int64_t pair_out;   // float[P][H] (used when the caller passes no pair_out)
  int64_t sh_part;    // float[2*4][T][Is]: shared gate and up partial sums per slice
  int64_t sh_h;       // float[T][Is]: shared expert h
  int64_t sh_out;     // float[2][T][H]: shared expert output slices
  int64_t total;
};

static_assert(sizeof(ActEntry) == 40, "active-expert entries are 40 bytes");
__host__ inline ActEntry* act_entries(uint8_t* ws, const WsLayout& L) {
  return reinterpret_cast<ActEntry*>(ws + L.act + kActHdrBytes);
}

__host__ inline WsLayout ws_layout(const moe_cfg& c, int T) {
  WsLayout L{};
  int64_t P = (int64_t)T * c.top_k;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    int64_t r = o;
    o += align256(bytes > 0 ? bytes : 0);
    return r;
  };
  L.counters = take(kCounters * 4);
  L.logits = take((int64_t)T * c.n_experts * 8);
  L.ghist = take((P + 1023) / 1024 * c.n_experts * 4);
  const bool pf = prefill_eligible(c, T);
  // chunks of kDecGPW (gate/up) and kDecGPWd (down) reduction groups per decode work item
  const int64_t nch_gu = (c.hidden / c.group + kDecGPW - 1) / kDecGPW;
  const int64_t nch_dn = (c.inter / c.group + kDecGPWd - 1) / kDecGPWd;
  L.act = take(pf ? 0 : kActHdrBytes + 40 * (int64_t)c.n_experts);
  L.osx = take(pf ? 0 : (int64_t)T * (c.hidden / c.group) * 4);
  L.osh = take(pf ? 0 : P * (c.inter / c.group) * 4);
  L.gpart = take(pf ? 0 : 2 * nch_gu * P * c.inter * 4);
  L.hdec = take(pf ? 0 : 2 * P * c.inter * 2);
  L.dpart = take(pf ? 0 : nch_dn * P * c.hidden * 4);
  L.x16 = take(pf ? (int64_t)T * c.hidden * 2 : 0);
  L.xshift = take(pf ? (int64_t)T * 4 : 0);
  L.h16 = take(pf ? P * c.inter * 2 : 0);
  L.tiles = take(pf ? (1 + 2 * prefill_max_tiles(P, c.n_experts)) * 4 : 0);
  L.vchk = take(pf ? 2 * ((std::max<int64_t>(P, c.n_experts) + 255) / 256) * 4 : 0);
  L.pair_out = take(pf ? P * c.hidden * 4 : 0);
  L.sh_part = take(8 * (int64_t)T * c.shared_inter * 4);
  L.sh_h = take((int64_t)T * c.shared_inter * 4);
  L.sh_out = take(2 * (int64_t)T * c.hidden * 4);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------- phase trace
// Builds with -DMOE_TRACE only: thread 0 of a block stores the constant-rate
// real-time counter (100 MHz) at named points of a kernel into a per-source
// device array, which moe_trace_read_<source> copies to the host.  Other builds
// compile the marks to nothing.
#ifdef MOE_TRACE
#define MOE_TRACE_DECL static __device__ unsigned long long g_moe_trace[1 << 15];
#define MOE_TR(slot)                                                           \
  do {                                                                         \
    if (threadIdx.x == 0) g_moe_trace[(slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
// the same, by lane 0 of each wave
#define MOE_TRW(slot)                                                                  \
  do {                                                                                 \
    if ((threadIdx.x & 63) == 0) g_moe_trace[(slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define MOE_TRACE_EXPORT(name)                                                             \
  extern "C" int moe_trace_read_##name(void* dst, size_t n) {                              \
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_moe_trace), n, 0, hipMemcpyDeviceToHost); \
  }
#else
#define MOE_TRACE_DECL
#define MOE_TR(slot) \
  do {               \
  } while (0)
#define MOE_TRW(slot) \
  do {                \
  } while (0)
#define MOE_TRACE_EXPORT(name)
#endif

// ---------------------------------------------------------------- profiling
enum KernelId {
  KID_LOGITS = 0, KID_TOPK, KID_PERMUTE, KID_PLAN, KID_GATEUP, KID_DOWN, KID_SH_GATEUP,
  KID_SH_DOWN, KID_COMBINE, KID_RMSNORM, KID_ZERO, KID_XPREP, KID_SWIGLU, KID_ROUTE, KID_TABLE,
  KID_CACHE, KID_STREAM, KID_COUNT
};
// when profiling is on: a pair of events for the next launch of kernel kid
bool prof_events(int kid, hipEvent_t* b, hipEvent_t* e);

// launch a kernel; when profiling is on, with start and end events that the
// launch itself timestamps
#define MOE_LAUNCH(kid, kernel, grid, block, shmem, stream, ...)                          \
  do {                                                                                    \
    hipEvent_t _moe_b, _moe_e;                                                            \
    if (::moe::prof_events(kid, &_moe_b, &_moe_e))                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, _moe_b, _moe_e, 0, __VA_ARGS__); \
    else                                                                                  \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                \
  } while (0)

// ---------------------------------------------------------------- launchers
struct FwdArgs {
  const moe_cfg* c;
  const moe_expert_ref* table;  // this layer's device table
  const void* sg;               // shared expert (or null)
  const void* su;
  const void* sd;
  const uint16_t* x;
  int T;
  const int32_t* ids;
  const float* w;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  float* out;
  float* pair_out;              // null: workspace
  float* resid;                 // or null: resid[t] += out[t] as the combine writes out[t]
  uint8_t* ws;
  hipStream_t side;             // shared-expert stream, fork and join events (or null)
  hipEvent_t ev_fork, ev_join;
  int pre_entries = 0;          // the routing kernel stored the active experts' entries
};

hipError_t launch_prefill(const FwdArgs& f, const WsLayout& L, float* pair_out, hipStream_t s);
hipError_t launch_decode(const FwdArgs& f, const WsLayout& L, float* shared_out, int nsh,
                         hipEvent_t join, hipStream_t s);
hipError_t launch_shared(const FwdArgs& f, const WsLayout& L, hipStream_t s, float** out,
                         int* nslices);
// the routing input: bf16 rows x, or (resid != null) x = bf16(RMSNorm(resid)),
// formed by the routing kernels themselves and written to xn
struct RouteIn {
  const uint16_t* x;
  const float* resid;
  float eps;
  uint16_t* xn;
  // optional (a layer call): the layer's table; the one-launch routing then also
  // stores the active experts' entries at `entries`, and the routing of 3 to 8
  // tokens does the decode plan's work (the active list at act_hdr / entries and
  // the offset sums osx of the gate/up codec, whose pair offsets and group size
  // are given); either sets *wrote_entries
  const moe_expert_ref* table = nullptr;
  ActEntry* entries = nullptr;
  int* wrote_entries = nullptr;
  int32_t* act_hdr = nullptr;
  float* osx = nullptr;
  int32_t* ctr0 = nullptr;  // the workspace's counters (the routing verdict)
  int codec = 0;
};
// the decode plan's work done by the routing kernel of 3 to 8 tokens
struct PlanIn {
  const moe_expert_ref* table;
  int32_t* act_hdr;
  ActEntry* act;
  const uint16_t* x;  // the experts' input rows (bf16)
  float* osx;         // [T][H/G]
  int32_t* ctr0;
  int H, G, pairs;
  float off[64];      // the codec's pair offsets
};
hipError_t launch_route(const moe_cfg& c, const RouteIn& in, int T, const float* wr,
                        const float* bias, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_pairs, int32_t* pair_pos, double* logits,
                        int32_t* ghist, int32_t* counters, hipStream_t s);
hipError_t launch_forward(const FwdArgs& f, hipStream_t s);
hipError_t launch_rmsnorm(float* resid, const float* add, int T, int H, float eps, uint16_t* y,
                          hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_set_table(moe_expert_ref* dst, const moe_expert_ref* host, int n,
                            hipStream_t s);
int64_t cache_state_bytes(int E, int S);
hipError_t launch_cache_init(uint8_t* state, int E, int S, int policy, double decay,
                             uint64_t arena, int64_t slot_bytes, int64_t bytes_gu,
                             int64_t bytes_dn, const moe_expert_ref* host_home,
                             moe_expert_ref* table, hipStream_t s);
hipError_t launch_cache_step(const int32_t* offsets, moe_expert_ref* table, uint8_t* state,
                             hipStream_t s);

}  // namespace moe
