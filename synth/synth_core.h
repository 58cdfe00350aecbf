/* synth_core.h -- seeded, counter-based synthetic input generator.
 *
 * Input generation only: this header holds none of the routed-MoE arithmetic.
 * It is included by the host generator (synth_host.c, built with gcc) and by the
 * device fill kernels (synth_dev.hip, built with hipcc); the includer defines
 * SYNTH_FN before including, so both compile the very same integer and IEEE
 * double operations and produce identical bytes.
 *
 * Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Output i of a stream with key k
 * is fin(k + (i + 1) * GAMMA), fin being the published 64-bit finaliser.  A stream
 * key is derived from (seed, layer, field, expert, matrix) by chaining fin().
 *
 * Only integer operations and correctly rounded IEEE double multiply/add are used
 * for anything generated on the device, so host and device agree bit for bit.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H
#include <stdint.h>

#ifndef SYNTH_FN
#error "define SYNTH_FN (function qualifiers) before including synth_core.h"
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

/* stream fields */
enum {
  SYN_CODES = 1,       /* packed code bytes of one matrix of one expert        */
  SYN_SCALES = 2,      /* group scales of one matrix of one expert             */
  SYN_X = 3,           /* activations                                          */
  SYN_ROUTER = 4,      /* router matrix                                        */
  SYN_BIAS_PERM = 5,   /* permutation that assigns Zipf ranks to experts       */
  SYN_SLOT_PERM = 6,   /* permutation of physical slots (pointer-table remap)  */
  SYN_SHARED = 7,      /* shared-expert bf16 weights                           */
  SYN_CODES_CONST = 8  /* reserved for structured tests                        */
};

SYNTH_FN uint64_t syn_fin(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* key of the stream (seed, layer, field, expert, matrix) */
SYNTH_FN uint64_t syn_key(uint64_t seed, uint64_t layer, uint64_t field,
                          uint64_t expert, uint64_t matrix) {
  uint64_t k = syn_fin(seed + SYNTH_GAMMA);
  k = syn_fin(k ^ (layer + 1) * SYNTH_GAMMA);
  k = syn_fin(k ^ (field + 1) * SYNTH_GAMMA);
  k = syn_fin(k ^ (expert + 1) * SYNTH_GAMMA);
  k = syn_fin(k ^ (matrix + 1) * SYNTH_GAMMA);
  return k;
}

/* output i of stream key */
SYNTH_FN uint64_t syn_draw(uint64_t key, uint64_t i) {
  return syn_fin(key + (i + 1) * SYNTH_GAMMA);
}

/* uniform double in [0, 1) with 53 random bits (exact) */
SYNTH_FN double syn_u01(uint64_t r) {
  return (double)(r >> 11) * 0x1.0p-53;
}

/* IEEE binary32 -> bfloat16, round to nearest even (no NaN inputs occur here) */
SYNTH_FN uint16_t syn_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* IEEE binary32 -> binary16, round to nearest even, for finite normal-range
 * inputs in [2^-14, 65504] in magnitude (the scales drawn here); exact bit ops. */
SYNTH_FN uint16_t syn_f32_to_f16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  uint32_t sign = (u >> 16) & 0x8000u;
  int32_t e = (int32_t)((u >> 23) & 0xFF) - 127 + 15;
  uint32_t m = u & 0x7FFFFFu;
  /* keep 10 mantissa bits, RNE on the 13 dropped bits */
  uint32_t half = ((uint32_t)e << 10) | (m >> 13);
  uint32_t rem = m & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (half & 1u))) half += 1u;
  return (uint16_t)(sign | half);
}

/* One 32-bit word of a packed code stream: word j takes the low (j even) or the
 * high (j odd) half of draw j/2.  Codes drawn uniformly over all 2^bits values
 * make every packed bit i.i.d. uniform, so the packed bytes are uniform bytes. */
SYNTH_FN uint32_t syn_code_word(uint64_t key, uint64_t j) {
  uint64_t r = syn_draw(key, j >> 1);
  return (j & 1) ? (uint32_t)(r >> 32) : (uint32_t)r;
}

/* Scale j: uniform in [lo, lo + width) computed in double (one multiply, one
 * add, each correctly rounded), rounded to binary32, then to the 16-bit type
 * (is_f16 ? binary16 : bfloat16), both round-to-nearest-even. */
SYNTH_FN uint16_t syn_scale(uint64_t key, uint64_t j, double lo, double width, int is_f16) {
  double u = syn_u01(syn_draw(key, j));
  double p = u * width;
  double d = lo + p;
  float f = (float)d;
  return is_f16 ? syn_f32_to_f16(f) : syn_f32_to_bf16(f);
}

/* Shared-expert weight j: uniform in [-a, a) as 2*a*u - a in double, to binary32,
 * to bfloat16 (RNE). */
SYNTH_FN uint16_t syn_uniform_bf16(uint64_t key, uint64_t j, double a) {
  double u = syn_u01(syn_draw(key, j));
  double p = u * (2.0 * a);
  double d = p - a;
  return syn_f32_to_bf16((float)d);
}

#endif /* SYNTH_CORE_H */
