/* synth_host.c -- host side of the seeded synthetic input generator.
 *
 * Input generation only (no routed-MoE arithmetic).  Built with gcc
 * (-ffp-contract=off) into libsynth.so; loaded from Python with ctypes.
 * Large fills run in parallel with OpenMP; every element depends only on its
 * own counter, so the thread count never changes the bytes.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define SYNTH_FN static inline
#include "synth_core.h"

#define SYN_PI 3.14159265358979323846

uint64_t syn_stream_key(uint64_t seed, uint64_t layer, uint64_t field, uint64_t expert,
                        uint64_t matrix) {
  return syn_key(seed, layer, field, expert, matrix);
}

uint64_t syn_draw_at(uint64_t key, uint64_t i) { return syn_draw(key, i); }

/* nbytes must be a multiple of 4 */
void syn_fill_codes(uint8_t* dst, uint64_t nbytes, uint64_t seed, uint64_t layer,
                    uint64_t expert, uint64_t matrix) {
  uint64_t key = syn_key(seed, layer, SYN_CODES, expert, matrix);
  uint32_t* w = (uint32_t*)dst;
  int64_t nw = (int64_t)(nbytes / 4);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nw; ++j) w[j] = syn_code_word(key, (uint64_t)j);
}

void syn_fill_scales(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t layer, uint64_t expert,
                     uint64_t matrix, double lo, double width, int is_f16) {
  uint64_t key = syn_key(seed, layer, SYN_SCALES, expert, matrix);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) dst[j] = syn_scale(key, (uint64_t)j, lo, width, is_f16);
}

void syn_fill_uniform_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t layer,
                           uint64_t field, uint64_t expert, uint64_t matrix, double a) {
  uint64_t key = syn_key(seed, layer, field, expert, matrix);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) dst[j] = syn_uniform_bf16(key, (uint64_t)j, a);
}

/* Box-Muller normal sample j of stream key with standard deviation sd, in double. */
static double syn_normal(uint64_t key, uint64_t j, double sd) {
  uint64_t p = j >> 1;
  double u1 = 1.0 - syn_u01(syn_draw(key, 2 * p));   /* (0, 1] */
  double u2 = syn_u01(syn_draw(key, 2 * p + 1));     /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double z = (j & 1) ? r * sin(2.0 * SYN_PI * u2) : r * cos(2.0 * SYN_PI * u2);
  return z * sd;
}

/* normal(0, sd^2) rounded to binary32 then to bfloat16 (RNE) */
void syn_fill_normal_bf16(uint16_t* dst, uint64_t n, uint64_t seed, uint64_t layer,
                          uint64_t field, uint64_t expert, double sd) {
  uint64_t key = syn_key(seed, layer, field, expert, 0);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    dst[j] = syn_f32_to_bf16((float)syn_normal(key, (uint64_t)j, sd));
}

/* normal(0, sd^2) rounded to binary32 */
void syn_fill_normal_f32(float* dst, uint64_t n, uint64_t seed, uint64_t layer, uint64_t field,
                         uint64_t expert, double sd) {
  uint64_t key = syn_key(seed, layer, field, expert, 0);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) dst[j] = (float)syn_normal(key, (uint64_t)j, sd);
}

/* Seeded permutation of 0..n-1 by Fisher-Yates (Durstenfeld): for i = n-1 down
 * to 1 swap a[i] with a[draw(i) mod (i+1)]. */
void syn_permutation(int32_t* dst, int32_t n, uint64_t seed, uint64_t layer, uint64_t field) {
  uint64_t key = syn_key(seed, layer, field, 0, 0);
  for (int32_t i = 0; i < n; ++i) dst[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(syn_draw(key, (uint64_t)i) % (uint64_t)(i + 1));
    int32_t t = dst[i];
    dst[i] = dst[j];
    dst[j] = t;
  }
}
