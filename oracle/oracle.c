/* oracle.c -- plain fp64 CPU oracle of the routed mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file's library; only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code with the HIP library: it reads the
 * packed weight bytes by its own reading of the format definition and computes
 * every step as written below, in double precision, in the plain order.
 *
 * What is computed (the routed-MoE layer of GLM-5.3-Flash-class models):
 *  - routing: top-8 of 288 experts per token per MoE layer (page "GLM-5.3-Flash
 *    EXL3 3.05bpw on 1x RTX 3090 -- RAM/NVMe expert tiering", field summary;
 *    page "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX PRO 6000 - GPU expert cache,
 *    host-RAM streaming", field config.expert_cache.layout).  The pages do not
 *    print the router function; it is read as a softmax over router logits with
 *    the top-k weights renormalised to sum to one, the logits being x.Wr^T plus
 *    an optional per-expert bias that takes part in both selection and weights.
 *  - grouping: the picks are grouped per expert (page "0xSero/glm53-flash-offload",
 *    paragraph "Elastic CLOCK expert cache": the picks are deduplicated per
 *    layer; paragraph "Batched decode": streams share the per-layer expert union).
 *  - experts: three matrices gate, up, down per expert, each reached through its
 *    own per-layer pointer table (RTX PRO 6000 page, field
 *    config.expert_cache.mechanism), combined as SwiGLU: h = silu(gate.x) * (up.x),
 *    y = down.h, silu(z) = z / (1 + exp(-z)).
 *  - combine: out[t] = sum over k (ascending) of w[t,k] * y[t,k], plus the
 *    always-on shared expert's output when present (glm53-flash-offload page,
 *    paragraph "Decode kernels (fast mode)": the shared expert is a separate
 *    expert computed beside the routed ones).
 *  - stack glue: x <- x + MoE(bf16(rmsnorm(x))), eps 1e-6, unit gain.
 *
 * Packed weight format (our own; the pages name their EXL3 codec but do not
 * define it).  A matrix W[N][Kd] (N outputs, Kd reduction), N % 64 == 0, in
 * groups of G consecutive reduction elements with one 16-bit scale per (row,
 * group); value W[n][k] = (c - 2^(bits-1)) * s[n][k/G] for the stored unsigned
 * code c.  The codes region is a sequence of tiles t = (n/64)*(Kd/G) + g, one per
 * 64 rows and one group; a tile holds 64 units (unit u = row 64*(n/64)+u) of
 * bits*G/8 bytes split into C = bits*G/128 chunks of 16 bytes: chunk j of tile t
 * starts at byte (t*C + j)*1024 and unit u's part of it at +16u; the unit's
 * 32-bit little-endian words are the chunks' words in order.  Scales follow at
 * the next 256-byte boundary in the same tile order: tile t holds the 64 scales
 * of its rows, s[n][g] at index t*64 + n%64.
 * Code i of a unit (reduction index g*G + i), P = i/2, half h = i%2:
 *   4-bit, G = 32 or 128 (4 or 16 words): c = (w[P/4] >> (16h + 4*(P%4))) & 15
 *   2-bit, G = 128 (8 words):  c = (w[P/8] >> (16h + 2*(P%8))) & 3
 *   3-bit, G = 128 (12 words): P < 60: c = (w[P/5] >> (16h + off[P%5])) & 7 with
 *                              off = {1,4,7,10,13};
 *                              P >= 60, m = P-60: bit b of c = bit 16h of w[3m+b].
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ threads */
/* OpenMP threads of the oracle's parallel loops (the CPU baseline is timed at the
 * host's full thread count and at one thread). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------ scalar types */
double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double orc_f16_to_double(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* double -> bfloat16 bits, round to nearest even, from the exact double value */
uint16_t orc_double_to_bf16(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0;
  int s = v < 0;
  double a = fabs(v);
  int e;
  double fr = frexp(a, &e);            /* a = fr * 2^e, fr in [0.5, 1) */
  /* bf16 normal: 8 significant bits; value = m * 2^(e-8), m in [128, 256) */
  double m = ldexp(fr, 8);
  double fl = floor(m);
  double rem = m - fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  double r = ldexp(fl, e - 8);
  float f = (float)r;                  /* exact: r has 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u >> 16) | (s ? 0x8000 : 0));
}

/* ------------------------------------------------------------ format reading */
typedef struct {
  int rows, cols, bits, group, scale_f16;
} orc_mat;

static int64_t orc_align256(int64_t n) { return (n + 255) / 256 * 256; }

static int64_t orc_codes_bytes(const orc_mat* m) {
  return (int64_t)(m->rows / 64) * (m->cols / m->group) * 64 * (m->bits * m->group / 8);
}

int64_t orc_matrix_bytes(int rows, int cols, int bits, int group) {
  orc_mat m = {rows, cols, bits, group, 0};
  return orc_align256(orc_codes_bytes(&m)) + orc_align256((int64_t)rows * (cols / group) * 2);
}

/* word w of the unit of (row n, group g) */
static uint32_t orc_unit_word(const uint8_t* blob, const orc_mat* m, int n, int g, int w) {
  int ng = m->cols / m->group;
  int C = m->bits * m->group / 128;
  int64_t t = (int64_t)(n / 64) * ng + g;
  int u = n % 64;
  int j = w / 4;
  int64_t off = (t * C + j) * 1024 + 16 * u + 4 * (w % 4);
  uint32_t v;
  memcpy(&v, blob + off, 4);
  return v;
}

/* unsigned code i of the unit of (row n, group g) */
int orc_code(const uint8_t* blob, int rows, int cols, int bits, int group, int n, int g, int i) {
  orc_mat m = {rows, cols, bits, group, 0};
  int P = i / 2, h = i % 2;
  if (bits == 4) {
    uint32_t w = orc_unit_word(blob, &m, n, g, P / 4);
    return (int)((w >> (16 * h + 4 * (P % 4))) & 15u);
  }
  if (bits == 2) {
    uint32_t w = orc_unit_word(blob, &m, n, g, P / 8);
    return (int)((w >> (16 * h + 2 * (P % 8))) & 3u);
  }
  if (bits == 3) {
    static const int off[5] = {1, 4, 7, 10, 13};
    if (P < 60) {
      uint32_t w = orc_unit_word(blob, &m, n, g, P / 5);
      return (int)((w >> (16 * h + off[P % 5])) & 7u);
    }
    int mm = P - 60, c = 0;
    for (int b = 0; b < 3; ++b) {
      uint32_t w = orc_unit_word(blob, &m, n, g, 3 * mm + b);
      c |= (int)((w >> (16 * h)) & 1u) << b;
    }
    return c;
  }
  return -1;
}

double orc_scale(const uint8_t* blob, int rows, int cols, int bits, int group, int scale_f16,
                 int n, int g) {
  orc_mat m = {rows, cols, bits, group, scale_f16};
  int ng = cols / group;
  /* scales in tile order: tile (n/64)*ng + g, 64 scales, row n%64 within it */
  int64_t off = orc_align256(orc_codes_bytes(&m)) + 2 * (((int64_t)(n / 64) * ng + g) * 64 + n % 64);
  uint16_t s;
  memcpy(&s, blob + off, 2);
  return scale_f16 ? orc_f16_to_double(s) : orc_bf16_to_double(s);
}

/* dequantised row n: out[k] = (c - 2^(bits-1)) * s[n][k/G] for k in [0, cols) */
void orc_dequant_row(const uint8_t* blob, int rows, int cols, int bits, int group, int scale_f16,
                     int n, double* out) {
  int ng = cols / group;
  int zero = 1 << (bits - 1);
  for (int g = 0; g < ng; ++g) {
    double s = orc_scale(blob, rows, cols, bits, group, scale_f16, n, g);
    for (int i = 0; i < group; ++i) {
      int c = orc_code(blob, rows, cols, bits, group, n, g, i);
      out[g * group + i] = (double)(c - zero) * s;
    }
  }
}

/* y[n] = sum_k W[n][k] * v[k], k ascending, fp64 */
void orc_matvec(const uint8_t* blob, int rows, int cols, int bits, int group, int scale_f16,
                const double* v, double* y) {
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
    for (int n = 0; n < rows; ++n) {
      orc_dequant_row(blob, rows, cols, bits, group, scale_f16, n, row);
      double acc = 0.0;
      for (int k = 0; k < cols; ++k) acc += row[k] * v[k];
      y[n] = acc;
    }
    free(row);
  }
}

/* y[n] = sum_k W[n][k] * v[k] for a row-major bfloat16 matrix, fp64 */
void orc_matvec_bf16(const uint16_t* W, int rows, int cols, const double* v, double* y) {
#pragma omp parallel for schedule(static)
  for (int n = 0; n < rows; ++n) {
    double acc = 0.0;
    for (int k = 0; k < cols; ++k) acc += orc_bf16_to_double(W[(int64_t)n * cols + k]) * v[k];
    y[n] = acc;
  }
}

/* ------------------------------------------------------------ routing */
/* Router logits, top-k and weights for T tokens.
 *   logits[t][e] = sum_h x[t][h] * Wr[e][h] (h ascending) + bias[e]
 *   top-k: experts ordered by logit descending, ties to the lower id; ids[t][k]
 *   lists the first K in that order.
 *   w[t][k] = exp(l_k - l_0) / sum_{j<K} exp(l_j - l_0): the softmax over all E
 *   experts restricted to the chosen K and renormalised (the common factor
 *   sum_e exp(l_e - l_0) cancels).
 * gap[t] (optional) = l_(K-1) - l_(K) in that order, the margin of the K-th pick
 * over the first expert left out (0 when K == E).
 * logits_out (optional) receives the T x E logits. */
void orc_route(int T, int H, int E, int K, const uint16_t* x_bf16, const float* Wr,
               const float* bias, int32_t* ids, double* w, double* gap, double* logits_out) {
#pragma omp parallel
  {
    double* l = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
          acc += orc_bf16_to_double(x_bf16[(int64_t)t * H + h]) * (double)Wr[(int64_t)e * H + h];
        l[e] = acc + (bias ? (double)bias[e] : 0.0);
        if (logits_out) logits_out[(int64_t)t * E + e] = l[e];
      }
      memset(taken, 0, (size_t)E);
      for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;  /* strict: lower id wins ties */
        taken[best] = 1;
        ids[t * K + k] = best;
      }
      double l0 = l[ids[t * K]];
      double den = 0.0;
      for (int k = 0; k < K; ++k) den += exp(l[ids[t * K + k]] - l0);
      for (int k = 0; k < K; ++k) w[t * K + k] = exp(l[ids[t * K + k]] - l0) / den;
      if (gap) {
        int next = -1;
        for (int e = 0; e < E; ++e)
          if (!taken[e] && (next < 0 || l[e] > l[next])) next = e;
        gap[t] = next < 0 ? 0.0 : l[ids[t * K + K - 1]] - l[next];
      }
    }
    free(l);
    free(taken);
  }
}

/* Grouping of the T*K picks by expert.  Pair p = t*K + k picks expert ids[p].
 * Pairs are listed expert by expert (ascending logical id) and, within an
 * expert, by ascending pair index:
 *   offsets[e] .. offsets[e+1]-1 are expert e's positions in sorted_pairs,
 *   sorted_pairs[i] = the pair at position i, pair_pos[p] = position of pair p.
 * Pairs whose id is outside [0, E) are left out (pair_pos = -1). */
void orc_permute(int T, int K, int E, const int32_t* ids, int32_t* offsets, int32_t* sorted_pairs,
                 int32_t* pair_pos) {
  int P = T * K, pos = 0;
  for (int p = 0; p < P; ++p) pair_pos[p] = -1;
  for (int e = 0; e < E; ++e) {
    offsets[e] = pos;
    for (int p = 0; p < P; ++p)
      if (ids[p] == e) {
        sorted_pairs[pos] = p;
        pair_pos[p] = pos;
        ++pos;
      }
  }
  offsets[E] = pos;
}

/* ------------------------------------------------------------ experts */
static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert on packed weights: y = down . (silu(gate.x) * (up.x)).
 * gate/up are [I][H], down is [H][I]. */
void orc_expert_ffn(int H, int I, int bits, int group, int scale_f16, const uint8_t* gate,
                    const uint8_t* up, const uint8_t* down, const double* x, double* y) {
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* u = (double*)malloc(sizeof(double) * (size_t)I);
  orc_matvec(gate, I, H, bits, group, scale_f16, x, g);
  orc_matvec(up, I, H, bits, group, scale_f16, x, u);
  for (int i = 0; i < I; ++i) g[i] = orc_silu(g[i]) * u[i];
  orc_matvec(down, H, I, bits, group, scale_f16, g, y);
  free(g);
  free(u);
}

/* The same FFN for n input vectors X[n][H] at once, Y[n][H]: each dequantised
 * row is formed once and applied to every vector, with the per-vector arithmetic
 * (k ascending, fp64) of orc_matvec, so Y[j] equals orc_expert_ffn of X[j] bit
 * for bit.  Only the tests use it, to check many pairs of one expert quickly. */
static void orc_matmul_rows(const uint8_t* blob, int rows, int cols, int bits, int group,
                            int scale_f16, int n, const double* V, double* Yt) {
  /* Yt[r][j] = sum_k W[r][k] * V[j][k] */
#pragma omp parallel
  {
    double* row = (double*)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
    for (int r = 0; r < rows; ++r) {
      orc_dequant_row(blob, rows, cols, bits, group, scale_f16, r, row);
      for (int j = 0; j < n; ++j) {
        const double* v = V + (int64_t)j * cols;
        double acc = 0.0;
        for (int k = 0; k < cols; ++k) acc += row[k] * v[k];
        Yt[(int64_t)r * n + j] = acc;
      }
    }
    free(row);
  }
}

void orc_expert_ffn_multi(int H, int I, int bits, int group, int scale_f16, const uint8_t* gate,
                          const uint8_t* up, const uint8_t* down, int n, const double* X,
                          double* Y) {
  double* g = (double*)malloc(sizeof(double) * (size_t)I * n);
  double* u = (double*)malloc(sizeof(double) * (size_t)I * n);
  double* h = (double*)malloc(sizeof(double) * (size_t)I * n);
  double* yt = (double*)malloc(sizeof(double) * (size_t)H * n);
  orc_matmul_rows(gate, I, H, bits, group, scale_f16, n, X, g);
  orc_matmul_rows(up, I, H, bits, group, scale_f16, n, X, u);
  for (int i = 0; i < I; ++i)
    for (int j = 0; j < n; ++j)
      h[(int64_t)j * I + i] = orc_silu(g[(int64_t)i * n + j]) * u[(int64_t)i * n + j];
  orc_matmul_rows(down, H, I, bits, group, scale_f16, n, h, yt);
  for (int r = 0; r < H; ++r)
    for (int j = 0; j < n; ++j) Y[(int64_t)j * H + r] = yt[(int64_t)r * n + j];
  free(g);
  free(u);
  free(h);
  free(yt);
}

/* Same FFN with row-major bfloat16 weights (the shared expert). */
void orc_shared_ffn(int H, int Is, const uint16_t* gate, const uint16_t* up, const uint16_t* down,
                    const double* x, double* y) {
  double* g = (double*)malloc(sizeof(double) * (size_t)Is);
  double* u = (double*)malloc(sizeof(double) * (size_t)Is);
  orc_matvec_bf16(gate, Is, H, x, g);
  orc_matvec_bf16(up, Is, H, x, u);
  for (int i = 0; i < Is; ++i) g[i] = orc_silu(g[i]) * u[i];
  orc_matvec_bf16(down, H, Is, g, y);
  free(g);
  free(u);
}

/* One routed-MoE layer for given routing.
 *   x_bf16 [T][H]; ids, w [T][K]; expert e's matrices at gate_tab[e], up_tab[e],
 *   down_tab[e] (the per-layer pointer tables, indexed by logical id).
 *   pair_out [T*K][H] (optional): y of pair p = t*K + k, before weighting.
 *   out [T][H] = sum_k w[t][k] * y[t*K+k] (k ascending) + shared(x_t) if given.
 * Pairs with an id outside [0, E) contribute nothing (pair_out row = 0). */
void orc_moe_layer(int T, int H, int I, int E, int K, int bits, int group, int scale_f16,
                   const uint16_t* x_bf16, const int32_t* ids, const double* w,
                   const uint8_t* const* gate_tab, const uint8_t* const* up_tab,
                   const uint8_t* const* down_tab, int Is, const uint16_t* sg,
                   const uint16_t* su, const uint16_t* sd, double* out, double* pair_out) {
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* y = (double*)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) xv[h] = orc_bf16_to_double(x_bf16[(int64_t)t * H + h]);
    for (int h = 0; h < H; ++h) out[(int64_t)t * H + h] = 0.0;
    for (int k = 0; k < K; ++k) {
      int p = t * K + k, e = ids[p];
      if (e < 0 || e >= E) {
        for (int h = 0; h < H; ++h) y[h] = 0.0;
      } else {
        orc_expert_ffn(H, I, bits, group, scale_f16, gate_tab[e], up_tab[e], down_tab[e], xv, y);
        for (int h = 0; h < H; ++h) out[(int64_t)t * H + h] += w[p] * y[h];
      }
      if (pair_out)
        for (int h = 0; h < H; ++h) pair_out[(int64_t)p * H + h] = y[h];
    }
    if (Is > 0 && sg) {
      orc_shared_ffn(H, Is, sg, su, sd, xv, y);
      for (int h = 0; h < H; ++h) out[(int64_t)t * H + h] += y[h];
    }
  }
  free(xv);
  free(y);
}

/* ------------------------------------------------------------ stack glue */
/* r = x / sqrt(mean(x^2) + eps) (unit gain) */
void orc_rmsnorm(int H, const double* x, double eps, double* r) {
  double ss = 0.0;
  for (int h = 0; h < H; ++h) ss += x[h] * x[h];
  double inv = 1.0 / sqrt(ss / H + eps);
  for (int h = 0; h < H; ++h) r[h] = x[h] * inv;
}

/* bf16 bits of rmsnorm(x) for T rows: the MoE input of one stack layer */
void orc_rmsnorm_bf16(int T, int H, const double* x, double eps, uint16_t* out) {
  double* r = (double*)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    orc_rmsnorm(H, x + (int64_t)t * H, eps, r);
    for (int h = 0; h < H; ++h) out[(int64_t)t * H + h] = orc_double_to_bf16(r[h]);
  }
  free(r);
}
