/* moe_oracle.c -- plain CPU reference of the routed-expert MoE layer (fp64).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the benchmark's
 * CPU baseline, never by the product path. It shares no code with the HIP library.
 *
 * Source: "Optimizing On-Device Inference for Apple Silicon". Each function names
 * the section it follows. Readings taken where the page is silent:
 *   - softmax over the router logits, restricted to the k selected experts (the
 *     partition function of the full softmax cancels in the renormalisation);
 *   - selection is by logit, ties going to the lower expert id; ids are reported
 *     in ascending order;
 *   - the shared expert has routing weight 1 and the same SwiGLU shape;
 *   - int4 codes are unsigned 0..15, grouped by 64 consecutive elements along the
 *     reduction axis of each output row, low nibble first.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 64

static double bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void oracle_bf16_to_f64(const uint16_t *src, int64_t n, double *dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = bf16_to_double(src[i]);
}

int oracle_check_layer(const oracle_layer *L) {
  if (!L || L->hidden <= 0 || L->inter <= 0 || L->n_experts <= 0) return -1;
  if (L->top_k < 1 || L->top_k > L->n_experts) return -1;
  if (L->n_shared < 0 || L->n_shared > 1) return -1;
  if (!L->router_w) return -1;
  if (L->fmt == ORACLE_FMT_INT4_G64) {
    if (L->hidden % GROUP || L->inter % GROUP) return -1;
    if (!L->w13_q || !L->w13_s || !L->w13_b || !L->w2_q || !L->w2_s || !L->w2_b) return -1;
  } else if (L->fmt == ORACLE_FMT_F32) {
    if (!L->w13_f || !L->w2_f) return -1;
  } else {
    return -1;
  }
  return 0;
}

/* Section "Dequantize weights during matrix multiplication": one 4-bit code per
 * weight, one bf16 scale and one bf16 bias per group of 64 weights. */
static double dq_int4(const uint8_t *codes, const uint16_t *scale, const uint16_t *bias,
                      int64_t K, int64_t r, int64_t c) {
  uint8_t byte = codes[r * (K / 2) + c / 2];
  int q = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  int64_t g = r * (K / GROUP) + c / GROUP;
  return bf16_to_double(scale[g]) * (double)q + bf16_to_double(bias[g]);
}

int oracle_dequant(const uint8_t *codes, const uint16_t *scale, const uint16_t *bias,
                   int64_t rows, int64_t K, double *out) {
  if (!codes || !scale || !bias || !out || rows < 0 || K <= 0 || K % GROUP) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < K; ++c) out[r * K + c] = dq_int4(codes, scale, bias, K, r, c);
  return 0;
}

/* Element (r, c) of W13 (rows 2I, reduction H) or W2 (rows H, reduction I) of expert e. */
static double w13_at(const oracle_layer *L, int32_t e, int64_t r, int64_t c) {
  const int64_t H = L->hidden, I2 = 2 * (int64_t)L->inter;
  if (L->fmt == ORACLE_FMT_F32) return (double)L->w13_f[((int64_t)e * I2 + r) * H + c];
  const int64_t rows0 = (int64_t)e * I2;
  return dq_int4(L->w13_q + rows0 * (H / 2), L->w13_s + rows0 * (H / GROUP),
                 L->w13_b + rows0 * (H / GROUP), H, r, c);
}

static double w2_at(const oracle_layer *L, int32_t e, int64_t r, int64_t c) {
  const int64_t H = L->hidden, I = L->inter;
  if (L->fmt == ORACLE_FMT_F32) return (double)L->w2_f[((int64_t)e * H + r) * I + c];
  const int64_t rows0 = (int64_t)e * H;
  return dq_int4(L->w2_q + rows0 * (I / 2), L->w2_s + rows0 * (I / GROUP),
                 L->w2_b + rows0 * (I / GROUP), I, r, c);
}

/* Section "Qwen creates three distinct workload shapes": the router scores every
 * expert for a token. */
static void logits_one(const oracle_layer *L, const double *xt, double *z) {
  const int64_t H = L->hidden;
  for (int32_t e = 0; e < L->n_experts; ++e) {
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h) acc += xt[h] * (double)L->router_w[(int64_t)e * H + h];
    if (L->router_b) acc += (double)L->router_b[e];
    z[e] = acc;
  }
}

int oracle_logits(const oracle_layer *L, const double *x, int64_t T, double *z) {
  if (oracle_check_layer(L) || !x || !z || T < 0) return -1;
  for (int64_t t = 0; t < T; ++t) logits_one(L, x + t * L->hidden, z + t * L->n_experts);
  return 0;
}

/* Selects k experts from logits z: repeatedly take the largest logit not yet taken,
 * the lower id winning a tie. Weights are the softmax of the selected logits. */
static void select_one(const oracle_layer *L, const double *z, unsigned char *taken,
                       int32_t *ids, double *w, double *margin) {
  const int32_t E = L->n_experts, k = L->top_k;
  memset(taken, 0, (size_t)E);
  double kth = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || z[e] > z[best])) best = e;
    taken[best] = 1;
    kth = z[best];
  }
  if (margin) {
    int32_t next = -1;
    for (int32_t e = 0; e < E; ++e)
      if (!taken[e] && (next < 0 || z[e] > z[next])) next = e;
    *margin = next < 0 ? INFINITY : kth - z[next];
  }
  /* ascending id order */
  int32_t j = 0;
  double zmax = -INFINITY;
  for (int32_t e = 0; e < E; ++e)
    if (taken[e]) {
      ids[j++] = e;
      if (z[e] > zmax) zmax = z[e];
    }
  double denom = 0.0;
  for (j = 0; j < k; ++j) denom += exp(z[ids[j]] - zmax);
  for (j = 0; j < k; ++j) w[j] = exp(z[ids[j]] - zmax) / denom;
}

int oracle_route(const oracle_layer *L, const double *x, int64_t T, int32_t *ids,
                 double *w, double *margin) {
  if (oracle_check_layer(L) || !x || !ids || !w || T < 0) return -1;
  const int32_t E = L->n_experts, k = L->top_k;
  double *z = (double *)malloc(sizeof(double) * (size_t)E);
  unsigned char *taken = (unsigned char *)malloc((size_t)E);
  if (!z || !taken) {
    free(z);
    free(taken);
    return -1;
  }
  for (int64_t t = 0; t < T; ++t) {
    logits_one(L, x + t * L->hidden, z);
    select_one(L, z, taken, ids + t * k, w + t * k, margin ? margin + t : NULL);
  }
  free(z);
  free(taken);
  return 0;
}

/* Section "Keep expert routing on the GPU": a histogram of assignments per expert,
 * an exclusive prefix scan of the counts into start offsets, and a scatter that
 * places each assignment in its expert's contiguous range. */
int oracle_group(const oracle_layer *L, const int32_t *ids, int64_t T, int32_t *counts,
                 int32_t *offsets, int32_t *sorted_tok, int32_t *slot_of) {
  if (oracle_check_layer(L) || !ids || !counts || !offsets || T < 0) return -1;
  const int32_t E = L->n_experts, k = L->top_k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * k; ++i) {
    if (ids[i] < 0 || ids[i] >= E) return -1;
    counts[ids[i]]++;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  if (sorted_tok && slot_of) {
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!fill) return -1;
    for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t t = 0; t < T; ++t)
      for (int32_t j = 0; j < k; ++j) {
        int32_t e = ids[t * k + j];
        sorted_tok[fill[e]] = (int32_t)t;
        slot_of[t * k + j] = fill[e];
        fill[e]++;
      }
    free(fill);
  }
  return 0;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* Section "Reduce intermediate and state traffic": the two input projections with
 * their gated activation, then the output projection. scratch holds 2I doubles. */
static void expert_one(const oracle_layer *L, int32_t e, const double *x, double *out,
                       double *scratch) {
  const int64_t H = L->hidden, I = L->inter;
  double *a = scratch;
  for (int64_t i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      g += w13_at(L, e, i, h) * x[h];
      u += w13_at(L, e, I + i, h) * x[h];
    }
    a[i] = silu(g) * u;
  }
  for (int64_t j = 0; j < H; ++j) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) acc += w2_at(L, e, j, i) * a[i];
    out[j] = acc;
  }
}

int oracle_expert(const oracle_layer *L, int32_t e, const double *x, double *out) {
  if (oracle_check_layer(L) || !x || !out) return -1;
  if (e < 0 || e >= L->n_experts + L->n_shared) return -1;
  double *scratch = (double *)malloc(sizeof(double) * 2 * (size_t)L->inter);
  if (!scratch) return -1;
  expert_one(L, e, x, out, scratch);
  free(scratch);
  return 0;
}

/* The whole layer for each token: route, run the selected experts and the shared
 * expert, and sum their outputs weighted by the routing scores (shared weight 1). */
int oracle_moe(const oracle_layer *L, const double *x, int64_t T, double *y, int nthreads) {
  if (oracle_check_layer(L) || !x || !y || T < 0) return -1;
  const int64_t H = L->hidden, I = L->inter;
  const int32_t E = L->n_experts, k = L->top_k;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double *z = (double *)malloc(sizeof(double) * (size_t)E);
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *scratch = (double *)malloc(sizeof(double) * 2 * (size_t)I);
    int32_t ids[64];
    double w[64];
    if (!z || !taken || !o || !scratch || k > 64) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t t = 0; t < T; ++t) {
        const double *xt = x + t * H;
        double *yt = y + t * H;
        for (int64_t h = 0; h < H; ++h) yt[h] = 0.0;
        logits_one(L, xt, z);
        select_one(L, z, taken, ids, w, NULL);
        if (L->n_shared) {
          expert_one(L, E, xt, o, scratch);
          for (int64_t h = 0; h < H; ++h) yt[h] += o[h];
        }
        for (int32_t j = 0; j < k; ++j) {
          expert_one(L, ids[j], xt, o, scratch);
          for (int64_t h = 0; h < H; ++h) yt[h] += w[j] * o[h];
        }
      }
    }
    free(z);
    free(taken);
    free(o);
    free(scratch);
  }
  return failed ? -1 : 0;
}

int oracle_rmsnorm(const double *h, int64_t T, int32_t H, double eps, double *out) {
  if (!h || !out || T < 0 || H <= 0) return -1;
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int32_t i = 0; i < H; ++i) ss += h[t * H + i] * h[t * H + i];
    double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int32_t i = 0; i < H; ++i) out[t * H + i] = h[t * H + i] * inv;
  }
  return 0;
}

/* Round to the nearest bf16 value, ties to even (8 significant bits; below 2^-126 the
 * bf16 subnormal grid of spacing 2^-133). The stack of layers rounds each normalised row
 * to the activation dtype before the layer reads it; this is that rounding, done once
 * from the exact value. Every step below is exact in double except the one nearbyint. */
static uint16_t round_bf16_one(double v) {
  if (isnan(v)) return 0x7FC0;
  double r;
  if (fabs(v) < 0x1p-126) {
    r = nearbyint(v * 0x1p133) * 0x1p-133;
  } else {
    int e;
    const double m = frexp(v, &e); /* v = m 2^e, 0.5 <= |m| < 1 */
    r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
  }
  const float f = (float)r; /* exact (or +-inf past the bf16 range) */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

void oracle_round_bf16(const double *src, int64_t n, uint16_t *dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = round_bf16_one(src[i]);
}

/* Decode attention of one query token over a KV cache, grouped-query form ("Optimizing
 * On-Device Inference for Apple Silicon", sections "Qwen creates three distinct workload
 * shapes" -- query heads share key-value heads, eight to one -- and "Read the attention
 * cache efficiently"). Readings where the page is silent: query head h reads key-value
 * head h / (n_q / n_kv) (consecutive heads share one); scores are scale * q.k; the
 * weights are the softmax over all ctx cached positions. The largest score is subtracted
 * before exponentiating, which leaves the softmax unchanged in exact arithmetic.
 *   q    [n_q, D] fp64;  k, v  bf16 bit patterns, head g's row t at g * head_stride + t * D
 *   out  [n_q, D] fp64 */
int oracle_attn_decode(const double *q, const uint16_t *k, const uint16_t *v, int32_t n_q,
                       int32_t n_kv, int32_t D, int64_t ctx, int64_t head_stride, double scale,
                       double *out) {
  if (!q || !k || !v || !out || n_q <= 0 || n_kv <= 0 || n_q % n_kv || D <= 0 || ctx <= 0 ||
      head_stride < ctx * D)
    return -1;
  const int32_t G = n_q / n_kv;
  double *s = (double *)malloc((size_t)ctx * sizeof(double));
  if (!s) return -1;
  for (int32_t h = 0; h < n_q; ++h) {
    const int64_t base = (int64_t)(h / G) * head_stride;
    double m = -INFINITY;
    for (int64_t t = 0; t < ctx; ++t) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += q[(int64_t)h * D + d] * bf16_to_double(k[base + t * D + d]);
      s[t] = scale * dot;
      if (s[t] > m) m = s[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < ctx; ++t) {
      s[t] = exp(s[t] - m);
      z += s[t];
    }
    for (int32_t d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int64_t t = 0; t < ctx; ++t) acc += s[t] * bf16_to_double(v[base + t * D + d]);
      out[(int64_t)h * D + d] = acc / z;
    }
  }
  free(s);
  return 0;
}

/* Gated DeltaNet recurrence over T tokens ("Optimizing On-Device Inference for Apple
 * Silicon", sections "Qwen creates three distinct workload shapes" -- a learned gate decides
 * how much of the fixed-size state to keep, a delta update writes the current token -- and
 * "Keep recurrent state on chip": fp32 state and gate, bf16 queries and keys). Reading taken
 * where the page gives no formula: the gated delta rule
 *     S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,   o_t = S_t q_t,
 * with S of value head j a d_v x d_k matrix and value head j reading key head
 * j / (n_v / n_k) for q and k.
 *   q, k   bf16 bits [T, n_k, d_k];  v bf16 bits [T, n_v, d_v];  alpha, beta fp32 [T, n_v]
 *   state  fp64 [n_v, d_v, d_k]: S_0 on entry, S_T on return;  out fp64 [T, n_v, d_v] */
int oracle_gdn_scan(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                    const float *beta, int64_t T, int32_t n_k, int32_t n_v, int32_t d_k,
                    int32_t d_v, double *state, double *out, int nthreads) {
  if (!q || !k || !v || !alpha || !beta || !state || !out || T < 0 || n_k <= 0 || n_v <= 0 ||
      n_v % n_k || d_k <= 0 || d_v <= 0)
    return -1;
  const int32_t rep = n_v / n_k;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int32_t j = 0; j < n_v; ++j) {
    const int32_t kh = j / rep;
    double *S = state + (int64_t)j * d_v * d_k;
    double *kt = (double *)malloc((size_t)d_k * sizeof(double));
    double *qt = (double *)malloc((size_t)d_k * sizeof(double));
    if (!kt || !qt) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
      free(kt);
      free(qt);
      continue;
    }
    for (int64_t t = 0; t < T; ++t) {
      const double a = alpha[t * n_v + j], b = beta[t * n_v + j];
      for (int32_t e = 0; e < d_k; ++e) {
        kt[e] = bf16_to_double(k[(t * n_k + kh) * d_k + e]);
        qt[e] = bf16_to_double(q[(t * n_k + kh) * d_k + e]);
      }
      for (int32_t i = 0; i < d_v; ++i) {
        double *row = S + (int64_t)i * d_k;
        double sk = 0.0;
        for (int32_t e = 0; e < d_k; ++e) sk += row[e] * kt[e];
        const double c = b * (bf16_to_double(v[(t * n_v + j) * d_v + i]) - a * sk);
        double o = 0.0;
        for (int32_t e = 0; e < d_k; ++e) {
          row[e] = a * row[e] + c * kt[e];
          o += row[e] * qt[e];
        }
        out[(t * n_v + j) * d_v + i] = o;
      }
    }
    free(kt);
    free(qt);
  }
  return failed ? -1 : 0;
}
