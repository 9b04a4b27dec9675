/* moe_oracle.h -- plain CPU reference of the routed-expert MoE layer (fp64).
 *
 * TEST INFRASTRUCTURE ONLY. This oracle exists to check the HIP path. It may be
 * loaded only by the test suite, the package's smoke check and the benchmark's CPU
 * baseline; the product path never calls it and shares no code with it.
 *
 * What it computes follows "Optimizing On-Device Inference for Apple Silicon":
 *   - section "Qwen creates three distinct workload shapes": a router scores E experts
 *     and selects k of them, plus one shared expert that every token uses;
 *   - section "Dequantize weights during matrix multiplication": each weight is a
 *     4-bit code, every 64 consecutive weights share one bf16 scale and one bf16 bias,
 *     w = scale * code + bias;
 *   - section "Keep expert routing on the GPU": assignments are counted per expert,
 *     an exclusive prefix scan of the counts gives the group offsets, and rows are
 *     placed contiguously by expert;
 *   - section "Reduce intermediate and state traffic": an expert is two input
 *     projections with their gated activation (SwiGLU) and an output projection whose
 *     result is scaled by the routing score and summed with the shared-expert result.
 * Every value is exact input data widened to double; every sum is accumulated in
 * double in plain index order.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_FMT_F32 = 0, ORACLE_FMT_INT4_G64 = 1 };

typedef struct {
  int32_t hidden, inter, n_experts, top_k, n_shared, fmt;
  const float *router_w;              /* [E, H] */
  const float *router_b;              /* [E] or NULL */
  /* int4 group-64: codes [E+S, rows, K/2] (low nibble = even element), scale and bias
     as bf16 bit patterns [E+S, rows, K/64]; W13 rows 0..I-1 gate, I..2I-1 up. */
  const uint8_t *w13_q, *w2_q;
  const uint16_t *w13_s, *w13_b, *w2_s, *w2_b;
  /* fp32: W13 [E+S, 2I, H], W2 [E+S, H, I] */
  const float *w13_f, *w2_f;
} oracle_layer;

/* Returns 0 on success, -1 on an invalid layer or argument. */
int oracle_check_layer(const oracle_layer *L);

/* Widen bf16 bit patterns to double (exact). */
void oracle_bf16_to_f64(const uint16_t *src, int64_t n, double *dst);

/* Dequantise one int4 group-64 matrix [rows, K] to double: w = s*q + b. */
int oracle_dequant(const uint8_t *codes, const uint16_t *scale, const uint16_t *bias,
                   int64_t rows, int64_t K, double *out);

/* Router logits z[t,e] = sum_h x[t,h] * W_r[e,h] (+ b[e]). */
int oracle_logits(const oracle_layer *L, const double *x, int64_t T, double *z);

/* Top-k selection by (logit desc, id asc); softmax restricted to the selected logits.
 * ids[t,j] ascending expert id, w[t,j] the matching weight. margin[t] (optional) is
 * z_(k) - z_(k+1), the gap between the k-th and (k+1)-th largest logits. */
int oracle_route(const oracle_layer *L, const double *x, int64_t T, int32_t *ids,
                 double *w, double *margin);

/* Grouping of the T*k assignments by expert (stable: tokens ascending inside a group).
 * counts[E], offsets[E+1] (exclusive scan, offsets[E] = k*T), sorted_tok[k*T],
 * slot_of[T,k] = position of assignment (t,j) in sorted_tok. */
int oracle_group(const oracle_layer *L, const int32_t *ids, int64_t T, int32_t *counts,
                 int32_t *offsets, int32_t *sorted_tok, int32_t *slot_of);

/* One expert (SwiGLU) applied to one token: out[H] = W2 (silu(W1 x) * (W3 x)). */
int oracle_expert(const oracle_layer *L, int32_t e, const double *x, double *out);

/* Full layer: y[t] = shared(x_t) + sum_j w[t,j] * expert_{ids[t,j]}(x_t).
 * nthreads <= 0 uses the OpenMP default. */
int oracle_moe(const oracle_layer *L, const double *x, int64_t T, double *y, int nthreads);

/* RMSNorm with unit gain: out[t] = h[t] / sqrt(mean(h[t]^2) + eps). */
int oracle_rmsnorm(const double *h, int64_t T, int32_t H, double eps, double *out);

/* Round each value to the nearest bf16, ties to even (one rounding from the exact value);
 * returns bf16 bit patterns. */
void oracle_round_bf16(const double *src, int64_t n, uint16_t *dst);

/* Decode attention of one token: out[h] = softmax_t(scale * q[h].k[g, t]) v[g, t] with
 * g = h / (n_q / n_kv); k and v bf16 bit patterns, head g's row t at g * head_stride + t * D. */
int oracle_attn_decode(const double *q, const uint16_t *k, const uint16_t *v, int32_t n_q,
                       int32_t n_kv, int32_t D, int64_t ctx, int64_t head_stride, double scale,
                       double *out);

/* Gated DeltaNet recurrence: S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
 * o_t = S_t q_t per value head (state fp64 [n_v, d_v, d_k], S_0 in, S_T out); q, k bf16 bits
 * [T, n_k, d_k], v bf16 bits [T, n_v, d_v], alpha, beta [T, n_v]; out fp64 [T, n_v, d_v]. */
int oracle_gdn_scan(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                    const float *beta, int64_t T, int32_t n_k, int32_t n_v, int32_t d_k,
                    int32_t d_v, double *state, double *out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
