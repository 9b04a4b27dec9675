/* Runs every entry point of the CPU oracle on small seeded inputs, for a build of the oracle
 * under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py builds
 * and runs it). The inputs come from a plain 64-bit linear congruential generator and hold
 * none of the layer's arithmetic; the checks are the invariants the oracle must keep whatever
 * the data: routing weights sum to one and are positive, each token takes k distinct experts
 * in ascending order, the grouping is a permutation with exclusive-scan offsets, a zero
 * router gives experts 0..k-1 with equal weights, x = 0 gives y = 0, a code of 0 dequantises
 * to the bias and a code of 15 to 15 scale + bias, and every output is finite. Any failure, or
 * any report from the sanitizers, ends the program with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/moe_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 32);
}
/* uniform in [-1, 1) */
static double next_unit(void) { return (double)next_u32() / 2147483648.0 - 1.0; }
/* bf16 bit pattern of a float (truncation is enough for test data) */
static uint16_t bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int failures = 0;
#define CHECK(cond, ...)                       \
  do {                                         \
    if (!(cond)) {                             \
      fprintf(stderr, "FAIL: " __VA_ARGS__);   \
      fprintf(stderr, "\n");                   \
      ++failures;                              \
    }                                          \
  } while (0)

enum { H = 128, I = 64, E = 8, K = 2, S = 1, T = 5, NE = E + S };

int main(void) {
  /* int4 layer: codes [NE, rows, cols/2], scales and biases [NE, rows, cols/64] */
  const size_t n13q = (size_t)NE * 2 * I * (H / 2), n13s = (size_t)NE * 2 * I * (H / 64);
  const size_t n2q = (size_t)NE * H * (I / 2), n2s = (size_t)NE * H * (I / 64);
  uint8_t *w13_q = malloc(n13q), *w2_q = malloc(n2q);
  uint16_t *w13_s = malloc(2 * n13s), *w13_b = malloc(2 * n13s);
  uint16_t *w2_s = malloc(2 * n2s), *w2_b = malloc(2 * n2s);
  float *router_w = malloc(sizeof(float) * E * H), *router_b = malloc(sizeof(float) * E);
  for (size_t i = 0; i < n13q; ++i) w13_q[i] = (uint8_t)next_u32();
  for (size_t i = 0; i < n2q; ++i) w2_q[i] = (uint8_t)next_u32();
  for (size_t i = 0; i < n13s; ++i) {
    w13_s[i] = bf16_bits((float)(0.002 + 0.001 * fabs(next_unit())));
    w13_b[i] = bf16_bits((float)(-0.016 * fabs(next_unit())));
  }
  for (size_t i = 0; i < n2s; ++i) {
    w2_s[i] = bf16_bits((float)(0.002 + 0.001 * fabs(next_unit())));
    w2_b[i] = bf16_bits((float)(-0.016 * fabs(next_unit())));
  }
  for (int i = 0; i < E * H; ++i) router_w[i] = (float)(0.1 * next_unit());
  for (int e = 0; e < E; ++e) router_b[e] = (float)(0.01 * next_unit());
  oracle_layer L = {H, I, E, K, S, ORACLE_FMT_INT4_G64, router_w, router_b,
                    w13_q, w2_q, w13_s, w13_b, w2_s, w2_b, NULL, NULL};
  CHECK(oracle_check_layer(&L) == 0, "valid layer rejected");

  double x[T * H];
  for (int i = 0; i < T * H; ++i) x[i] = next_unit();
  for (int h = 0; h < H; ++h) x[(T - 1) * H + h] = 0.0; /* last token: x = 0 */

  double z[T * E], w[T * K], margin[T], y[T * H];
  int32_t ids[T * K], counts[E], offsets[E + 1], sorted_tok[T * K], slot_of[T * K];
  CHECK(oracle_logits(&L, x, T, z) == 0, "logits");
  CHECK(oracle_route(&L, x, T, ids, w, margin) == 0, "route");
  for (int t = 0; t < T; ++t) {
    double sum = 0.0;
    for (int j = 0; j < K; ++j) {
      CHECK(ids[t * K + j] >= 0 && ids[t * K + j] < E, "id out of range");
      CHECK(j == 0 || ids[t * K + j] > ids[t * K + j - 1], "ids not ascending");
      CHECK(w[t * K + j] > 0.0, "weight not positive");
      sum += w[t * K + j];
    }
    CHECK(fabs(sum - 1.0) <= 1e-15, "weights of token %d sum to %.17g", t, sum);
    CHECK(margin[t] >= 0.0, "negative margin");
  }
  CHECK(oracle_group(&L, ids, T, counts, offsets, sorted_tok, slot_of) == 0, "group");
  CHECK(offsets[0] == 0 && offsets[E] == K * T, "offsets ends");
  for (int e = 0; e < E; ++e) CHECK(offsets[e + 1] - offsets[e] == counts[e], "scan");
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int s = slot_of[t * K + j];
      CHECK(s >= 0 && s < K * T && sorted_tok[s] == t, "slot_of / sorted_tok disagree");
    }
  CHECK(oracle_moe(&L, x, T, y, 2) == 0, "moe");
  for (int i = 0; i < T * H; ++i) CHECK(isfinite(y[i]), "y not finite");
  for (int h = 0; h < H; ++h) CHECK(y[(T - 1) * H + h] == 0.0, "x = 0 does not give y = 0");
  double ex[H];
  CHECK(oracle_expert(&L, E, x, ex) == 0, "expert");

  /* zero router, no bias: every logit ties, experts 0..K-1 with weight 1/K */
  float *zero_w = calloc((size_t)E * H, sizeof(float));
  oracle_layer Lz = L;
  Lz.router_w = zero_w;
  Lz.router_b = NULL;
  CHECK(oracle_route(&Lz, x, T, ids, w, margin) == 0, "route (ties)");
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      CHECK(ids[t * K + j] == j, "tie not broken towards the lower id");
      CHECK(w[t * K + j] == 1.0 / K, "tied weights not equal");
    }

  /* dequantisation closed forms on one row of one group: codes 0 and 15 */
  uint8_t codes[32];
  memset(codes, 0, sizeof codes);
  codes[1] = 0xF0; /* element 3 = 15, element 2 = 0 */
  const uint16_t sc = bf16_bits(0.5f), bi = bf16_bits(-2.0f);
  double dq[64];
  CHECK(oracle_dequant(codes, &sc, &bi, 1, 64, dq) == 0, "dequant");
  CHECK(dq[0] == -2.0 && dq[2] == -2.0 && dq[3] == 15 * 0.5 - 2.0, "dequant closed form");

  /* RMSNorm and bf16 rounding */
  double nrm[T * H];
  uint16_t nb[T * H];
  CHECK(oracle_rmsnorm(x, T, H, 1e-6, nrm) == 0, "rmsnorm");
  oracle_round_bf16(nrm, T * H, nb);
  uint16_t xb[4] = {0x3F80, 0xBF80, 0x0000, 0x7F80};
  double xd[4];
  oracle_bf16_to_f64(xb, 4, xd);
  CHECK(xd[0] == 1.0 && xd[1] == -1.0 && xd[2] == 0.0 && isinf(xd[3]), "bf16 widening");

  /* decode attention: 4 query heads over 2 KV heads, 3 positions, D = 8 */
  enum { NQ = 4, NKV = 2, D = 8, CTX = 3 };
  double q[NQ * D], ao[NQ * D];
  uint16_t kc[NKV * CTX * D], vc[NKV * CTX * D];
  for (int i = 0; i < NQ * D; ++i) q[i] = next_unit();
  for (int i = 0; i < NKV * CTX * D; ++i) {
    kc[i] = bf16_bits((float)next_unit());
    vc[i] = bf16_bits((float)next_unit());
  }
  CHECK(oracle_attn_decode(q, kc, vc, NQ, NKV, D, CTX, CTX * D, 0.35, ao) == 0, "attention");
  for (int i = 0; i < NQ * D; ++i) CHECK(isfinite(ao[i]) && fabs(ao[i]) <= 1.0, "attention out");

  /* DeltaNet scan: 3 tokens, 1 key head, 2 value heads, d = 4 */
  enum { GT = 3, NK = 1, NV = 2, DK = 4, DV = 4 };
  uint16_t gq[GT * NK * DK], gk[GT * NK * DK], gv[GT * NV * DV];
  float al[GT * NV], be[GT * NV];
  double st[NV * DV * DK], go[GT * NV * DV];
  for (int i = 0; i < GT * NK * DK; ++i) {
    gq[i] = bf16_bits((float)next_unit());
    gk[i] = bf16_bits((float)(0.5 * next_unit()));
  }
  for (int i = 0; i < GT * NV * DV; ++i) gv[i] = bf16_bits((float)next_unit());
  for (int i = 0; i < GT * NV; ++i) {
    al[i] = (float)(0.5 + 0.4 * fabs(next_unit()));
    be[i] = (float)(0.5 * fabs(next_unit()));
  }
  memset(st, 0, sizeof st);
  CHECK(oracle_gdn_scan(gq, gk, gv, al, be, GT, NK, NV, DK, DV, st, go, 2) == 0, "gdn scan");
  for (int i = 0; i < GT * NV * DV; ++i) CHECK(isfinite(go[i]), "gdn out not finite");

  /* argument checks answer with -1 */
  CHECK(oracle_moe(&L, x, -1, y, 1) == -1, "negative T accepted");
  oracle_layer Lbad = L;
  Lbad.top_k = E + 1;
  CHECK(oracle_check_layer(&Lbad) == -1, "k > E accepted");

  free(zero_w);
  free(w13_q); free(w2_q); free(w13_s); free(w13_b); free(w2_s); free(w2_b);
  free(router_w); free(router_b);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitize driver: all checks passed\n");
  return 0;
}
