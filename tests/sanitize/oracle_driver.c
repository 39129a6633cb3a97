/* Drives every entry point of the fp64 CPU oracle (oracle/spec_oracle.h) over
 * small seeded inputs and their edge cases: rows that define no distribution
 * (all -inf, a NaN, a +inf), tokens outside [0, V), one-token rows, zero and
 * equal weights, filter parameters at and past their limits, one and several
 * OpenMP threads.  Built with AddressSanitizer and UndefinedBehaviorSanitizer
 * by tests/test_sanitizers_cpu.py; it checks return codes and the ranges of
 * the outputs only (the oracle's values are pinned elsewhere). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double unit(void) { /* xorshift64*, uniform in [0, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);    \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

static uint16_t bf16_of(float x) { /* truncation is enough for test rows */
  uint32_t b;
  memcpy(&b, &x, 4);
  return (uint16_t)(b >> 16);
}

/* rows [n][V] of logits 3*gauss-ish, in f32 or as bf16 codes */
static void *rows(int dtype, int64_t n, int V) {
  void *p = malloc((size_t)(n * V) * (dtype ? 2 : 4));
  for (int64_t i = 0; i < n * V; ++i) {
    float x = (float)(3.0 * (unit() + unit() + unit() - 1.5));
    if (dtype) ((uint16_t *)p)[i] = bf16_of(x);
    else ((float *)p)[i] = x;
  }
  return p;
}

static void set(void *p, int dtype, int64_t i, float x) {
  if (dtype) ((uint16_t *)p)[i] = bf16_of(x);
  else ((float *)p)[i] = x;
}

static void fill_row(void *p, int dtype, int64_t r, int V, float x) {
  for (int v = 0; v < V; ++v) set(p, dtype, r * V + v, x);
}

int main(void) {
  for (int dtype = 0; dtype <= 1; ++dtype) {
    for (int V = 1; V <= 300; V += 37) {
      const int B = 6, K = 4;
      const double T = 0.7;
      void *tgt = rows(dtype, (int64_t)B * (K + 1), V);
      void *dft = rows(dtype, (int64_t)B * K, V);
      int32_t tok[6 * 4];
      float uni[6 * 5];
      for (int i = 0; i < B * K; ++i) tok[i] = (int32_t)(unit() * V);
      for (int i = 0; i < B * (K + 1); ++i) uni[i] = (float)unit();
      tok[1 * K + 2] = V;  /* sequence 1: a token past V */
      tok[2 * K + 0] = -1; /* sequence 2: a negative token */
      fill_row(tgt, dtype, 3 * (K + 1) + 1, V, -INFINITY); /* sequence 3: no distribution */
      set(dft, dtype, (int64_t)(4 * K + 3) * V + V / 2, NAN);  /* sequence 4: a NaN */
      set(tgt, dtype, (int64_t)(5 * (K + 1)) * V, INFINITY);  /* sequence 5: a +inf */
      double ts[6 * 5 * 2], ds[6 * 4 * 2], probs[6 * 4 * 2], adist[6 * 4], ddist[6];
      int32_t nacc[6], out[6 * 5], nemit[6], kind[6];
      for (int nt = 1; nt <= 3; nt += 2) {
        CHECK(oracle_verify(tgt, dft, dtype, B, K, V, T, tok, uni, ts, ds, nacc, out, nemit,
                            probs, adist, ddist, kind, nt) == 0);
        for (int b = 0; b < B; ++b) {
          CHECK(nacc[b] >= -1 && nacc[b] <= K);
          if (nacc[b] >= 0) {
            CHECK(nemit[b] == nacc[b] + 1);
            CHECK(out[b * (K + 1) + nacc[b]] >= 0 && out[b * (K + 1) + nacc[b]] < V);
          }
        }
        CHECK(nacc[1] == -1 && nacc[2] == -1 && nacc[3] == -1 && nacc[4] == -1 && nacc[5] == -1);
      }
      int32_t n_in[6] = {0, K, -1, K + 1, 2, 1}, tk[6];
      CHECK(oracle_final_draw(tgt, dft, dtype, B, K, V, T, uni, n_in, tk, ddist, kind, 2) == 0);
      CHECK(tk[2] == -1 && tk[3] == -1);
      int32_t am[6 * 5];
      CHECK(oracle_greedy_verify(tgt, dtype, B, K, V, tok, am, nacc, out, nemit, 2) == 0);
      int32_t st[6 * 5];
      double sd[6 * 5];
      CHECK(oracle_sample_rows(tgt, dtype, (int64_t)B * (K + 1), V, T, uni, st, sd, 3) == 0);
      for (int i = 0; i < B * (K + 1); ++i) CHECK(st[i] >= -1 && st[i] < V);
      const int ks[] = {0, 1, 5, V, V + 3};
      const double ps[] = {1e-6, 0.5, 0.9, 1.0, 2.0};
      for (int a = 0; a < 5; ++a)
        for (int c = 0; c < 5; ++c) {
          double thr = 0.0;
          const int rc = oracle_filter_threshold(tgt, dtype, V, T, ks[a], ps[c], &thr);
          CHECK(rc == 0 && !isnan(thr));
        }
      double thr = 0.0;
      CHECK(oracle_filter_threshold(tgt, dtype, V, T, 3, 0.0, &thr) == -1);
      CHECK(oracle_filter_threshold(tgt, dtype, V, T, 3, NAN, &thr) == -1);
      double tthr[6 * 5], dthr[6 * 4];
      CHECK(oracle_verify_filtered(tgt, dft, dtype, B, K, V, T, 5, 0.9, tok, uni, tthr, dthr, ts,
                                   ds, nacc, out, nemit, probs, adist, ddist, kind, 2) == 0);
      int32_t idx = -5;
      CHECK(oracle_argmax_row(tgt, dtype, V, &idx) == 0 && idx >= 0 && idx < V);
      double M = 0.0, S = 0.0;
      double *prob = malloc(sizeof(double) * (size_t)V);
      CHECK(oracle_softmax_row(tgt, dtype, V, T, prob, &M, &S) == 0 && S >= 1.0);
      CHECK(oracle_softmax_row((char *)tgt + (size_t)(3 * (K + 1) + 1) * V * (dtype ? 2 : 4),
                               dtype, V, T, prob, &M, &S) == -1);
      free(prob);
      free(tgt);
      free(dft);
    }
  }
  /* the distribution-level helpers */
  const int V = 9, K = 2;
  double q[3 * 9], p[2 * 9], w[9];
  for (int i = 0; i < 3 * V; ++i) q[i] = 1.0 / V;
  for (int i = 0; i < 2 * V; ++i) p[i] = (i % V == 0) ? 1.0 : 0.0;
  CHECK(oracle_residual_weights(q, q, V, w) == 1); /* q == p: the q fallback */
  CHECK(oracle_residual_weights(q, p, V, w) == 0);
  double zero[9] = {0};
  double d = 0.0;
  CHECK(oracle_inverse_cdf(zero, V, 0.5, &d) == -1);
  CHECK(oracle_inverse_cdf(q, V, 0.0, &d) == 0);
  CHECK(oracle_accept(0.0, 0.0, 0.3, &d) == 0);
  CHECK(oracle_accept(0.2, 0.0, 0.3, &d) == 1);
  int32_t tok[4 * 2] = {0, 1, 3, 3, 8, 0, 9, 2};
  float uni[4 * 3] = {0.1f, 0.5f, 0.9f, 0.99f, 0.0f, 0.3f, 0.2f, 0.2f, 0.2f, 0.7f, 0.7f, 0.7f};
  int32_t nacc[4], out[4 * 3], kind[4];
  double adist[4 * 2], ddist[4];
  CHECK(oracle_verify_dists(q, p, K, V, 4, tok, uni, nacc, out, adist, ddist, kind) == 0);
  CHECK(nacc[3] == -1); /* token 9 lies outside [0, 9) */
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle driver: ok\n");
  return 0;
}
