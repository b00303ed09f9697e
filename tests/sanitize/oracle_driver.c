/*
 * Drives every path of the C oracle (oracle/kda_oracle.c) on small inputs so
 * that an AddressSanitizer + UndefinedBehaviorSanitizer build, and a
 * ThreadSanitizer build, can check its memory accesses, arithmetic and
 * worker threads.  Built and run by tests/test_sanitizers.py; the exit status
 * is 0 when every call returned what it should and the outputs of one thread
 * and of several threads agree bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_kda_recurrence_gated(int dtype, const void *q, const void *k, const void *v,
                                const void *g, const void *beta, const int64_t *cu,
                                int num_seqs, int hqk, int hv, double scale,
                                int use_l2norm, const double *a_log,
                                const double *dt_bias, double lower_bound,
                                const double *s0, double *out, double *s_final,
                                const int *heads, int n_heads, int n_threads);
int oracle_kda_recurrence(int dtype, const void *q, const void *k, const void *v,
                          const void *g, const void *beta, const int64_t *cu,
                          int num_seqs, int hqk, int hv, double scale,
                          int use_l2norm, const double *s0, double *out,
                          double *s_final, const int *heads, int n_heads,
                          int n_threads);

#define D 128
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static uint16_t to_bf16(float f) { uint32_t b; memcpy(&b, &f, 4); return (uint16_t)(b >> 16); }
static uint16_t to_f16(double x) { /* |x| < 2; below fp16's normal range: zero */
  const unsigned s = x < 0 ? 1u : 0u;
  x = fabs(x);
  int e;
  const double m = frexp(x, &e); /* x = m 2^e, m in [0.5, 1) */
  const int ex = e - 1 + 15;
  if (x == 0.0 || ex < 1) return (uint16_t)(s << 15);
  const unsigned man = (unsigned)((m * 2.0 - 1.0) * 1024.0);
  return (uint16_t)((s << 15) | ((unsigned)ex << 10) | man);
}

/* Fills an array of n elements of the given storage type with values a*u+b. */
static void *fill(int dtype, size_t n, double a, double b) {
  void *p = malloc(n * (dtype == 0 ? 4 : 2));
  for (size_t i = 0; i < n; ++i) {
    const double x = a * uni() + b;
    if (dtype == 0) ((float *)p)[i] = (float)x;
    else if (dtype == 1) ((uint16_t *)p)[i] = to_bf16((float)x);
    else ((uint16_t *)p)[i] = to_f16(x);
  }
  return p;
}

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); ++failures; } } while (0)

int main(void) {
  const int64_t cu[4] = {0, 5, 5, 22}; /* three sequences, the middle one empty */
  const int N = 3, hqk = 2, hv = 4, T = 22;
  const double scale = 1.0 / sqrt(128.0);
  double *s0 = malloc(sizeof(double) * N * hv * D * D);
  for (size_t i = 0; i < (size_t)N * hv * D * D; ++i) s0[i] = 0.1 * uni();
  double a_log[4], dt_bias[4 * D];
  for (int h = 0; h < hv; ++h) a_log[h] = 0.5 * uni();
  for (int i = 0; i < hv * D; ++i) dt_bias[i] = uni();
  const int heads[2] = {3, 1};
  for (int dtype = 0; dtype < 3; ++dtype) {
    void *q = fill(dtype, (size_t)T * hqk * D, 1.0, 0.0), *k = fill(dtype, (size_t)T * hqk * D, 1.0, 0.0);
    void *v = fill(dtype, (size_t)T * hv * D, 1.0, 0.0), *g = fill(dtype, (size_t)T * hv * D, 0.25, -0.3);
    void *beta = fill(dtype, (size_t)T * hv, 2.0, 0.0);
    const size_t no = (size_t)T * hv * D, ns = (size_t)N * hv * D * D;
    double *o1 = calloc(no, 8), *o3 = calloc(no, 8), *f1 = calloc(ns, 8), *f3 = calloc(ns, 8);
    for (int gate = 0; gate < 2; ++gate)
      for (int l2 = 0; l2 < 2; ++l2) {
        const double *al = gate ? a_log : NULL, *db = gate ? dt_bias : NULL;
        EXPECT(oracle_kda_recurrence_gated(dtype, q, k, v, g, beta, cu, N, hqk, hv, scale, l2, al,
                                           db, -5.0, s0, o1, f1, NULL, 0, 1) == 0);
        EXPECT(oracle_kda_recurrence_gated(dtype, q, k, v, g, beta, cu, N, hqk, hv, scale, l2, al,
                                           db, -5.0, s0, o3, f3, NULL, 0, 3) == 0);
        EXPECT(memcmp(o1, o3, no * 8) == 0 && memcmp(f1, f3, ns * 8) == 0);
        for (size_t i = 0; i < no; ++i) EXPECT(isfinite(o1[i]));
      }
    /* zero start, no final state, a subset of heads, more threads than units */
    EXPECT(oracle_kda_recurrence(dtype, q, k, v, g, beta, cu, N, hqk, hv, scale, 1, NULL, o1,
                                 NULL, heads, 2, 8) == 0);
    /* bad arguments are refused before any work */
    const int bad_head[1] = {4};
    EXPECT(oracle_kda_recurrence(dtype, q, k, v, g, beta, cu, N, hqk, hv, scale, 1, NULL, o1,
                                 NULL, bad_head, 1, 1) == -1);
    EXPECT(oracle_kda_recurrence(dtype, q, k, v, g, beta, cu, N, 3, hv, scale, 1, NULL, o1, NULL,
                                 NULL, 0, 1) == -1);
    EXPECT(oracle_kda_recurrence_gated(dtype, q, k, v, g, beta, cu, N, hqk, hv, scale, 1, a_log,
                                       NULL, -5.0, NULL, o1, NULL, NULL, 0, 1) == -1);
    EXPECT(oracle_kda_recurrence(3, q, k, v, g, beta, cu, N, hqk, hv, scale, 1, NULL, o1, NULL,
                                 NULL, 0, 1) == -1);
    free(q); free(k); free(v); free(g); free(beta);
    free(o1); free(o3); free(f1); free(f3);
  }
  free(s0);
  if (failures) return 1;
  printf("oracle driver: ok\n");
  return 0;
}
