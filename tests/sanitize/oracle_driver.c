/*
 * oracle_driver.c -- runs the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py with gcc
 * -fsanitize=address,undefined -fno-sanitize-recover=all).  Test infrastructure.
 *
 * Calls every oracle entry point over shapes that reach each loop bound and
 * edge: ragged sequences with no cached rows, one new row and several, full
 * and zero rotation, fp32, bf16 and f64 caches, row subsets, and the rejected
 * configurations.  It also checks two closed forms on the way, so that a run
 * that computes nonsense does not pass for clean: with every attended key equal
 * the attention output is the mean of the attended values, and a single key
 * returns its value.  Exit status 0 means clean and correct.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qsa_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {                     /* xorshift64*, uniform in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

static void fill(double *x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = urand();
}

static uint16_t to_bf16_bits(double x) {        /* storage only: the oracle rounds, this truncates */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static int failures = 0;
#define CHECK(c, ...)                     \
  do {                                    \
    if (!(c)) {                           \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      ++failures;                         \
    }                                     \
  } while (0)

/* One call over a ragged batch; dtype: 0 f64, 1 f32, 2 bf16 cache storage. */
static void run_case(int B, int L, int Hq, int Hkv, int D, int r, int dtype, int use_rows, int equal_keys) {
  qsa_oracle_cfg c = {B, L, Hq, Hkv, D, r, 1e4, 1e-6, 0.0, dtype == 2 ? 8 : dtype == 1 ? 24 : 53};
  int32_t *n = malloc(sizeof(int32_t) * B);
  int64_t *off = malloc(sizeof(int64_t) * B);
  int64_t rows_total = 0;
  for (int b = 0; b < B; ++b) {
    n[b] = (b * 7) % 5;                         /* includes sequences with no cached rows */
    off[b] = rows_total;
    rows_total += n[b] + L;
  }
  const size_t nq = (size_t)B * L * Hq * 2 * D, nk = (size_t)B * L * Hkv * D;
  const size_t ncache = (size_t)rows_total * Hkv * D;
  double *q_gate = malloc(sizeof(double) * nq), *k_new = malloc(sizeof(double) * nk),
         *v_new = malloc(sizeof(double) * nk), *w_q = malloc(sizeof(double) * D),
         *w_k = malloc(sizeof(double) * D), *k_rows = malloc(sizeof(double) * nk),
         *v_rows = malloc(sizeof(double) * nk), *kc = malloc(sizeof(double) * ncache),
         *vc = malloc(sizeof(double) * ncache);
  int32_t *pos = malloc(sizeof(int32_t) * B * L);
  fill(q_gate, nq);
  fill(k_new, nk);
  fill(v_new, nk);
  fill(w_q, D);
  fill(w_k, D);
  fill(kc, ncache);
  fill(vc, ncache);
  if (equal_keys) {
    for (size_t i = 0; i < ncache; ++i) kc[i] = kc[i % ((size_t)Hkv * D)];
  }
  for (int b = 0; b < B; ++b)
    for (int l = 0; l < L; ++l) pos[b * L + l] = n[b] + l;

  void *kst = kc, *vst = vc;
  float *kf = NULL, *vf = NULL;
  uint16_t *kb = NULL, *vb = NULL;
  if (dtype == 1) {
    kf = malloc(sizeof(float) * ncache);
    vf = malloc(sizeof(float) * ncache);
    for (size_t i = 0; i < ncache; ++i) {
      kf[i] = (float)kc[i];
      vf[i] = (float)vc[i];
    }
    kst = kf;
    vst = vf;
  } else if (dtype == 2) {
    kb = malloc(sizeof(uint16_t) * ncache);
    vb = malloc(sizeof(uint16_t) * ncache);
    for (size_t i = 0; i < ncache; ++i) {
      kb[i] = to_bf16_bits(kc[i]);
      vb[i] = to_bf16_bits(vc[i]);
    }
    kst = kb;
    vst = vb;
  }
  CHECK(qsa_oracle_new_kv(&c, k_new, v_new, w_k, pos, k_rows, v_rows) == 0, "new_kv");

  const int64_t total = (int64_t)B * L * Hq;
  int64_t nr = use_rows ? (total + 1) / 2 : 0;
  int64_t *rows = NULL;
  if (use_rows) {
    rows = malloc(sizeof(int64_t) * nr);
    for (int64_t i = 0; i < nr; ++i) rows[i] = (2 * i + 1) % total;
  }
  const int64_t count = use_rows ? nr : total;
  double *out = malloc(sizeof(double) * count * D), *att = malloc(sizeof(double) * count * D);
  /* keys of the new rows from the cache (the rows passed as NULL): the cache rows
   * n_b .. n_b + L - 1 hold whatever fill() put there, which is fine here */
  CHECK(qsa_oracle_attention(&c, q_gate, w_q, kst, vst, dtype, off, n, pos, NULL, NULL, rows, nr, out, att) == 0,
        "attention from the cache");
  CHECK(qsa_oracle_attention(&c, q_gate, w_q, kst, vst, dtype, off, n, pos, k_rows, v_rows, rows, nr, out, att) == 0,
        "attention with new rows");
  for (int64_t i = 0; i < count * D; ++i) CHECK(isfinite(out[i]) && isfinite(att[i]), "finite output");

  /* closed forms, on the call with new rows */
  for (int64_t i = 0; i < count; ++i) {
    const int64_t f = rows ? rows[i] : i;
    const int h = (int)(f % Hq), l = (int)((f / Hq) % L), b = (int)(f / Hq / L), g = h / (Hq / Hkv);
    const int64_t keys = (int64_t)n[b] + l + 1;
    if (keys == 1) {                            /* one key: its value */
      const double *v = v_rows + (((int64_t)b * L) * Hkv + g) * D;
      for (int d = 0; d < D; ++d) CHECK(fabs(att[i * D + d] - v[d]) < 1e-12, "single key returns its value");
    }
  }
  if (equal_keys && dtype == 0) {              /* every cached key equal, no new rows: mean of values */
    CHECK(qsa_oracle_attention(&c, q_gate, w_q, kst, vst, dtype, off, n, pos, NULL, NULL, rows, nr, out, att) == 0,
          "attention, equal keys");
    for (int64_t i = 0; i < count; ++i) {
      const int64_t f = rows ? rows[i] : i;
      const int h = (int)(f % Hq), l = (int)((f / Hq) % L), b = (int)(f / Hq / L), g = h / (Hq / Hkv);
      const int64_t keys = (int64_t)n[b] + l + 1;
      for (int d = 0; d < D; ++d) {
        double mean = 0.0;
        for (int64_t j = 0; j < keys; ++j) mean += vc[((off[b] + j) * Hkv + g) * D + d];
        mean /= (double)keys;
        CHECK(fabs(att[i * D + d] - mean) < 1e-12, "equal keys give the mean of the values");
      }
    }
  }

  /* rejected configurations */
  qsa_oracle_cfg bad = c;
  bad.rotary_dim = r + 1;
  CHECK(qsa_oracle_new_kv(&bad, k_new, v_new, w_k, pos, k_rows, v_rows) == -1, "odd rotary_dim rejected");
  bad = c;
  bad.num_kv_heads = Hq + 1;
  CHECK(qsa_oracle_attention(&bad, q_gate, w_q, kst, vst, dtype, off, n, pos, NULL, NULL, NULL, 0, out, NULL) == -1,
        "head groups rejected");
  int64_t badrow = total;
  CHECK(qsa_oracle_attention(&c, q_gate, w_q, kst, vst, dtype, off, n, pos, NULL, NULL, &badrow, 1, out, NULL) == -1,
        "row index past the end rejected");

  free(n); free(off); free(q_gate); free(k_new); free(v_new); free(w_q); free(w_k); free(k_rows);
  free(v_rows); free(kc); free(vc); free(pos); free(kf); free(vf); free(kb); free(vb); free(rows);
  free(out); free(att);
}

int main(void) {
  CHECK(qsa_oracle_round(1.0 + 3.0 / 256.0, 8) == 1.0 + 1.0 / 64.0, "round ties to even");
  CHECK(qsa_oracle_round(INFINITY, 8) == INFINITY, "round keeps inf");
  run_case(3, 1, 4, 1, 64, 16, 0, 0, 0);
  run_case(3, 1, 4, 2, 64, 64, 0, 0, 1);        /* full rotation, equal keys */
  run_case(2, 4, 12, 1, 32, 0, 1, 1, 0);        /* no rotation, fp32 cache, row subset */
  run_case(4, 3, 8, 2, 128, 32, 2, 0, 0);       /* bf16 cache */
  run_case(1, 5, 2, 2, 16, 8, 2, 1, 1);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer run: clean\n");
  return 0;
}
