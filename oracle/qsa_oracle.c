/*
 * qsa_oracle.c -- plain CPU oracle for the gated grouped-query attention core.
 *
 * TEST INFRASTRUCTURE ONLY (see qsa_oracle.h).  Slow on purpose: one query
 * row at a time, every sum a straight loop in double, no blocking or fusion.
 * OpenMP only distributes independent rows over host cores.
 */
#include "qsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Round to `bits` significand bits, ties to even.  frexp gives x = m * 2^e with
 * 0.5 <= |m| < 1; scaling m by 2^bits puts the kept bits left of the binary
 * point, and nearbyint rounds in the default mode (to nearest, ties to even). */
double qsa_oracle_round(double x, int bits) {
  if (bits >= 53 || x == 0.0 || !isfinite(x)) return x;
  int e;
  double m = frexp(x, &e);
  return ldexp(nearbyint(ldexp(m, bits)), e - bits);
}

static int cfg_ok(const qsa_oracle_cfg *c) {
  if (!c || c->batch < 0 || c->q_len < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1)
    return 0;
  if (c->num_q_heads % c->num_kv_heads) return 0;
  if (c->head_dim < 2 || c->rotary_dim < 0 || c->rotary_dim > c->head_dim) return 0;
  if (c->rotary_dim & 1) return 0;
  return 1;
}

static double scale_of(const qsa_oracle_cfg *c) {
  return c->softmax_scale != 0.0 ? c->softmax_scale : 1.0 / sqrt((double)c->head_dim);
}

/* RMS norm over one head: y_d = x_d * w_d / sqrt(mean(x^2) + eps). */
static void rms_norm(const double *x, const double *w, int D, double eps, double *y) {
  double ss = 0.0;
  for (int d = 0; d < D; ++d) ss += x[d] * x[d];
  double inv = 1.0 / sqrt(ss / D + eps);
  for (int d = 0; d < D; ++d) y[d] = x[d] * inv * w[d];
}

/* Rotary embedding on the first r dims, half-split pairing: dim i is paired
 * with dim i + r/2, rotated by angle p * theta^(-2i/r).  Dims r..D-1 untouched. */
static void rope(double *x, int r, double theta, double p) {
  int h = r / 2;
  for (int i = 0; i < h; ++i) {
    double freq = pow(theta, -2.0 * (double)i / (double)r);
    double a = p * freq;
    double c = cos(a), s = sin(a);
    double x0 = x[i], x1 = x[i + h];
    x[i] = x0 * c - x1 * s;
    x[i + h] = x1 * c + x0 * s;
  }
}

static double load(const void *base, int32_t dtype, int64_t idx) {
  switch (dtype) {
    case QSA_ORACLE_F64:
      return ((const double *)base)[idx];
    case QSA_ORACLE_F32:
      return (double)((const float *)base)[idx];
    default: {
      /* bf16: the upper 16 bits of a binary32 */
      uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
      float f;
      memcpy(&f, &u, sizeof f);
      return (double)f;
    }
  }
}

int qsa_oracle_new_kv(const qsa_oracle_cfg *c, const double *k_new, const double *v_new,
                      const double *w_k, const int32_t *positions, double *k_rows,
                      double *v_rows) {
  if (!cfg_ok(c)) return -1;
  const int B = c->batch, L = c->q_len, Hkv = c->num_kv_heads, D = c->head_dim;
  const int64_t n = (int64_t)B * L * Hkv;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t bl = i / Hkv;
    const double *k = k_new + i * D;
    double *ko = k_rows + i * D;
    rms_norm(k, w_k, D, c->rms_eps, ko);
    rope(ko, c->rotary_dim, c->rope_theta, (double)positions[bl]);
    for (int d = 0; d < D; ++d) {
      ko[d] = qsa_oracle_round(ko[d], c->store_bits);
      v_rows[i * D + d] = qsa_oracle_round(v_new[i * D + d], c->store_bits);
    }
  }
  return 0;
}

int qsa_oracle_attention(const qsa_oracle_cfg *c, const double *q_gate, const double *w_q,
                         const void *k_cache, const void *v_cache, int32_t cache_dtype,
                         const int64_t *seq_offset, const int32_t *seq_lens,
                         const int32_t *positions, const double *k_rows,
                         const double *v_rows, const int64_t *rows, int64_t n_rows,
                         double *out, double *attn) {
  if (!cfg_ok(c)) return -1;
  if ((k_rows == NULL) != (v_rows == NULL)) return -1;
  const int B = c->batch, L = c->q_len, Hq = c->num_q_heads, Hkv = c->num_kv_heads;
  const int D = c->head_dim, G = Hq / Hkv;
  const double scale = scale_of(c);
  const int64_t total = (int64_t)B * L * Hq;
  const int64_t count = rows ? n_rows : total;
  for (int64_t i = 0; i < count; ++i) {
    int64_t f = rows ? rows[i] : i;
    if (f < 0 || f >= total) return -1;
  }
  int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < count; ++i) {
    const int64_t f = rows ? rows[i] : i;
    const int h = (int)(f % Hq);
    const int64_t bl = f / Hq;
    const int l = (int)(bl % L);
    const int b = (int)(bl / L);
    const int g = h / G;                      /* contiguous query-head groups */
    const int64_t n = seq_lens[b];
    const int64_t nkeys = n + l + 1;          /* row l sees keys 0 .. n+l */

    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)nkeys);
    double *o = (double *)calloc((size_t)D, sizeof(double));
    if (!q || !s || !o) {
#pragma omp atomic write
      err = 1;
      free(q); free(s); free(o);
      continue;
    }

    /* split: query half of head h */
    const double *qh = q_gate + f * 2 * D;
    const double *zh = qh + D;
    rms_norm(qh, w_q, D, c->rms_eps, q);
    rope(q, c->rotary_dim, c->rope_theta, (double)positions[bl]);

    /* scores over keys 0 .. n+l of KV head g */
    for (int64_t j = 0; j < nkeys; ++j) {
      double acc = 0.0;
      if (j >= n && k_rows) {
        const double *kr = k_rows + (((int64_t)b * L + (j - n)) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) acc += q[d] * kr[d];
      } else {
        const int64_t base = ((seq_offset[b] + j) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) acc += q[d] * load(k_cache, cache_dtype, base + d);
      }
      s[j] = scale * acc;
    }

    /* softmax, max-subtracted */
    double m = s[0];
    for (int64_t j = 1; j < nkeys; ++j) m = s[j] > m ? s[j] : m;
    double sum = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
      s[j] = exp(s[j] - m);
      sum += s[j];
    }

    /* weighted sum of values */
    for (int64_t j = 0; j < nkeys; ++j) {
      const double p = s[j] / sum;
      if (j >= n && v_rows) {
        const double *vr = v_rows + (((int64_t)b * L + (j - n)) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) o[d] += p * vr[d];
      } else {
        const int64_t base = ((seq_offset[b] + j) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) o[d] += p * load(v_cache, cache_dtype, base + d);
      }
    }

    /* gate */
    double *dst = out + i * D;
    for (int d = 0; d < D; ++d) {
      const double sig = 1.0 / (1.0 + exp(-zh[d]));
      if (attn) attn[i * D + d] = o[d];
      dst[d] = qsa_oracle_round(o[d] * sig, c->store_bits);
    }
    free(q); free(s); free(o);
  }
  return err ? -1 : 0;
}

int qsa_oracle_linear(const double *x, const double *w, int64_t M, int64_t N, int64_t K, int32_t store_bits,
                      double *y) {
  if (M < 0 || N < 0 || K < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M * N; ++i) {
    const int64_t m = i / N, n = i % N;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += x[m * K + k] * w[n * K + k];
    y[i] = qsa_oracle_round(acc, store_bits);
  }
  return 0;
}

int qsa_oracle_qkv_proj(const qsa_oracle_cfg *c, int32_t hidden, const double *x, const double *w_qkv,
                        double *q_gate, double *k_new, double *v_new) {
  if (!cfg_ok(c) || hidden < 1) return -1;
  const int64_t M = (int64_t)c->batch * c->q_len, D = c->head_dim;
  const int64_t nq = (int64_t)c->num_q_heads * 2 * D, nk = (int64_t)c->num_kv_heads * D, n = nq + 2 * nk;
  double *y = (double *)malloc(sizeof(double) * (size_t)(M * n));
  if (!y) return -1;
  qsa_oracle_linear(x, w_qkv, M, n, hidden, c->store_bits, y);
  /* the split: the first 2 Hq D features of each row are q_gate, then k, then v */
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t f = 0; f < nq; ++f) q_gate[m * nq + f] = y[m * n + f];
    for (int64_t f = 0; f < nk; ++f) k_new[m * nk + f] = y[m * n + nq + f];
    for (int64_t f = 0; f < nk; ++f) v_new[m * nk + f] = y[m * n + nq + nk + f];
  }
  free(y);
  return 0;
}

int qsa_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
