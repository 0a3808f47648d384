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

/* ------------------------------------------------------------------ Turbo8 */

double qsa_oracle_e4m3_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

uint8_t qsa_oracle_e4m3_code(double x) {
  const uint8_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0;
  double a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;              /* saturate: 1.75 * 2^8 */
  if (a < ldexp(1.0, -6)) {                        /* subnormal grid m * 2^-9; m = 8 is 2^-6 */
    const double m = nearbyint(ldexp(a, 9));       /* ties to even */
    return sign | (uint8_t)m;
  }
  int e;
  frexp(a, &e);                                    /* a = f * 2^e, 0.5 <= f < 1: exponent e - 1 */
  const int ex = e - 1;                            /* -6 .. 8 */
  const double q = nearbyint(ldexp(a, 3 - ex));    /* 8 .. 16, ties to even */
  return sign | (uint8_t)(((ex + 7) << 3) + (int)q - 8);   /* q = 16 carries into the exponent */
}

int qsa_oracle_wht(const double *x, int n, double *y) {
  if (n < 1 || (n & (n - 1))) return -1;
  const double norm = 1.0 / sqrt((double)n);
  for (int i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j) acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -x[j] : x[j];
    y[i] = acc * norm;
  }
  return 0;
}

static uint16_t bf16_bits(double x) {           /* RNE to bf16, as bits */
  float f = (float)qsa_oracle_round(x, 8);
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int qsa_oracle_turbo8_quantize(const double *x, int n, uint8_t *codes, uint16_t *scale_bits) {
  if (n < 16 || n % 16) return -1;
  for (int g = 0; g < n / 16; ++g) {
    float xf[16], amax = 0.f;
    for (int i = 0; i < 16; ++i) {
      xf[i] = (float)x[16 * g + i];                /* the row in fp32 */
      amax = fabsf(xf[i]) > amax ? fabsf(xf[i]) : amax;
    }
    const float sq = amax / 448.0f;                /* fp32 division */
    const uint16_t sb = bf16_bits((double)sq);
    const float s = (float)bf16_value(sb);
    scale_bits[g] = sb;
    for (int i = 0; i < 16; ++i) {
      if (s == 0.f) {
        codes[16 * g + i] = 0;
        continue;
      }
      float q = xf[i] / s;                         /* fp32 quotient */
      q = q > 448.f ? 448.f : (q < -448.f ? -448.f : q);
      codes[16 * g + i] = qsa_oracle_e4m3_code((double)q);
    }
  }
  return 0;
}

int qsa_oracle_turbo8_new_kv(const qsa_oracle_cfg *c, const double *k_new, const double *v_new,
                             const double *w_k, const int32_t *positions, uint8_t *k_codes,
                             uint16_t *k_scales, uint8_t *v_codes, uint16_t *v_scales) {
  if (!cfg_ok(c) || c->head_dim % 16 || (c->head_dim & (c->head_dim - 1))) return -1;
  const int L = c->q_len, Hkv = c->num_kv_heads, D = c->head_dim;
  const int64_t n = (int64_t)c->batch * L * Hkv;
  int err = 0;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double *t = (double *)malloc(sizeof(double) * (size_t)D);
    double *r = (double *)malloc(sizeof(double) * (size_t)D);
    if (!t || !r) {
#pragma omp atomic write
      err = 1;
      free(t); free(r);
      continue;
    }
    rms_norm(k_new + i * D, w_k, D, c->rms_eps, t);
    rope(t, c->rotary_dim, c->rope_theta, (double)positions[i / Hkv]);
    qsa_oracle_wht(t, D, r);
    qsa_oracle_turbo8_quantize(r, D, k_codes + i * D, k_scales + i * (D / 16));
    qsa_oracle_wht(v_new + i * D, D, r);
    qsa_oracle_turbo8_quantize(r, D, v_codes + i * D, v_scales + i * (D / 16));
    free(t); free(r);
  }
  return err ? -1 : 0;
}

/* one decoded Turbo8 row: codes [D] times their group scales [D/16] */
static void turbo8_row(const uint8_t *codes, const uint16_t *scales, int D, double *out) {
  for (int d = 0; d < D; ++d) out[d] = qsa_oracle_e4m3_value(codes[d]) * bf16_value(scales[d / 16]);
}

int qsa_oracle_turbo8_attention(const qsa_oracle_cfg *c, const double *q_gate, const double *w_q,
                                const uint8_t *k_codes, const uint16_t *k_scales, const uint8_t *v_codes,
                                const uint16_t *v_scales, const int64_t *seq_offset, const int32_t *seq_lens,
                                const int32_t *positions, const uint8_t *nk_codes, const uint16_t *nk_scales,
                                const uint8_t *nv_codes, const uint16_t *nv_scales, const int64_t *rows,
                                int64_t n_rows, double *out) {
  if (!cfg_ok(c) || c->head_dim % 16 || (c->head_dim & (c->head_dim - 1))) return -1;
  const int given = (nk_codes != NULL) + (nk_scales != NULL) + (nv_codes != NULL) + (nv_scales != NULL);
  if (given != 0 && given != 4) return -1;
  const int B = c->batch, L = c->q_len, Hq = c->num_q_heads, Hkv = c->num_kv_heads;
  const int D = c->head_dim, G = Hq / Hkv;
  const double scale = scale_of(c);
  const int64_t total = (int64_t)B * L * Hq;
  const int64_t count = rows ? n_rows : total;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t f = rows ? rows[i] : i;
    if (f < 0 || f >= total) return -1;
  }
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < count; ++i) {
    const int64_t f = rows ? rows[i] : i;
    const int h = (int)(f % Hq);
    const int64_t bl = f / Hq;
    const int l = (int)(bl % L), b = (int)(bl / L), g = h / G;
    const int64_t n = seq_lens[b], nkeys = n + l + 1;
    double *q0 = (double *)malloc(sizeof(double) * (size_t)D);
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *kv = (double *)malloc(sizeof(double) * (size_t)D);
    double *o = (double *)calloc((size_t)D, sizeof(double));
    double *ob = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)nkeys);
    if (!q0 || !q || !kv || !o || !ob || !s) {
#pragma omp atomic write
      err = 1;
      free(q0); free(q); free(kv); free(o); free(ob); free(s);
      continue;
    }
    const double *qh = q_gate + f * 2 * D, *zh = qh + D;
    rms_norm(qh, w_q, D, c->rms_eps, q0);
    rope(q0, c->rotary_dim, c->rope_theta, (double)positions[bl]);
    qsa_oracle_wht(q0, D, q);                       /* WHT(Q) bookend */
    for (int64_t j = 0; j < nkeys; ++j) {
      if (j >= n && nk_codes) {
        const int64_t r = ((int64_t)b * L + (j - n)) * Hkv + g;
        turbo8_row(nk_codes + r * D, nk_scales + r * (D / 16), D, kv);
      } else {
        const int64_t r = (seq_offset[b] + j) * Hkv + g;
        turbo8_row(k_codes + r * D, k_scales + r * (D / 16), D, kv);
      }
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += q[d] * kv[d];
      s[j] = scale * acc;
    }
    double m = s[0];
    for (int64_t j = 1; j < nkeys; ++j) m = s[j] > m ? s[j] : m;
    double sum = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
      s[j] = exp(s[j] - m);
      sum += s[j];
    }
    for (int64_t j = 0; j < nkeys; ++j) {
      if (j >= n && nv_codes) {
        const int64_t r = ((int64_t)b * L + (j - n)) * Hkv + g;
        turbo8_row(nv_codes + r * D, nv_scales + r * (D / 16), D, kv);
      } else {
        const int64_t r = (seq_offset[b] + j) * Hkv + g;
        turbo8_row(v_codes + r * D, v_scales + r * (D / 16), D, kv);
      }
      const double p = s[j] / sum;
      for (int d = 0; d < D; ++d) o[d] += p * kv[d];
    }
    qsa_oracle_wht(o, D, ob);                       /* iWHT(out) bookend: the transform is its own inverse */
    double *dst = out + i * D;
    for (int d = 0; d < D; ++d) dst[d] = qsa_oracle_round(ob[d] / (1.0 + exp(-zh[d])), c->store_bits);
    free(q0); free(q); free(kv); free(o); free(ob); free(s);
  }
  return err ? -1 : 0;
}

/* ---- bf16 K + Turbo4 V ------------------------------------------------- */

static double npdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * acos(-1.0)); }

/* P(lo < X < hi) for X ~ N(0, 1), from whichever tail keeps the precision */
static double nmass(double lo, double hi) {
  const double r2 = sqrt(2.0);
  if (hi <= 0.0) return 0.5 * (erfc(-hi / r2) - erfc(-lo / r2));
  if (lo >= 0.0) return 0.5 * (erfc(lo / r2) - erfc(hi / r2));
  return 1.0 - 0.5 * erfc(-lo / r2) - 0.5 * erfc(hi / r2);
}

int qsa_oracle_lloyd_max_normal(int levels, double *c) {
  if (levels < 2 || levels > 256) return -1;
  double nc[256];
  for (int i = 0; i < levels; ++i) c[i] = -3.0 + 6.0 * (i + 0.5) / levels;
  for (int it = 0; it < 200000; ++it) {
    double change = 0.0;
    for (int i = 0; i < levels; ++i) {
      const double lo = i == 0 ? -INFINITY : 0.5 * (c[i - 1] + c[i]);
      const double hi = i == levels - 1 ? INFINITY : 0.5 * (c[i] + c[i + 1]);
      nc[i] = (npdf(lo) - npdf(hi)) / nmass(lo, hi);      /* the cell's conditional mean */
      change = fmax(change, fabs(nc[i] - c[i]));
    }
    for (int i = 0; i < levels; ++i) c[i] = nc[i];
    if (change < 1e-16) break;
  }
  for (int i = 0; i < levels / 2; ++i) {                  /* exact symmetry */
    const double m = 0.5 * (c[levels - 1 - i] - c[i]);
    c[i] = -m;
    c[levels - 1 - i] = m;
  }
  return 0;
}

int qsa_oracle_turbo4_quantize(const double *x, int n, const double *cb, uint8_t *codes, uint8_t *scales) {
  if (n < 16 || n % 16) return -1;
  for (int g = 0; g < n / 16; ++g) {
    const double *xg = x + 16 * g;
    uint8_t *cg = codes + 8 * g;
    double ss = 0.0;
    for (int i = 0; i < 16; ++i) ss += xg[i] * xg[i];
    for (int i = 0; i < 8; ++i) cg[i] = 0;
    if (ss == 0.0) {
      scales[g] = 0;
      continue;
    }
    const double sigma = sqrt(ss / 16.0);
    double cc = 0.0;
    for (int i = 0; i < 16; ++i) {
      const double u = xg[i] / sigma;
      int idx = 0;                                         /* nearest level: thresholds below u */
      for (int j = 0; j < 15; ++j)
        if (0.5 * (cb[j] + cb[j + 1]) < u) idx = j + 1;
      cc += cb[idx] * cb[idx];
      cg[i / 2] |= (uint8_t)(idx << (4 * (i & 1)));
    }
    scales[g] = qsa_oracle_e4m3_code(sqrt(ss / cc));    /* matched L2 norm */
  }
  return 0;
}

int qsa_oracle_turbo4_dequantize(const uint8_t *codes, const uint8_t *scales, int n, const double *cb, double *x) {
  if (n < 16 || n % 16) return -1;
  for (int i = 0; i < n; ++i) x[i] = qsa_oracle_e4m3_value(scales[i / 16]) * cb[(codes[i / 2] >> (4 * (i & 1))) & 15];
  return 0;
}

int qsa_oracle_bf16k_turbo4v_new_kv(const qsa_oracle_cfg *c, const double *k_new, const double *v_new,
                                    const double *w_k, const int32_t *positions, const double *cb, double *k_rows,
                                    uint8_t *v_codes, uint8_t *v_scales) {
  if (!cfg_ok(c) || c->head_dim % 16 || (c->head_dim & (c->head_dim - 1))) return -1;
  const int L = c->q_len, Hkv = c->num_kv_heads, D = c->head_dim;
  const int64_t n = (int64_t)c->batch * L * Hkv;
  int err = 0;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double *r = (double *)malloc(sizeof(double) * (size_t)D);
    if (!r) {
#pragma omp atomic write
      err = 1;
      continue;
    }
    double *ko = k_rows + i * D;                           /* K: the bf16 cache's row */
    rms_norm(k_new + i * D, w_k, D, c->rms_eps, ko);
    rope(ko, c->rotary_dim, c->rope_theta, (double)positions[i / Hkv]);
    for (int d = 0; d < D; ++d) ko[d] = qsa_oracle_round(ko[d], 8);
    qsa_oracle_wht(v_new + i * D, D, r);                   /* V: rotated, then Turbo4 */
    qsa_oracle_turbo4_quantize(r, D, cb, v_codes + i * (D / 2), v_scales + i * (D / 16));
    free(r);
  }
  return err ? -1 : 0;
}

int qsa_oracle_bf16k_turbo4v_attention(const qsa_oracle_cfg *c, const double *q_gate, const double *w_q,
                                       const uint16_t *k_cache, const uint8_t *v_codes, const uint8_t *v_scales,
                                       const int64_t *seq_offset, const int32_t *seq_lens, const int32_t *positions,
                                       const double *cb, const double *nk_rows, const uint8_t *nv_codes,
                                       const uint8_t *nv_scales, const int64_t *rows, int64_t n_rows, double *out) {
  if (!cfg_ok(c) || c->head_dim % 16 || (c->head_dim & (c->head_dim - 1))) return -1;
  const int given = (nk_rows != NULL) + (nv_codes != NULL) + (nv_scales != NULL);
  if (given != 0 && given != 3) return -1;
  const int B = c->batch, L = c->q_len, Hq = c->num_q_heads, Hkv = c->num_kv_heads;
  const int D = c->head_dim, G = Hq / Hkv;
  const double scale = scale_of(c);
  const int64_t total = (int64_t)B * L * Hq;
  const int64_t count = rows ? n_rows : total;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t f = rows ? rows[i] : i;
    if (f < 0 || f >= total) return -1;
  }
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < count; ++i) {
    const int64_t f = rows ? rows[i] : i;
    const int h = (int)(f % Hq);
    const int64_t bl = f / Hq;
    const int l = (int)(bl % L), b = (int)(bl / L), g = h / G;
    const int64_t n = seq_lens[b], nkeys = n + l + 1;
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *vv = (double *)malloc(sizeof(double) * (size_t)D);
    double *o = (double *)calloc((size_t)D, sizeof(double));
    double *ob = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)nkeys);
    if (!q || !vv || !o || !ob || !s) {
#pragma omp atomic write
      err = 1;
      free(q); free(vv); free(o); free(ob); free(s);
      continue;
    }
    const double *qh = q_gate + f * 2 * D, *zh = qh + D;
    rms_norm(qh, w_q, D, c->rms_eps, q);
    rope(q, c->rotary_dim, c->rope_theta, (double)positions[bl]);   /* K is not rotated: no WHT(Q) */
    for (int64_t j = 0; j < nkeys; ++j) {
      double acc = 0.0;
      if (j >= n && nk_rows) {
        const double *kr = nk_rows + (((int64_t)b * L + (j - n)) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) acc += q[d] * kr[d];
      } else {
        const int64_t r = ((seq_offset[b] + j) * Hkv + g) * D;
        for (int d = 0; d < D; ++d) acc += q[d] * load(k_cache, QSA_ORACLE_BF16, r + d);
      }
      s[j] = scale * acc;
    }
    double m = s[0];
    for (int64_t j = 1; j < nkeys; ++j) m = s[j] > m ? s[j] : m;
    double sum = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
      s[j] = exp(s[j] - m);
      sum += s[j];
    }
    for (int64_t j = 0; j < nkeys; ++j) {
      if (j >= n && nv_codes) {
        const int64_t r = ((int64_t)b * L + (j - n)) * Hkv + g;
        qsa_oracle_turbo4_dequantize(nv_codes + r * (D / 2), nv_scales + r * (D / 16), D, cb, vv);
      } else {
        const int64_t r = (seq_offset[b] + j) * Hkv + g;
        qsa_oracle_turbo4_dequantize(v_codes + r * (D / 2), v_scales + r * (D / 16), D, cb, vv);
      }
      const double p = s[j] / sum;
      for (int d = 0; d < D; ++d) o[d] += p * vv[d];
    }
    qsa_oracle_wht(o, D, ob);                              /* iWHT(out): V is rotated */
    double *dst = out + i * D;
    for (int d = 0; d < D; ++d) dst[d] = qsa_oracle_round(ob[d] / (1.0 + exp(-zh[d])), c->store_bits);
    free(q); free(vv); free(o); free(ob); free(s);
  }
  return err ? -1 : 0;
}

int qsa_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
