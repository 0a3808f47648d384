/*
 * qsa_oracle.h -- plain CPU oracle for the gated grouped-query attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library under gated_gqa_attention_amd/.
 *
 * What it computes (per new row l of sequence b and query head h):
 *   split  : the q_proj output of one head is [query(D) | gate(D)]
 *            (mlxd PR #99 "stage D6", Summary: doubled q_proj -> split into
 *            queries and gate -> o_proj(attn * sigmoid(gate)); Atlas
 *            qwen3_5/mod.rs, Qwen35ForwardConfig::q_total)
 *   norm   : per-head RMS norm of q and k over D, times a [D] weight
 *            (mlxd PR #99 config audit table, has_qk_norm; Atlas
 *            FullAttentionLayer q_norm / k_norm)
 *   rope   : rotation of only the first rotary_dim dims of q and k
 *            (mlxd PR #99 Summary, partial_rotary_factor; Atlas
 *            Qwen35ForwardConfig::rotary_dim doc comment)
 *   append : roped K and raw V of the new rows stored at slot n_b + l
 *            (Atlas qwen3_5/mod.rs module doc: KV append at cache_pos,
 *            attention over cache_pos + 1 keys)
 *   attend : softmax(scale * q.K^T) V over keys 0 .. n_b + l, with the
 *            query heads of one KV head forming a contiguous group
 *            (DS4Server issue #113, Reproduction: query heads divided
 *            within their KV groups)
 *   gate   : out = attn * sigmoid(gate), rounded to the storage dtype.
 *
 * All arithmetic is IEEE double.  Inputs are the stored (bf16 or fp32)
 * values widened exactly.  Rounding to the storage dtype is round to
 * nearest, ties to even, written from its definition.
 */
#ifndef QSA_ORACLE_H
#define QSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage codes for cache buffers handed to the oracle. */
enum { QSA_ORACLE_F64 = 0, QSA_ORACLE_F32 = 1, QSA_ORACLE_BF16 = 2 };

typedef struct {
  int32_t batch;          /* B */
  int32_t q_len;          /* L, new rows per sequence */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv, Hq % Hkv == 0 */
  int32_t head_dim;       /* D */
  int32_t rotary_dim;     /* r, even, 0 <= r <= D; 0 disables the rotation */
  double rope_theta;      /* theta */
  double rms_eps;         /* eps inside the square root */
  double softmax_scale;   /* 0 selects 1/sqrt(D) */
  int32_t store_bits;     /* significand bits of the storage dtype: 8 bf16, 24 fp32, 53 keeps double */
} qsa_oracle_cfg;

/* Round x to a binary floating-point value with `bits` significand bits,
 * ties to even.  bits >= 53 returns x. */
double qsa_oracle_round(double x, int bits);

/* New cache rows.  k_new, v_new: [B][L][Hkv][D]; w_k: [D]; positions: [B][L].
 * Writes k_rows = round(rope(rmsnorm(k_new) * w_k)) and v_rows = round(v_new),
 * both [B][L][Hkv][D].  Returns 0, or -1 on an invalid configuration. */
int qsa_oracle_new_kv(const qsa_oracle_cfg *cfg, const double *k_new, const double *v_new,
                      const double *w_k, const int32_t *positions, double *k_rows,
                      double *v_rows);

/* Gated attention of the new rows.
 *   q_gate     [B][L][Hq][2D]   per head [query | gate]
 *   w_q        [D]
 *   k_cache,
 *   v_cache    token-major rows of [Hkv][D] in storage `cache_dtype`; sequence b
 *              starts at row seq_offset[b]
 *   seq_lens   [B] cached rows before this call (n_b)
 *   positions  [B][L] rotary positions of the new rows
 *   k_rows,
 *   v_rows     [B][L][Hkv][D] new rows from qsa_oracle_new_kv, used for keys
 *              n_b .. n_b+L-1; both NULL means those keys are read from the cache
 *   rows       flat (b*L + l)*Hq + h indices to evaluate, or NULL for all
 *   out        [n_rows][D] (or [B][L][Hq][D] when rows is NULL): gated output
 *              rounded to the storage dtype
 *   attn       optional, same shape: the attention output before the gate,
 *              unrounded
 * Row l of sequence b attends to keys 0 .. n_b + l.  Returns 0 or -1. */
int qsa_oracle_attention(const qsa_oracle_cfg *cfg, const double *q_gate, const double *w_q,
                         const void *k_cache, const void *v_cache, int32_t cache_dtype,
                         const int64_t *seq_offset, const int32_t *seq_lens,
                         const int32_t *positions, const double *k_rows,
                         const double *v_rows, const int64_t *rows, int64_t n_rows,
                         double *out, double *attn);

/* A linear layer: y[m][n] = sum_k x[m][k] w[n][k] in double, rounded to
 * store_bits significand bits.  x [M][K], w [N][K] (row-major, a linear
 * layer's weight), y [M][N].  Returns 0, or -1 on a negative size. */
int qsa_oracle_linear(const double *x, const double *w, int64_t M, int64_t N, int64_t K, int32_t store_bits,
                      double *y);

/* The fused q/k/v projection of the rows x [B*L][hidden] (mlxd PR #99 Summary:
 * doubled q_proj -> split into queries and gate; Atlas FullAttentionLayer
 * q_proj / k_proj / v_proj, Qwen35Kernels qkv_split).  w_qkv holds the q_proj
 * rows ([Hq][2D]: per head its query rows, then its gate rows), then the k_proj
 * rows [Hkv][D], then the v_proj rows [Hkv][D], each over hidden inputs.  Writes
 * q_gate [B*L][Hq][2D], k_new and v_new [B*L][Hkv][D], rounded to storage.
 * Returns 0 or -1. */
int qsa_oracle_qkv_proj(const qsa_oracle_cfg *cfg, int32_t hidden, const double *x, const double *w_qkv,
                        double *q_gate, double *k_new, double *v_new);

/* ---- Turbo8 KV cache (Atlas docs, spark_model/forward/qwen3_5/mod.rs:
 * MetalKvDtype::Turbo8 -- FP8 E4M3 data plus bf16 scales for groups of 16
 * elements, in the Walsh-Hadamard rotated basis; LayerKvCache::alloc -- one
 * byte per element and two bytes per group of 16, for K and for V;
 * Qwen35Kernels -- quantizing appends, dequantizing decode attention, and the
 * WHT(Q) / iWHT(out) bookends).  Readings where the page is silent: the scale
 * of a group is its largest magnitude over 448 (the largest E4M3 value),
 * rounded to bf16; codes round x / scale to nearest E4M3, ties to even,
 * saturating at +-448; the rotation is the orthonormal Walsh-Hadamard
 * transform over head_dim (Sylvester order, divided by sqrt(head_dim)), which
 * is its own inverse.  The quantizer takes its decisions in fp32, as the GPU
 * does: row values rounded to fp32, scale = bf16(amax / 448) with an fp32
 * division, code = E4M3(fp32 quotient). */

/* Value of an FP8 E4M3 code (OCP: bias 7, 3 mantissa bits, no infinity,
 * S.1111.111 is NaN). */
double qsa_oracle_e4m3_value(uint8_t code);
/* Code of x: round to nearest E4M3 value, ties to even, saturating at +-448
 * (NaN is never produced). */
uint8_t qsa_oracle_e4m3_code(double x);
/* Orthonormal Walsh-Hadamard transform: y[i] = n^-1/2 sum_j (-1)^popcount(i & j) x[j];
 * n a power of two.  y may not alias x.  Returns 0 or -1. */
int qsa_oracle_wht(const double *x, int n, double *y);
/* Quantize n values (n % 16 == 0) to Turbo8: codes[n] and scale_bits[n/16]
 * (bf16 bit patterns).  Returns 0 or -1. */
int qsa_oracle_turbo8_quantize(const double *x, int n, uint8_t *codes, uint16_t *scale_bits);
/* New cache rows in Turbo8: K = quantize(WHT(rope(rmsnorm(k_new) * w_k))),
 * V = quantize(WHT(v_new)), each [B][L][Hkv][D] codes and [B][L][Hkv][D/16]
 * scale bits.  Returns 0 or -1. */
int qsa_oracle_turbo8_new_kv(const qsa_oracle_cfg *cfg, const double *k_new, const double *v_new,
                             const double *w_k, const int32_t *positions, uint8_t *k_codes,
                             uint16_t *k_scales, uint8_t *v_codes, uint16_t *v_scales);
/* Gated attention over a Turbo8 cache: like qsa_oracle_attention, with the
 * query rotated by WHT after its norm and rotary embedding, keys and values
 * decoded from codes x scales (cache rows token-major [rows][Hkv][D] codes,
 * [rows][Hkv][D/16] scale bits; new rows from qsa_oracle_turbo8_new_kv, or
 * all four NULL when they are already in the cache), and the attention output
 * rotated back by WHT before the gate.  Returns 0 or -1. */
int qsa_oracle_turbo8_attention(const qsa_oracle_cfg *cfg, const double *q_gate, const double *w_q,
                                const uint8_t *k_codes, const uint16_t *k_scales, const uint8_t *v_codes,
                                const uint16_t *v_scales, const int64_t *seq_offset, const int32_t *seq_lens,
                                const int32_t *positions, const uint8_t *nk_codes, const uint16_t *nk_scales,
                                const uint8_t *nv_codes, const uint16_t *nv_scales, const int64_t *rows,
                                int64_t n_rows, double *out);

/* ---- bf16 K + Turbo4 V (Atlas docs, spark_model/forward/qwen3_5/mod.rs:
 * MetalKvDtype::Bf16KTurbo4V -- K raw bf16 (not rotated), V Turbo4: 4-bit
 * Lloyd-Max codebook indices plus an FP8 scale per group of 16 elements,
 * matched-norm L2, in the Walsh-Hadamard rotated basis; LayerKvCache::alloc --
 * K two bytes per element, V half a byte per element and one scale byte per
 * 16; the iWHT(out) bookend only, since only V is rotated).  Readings where
 * the page is silent (parity against the page unpinned): the codebook is the
 * 16-level Lloyd-Max quantizer of the standard normal (the WHT makes a row's
 * coordinates near Gaussian), ascending, index 0 the most negative; a group's
 * indices are the levels nearest to x / sigma (sigma its RMS, the lower index
 * on a tie) and its scale is sqrt(sum x^2 / sum c^2) rounded to E4M3 (the
 * reconstruction keeps the group's L2 norm), a zero group taking scale 0;
 * codes pack two per byte, element 2i in the low nibble. */

/* The Lloyd-Max quantizer of N(0, 1) with `levels` levels (Lloyd's iteration
 * on the exact cell masses and conditional means), ascending, exactly
 * symmetric.  Returns 0 or -1. */
int qsa_oracle_lloyd_max_normal(int levels, double *centroids);
/* Turbo4: codes[n/2] (two per byte) and E4M3 scales[n/16] of x[n] under the
 * 16-level codebook cb.  Returns 0 or -1. */
int qsa_oracle_turbo4_quantize(const double *x, int n, const double *cb, uint8_t *codes, uint8_t *scales);
int qsa_oracle_turbo4_dequantize(const uint8_t *codes, const uint8_t *scales, int n, const double *cb, double *x);
/* New rows: K = bf16(rope(rmsnorm(k_new) * w_k)) as double [B][L][Hkv][D];
 * V = turbo4(WHT(v_new)): codes [B][L][Hkv][D/2], scales [B][L][Hkv][D/16]. */
int qsa_oracle_bf16k_turbo4v_new_kv(const qsa_oracle_cfg *cfg, const double *k_new, const double *v_new,
                                    const double *w_k, const int32_t *positions, const double *cb, double *k_rows,
                                    uint8_t *v_codes, uint8_t *v_scales);
/* Gated attention with K from a bf16 cache (bit patterns, [rows][Hkv][D]) and
 * V decoded from Turbo4 rows ([rows][Hkv][D/2] codes, [rows][Hkv][D/16]
 * scales), the attention output rotated back by WHT before the gate; new rows
 * from qsa_oracle_bf16k_turbo4v_new_kv, or all three NULL when they are in the
 * cache.  Returns 0 or -1. */
int qsa_oracle_bf16k_turbo4v_attention(const qsa_oracle_cfg *cfg, const double *q_gate, const double *w_q,
                                       const uint16_t *k_cache, const uint8_t *v_codes, const uint8_t *v_scales,
                                       const int64_t *seq_offset, const int32_t *seq_lens, const int32_t *positions,
                                       const double *cb, const double *nk_rows, const uint8_t *nv_codes,
                                       const uint8_t *nv_scales, const int64_t *rows, int64_t n_rows, double *out);

/* Number of OpenMP threads the oracle runs with. */
int qsa_oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
