/*
 * qsa.h -- C ABI of the gated grouped-query attention core for AMD MI355X (gfx950).
 *
 * The operation is the full-attention core of a Qwen3.5 decoder layer:
 *
 *   1. split the doubled q_proj output of every query head into a query half
 *      and a gate half (mlxd PR #99 "stage D6", Summary: doubled q_proj, split
 *      into queries and gate, o_proj(attn * sigmoid(gate)); Atlas
 *      spark_model/forward/qwen3_5/mod.rs, Qwen35ForwardConfig::q_total);
 *   2. RMS-normalise every query head and every new key head over head_dim and
 *      scale by a [head_dim] weight (mlxd PR #99, config audit table,
 *      has_qk_norm; Atlas FullAttentionLayer q_norm / k_norm);
 *   3. rotate only the first rotary_dim dims of query and key (partial RoPE;
 *      mlxd PR #99 Summary, partial_rotary_factor; Atlas
 *      Qwen35ForwardConfig::rotary_dim);
 *   4. append the rotated keys and the values of the new rows to the KV cache
 *      at slot seq_lens[b] + l, then attend over keys 0 .. seq_lens[b] + l
 *      (Atlas qwen3_5/mod.rs module doc: KV append at cache_pos, attention at
 *      cache_pos + 1);
 *   5. grouped-query softmax attention, the query heads of KV head g being the
 *      contiguous group g*G .. g*G+G-1, G = num_q_heads / num_kv_heads
 *      (DS4Server issue #113, Reproduction: query heads divided within their
 *      KV groups; Atlas Qwen35ForwardConfig: 16 query / 4 KV heads);
 *   6. multiply by sigmoid(gate) (mlxd PR #99 Summary; Atlas sigmoid_gate).
 *
 * Conventions fixed by this interface where the pages leave them open:
 *   - per head the q_proj output is [query(D) | gate(D)] (head-blocked halves);
 *   - RMS norm: x * w / sqrt(mean(x^2) + eps), with the weight w applied as
 *     given (a checkpoint that stores zero-centred weights passes 1 + w);
 *   - rotation pairs dim i with dim i + rotary_dim/2, angle
 *     position * rope_theta^(-2i/rotary_dim); rotary_dim = 0 disables it;
 *   - softmax scale 1/sqrt(head_dim) unless softmax_scale is set;
 *   - the cache stores K after norm and rotation and V as given, rounded to the
 *     storage dtype (round to nearest even);
 *   - new row l of a call sees new rows 0 .. l (causal by row order).
 *
 * Memory and ownership.  Every buffer is device memory allocated and owned by
 * the caller: inputs, the KV cache, the output and the workspace.  The
 * library allocates nothing, never synchronises, and launches all work on
 * cfg->stream; calls return as soon as the work is queued.  The library owns
 * only its code objects.  seq_lens is never advanced by the library: the
 * caller owns the cache position.
 *
 * Errors.  Every entry point validates its arguments on the host before any
 * launch and returns a negative qsa_status on failure, with a message for the
 * calling thread in qsa_last_error().  Nothing falls back to another path.
 * Values that live on the device (seq_lens, seq_offset, capacity, block_table)
 * are checked by the kernels: a sequence whose rows would leave the cache,
 * exceed its capacity or exceed cfg->max_seq_len gets NaN outputs, its cache
 * is not written, and bit 0 of the int32 at the start of the workspace is set
 * (sticky until the caller clears it).  A paged sequence whose table names a
 * block outside the cache gets NaN outputs and sets that bit too; nothing is
 * read or written outside the cache (a new row whose own block is valid may
 * still be stored there).  Paged caches: the attention call takes them on the short-query route
 * (decode, verify, batched decode: q_len * G <= 48, q_len <= 16, bf16) with key
 * chunks of at most 127 blocks, and returns QSA_ERR_UNSUPPORTED otherwise;
 * qsa_append_kv takes them always.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_INVALID = -1,      /* malformed argument (NULL pointer, bad size, odd rotary_dim, ...) */
  QSA_ERR_UNSUPPORTED = -2,  /* well-formed but not supported (head_dim, dtype, group size) */
  QSA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than qsa_workspace_size() */
  QSA_ERR_DEVICE = -4        /* a HIP launch failed, or the device is not gfx950 */
} qsa_status;

typedef enum {
  QSA_BF16 = 0,              /* bfloat16 activations, cache, norm weights and output; fp32 accumulation */
  QSA_F32 = 1                /* fp32 everywhere */
} qsa_dtype;

/* Storage of the KV cache. */
typedef enum {
  QSA_KV_NATIVE = 0,         /* rows in cfg->dtype */
  QSA_KV_TURBO8 = 1,         /* Turbo8 (Atlas qwen3_5/mod.rs, MetalKvDtype::Turbo8: FP8 E4M3 data and a
                                bf16 scale per 16 elements, in the Walsh-Hadamard rotated basis): k / v
                                hold one E4M3 code per element ([rows][Hkv][D] bytes) and k_scales /
                                v_scales one bf16 scale per 16 consecutive elements of a row
                                ([rows][Hkv][D/16]).  A group's scale is its largest magnitude over
                                448 rounded to bf16, a code is value / scale rounded to nearest E4M3
                                (ties to even, saturating at +-448), and rows are stored after the
                                orthonormal Walsh-Hadamard transform over head_dim (keys after their
                                norm and rotation), which the attention applies to the queries and
                                undoes on its output.  bf16 activations only; contiguous caches on
                                the short-query route. */
  QSA_KV_BF16K_TURBO4V = 2   /* bf16 K + Turbo4 V (Atlas qwen3_5/mod.rs, MetalKvDtype::Bf16KTurbo4V: K raw
                                bf16, not rotated; V as 4-bit Lloyd-Max codebook indices and an FP8 scale
                                per 16 elements, matched-norm L2, in the Walsh-Hadamard rotated basis):
                                k holds the bf16 cache's K rows ([rows][Hkv][D]); v holds two 4-bit
                                indices per byte ([rows][Hkv][D/2], element 2i in the low nibble) into
                                the 16-level Lloyd-Max quantizer of the standard normal (ascending),
                                and v_scales one E4M3 scale byte per 16 elements ([rows][Hkv][D/16]);
                                k_scales is not used.  A group's indices are the levels nearest to
                                x / RMS(group) and its scale is sqrt(sum x^2 / sum level^2) rounded to
                                E4M3, so the decoded group keeps the group's L2 norm; V rows are stored
                                after the orthonormal Walsh-Hadamard transform, which the attention
                                undoes on its output.  bf16 activations, head_dim 256; contiguous
                                caches on the short-query route. */
} qsa_kv_dtype;

/* One call's shape, numerics and execution context. */
typedef struct {
  int32_t batch;             /* B >= 1 sequences */
  int32_t q_len;             /* L >= 1 new rows per sequence */
  int32_t num_q_heads;       /* Hq >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;          /* D: 64, 128 or 256 */
  int32_t rotary_dim;        /* r: even, 0 <= r <= D; 0 = no rotation */
  float rope_theta;          /* theta > 0 */
  float rms_eps;             /* eps >= 0, added to mean(x^2) inside the square root */
  float softmax_scale;       /* > 0, or 0 for 1/sqrt(D) */
  int32_t dtype;             /* qsa_dtype */
  int32_t max_seq_len;       /* host bound: seq_lens[b] + q_len <= max_seq_len for every b */
  int32_t force_splits;      /* 0 = automatic; k > 0 plans k key chunks for max_seq_len (tests) */
  const void *q_norm_w;      /* device [D] query norm weight, in dtype */
  const void *k_norm_w;      /* device [D] key norm weight, in dtype */
  void *workspace;           /* device scratch, zero-filled before its first use */
  size_t workspace_bytes;    /* >= qsa_workspace_size(cfg) */
  void *stream;              /* hipStream_t to launch on; NULL = the null stream */
  void *timing_begin;        /* optional hipEvent_t, recorded on stream right before the call's
                                attention kernel (the one that reads the KV cache) is launched;
                                NULL for none.  For profilers and benchmarks; leave both NULL
                                while the stream is being captured into a graph. */
  void *timing_end;          /* optional hipEvent_t, recorded right after that launch */
} qsa_cfg;

/* KV cache of one attention layer.  Token-major: a row is [num_kv_heads][head_dim]
 * elements of cfg->dtype, and row t of sequence b sits at element offset
 * row(b, t) * num_kv_heads * head_dim of k (and of v), where
 *   contiguous (block_table == NULL): row(b, t) = seq_offset[b] + t; sequences
 *     may be packed back to back (ragged batches) or strided uniformly;
 *   paged (block_table != NULL): row(b, t) = block_table[b][t / block_size] *
 *     block_size + t % block_size; a sequence's rows live in blocks of
 *     block_size rows that the caller hands out as the sequence grows
 *     (TensorFold issue #503: grow-as-used K/V; Atlas qwen3_5/mod.rs module
 *     doc: paged KV in the production decode path).  seq_offset is not read.
 * The two layouts give bitwise the same results for the same rows. */
typedef struct {
  void *k;                   /* device base of the K rows */
  void *v;                   /* device base of the V rows */
  const int64_t *seq_offset; /* device [B]: first row of sequence b (64-bit: caches may exceed 2^31
                                elements); contiguous layout only */
  const int32_t *capacity;   /* device [B]: rows owned by sequence b, or NULL for "up to num_rows"
                                (contiguous) / "max_blocks * block_size" (paged) */
  int64_t num_rows;          /* host: rows allocated in k and in v (paged: a multiple of block_size) */
  const int32_t *block_table; /* device [B][max_blocks] physical block ids, or NULL (contiguous) */
  int32_t block_size;        /* paged: rows per block, a power of two in [64, 65536] */
  int32_t max_blocks;        /* paged: entries per sequence in block_table (row stride) */
  int32_t kv_dtype;          /* qsa_kv_dtype; 0 = rows in cfg->dtype */
  void *k_scales;            /* QSA_KV_TURBO8: device [rows][Hkv][D/16] bf16 group scales of k */
  void *v_scales;            /* QSA_KV_TURBO8: the same for v; QSA_KV_BF16K_TURBO4V: [rows][Hkv][D/16]
                                E4M3 scale bytes of v */
} qsa_kv_cache;

/* Bytes of workspace a call with this cfg needs (split-K partials, the
 * prepared queries of long calls and a 256-byte header holding the device
 * error bits).  The workspace must be zero-filled once before its first use.
 * Calls that share a workspace must be ordered on one stream.  Returns 0 if
 * cfg is invalid (see qsa_last_error()). */
size_t qsa_workspace_size(const qsa_cfg *cfg);

/* Steps 2-4 for the keys only: normalise and rotate k_new, round, and write it
 * with v_new to rows seq_lens[b] + l of the cache.
 *   k_new, v_new : device [B][L][Hkv][D] in cfg->dtype (raw k_proj / v_proj outputs)
 *   seq_lens     : device [B] int32, cached rows before this call
 *   positions    : device [B][L] int32, rotary positions of the new rows
 * cfg->workspace may be NULL here (then device-side range errors only skip
 * the write).  Returns a qsa_status. */
int qsa_append_kv(const void *k_new, const void *v_new, const qsa_kv_cache *kv,
                  const int32_t *seq_lens, const int32_t *positions, const qsa_cfg *cfg);

/* Steps 1-6.  Equivalent to qsa_append_kv followed by gated attention over the
 * cache.
 *   q_gate       : device [B][L][Hq][2D], per head [query | gate]
 *   k_new, v_new : device [B][L][Hkv][D]; both NULL when the new rows are
 *                  already in the cache (then the cache is only read)
 *   seq_lens     : device [B] int32, cached rows before this call
 *   positions    : device [B][L] int32, rotary positions of the new rows
 *   out          : device [B][L][Hq][D] in cfg->dtype; must not alias any input
 * Returns a qsa_status. */
int qsa_gated_attention(const void *q_gate, const void *k_new, const void *v_new,
                        const qsa_kv_cache *kv, const int32_t *seq_lens,
                        const int32_t *positions, const qsa_cfg *cfg, void *out);

/* The projections on either side of the core, for the few rows of decode and
 * speculative verify (mlxd PR #99 Summary: doubled q_proj -> split into queries
 * and gate -> o_proj(attn * sigmoid(gate)); Atlas FullAttentionLayer q_proj /
 * k_proj / v_proj / o_proj and Qwen35Kernels qkv_split).  Only the shape
 * fields of cfg (batch, q_len, num_q_heads, num_kv_heads, head_dim, dtype) and
 * cfg->stream are read; rows = batch * q_len <= 64; bf16 only; hidden a
 * multiple of 256; num_q_heads * head_dim a multiple of 256.  Accumulation is
 * fp32 and each output is rounded once (nearest even).  Weights are row-major
 * [out_features][in_features] (a linear layer's weight), device memory owned
 * by the caller; outputs must not alias inputs.  Asynchronous on cfg->stream;
 * returns a qsa_status.
 *
 * qsa_qkv_proj: x [rows][hidden]; w_qkv [2 Hq D + 2 Hkv D][hidden] holding the
 * q_proj rows (per head h: its D query rows, then its D gate rows), then the
 * k_proj rows, then the v_proj rows.  Writes q_gate [rows][Hq][2D] (per head
 * [query | gate], the layout qsa_gated_attention reads), k_new [rows][Hkv][D]
 * and v_new [rows][Hkv][D]: the split of the doubled q_proj output is where the
 * products are stored. */
int qsa_qkv_proj(const void *x, const void *w_qkv, int32_t hidden, const qsa_cfg *cfg, void *q_gate,
                 void *k_new, void *v_new);

/* qsa_o_proj: y [rows][hidden] = attn W_o^T with attn [rows][Hq D] (the gated
 * output of qsa_gated_attention) and w_o [hidden][Hq D]. */
int qsa_o_proj(const void *attn, const void *w_o, int32_t hidden, const qsa_cfg *cfg, void *y);

/* One decode step of the GatedDeltaNet (linear-attention) layer that hybrid
 * Qwen3.5 interleaves with the gated attention layers (Atlas docs,
 * spark_model/forward/qwen3_5/mod.rs: LinearAttentionLayer, LinearAttentionState,
 * LinearAttentionScratch, Qwen35ForwardConfig GDN sizes, Qwen35Kernels
 * causal_conv1d_update_l2norm, gdn_compute_gate, sigmoid_bf16_to_f32,
 * gated_delta_rule_decode), for a batch of sequences with one new token each.
 * The pages give the tensors and kernel names; the rule is the published gated
 * delta rule:
 *   conv   : per channel c, the conv state row (the K latest inputs, oldest
 *            first) takes the new input; u_c = silu(sum_j conv_w[c][j] row[j])
 *   q, k   : per key head, x / sqrt(sum x^2 + 1e-6); q also / sqrt(Dk)
 *   gate   : g = -exp(a_log) softplus(a + dt_bias); beta = sigmoid(b)
 *   state  : per value head h (reading key head h / (Hv / Hk)),
 *            S <- exp(g) S;  S <- S + beta k (v - S^T k)^T;  o = S^T q
 *   output : y = o / sqrt(mean(o^2) + rms_eps) * norm_w * silu(z)
 * u = [q channels Hk Dk | k channels Hk Dk | v channels Hv Dv] (C channels).
 *
 * Arguments (device pointers, 16-byte aligned, owned by the caller):
 *   qkv        : [B][C] bf16, the in_proj_qkv output of each sequence's token
 *   z          : [B][Hv Dv] bf16, the in_proj_z output (the output gate)
 *   a, b       : [B][Hv] bf16, the in_proj_a / in_proj_b outputs
 *   conv_w     : [C][K] bf16;  a_log : [Hv] fp32;  dt_bias : [Hv] bf16;
 *   norm_w     : [Dv] bf16
 *   conv_state : [B][C][K] fp32, read and updated in place
 *   state      : [B][Hv][Dk][Dv] fp32, read and updated in place
 *   y          : [B][Hv][Dv] bf16, written; must not alias any other argument
 * Supported: Dk = Dv = 128, Hv / Hk in {1, 2, 4}, 1 <= K <= 4, batch >= 0.
 * Arithmetic is fp32 (y rounded to bf16 once).  Asynchronous on cfg->stream;
 * returns a qsa_status (invalid or unsupported arguments are refused before
 * anything runs). */
typedef struct qsa_gdn_cfg {
  int32_t batch;        /* B: sequences */
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv (the state heads) */
  int32_t k_head_dim;   /* Dk */
  int32_t v_head_dim;   /* Dv */
  int32_t conv_kernel;  /* K */
  float rms_eps;        /* of the output norm */
  void *stream;         /* hipStream_t, NULL for the default stream */
} qsa_gdn_cfg;

int qsa_gdn_decode(const void *qkv, const void *z, const void *a, const void *b, const void *conv_w,
                   const float *a_log, const void *dt_bias, const void *norm_w, float *conv_state, float *state,
                   void *y, const qsa_gdn_cfg *cfg);

/* Bytes of device scratch that qsa_gated_attention_noalloc holds per GPU. */
#define QSA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* qsa_gated_attention without a caller workspace, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, result
 * and errors as qsa_gated_attention, except that cfg->workspace and
 * cfg->workspace_bytes are ignored: the call uses a scratch array of
 * QSA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (set up, and cleared once, on the first call on that
 * GPU, which must be current).  It calls no hipMalloc, hipFree or allocating
 * routine.  A call whose plan needs more scratch than that returns
 * QSA_ERR_WORKSPACE (qsa_workspace_size() tells the need).  Every call on one
 * GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, no ordering between them) race and give wrong results.  Device-side
 * range errors show as NaN outputs only (the error bits stay in the scratch
 * array, which the caller cannot read). */
int qsa_gated_attention_noalloc(const void *q_gate, const void *k_new, const void *v_new,
                                const qsa_kv_cache *kv, const int32_t *seq_lens,
                                const int32_t *positions, const qsa_cfg *cfg, void *out);

/* Human-readable launch plan for cfg (route, chunking, grid), written to buf.
 * Returns the number of characters the full text needs, or a negative
 * qsa_status if cfg is invalid. */
int qsa_describe_plan(const qsa_cfg *cfg, char *buf, size_t buf_len);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *qsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
