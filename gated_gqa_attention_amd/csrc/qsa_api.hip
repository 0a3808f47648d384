// qsa_api.hip -- the C ABI (include/qsa.h): host-side validation, launch
// planning, workspace sizing and kernel launches.  Nothing here allocates,
// synchronises or falls back to another path: an unsupported request is an
// error, as the pages' engines do at admission (mlxd PR #99, Decision R1 and
// the first reply: reject at load rather than approximate; Atlas
// Qwen35Kernels::resolve: fail loudly).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qsa.h"
#include "qsa_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

enum Route { kRouteF32 = 0, kRouteFused = 1, kRoutePrepared = 2 };
const char *route_name(int r) {
  return r == kRouteF32 ? "f32_rows" : r == kRouteFused ? "fused_splitk" : "prepared_tiles";
}

struct Plan {
  int route = 0;
  int rows = 0, tiles = 0, chunks = 1, chunk_keys = 0, even_split = 0;
  int64_t blocks = 0;
  size_t off_ml = 0, off_o = 0, off_tinfo = 0, off_qt = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate_cfg(const qsa_cfg *c) {
  if (!c) return fail(QSA_ERR_INVALID, "cfg is NULL");
  if (c->batch < 1 || c->q_len < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1)
    return fail(QSA_ERR_INVALID, "batch, q_len, num_q_heads and num_kv_heads must be >= 1 (got %d, %d, %d, %d)",
                c->batch, c->q_len, c->num_q_heads, c->num_kv_heads);
  if (c->num_q_heads % c->num_kv_heads)
    return fail(QSA_ERR_INVALID, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", c->num_q_heads,
                c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not supported (64 | 128 | 256)", c->head_dim);
  if (c->rotary_dim < 0 || c->rotary_dim > c->head_dim || (c->rotary_dim & 1))
    return fail(QSA_ERR_INVALID, "rotary_dim %d must be even and in [0, head_dim=%d]", c->rotary_dim,
                c->head_dim);
  if (!(std::isfinite(c->rope_theta) && c->rope_theta > 0.f))
    return fail(QSA_ERR_INVALID, "rope_theta must be finite and > 0");
  if (!(std::isfinite(c->rms_eps) && c->rms_eps >= 0.f))
    return fail(QSA_ERR_INVALID, "rms_eps must be finite and >= 0");
  if (!(std::isfinite(c->softmax_scale) && c->softmax_scale >= 0.f))
    return fail(QSA_ERR_INVALID, "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  if (c->dtype != QSA_BF16 && c->dtype != QSA_F32)
    return fail(QSA_ERR_UNSUPPORTED, "dtype %d not supported (QSA_BF16 | QSA_F32)", c->dtype);
  if (c->max_seq_len < c->q_len || c->max_seq_len > (1 << 30))
    return fail(QSA_ERR_INVALID, "max_seq_len %d must be in [q_len=%d, 2^30]", c->max_seq_len, c->q_len);
  if (c->force_splits < 0) return fail(QSA_ERR_INVALID, "force_splits must be >= 0");
  if (!c->q_norm_w || !c->k_norm_w) return fail(QSA_ERR_INVALID, "q_norm_w and k_norm_w must be device pointers");
  return QSA_OK;
}

// row_tiles: the short-query route may cut a KV group's rows into row tiles (the bf16
// cache's kernel; the quantized caches' kernel takes a group's rows whole).
int make_plan(const qsa_cfg *c, Plan *pl, bool row_tiles = true) {
  const int64_t B = c->batch, L = c->q_len, Hq = c->num_q_heads, Hkv = c->num_kv_heads, D = c->head_dim;
  const int64_t G = Hq / Hkv;
  const int64_t rows_total = L * G;
  const size_t es = c->dtype == QSA_BF16 ? 2 : 4;
  const int64_t S = c->max_seq_len;
  Plan p;
  if (c->dtype == QSA_F32) {
    p.route = kRouteF32;
    p.rows = (int)std::min<int64_t>(rows_total, qsa::kTileRows);
    p.tiles = 1;
    p.chunks = 1;
    p.chunk_keys = (int)S;
    p.blocks = B * L * Hq;
  } else {
    // The short-query kernel packs L, G and Hq into one 32-bit argument,
    // keeps up to 48 prepared query rows and two (cos, sin) tables of L
    // positions x r/2 pairs in LDS beside its key ring, and rotates by whole
    // lanes, so r/2 must be a multiple of the head_dim/16 elements a lane holds.
    const bool fused = rows_total <= qsa::kMaxFusedRows && L <= qsa::kMaxFusedNewRows &&
                       c->num_q_heads <= 32767 && L * (c->rotary_dim / 2) <= qsa::kMaxFusedTable &&
                       (c->rotary_dim / 2) % (D / 16) == 0;
    p.route = fused ? kRouteFused : kRoutePrepared;
    // Short-query route: a KV group's rows in tiles of at most kFusedTileRows,
    // balanced (48 rows: two tiles of 24), so more workgroups share a group's
    // keys and each takes a longer key chunk: fewer split-K partials, and fewer
    // query rows to prepare per workgroup.
    const int64_t tile_rows = fused ? (row_tiles ? qsa::kFusedTileRows : qsa::kMaxFusedRows) : qsa::kPrefillTileRows;
    p.tiles = (int)cdiv(rows_total, tile_rows);
    p.rows = fused ? (int)cdiv(rows_total, p.tiles) : (int)std::min<int64_t>(rows_total, tile_rows);
    const int64_t base = B * Hkv * p.tiles;
    if (!fused) {
      // Tile route: a tile's keys are cut into chunks of equal length, just
      // enough of them to give every CU a workgroup (none shorter than 1024
      // keys; 32 when a test fixes the count).
      const int64_t min_keys = c->force_splits > 0 ? 32 : 1024;
      int64_t ch = c->force_splits > 0 ? c->force_splits : (base >= 256 ? 1 : cdiv(256, base));
      ch = std::min<int64_t>(std::min<int64_t>(ch, std::max<int64_t>(1, S / min_keys)), qsa::kMaxChunks);
      p.even_split = 1;
      p.chunk_keys = (int)std::min<int64_t>(min_keys, S);
      p.chunks = (int)ch;
    } else {
      // Short-query route: chunks of fixed length, the last one taking the
      // remainder.  One round of workgroups (one per CU) for short work; for
      // long work chunks of ~2048 keys (up to ~4096 of them), so ragged lengths
      // balance across the CUs (measured best between 1024 and 8192 keys).
      int64_t ck;
      if (c->force_splits > 0) {
        ck = std::max<int64_t>(1, S / c->force_splits);
      } else {
        const int64_t total = base * S;
        ck = std::max<int64_t>(qsa::kTileKeys, total / 256);
        if (ck > 2048) ck = std::max<int64_t>(2048, total / 4096);
      }
      ck = std::max<int64_t>(ck, cdiv(S, qsa::kMaxChunks));
      p.chunk_keys = (int)std::min<int64_t>(ck, S);
      // long chunks are cut to equal lengths (round(keys / chunk_keys) of them),
      // so no sequence's last chunk carries a remainder of almost a chunk; short
      // ones keep the fixed 64-key stage grid
      p.even_split = c->force_splits == 0 && p.chunk_keys >= 1024;
      p.chunks = (int)std::max<int64_t>(1, (S + (p.even_split ? p.chunk_keys / 2 : 0)) / p.chunk_keys);
    }
    // the short-query grid takes its work items in groups of 8 (one per XCD),
    // times the row tiles; items past the count return at once
    p.blocks = fused ? cdiv(B * Hkv * p.chunks, 8) * 8 * p.tiles : base * p.chunks;
  }
  if (p.blocks > 0x7fffffffLL) return fail(QSA_ERR_UNSUPPORTED, "launch grid too large (%lld workgroups)",
                                           (long long)p.blocks);
  if (B * L * Hq > 0x7fffffffLL)                        // the merge kernels index query rows in 32 bits
    return fail(QSA_ERR_UNSUPPORTED, "batch * q_len * num_q_heads too large (%lld)", (long long)(B * L * Hq));
  // split-K partial slots: chunks per (sequence, KV head, row tile); on the
  // tile route 2 chunks + 1 per pair of row tiles (the middle tile of an odd
  // count alone), for the pieces of the pair's equal key ranges
  const int64_t parts = p.route == kRoutePrepared ? B * Hkv * (p.tiles - p.tiles / 2) * (2 * p.chunks + 1)
                                                  : B * Hkv * p.tiles * p.chunks;
  // (tile route: (max, sum, scale, 0) and fp16 outputs per row; otherwise
  // (max, sum) and fp32 outputs)
  const bool tile_route = p.route == kRoutePrepared;
  size_t off = 256;
  if (p.chunks > 1) {
    p.off_ml = off;
    off = align256(off + (size_t)parts * p.rows * (tile_route ? 4 : 2) * 4);
    p.off_o = off;
    off = align256(off + (size_t)parts * p.rows * D * (tile_route ? 2 : 4));
    if (tile_route) {
      p.off_tinfo = off;
      off = align256(off + (size_t)(B * Hkv * p.tiles) * 4);
    }
  }
  if (p.route != kRouteFused) {
    p.off_qt = off;
    off = align256(off + (size_t)(B * L * Hq * D) * es);
  }
  p.total = off;
  *pl = p;
  return QSA_OK;
}

qsa::Params base_params(const qsa_cfg *c, const Plan &pl) {
  qsa::Params p{};
  p.B = c->batch;
  p.L = c->q_len;
  p.Hq = c->num_q_heads;
  p.Hkv = c->num_kv_heads;
  p.G = p.Hq / p.Hkv;
  p.D = c->head_dim;
  p.r = c->rotary_dim;
  p.rows = pl.rows;
  p.tiles = pl.tiles;
  p.chunks = pl.chunks;
  p.chunk_keys = pl.chunk_keys;
  p.even_split = pl.even_split;
  p.max_seq_len = c->max_seq_len;
  p.eps = c->rms_eps;
  p.scale = c->softmax_scale > 0.f ? c->softmax_scale : (float)(1.0 / std::sqrt((double)c->head_dim));
  p.scale_log2 = p.scale * qsa::kLog2e;
  p.rope_step = c->rotary_dim > 0 ? std::pow((double)c->rope_theta, -2.0 / (double)c->rotary_dim) : 1.0;
  p.wq = c->q_norm_w;
  p.wk = c->k_norm_w;
  return p;
}

int check_device() {
  static std::once_flag once;
  static int status = QSA_OK;
  static std::string msg;
  std::call_once(once, [] {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      status = QSA_ERR_DEVICE;
      msg = "no HIP device available";
      return;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      status = QSA_ERR_DEVICE;
      msg = std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950 only";
    }
  });
  if (status != QSA_OK) return fail(status, "%s", msg.c_str());
  return QSA_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b) return false;
  const char *pa = (const char *)a, *pb = (const char *)b;
  return pa < pb + nb && pb < pa + na;
}

int check_kv(const qsa_kv_cache *kv) {
  if (!kv) return fail(QSA_ERR_INVALID, "kv cache descriptor is NULL");
  if (!kv->k || !kv->v) return fail(QSA_ERR_INVALID, "kv->k and kv->v are required");
  if (kv->num_rows < 1) return fail(QSA_ERR_INVALID, "kv->num_rows must be >= 1");
  if (kv->k == kv->v) return fail(QSA_ERR_INVALID, "kv->k and kv->v must be different buffers");
  if (kv->kv_dtype != QSA_KV_NATIVE && kv->kv_dtype != QSA_KV_TURBO8 && kv->kv_dtype != QSA_KV_BF16K_TURBO4V)
    return fail(QSA_ERR_UNSUPPORTED,
                "kv->kv_dtype %d not supported (QSA_KV_NATIVE | QSA_KV_TURBO8 | QSA_KV_BF16K_TURBO4V)", kv->kv_dtype);
  if (kv->kv_dtype == QSA_KV_TURBO8 && (!kv->k_scales || !kv->v_scales))
    return fail(QSA_ERR_INVALID, "a Turbo8 cache needs kv->k_scales and kv->v_scales");
  if (kv->kv_dtype == QSA_KV_BF16K_TURBO4V && !kv->v_scales)
    return fail(QSA_ERR_INVALID, "a bf16-K / Turbo4-V cache needs kv->v_scales");
  if (kv->kv_dtype != QSA_KV_NATIVE && kv->block_table)
    return fail(QSA_ERR_UNSUPPORTED, "quantized caches are taken in the contiguous layout only");
  if (!kv->block_table) {
    if (!kv->seq_offset) return fail(QSA_ERR_INVALID, "kv->seq_offset is required for a contiguous cache");
    return QSA_OK;
  }
  const int32_t bs = kv->block_size;
  if (bs < 64 || bs > (1 << 16) || (bs & (bs - 1)))
    return fail(QSA_ERR_INVALID, "kv->block_size %d must be a power of two in [64, 65536]", bs);
  if (kv->max_blocks < 1) return fail(QSA_ERR_INVALID, "kv->max_blocks must be >= 1");
  if (kv->num_rows % bs) return fail(QSA_ERR_INVALID, "kv->num_rows must be a multiple of block_size for a paged cache");
  return QSA_OK;
}

// Quantized caches: bf16 activations, and the short-query route's whole-lane
// rotation (the quantizing append shares its key preparation); bf16 K +
// Turbo4 V at head_dim 256.
int check_quant(const qsa_cfg *c, const Plan &pl, int32_t kv_dtype) {
  const char *name = kv_dtype == QSA_KV_TURBO8 ? "Turbo8" : "bf16-K / Turbo4-V";
  if (c->dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "%s caches take bf16 activations only", name);
  if (kv_dtype == QSA_KV_BF16K_TURBO4V && c->head_dim != 256)
    return fail(QSA_ERR_UNSUPPORTED, "bf16-K / Turbo4-V caches take head_dim 256 only (head_dim %d)", c->head_dim);
  if (pl.route != kRouteFused)
    return fail(QSA_ERR_UNSUPPORTED,
                "%s caches are taken on the short-query route only (q_len <= 16, q_len * G <= 48, "
                "rotary_dim / 2 a multiple of head_dim / 16); this call plans route %s", name, route_name(pl.route));
  return QSA_OK;
}

// The 16-level Lloyd-Max quantizer of the standard normal distribution:
// Lloyd's iteration from evenly spread levels, each level moved to the mean of
// the normal over its cell (cells split at the midpoints between levels),
// until no level moves.  Computed once, in double; the kernels get fp32
// levels and fp32 midpoints.
struct Turbo4Codebook {
  float level[16], threshold[15];
  Turbo4Codebook() {
    const double inv_sqrt_2pi = 0.3989422804014327, r2 = 1.4142135623730951;
    auto density = [&](double x) { return std::isinf(x) ? 0.0 : inv_sqrt_2pi * std::exp(-0.5 * x * x); };
    auto upper_tail = [&](double x) { return 0.5 * std::erfc(x / r2); };   // P(X > x)
    double c[16];
    for (int i = 0; i < 16; ++i) c[i] = (i - 7.5) * 0.4;
    for (int round = 0; round < 200000; ++round) {
      double edges[17];
      edges[0] = -INFINITY;
      edges[16] = INFINITY;
      for (int i = 1; i < 16; ++i) edges[i] = 0.5 * (c[i - 1] + c[i]);
      double moved = 0.0;
      for (int i = 0; i < 16; ++i) {
        const double a = edges[i], b = edges[i + 1];
        // mass of the cell from the tail on its own side (no cancellation of two values near 1)
        const double mass = b <= 0.0 ? upper_tail(-b) - upper_tail(-a) : upper_tail(a) - upper_tail(b);
        const double mean = (density(a) - density(b)) / mass;
        moved = std::max(moved, std::fabs(mean - c[i]));
        c[i] = mean;
      }
      if (moved < 1e-16) break;
    }
    for (int i = 0; i < 8; ++i) {                       // exactly symmetric
      const double m = 0.5 * (c[15 - i] - c[i]);
      c[i] = -m;
      c[15 - i] = m;
    }
    for (int i = 0; i < 16; ++i) level[i] = (float)c[i];
    for (int i = 0; i < 15; ++i) threshold[i] = (float)(0.5 * (c[i] + c[i + 1]));
  }
};

qsa::QuantCache quant_of(const qsa_kv_cache *kv) {
  static const Turbo4Codebook cb;
  qsa::QuantCache c;
  c.fmt = kv->kv_dtype == QSA_KV_TURBO8 ? 0 : 1;
  c.k = kv->k;
  c.ks = kv->k_scales;
  c.v = kv->v;
  c.vs = kv->v_scales;
  for (int i = 0; i < 16; ++i) c.cb[i] = cb.level[i];
  for (int i = 0; i < 15; ++i) c.thr[i] = cb.threshold[i];
  return c;
}

int log2_of(int32_t x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

void fill_kv(qsa::Params &p, const qsa_kv_cache *kv, const int32_t *seq_lens, const int32_t *positions) {
  p.kc = kv->k;
  p.vc = kv->v;
  p.seq_offset = kv->seq_offset;
  p.capacity = kv->capacity;
  p.num_rows = kv->num_rows;
  p.btab = kv->block_table;
  p.bs_log2 = kv->block_table ? log2_of(kv->block_size) : 0;
  p.max_blocks = kv->block_table ? kv->max_blocks : 0;
  p.seq_lens = seq_lens;
  p.positions = positions;
}

}  // namespace

extern "C" {

const char *qsa_last_error(void) { return g_err.c_str(); }

size_t qsa_workspace_size(const qsa_cfg *cfg) {
  if (validate_cfg(cfg) != QSA_OK) return 0;
  Plan pl, whole;                                       // the bf16 cache's plan, and the quantized caches'
  if (make_plan(cfg, &pl) != QSA_OK || make_plan(cfg, &whole, false) != QSA_OK) return 0;
  return std::max(pl.total, whole.total);
}

int qsa_describe_plan(const qsa_cfg *cfg, char *buf, size_t len) {
  int rc = validate_cfg(cfg);
  if (rc != QSA_OK) return rc;
  Plan pl, whole;
  if ((rc = make_plan(cfg, &pl)) != QSA_OK || (rc = make_plan(cfg, &whole, false)) != QSA_OK) return rc;
  pl.total = std::max(pl.total, whole.total);           // what qsa_workspace_size asks for
  // the plan of a bf16 cache (a quantized cache's takes a KV group's rows whole);
  // merge: how split-K partials are combined -- "kernel" (a second kernel, launched
  // only when the grid splits keys) or "none"
  return snprintf(buf, len,
                  "route=%s rows=%d tiles=%d chunks=%d chunk_keys=%d workgroups=%lld threads=%d "
                  "workspace=%zu merge=%s",
                  route_name(pl.route), pl.rows, pl.tiles, pl.chunks, pl.chunk_keys, (long long)pl.blocks,
                  pl.route == kRoutePrepared ? qsa::kPrefillThreads : qsa::kThreads, pl.total,
                  pl.chunks > 1 ? "kernel" : "none");
}

int qsa_append_kv(const void *k_new, const void *v_new, const qsa_kv_cache *kv, const int32_t *seq_lens,
                  const int32_t *positions, const qsa_cfg *cfg) {
  int rc = validate_cfg(cfg);
  if (rc != QSA_OK) return rc;
  if ((rc = check_kv(kv)) != QSA_OK) return rc;
  if (!k_new || !v_new || !seq_lens || !positions)
    return fail(QSA_ERR_INVALID, "k_new, v_new, seq_lens and positions are required");
  if ((rc = check_device()) != QSA_OK) return rc;
  Plan pl;
  if ((rc = make_plan(cfg, &pl)) != QSA_OK) return rc;
  qsa::Params p = base_params(cfg, pl);
  fill_kv(p, kv, seq_lens, positions);
  p.k_new = k_new;
  p.v_new = v_new;
  p.err = cfg->workspace ? (int32_t *)cfg->workspace : nullptr;
  hipError_t e;
  if (kv->kv_dtype != QSA_KV_NATIVE) {
    if ((rc = check_quant(cfg, pl, kv->kv_dtype)) != QSA_OK) return rc;
    e = qsa::launch_quant_append(p, quant_of(kv), (hipStream_t)cfg->stream);
    if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "append launch failed: %s", hipGetErrorString(e));
    return QSA_OK;
  }
  e = qsa::launch_prologue(p, cfg->dtype, false, true, (hipStream_t)cfg->stream);
  if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "append launch failed: %s", hipGetErrorString(e));
  return QSA_OK;
}

}  // extern "C"

namespace {

// Everything of qsa_gated_attention after the workspace has been chosen: ws
// holds ws_bytes of device memory (the caller's workspace, or this device's
// scratch array for the allocation-free entry point).
int gated_attention_in(const void *q_gate, const void *k_new, const void *v_new, const qsa_kv_cache *kv,
                       const int32_t *seq_lens, const int32_t *positions, const qsa_cfg *cfg, void *out,
                       void *ws_ptr, size_t ws_bytes, const char *ws_name) {
  int rc = validate_cfg(cfg);
  if (rc != QSA_OK) return rc;
  if ((rc = check_kv(kv)) != QSA_OK) return rc;
  if (!q_gate || !seq_lens || !positions || !out)
    return fail(QSA_ERR_INVALID, "q_gate, seq_lens, positions and out are required");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(QSA_ERR_INVALID, "k_new and v_new must both be given or both be NULL");
  const size_t es = cfg->dtype == QSA_BF16 ? 2 : 4;
  const size_t nrow = (size_t)cfg->batch * cfg->q_len;
  const size_t out_bytes = nrow * cfg->num_q_heads * cfg->head_dim * es;
  // bytes of each cache tensor: elements times bytes per element (Turbo8 codes 1;
  // Turbo4 indices 1/2), scales per 16 elements (Turbo8 bf16 2, Turbo4 E4M3 1)
  const size_t elems = (size_t)kv->num_rows * cfg->num_kv_heads * cfg->head_dim;
  const int32_t kd = kv->kv_dtype;
  const size_t k_bytes = kd == QSA_KV_TURBO8 ? elems : elems * (kd == QSA_KV_BF16K_TURBO4V ? 2 : es);
  const size_t v_bytes = kd == QSA_KV_TURBO8 ? elems : kd == QSA_KV_BF16K_TURBO4V ? elems / 2 : elems * es;
  const size_t ks_bytes = kd == QSA_KV_TURBO8 ? elems / 8 : 0;
  const size_t vs_bytes = kd == QSA_KV_TURBO8 ? elems / 8 : kd == QSA_KV_BF16K_TURBO4V ? elems / 16 : 0;
  const size_t new_bytes = nrow * cfg->num_kv_heads * cfg->head_dim * es;
  if (overlaps(out, out_bytes, q_gate, 2 * out_bytes) || overlaps(out, out_bytes, k_new, new_bytes) ||
      overlaps(out, out_bytes, v_new, new_bytes) || overlaps(out, out_bytes, kv->k, k_bytes) ||
      overlaps(out, out_bytes, kv->v, v_bytes) || overlaps(out, out_bytes, kv->k_scales, ks_bytes) ||
      overlaps(out, out_bytes, kv->v_scales, vs_bytes))
    return fail(QSA_ERR_INVALID, "out must not alias q_gate, k_new, v_new or the cache");
  Plan pl;
  if ((rc = make_plan(cfg, &pl, kv->kv_dtype == QSA_KV_NATIVE)) != QSA_OK) return rc;
  if (kv->kv_dtype != QSA_KV_NATIVE && (rc = check_quant(cfg, pl, kv->kv_dtype)) != QSA_OK) return rc;
  if (kv->block_table) {
    // Paged caches on the short-query route only.  A workgroup holds the block
    // ids of its key chunk (at most 128): with fixed chunks the last one has
    // fewer than 2 chunk_keys keys, with equal chunks about 1.5 chunk_keys.
    if (pl.route != kRouteFused)
      return fail(QSA_ERR_UNSUPPORTED,
                  "paged caches are taken on the short-query route only (bf16, q_len <= 16, q_len * G <= 48); "
                  "this call plans route %s", route_name(pl.route));
    const int64_t span = 2 * (int64_t)pl.chunk_keys + cfg->q_len;
    if ((span >> log2_of(kv->block_size)) + 2 > 128)
      return fail(QSA_ERR_UNSUPPORTED, "key chunks of %d keys span more than 128 blocks of %d rows",
                  pl.chunk_keys, kv->block_size);
  }
  // the contract is qsa_workspace_size(cfg), whichever cache format this call has
  Plan whole;
  if ((rc = make_plan(cfg, &whole, false)) != QSA_OK) return rc;
  const size_t need = std::max(pl.total, whole.total);
  if (!ws_ptr || ws_bytes < need)
    return fail(QSA_ERR_WORKSPACE, "%s of %zu bytes needed, %zu %s", ws_name, need,
                ws_ptr ? ws_bytes : (size_t)0, ws_ptr ? "available" : "given");
  if ((rc = check_device()) != QSA_OK) return rc;

  qsa::Params p = base_params(cfg, pl);
  fill_kv(p, kv, seq_lens, positions);
  p.q_gate = q_gate;
  p.k_new = k_new;
  p.v_new = v_new;
  p.out = out;
  char *ws = (char *)ws_ptr;
  p.err = (int32_t *)ws;
  p.part_ml = pl.off_ml ? (float *)(ws + pl.off_ml) : nullptr;
  p.part_o = pl.off_o ? (float *)(ws + pl.off_o) : nullptr;
  p.tinfo = pl.off_tinfo ? (int32_t *)(ws + pl.off_tinfo) : nullptr;
  p.qt = pl.off_qt ? (void *)(ws + pl.off_qt) : nullptr;
  hipStream_t s = (hipStream_t)cfg->stream;
  const bool has_new = k_new != nullptr;

  // optional timing events: the dispatch times of the kernel that streams the KV cache
  qsa::Timing tm;
  tm.begin = (hipEvent_t)cfg->timing_begin;
  tm.end = (hipEvent_t)cfg->timing_end;

  hipError_t e = hipSuccess;
  switch (pl.route) {
    case kRouteF32:
      e = qsa::launch_prologue(p, QSA_F32, true, has_new, s);
      if (e == hipSuccess) e = qsa::launch_rows_f32(p, s, tm);
      break;
    case kRouteFused:
      if (kv->kv_dtype != QSA_KV_NATIVE) {                // V in the WHT basis: the merge rotates back
        e = qsa::launch_quant_bf16(p, quant_of(kv), s, tm);
        if (e == hipSuccess && pl.chunks > 1) e = qsa::launch_combine_wht_bf16(p, s);
      } else {
        e = qsa::launch_stream_bf16(p, s, tm);
        if (e == hipSuccess && pl.chunks > 1) e = qsa::launch_combine_bf16(p, s, false);
      }
      break;
    default:
      e = qsa::launch_prologue(p, QSA_BF16, true, has_new, s);
      if (e == hipSuccess) e = qsa::launch_tile_bf16(p, s, tm);
      if (e == hipSuccess && pl.chunks > 1) e = qsa::launch_combine_bf16(p, s, true);
      break;
  }
  if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(e));
  return QSA_OK;
}

// Scratch of the allocation-free entry point: one array per device, part of
// the library's code object, held until the process ends.  In host code its
// name is only a handle: the device address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)QSA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

__global__ void zero_words(uint4 *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// This device's scratch address, set up once per device: the symbol's address
// on the current device, and the array cleared once by a fill kernel on the
// caller's stream (the calls keep it in the state they found it in: the merge
// counters return to zero at the end of every call).
int scratch_for_current_device(hipStream_t s, void **ptr) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(QSA_ERR_DEVICE, "no current HIP device (or device index past 63)");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a)
      return fail(QSA_ERR_DEVICE, "scratch array not available on device %d: %s", dev, hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words, dim3(1024), dim3(256), 0, s, (uint4 *)a, kScratchBytes / 16);
    if ((e = hipGetLastError()) != hipSuccess)
      return fail(QSA_ERR_DEVICE, "scratch clear failed on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return QSA_OK;
}

// Shape checks of the projections: the rows, heads and head_dim of cfg, bf16,
// hidden a multiple of 256 (the K split of the projection kernel).
int validate_proj(const qsa_cfg *c, int32_t hidden) {
  if (!c) return fail(QSA_ERR_INVALID, "cfg is NULL");
  if (c->batch < 1 || c->q_len < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 ||
      c->num_q_heads % c->num_kv_heads)
    return fail(QSA_ERR_INVALID, "batch, q_len >= 1 and num_q_heads a multiple of num_kv_heads >= 1 required");
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(QSA_ERR_UNSUPPORTED, "head_dim %d not supported (64 | 128 | 256)", c->head_dim);
  if (c->dtype != QSA_BF16) return fail(QSA_ERR_UNSUPPORTED, "the projections take bf16 only");
  if ((int64_t)c->batch * c->q_len > qsa::kMaxLinearRows)
    return fail(QSA_ERR_UNSUPPORTED, "the projections take at most %d rows (batch * q_len = %lld)",
                qsa::kMaxLinearRows, (long long)c->batch * c->q_len);
  if (hidden < 256 || hidden % 256)
    return fail(QSA_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 256", hidden);
  if ((c->num_q_heads * c->head_dim) % 256)
    return fail(QSA_ERR_UNSUPPORTED, "num_q_heads * head_dim must be a multiple of 256");
  return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_gated_attention(const void *q_gate, const void *k_new, const void *v_new, const qsa_kv_cache *kv,
                        const int32_t *seq_lens, const int32_t *positions, const qsa_cfg *cfg, void *out) {
  if (!cfg) return fail(QSA_ERR_INVALID, "cfg is NULL");
  return gated_attention_in(q_gate, k_new, v_new, kv, seq_lens, positions, cfg, out, cfg->workspace,
                            cfg->workspace_bytes, "workspace");
}

int qsa_qkv_proj(const void *x, const void *w_qkv, int32_t hidden, const qsa_cfg *cfg, void *q_gate, void *k_new,
                 void *v_new) {
  int rc = validate_proj(cfg, hidden);
  if (rc != QSA_OK) return rc;
  if (!x || !w_qkv || !q_gate || !k_new || !v_new)
    return fail(QSA_ERR_INVALID, "x, w_qkv, q_gate, k_new and v_new are required");
  const int M = cfg->batch * cfg->q_len, D = cfg->head_dim;
  const int nq = cfg->num_q_heads * 2 * D, nk = cfg->num_kv_heads * D;
  const size_t xb = (size_t)M * hidden * 2, wb = (size_t)(nq + 2 * nk) * hidden * 2;
  const size_t qb = (size_t)M * nq * 2, kb = (size_t)M * nk * 2;
  const void *outs[3] = {q_gate, k_new, v_new};
  const size_t ob[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], ob[i], x, xb) || overlaps(outs[i], ob[i], w_qkv, wb))
      return fail(QSA_ERR_INVALID, "the outputs must not alias x or w_qkv");
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return fail(QSA_ERR_INVALID, "q_gate, k_new and v_new overlap");
  }
  if ((rc = check_device()) != QSA_OK) return rc;
  hipError_t e = qsa::launch_linear_bf16(x, w_qkv, M, nq + 2 * nk, hidden, q_gate, nq, nq, k_new, nq + nk, nk, v_new,
                                         nk, (hipStream_t)cfg->stream);
  if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "projection launch failed: %s", hipGetErrorString(e));
  return QSA_OK;
}

int qsa_o_proj(const void *attn, const void *w_o, int32_t hidden, const qsa_cfg *cfg, void *y) {
  int rc = validate_proj(cfg, hidden);
  if (rc != QSA_OK) return rc;
  if (!attn || !w_o || !y) return fail(QSA_ERR_INVALID, "attn, w_o and y are required");
  const int M = cfg->batch * cfg->q_len, K = cfg->num_q_heads * cfg->head_dim;
  if (overlaps(y, (size_t)M * hidden * 2, attn, (size_t)M * K * 2) ||
      overlaps(y, (size_t)M * hidden * 2, w_o, (size_t)hidden * K * 2))
    return fail(QSA_ERR_INVALID, "y must not alias attn or w_o");
  if ((rc = check_device()) != QSA_OK) return rc;
  hipError_t e = qsa::launch_linear_bf16(attn, w_o, M, hidden, K, y, hidden, hidden, y, hidden, hidden, y, hidden,
                                         (hipStream_t)cfg->stream);
  if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "projection launch failed: %s", hipGetErrorString(e));
  return QSA_OK;
}

int qsa_gdn_decode(const void *qkv, const void *z, const void *a, const void *b, const void *conv_w,
                   const float *a_log, const void *dt_bias, const void *norm_w, float *conv_state, float *state,
                   void *y, const qsa_gdn_cfg *cfg) {
  if (!cfg) return fail(QSA_ERR_INVALID, "cfg is NULL");
  const qsa_gdn_cfg &c = *cfg;
  if (c.batch < 0 || c.num_k_heads < 1 || c.num_v_heads < 1 || c.num_v_heads % c.num_k_heads)
    return fail(QSA_ERR_INVALID, "batch >= 0 and num_v_heads a multiple of num_k_heads >= 1 required");
  const int R = c.num_v_heads / c.num_k_heads;
  if (R != 1 && R != 2 && R != 4)
    return fail(QSA_ERR_UNSUPPORTED, "num_v_heads / num_k_heads = %d not supported (1 | 2 | 4)", R);
  if (c.k_head_dim != 128 || c.v_head_dim != 128)
    return fail(QSA_ERR_UNSUPPORTED, "k_head_dim %d, v_head_dim %d not supported (128, 128)", c.k_head_dim,
                c.v_head_dim);
  if (c.conv_kernel < 1 || c.conv_kernel > 4)
    return fail(QSA_ERR_UNSUPPORTED, "conv_kernel %d not supported (1 .. 4)", c.conv_kernel);
  if (!(c.rms_eps >= 0.f)) return fail(QSA_ERR_INVALID, "rms_eps must be >= 0");
  const void *ptrs[11] = {qkv, z, a, b, conv_w, a_log, dt_bias, norm_w, conv_state, state, y};
  for (const void *q : ptrs) {
    if (!q) return fail(QSA_ERR_INVALID, "every tensor argument is required");
    if ((uintptr_t)q % 16) return fail(QSA_ERR_INVALID, "tensor arguments must be 16-byte aligned");
  }
  const int64_t B = c.batch, Hk = c.num_k_heads, Hv = c.num_v_heads, D = 128, K = c.conv_kernel;
  const int64_t C = 2 * Hk * D + Hv * D;
  if (B * Hk > 0x7fffffff) return fail(QSA_ERR_UNSUPPORTED, "batch * num_k_heads too large");
  const size_t yb = (size_t)(B * Hv * D * 2);
  const struct { const void *p; size_t n; } others[10] = {
      {qkv, (size_t)(B * C * 2)}, {z, (size_t)(B * Hv * D * 2)}, {a, (size_t)(B * Hv * 2)},
      {b, (size_t)(B * Hv * 2)}, {conv_w, (size_t)(C * K * 2)}, {a_log, (size_t)(Hv * 4)},
      {dt_bias, (size_t)(Hv * 2)}, {norm_w, (size_t)(D * 2)}, {conv_state, (size_t)(B * C * K * 4)},
      {state, (size_t)(B * Hv * D * D * 4)}};
  for (const auto &o : others)
    if (overlaps(y, yb, o.p, o.n)) return fail(QSA_ERR_INVALID, "y must not alias any other argument");
  if (overlaps(conv_state, others[8].n, state, others[9].n))
    return fail(QSA_ERR_INVALID, "conv_state and state overlap");
  for (int i = 0; i < 8; ++i)
    if (overlaps(others[i].p, others[i].n, conv_state, others[8].n) ||
        overlaps(others[i].p, others[i].n, state, others[9].n))
      return fail(QSA_ERR_INVALID, "the states must not alias the inputs");
  int rc;
  if ((rc = check_device()) != QSA_OK) return rc;
  qsa::GdnParams p;
  p.qkv = (const qsa::bf16_t *)qkv;
  p.z = (const qsa::bf16_t *)z;
  p.a = (const qsa::bf16_t *)a;
  p.b = (const qsa::bf16_t *)b;
  p.conv_w = (const qsa::bf16_t *)conv_w;
  p.dt_bias = (const qsa::bf16_t *)dt_bias;
  p.norm_w = (const qsa::bf16_t *)norm_w;
  p.a_log = a_log;
  p.conv_state = conv_state;
  p.state = state;
  p.y = (qsa::bf16_t *)y;
  p.B = (int)B;
  p.Hk = (int)Hk;
  p.Hv = (int)Hv;
  p.K = (int)K;
  p.C = (int)C;
  p.eps = c.rms_eps;
  const hipError_t e = qsa::launch_gdn_decode(p, (hipStream_t)c.stream);
  if (e != hipSuccess) return fail(QSA_ERR_DEVICE, "GatedDeltaNet launch failed: %s", hipGetErrorString(e));
  return QSA_OK;
}

int qsa_gated_attention_noalloc(const void *q_gate, const void *k_new, const void *v_new, const qsa_kv_cache *kv,
                                const int32_t *seq_lens, const int32_t *positions, const qsa_cfg *cfg,
                                void *out) {
  int rc = validate_cfg(cfg);
  if (rc != QSA_OK) return rc;
  Plan pl, whole;
  if ((rc = make_plan(cfg, &pl)) != QSA_OK || (rc = make_plan(cfg, &whole, false)) != QSA_OK) return rc;
  pl.total = std::max(pl.total, whole.total);           // either cache format's plan fits
  if (pl.total > kScratchBytes)
    return fail(QSA_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use qsa_gated_attention with a workspace)", pl.total, kScratchBytes);
  if ((rc = check_device()) != QSA_OK) return rc;
  void *ws = nullptr;
  if ((rc = scratch_for_current_device((hipStream_t)cfg->stream, &ws)) != QSA_OK) return rc;
  return gated_attention_in(q_gate, k_new, v_new, kv, seq_lens, positions, cfg, out, ws, kScratchBytes,
                            "scratch");
}

}  // extern "C"
