// qsa_internal.h -- launch parameters and device helpers shared by the HIP kernels.
//
// Target: AMD CDNA4 (gfx950), 64-wide wavefronts, MFMA bf16 16x16x32.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;         // four wavefronts per workgroup
constexpr int kWave = 64;
constexpr int kTileKeys = 64;         // shortest key chunk the planner makes (one short-query stage)
constexpr int kTileRows = 64;         // query rows per tile of the fp32 route
constexpr int kPrefillRowTiles = 2;  // 16-row MFMA tiles per wavefront of the tile (prefill) kernel
constexpr int kPrefillThreads = 512;  // eight wavefronts per workgroup of the tile kernel
constexpr int kPrefillTileRows = 16 * kPrefillRowTiles * kPrefillThreads / kWave;   // query rows per workgroup
constexpr int kMaxFusedNewRows = 16;  // new rows a fused call may append per sequence
constexpr int kMaxPairs = 128;        // rotary pairs (rotary_dim / 2) supported
constexpr int kMaxChunks = 4096;      // key chunks per (sequence, KV head, tile)
constexpr int kMaxFusedTable = 512;   // (cos, sin) pairs a short-query call tabulates: L * r/2
constexpr int kMaxFusedRows = 48;     // query rows (group heads x new rows) of a short-query call
constexpr int kFusedTileRows = 32;    // query rows per workgroup of the bf16 short-query kernel
static_assert(2 * kFusedTileRows >= kMaxFusedRows && kFusedTileRows == 32,
              "the short-query kernel takes one row tile of up to 32 rows, or two of 17 .. 24");
constexpr float kLog2e = 1.4426950408889634f;

// Workspace layout (bytes, 256-aligned sections):
//   [0, 256)   header; int32 at 0 = sticky device error bits
//   part_ml    float [slots][chunks][rows][2]   per-chunk running max (log2 units) and sum
//   part_o     float [slots][chunks][rows][D]   per-chunk unnormalised outputs
//   qt         prepared queries [B][L][Hq][D] (bf16 or fp32)
//   tinfo      int32 [B][Hkv][tiles]            tile route: a split tile's partial slots
// where slots = B * Hkv * tiles.  On the tile route the partials are instead
// [B][Hkv][pairs][2 chunks + 1][rows] (pair_ranges), part_ml holding (max, sum,
// scale, 0) per row and part_o the fp16 output divided by the sum and the scale;
// tinfo holds the first and last slot of each tile's pieces within its pair
// (first | last << 16).
constexpr int32_t kErrRange = 1;

struct Params {
  int B, L, Hq, Hkv, G, D, r;
  int rows;           // query rows per tile
  int tiles;          // row tiles per (sequence, KV head)
  int chunks;         // grid extent in key chunks
  int chunk_keys;     // fixed chunks: keys per chunk (the last one also takes the remainder);
                      // even chunks: the shortest chunk
  int even_split;     // 1: a tile's keys are cut into up to `chunks` chunks of equal length
  int max_seq_len;
  float eps;
  float scale_log2;   // softmax scale * log2(e)
  float scale;        // softmax scale
  const void *q_gate;
  const void *k_new;
  const void *v_new;
  void *kc;
  void *vc;
  const int64_t *seq_offset;
  const int32_t *capacity;  // may be null
  int64_t num_rows;
  const int32_t *btab;      // paged caches: block table [B][max_blocks]; null when contiguous
  int bs_log2;              // paged: log2 of the rows per block
  int max_blocks;           // paged: block table row stride
  const int32_t *seq_lens;
  const int32_t *positions;
  const void *wq;
  const void *wk;
  void *out;
  int32_t *err;       // may be null
  float *part_ml;
  float *part_o;
  int32_t *tinfo;     // tile route with split tiles: each tile's piece slots
  void *qt;
  double rope_step;            // theta^(-2/r) (r > 0), computed on the host in double
};

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return (bf16_t)x; }  // v_cvt_pk_bf16_f32: nearest-even

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// cos/sin of the angle pos * inv, inv = theta^(-2i/r).  The angle reaches 3e4
// rad, so it is formed and reduced modulo 2*pi in double (two-part Cody-Waite
// constant), and only the reduced angle goes through fp32 sincos.
__device__ __forceinline__ void rope_angle_cs(int pos, double inv, float &c, float &s) {
  const double a = (double)pos * inv;
  const double k = rint(a * 0.15915494309189535);  // 1 / (2 pi)
  double red = fma(-k, 6.283185307179586, a);
  red = fma(-k, 2.4492935982947064e-16, red);
  sincosf((float)red, &s, &c);
}

// theta^(-2i/r) = step^i for 0 <= i < kMaxPairs, by binary powers in double
// (at most 14 roundings, ~1e-15 relative) of the host's step = theta^(-2/r): a
// scalar argument, where reading a per-lane entry of a table in the argument
// segment would be a slow vector load.
__device__ __forceinline__ double rope_freq(double step, int i) {
  double f = 1.0, sq = step;
#pragma unroll
  for (int bit = 0; bit < 7; ++bit) {                   // kMaxPairs = 2^7
    f = (i >> bit) & 1 ? f * sq : f;
    sq *= sq;
  }
  return f;
}

// Keys [0, kend) of one (sequence, row tile) are cut into max(1, kend / chunk_keys)
// chunks of chunk_keys keys; the last chunk also takes the remainder.
__device__ __forceinline__ int chunk_count(int64_t kend, int chunk_keys) {
  const int64_t c = kend / chunk_keys;
  return c < 1 ? 1 : (int)c;
}
// With even_split they are cut instead into min(chunks, max(1, round(kend /
// chunk_keys))) chunks of equal length: chunk c covers [c kend / nch,
// (c + 1) kend / nch).
__device__ __forceinline__ int tile_chunk_count(int64_t kend, int even_split, int chunks, int chunk_keys) {
  if (!even_split) return chunk_count(kend, chunk_keys);
  const int64_t c = (kend + chunk_keys / 2) / chunk_keys;
  return c < 1 ? 1 : (c > chunks ? chunks : (int)c);
}
__device__ __forceinline__ int64_t chunk_begin(int64_t kend, int even_split, int nch, int chunk_keys, int c) {
  return even_split ? (int64_t)c * kend / nch : (int64_t)c * chunk_keys;
}

// Tile route (prepared queries, tiles of `rows` query rows).  Keys tile t of
// sequence b can see: up to its last row's position, n_b + l_last.
__device__ __forceinline__ int64_t tile_keys(int n, int t, int rows, int R, int G) {
  return (int64_t)n + (min((t + 1) * rows, R) - 1) / G + 1;
}
// With more than one chunk per tile, tiles t and T - 1 - t of one (sequence,
// KV head) form a pair (the middle tile of an odd count stands alone).  The
// pair's keys, those of tile t followed by those of tile T - 1 - t (S in all),
// are cut into nw ranges of equal length, range v = [v S / nw, (v + 1) S / nw),
// with nw = min(most, max(1, round(S / chunk_keys))) and most = 2 chunks (one
// tile alone: chunks).  A range that crosses the boundary between the two
// tiles holds one piece of each.  The pieces' split-K partials take slot v of
// the pair for the first tile's piece and v + 1 for the second's, 2 chunks + 1
// slots per pair.
//
// floor(a / b) for integers 0 <= a < 2^53 and b >= 1, from the correctly
// rounded double quotient: it is exact when the quotient is an integer, and
// otherwise lies within a/b 2^-53 < 1/b of it, nearer than the next integer.
// On the GPU this is a short fp64 sequence where a 64-bit integer division is
// a long one.  Every numerator below is under 2^45.
__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
  return (int64_t)__builtin_floor((double)a / (double)b);
}
__device__ __forceinline__ int pair_ranges(int64_t S, int most, int chunk_keys) {
  const int64_t c = floor_div(S + chunk_keys / 2, chunk_keys);
  return c < 1 ? 1 : (c > most ? most : (int)c);
}
// The first key of range v, and the range that holds key x of the pair's S
// keys (0 <= x < S): the largest v with range_start(v) <= x.
__device__ __forceinline__ int64_t range_start(int v, int64_t S, int nw) { return floor_div((int64_t)v * S, nw); }
__device__ __forceinline__ int range_of(int64_t x, int64_t S, int nw) { return (int)floor_div((x + 1) * nw - 1, S); }

// Sequence bounds check shared by the prologue and the fp32 kernel.  Returns
// false when rows [0, n + L) of sequence b would leave the cache or pass its
// capacity (paged: the blocks its table row can name).  off: the first row
// (contiguous caches).
__device__ __forceinline__ bool seq_in_range(const Params &p, int b, int n, int64_t &off) {
  const int64_t total = (int64_t)n + p.L;
  bool ok;
  if (p.btab) {
    off = 0;
    ok = n >= 0 && total <= p.max_seq_len && total <= ((int64_t)p.max_blocks << p.bs_log2);
  } else {
    off = p.seq_offset[b];
    ok = n >= 0 && off >= 0 && total <= p.max_seq_len && off + total <= p.num_rows;
  }
  if (ok && p.capacity) ok = total <= (int64_t)p.capacity[b];
  return ok;
}

// Cache row of token t of sequence b (off from seq_in_range); -1 when a paged
// cache's table names a block outside the allocated rows.
__device__ __forceinline__ int64_t cache_row(const Params &p, int b, int64_t off, int64_t t) {
  if (!p.btab) return off + t;
  const int64_t blk = p.btab[(int64_t)b * p.max_blocks + (t >> p.bs_log2)];
  if (blk < 0 || blk >= (p.num_rows >> p.bs_log2)) return -1;
  return (blk << p.bs_log2) + (t & ((1 << p.bs_log2) - 1));
}

__device__ __forceinline__ void flag_error(const Params &p) {
  if (p.err) atomicOr(p.err, kErrRange);
}

// --------------------------------------------------------------- launchers
// Optional events that time one kernel.  When either is set the kernel goes
// through hipExtLaunchKernel, which stamps the events with the dispatch's own
// begin and end times (the interval a kernel-trace profiler reports).
struct Timing {
  hipEvent_t begin = nullptr, end = nullptr;
};

template <int THREADS = kThreads, typename Kernel, typename... Args>
inline void launch_kernel(Kernel kernel, int64_t blocks, hipStream_t s, const Timing &tm, Args... args) {
  if (tm.begin || tm.end)
    hipExtLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(THREADS), 0, s, tm.begin, tm.end, 0, args...);
  else
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(THREADS), 0, s, args...);
}

// (defined in the kernel translation units, called by the C ABI layer)
hipError_t launch_prologue(const Params &p, int dtype, bool do_q, bool do_kv, hipStream_t s);
hipError_t launch_rows_f32(const Params &p, hipStream_t s, const Timing &tm);
hipError_t launch_tile_bf16(const Params &p, hipStream_t s, const Timing &tm);
hipError_t launch_stream_bf16(const Params &p, hipStream_t s, const Timing &tm);
hipError_t launch_combine_bf16(const Params &p, hipStream_t s, bool per_row);   // per_row: the tile route's merge
hipError_t launch_combine_wht_bf16(const Params &p, hipStream_t s);              // partials in the WHT basis
// A quantized KV cache.  fmt 0, Turbo8: K and V codes [rows][Hkv][D] (E4M3)
// with bf16 scales [rows][Hkv][D/16].  fmt 1, bf16 K + Turbo4 V: K bf16
// [rows][Hkv][D] (no scales), V indices [rows][Hkv][D/2] (two per byte) with
// E4M3 scales [rows][Hkv][D/16]; cb / thr the Turbo4 levels and thresholds.
struct QuantCache {
  int fmt;
  void *k, *ks, *v, *vs;
  float cb[16], thr[15];
};
hipError_t launch_quant_bf16(const Params &p, const QuantCache &c, hipStream_t s, const Timing &tm);
hipError_t launch_quant_append(const Params &p, const QuantCache &c, hipStream_t s);
hipError_t launch_linear_bf16(const void *x, const void *w, int M, int N, int K, void *y0, int n0_end, int ld0,
                              void *y1, int n1_end, int ld1, void *y2, int ld2, hipStream_t s);
constexpr int kMaxLinearRows = 64;    // rows (tokens) a projection call takes

// One GatedDeltaNet decode step (qsa_gdn_decode): per sequence b, inputs qkv
// [B][C] (C = 2 Hk D + Hv D), z [B][Hv D], a and b [B][Hv]; parameters conv_w
// [C][K], a_log [Hv], dt_bias [Hv], norm_w [D]; states conv_state [B][C][K] and
// state [B][Hv][D][D] (fp32, updated in place); output y [B][Hv][D].  D = 128.
struct GdnParams {
  const bf16_t *qkv, *z, *a, *b, *conv_w, *dt_bias, *norm_w;
  const float *a_log;
  float *conv_state, *state;
  bf16_t *y;
  int B, Hk, Hv, K, C;
  float eps;
};
hipError_t launch_gdn_decode(const GdnParams &p, hipStream_t s);

}  // namespace qsa
