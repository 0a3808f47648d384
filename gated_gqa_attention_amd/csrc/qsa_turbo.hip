// qsa_turbo.hip -- gated grouped-query attention over a Turbo8 KV cache
// (gfx950): the cache holds K and V as FP8 E4M3 codes with a bf16 scale per
// group of 16 elements, in the Walsh-Hadamard rotated basis (Atlas docs,
// spark_model/forward/qwen3_5/mod.rs: MetalKvDtype::Turbo8, LayerKvCache::alloc
// with one byte per element and two per group of 16; Qwen35Kernels
// kv_cache_append_turbo8, attention_decode_turbo8 and the WHT bookends).
//
// Layout: codes [rows][Hkv][D] bytes, scales [rows][Hkv][D/16] bf16, for K
// and for V, token-major like the bf16 cache.
//
// turbo8_append_kernel: one workgroup per new row (b, l); 16 lanes per head
// row.  K: norm and partial rotation (norm_rope, as for the bf16 cache), then
// the WHT, then the group quantizer; V: WHT, then the quantizer.  Codes and
// scales are stored at row seq_lens[b] + l.
//
// turbo8_kernel: one workgroup per (sequence, KV head, key chunk), the short-
// query route's geometry (rows = the G query heads x L new rows, up to 48).
// The query rows are normalised, rotated, taken to the WHT basis (the WHT(Q)
// bookend: (H q).(H k) = q.k) and rounded to fp16 MFMA operands.  The chunk's
// keys stream through a ring of raw 64-key stages (codes and scales as
// stored, 36 KB per stage at head_dim 256, three in flight), copied straight
// from HBM into LDS.  Codes are decoded to code x scale (12 significant bits,
// which fp16's 11 keep better than bf16's 8): the V codes of a stage into one
// fp16 tile laid out like the bf16 kernel's V stages, the K codes per MFMA
// operand straight from the ring, so the stage step is the bf16 kernel's
// (attend_stage) on fp16 MFMAs.  The workgroup holding the sequence's end
// quantizes the new rows as the append does (when k_new is given: and stores
// them), decodes them and attends them first.  At the end a chunk that is
// the whole sequence rotates its rows back (the iWHT(out) bookend) and applies
// the gate; other chunks store their partials in the rotated basis and the
// merge kernel rotates each merged row once (the merge is linear, so rotating
// the merged row is rotating every chunk's).
#include "qsa_device.h"

namespace qsa {

namespace {

// One new row's K (norm, rotation, WHT, quantizer) or V (WHT, quantizer), for
// the 16 lanes that hold it; x holds the raw row and is left as the value the
// quantizer saw.
template <int D>
__device__ __forceinline__ void turbo8_new_row(float (&x)[D / 16], bool is_k, const float (&w)[D / 16], bool valid,
                                               float eps, int r, const float2 *cs, Turbo8Row<D> &q) {
  if (is_k) norm_rope<D>(x, w, valid, eps, r, cs);
  row_wht<D>(x);
  q.quantize(x);
}

}  // namespace

// Formats of a quantized cache, and what one launch reads of it.
constexpr int kT8 = 0;                                   // Turbo8: K and V as E4M3 codes + bf16 scales
constexpr int kB4 = 1;                                   // bf16 K + Turbo4 V (indices + E4M3 scales)

// The tensors of a quantized cache (read; the fused append writes the new
// rows through the same pointers) and the Turbo4 codebook.
struct QArgs {
  const void *k, *ks, *v, *vs;                           // K data and scales (none for bf16 K), V data and scales
  float cb[16];                                          // Turbo4 levels, ascending
  float thr[15];                                         // their decision thresholds (midpoints)
};

// ------------------------------------------------------------------ append
// One workgroup per new row (b, l); 16 lanes per head row.  Turbo8: K norm,
// rotation, WHT, group quantizer; V WHT, quantizer.  bf16 K + Turbo4 V: K norm
// and rotation rounded to bf16 (the bf16 cache's row); V WHT, Turbo4.  Stored
// at row seq_lens[b] + l.
template <int D, int FMT>
__global__ __launch_bounds__(kThreads) void quant_append_kernel(Params p, QArgs a) {
  constexpr int E = D / 16, ROWS = kThreads / 16, NG = D / 16;
  __shared__ __attribute__((aligned(16))) float2 cs[kMaxPairs];
  __shared__ float cbs[16];
  if constexpr (FMT == kB4) {
    if (threadIdx.x < 16) cbs[threadIdx.x] = a.cb[threadIdx.x];
  }
  float thr[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) thr[i] = a.thr[i];
  const int c16 = threadIdx.x & 15, hr = threadIdx.x / 16;
  const int64_t bl = blockIdx.x;
  const int b = (int)(bl / p.L), l = (int)(bl % p.L);
  const int half = p.r / 2;
  if (half > 0) {
    const int pos = p.positions[bl];
    for (int i = threadIdx.x; i < half; i += kThreads) {
      float c, s;
      rope_angle_cs(pos, rope_freq(p.rope_step, i), c, s);
      cs[i] = make_float2(c, s);
    }
  }
  __syncthreads();
  const int n = p.seq_lens[b];
  int64_t off;
  const bool ok = seq_in_range(p, b, n, off);
  if (!ok && threadIdx.x == 0) flag_error(p);
  float w[E];
  {
    RawE<E> wr;
    wr.load((const bf16_t *)p.wk + E * c16);
    wr.to_float(w);
  }
  const bf16_t *const k_new = (const bf16_t *)p.k_new, *const v_new = (const bf16_t *)p.v_new;
  const int njobs = 2 * p.Hkv;                          // K heads, then V heads
  for (int j0 = 0; j0 < njobs; j0 += ROWS) {
    const int job = j0 + hr;
    const bool valid = job < njobs;
    const int jb = valid ? job : njobs - 1;
    const bool is_k = jb < p.Hkv;
    const int head = is_k ? jb : jb - p.Hkv;
    RawE<E> raw;
    raw.load((is_k ? k_new : v_new) + (bl * p.Hkv + head) * D + E * c16);
    float x[E];
    raw.to_float(x);
    const int64_t row = (off + n + l) * p.Hkv + head;
    if constexpr (FMT == kT8) {
      Turbo8Row<D> q;
      turbo8_new_row<D>(x, is_k, w, valid, p.eps, p.r, cs, q);
      if (!valid || !ok) continue;
      uint8_t *codes = (uint8_t *)(is_k ? a.k : a.v) + row * D + E * c16;
#pragma unroll
      for (int c = 0; c < Turbo8Row<D>::CW; ++c) *(uint32_t *)(codes + 4 * c) = q.codes[c];
      if (c16 % Turbo8Row<D>::LPG == 0) ((bf16_t *)(is_k ? a.ks : a.vs))[row * NG + E * c16 / 16] = q.scale;
    } else {
      Turbo4Row<D> q4;
      if (is_k) {
        norm_rope<D>(x, w, valid, p.eps, p.r, cs);
      } else {
        row_wht<D>(x);
        q4.quantize(x, cbs, thr);
      }
      if (!valid || !ok) continue;
      if (is_k) {
#pragma unroll
        for (int j = 0; j < E; ++j) ((bf16_t *)a.k)[row * D + E * c16 + j] = (bf16_t)x[j];
      } else {
        uint8_t *const cs4 = (uint8_t *)a.v + row * (D / 2) + E * c16 / 2;
#pragma unroll
        for (int c = 0; c < Turbo4Row<D>::CW; ++c) {
          if constexpr (E >= 8)
            *(uint32_t *)(cs4 + 4 * c) = q4.codes[c];
          else
            *(uint16_t *)cs4 = (uint16_t)q4.codes[0];
        }
        if (c16 % Turbo4Row<D>::LPG == 0) ((uint8_t *)a.vs)[row * NG + E * c16 / 16] = (uint8_t)q4.scale;
      }
    }
  }
}

// ------------------------------------------------------------------ attention
// Stage layout of the raw ring (one slot per 64-key stage), copied straight
// from HBM by global_load_lds.  Turbo8: K codes [64][D] with each row's
// 16-byte units XOR-swizzled by the key (conflict-free reads of one column by
// 16 keys), K scales [64][D/16] bf16, V codes [64][D], V scales [64][D/16].
// Copy instruction q of a stage (64 lanes) has a kind: 0 K codes, 1 V codes,
// 2 K scales, 3 V scales; kind k copies UPK(k) units of UB(k) bytes per key,
// unit u of key r at LDS unit u ^ (r & SWZ(k)).
template <int D>
struct T8Geo {
  static constexpr int SK = Geo<D>::SK;
  static constexpr int UPR = D / 16;                    // 16-byte code units (= scale groups) per key row
  static constexpr int SWC = (UPR < 16 ? UPR : 16) - 1;
  static constexpr int CODES = SK * D, SCL = SK * D / 8;
  static constexpr int KC = 0, KS = CODES, VC = CODES + SCL, VS = 2 * CODES + SCL;
  static constexpr int SLOT = 2 * (CODES + SCL);
  static constexpr int NC = 2 * UPR;                    // 16-byte code copy instructions per stage (K, V)
  // scale copies: 16-byte units when a key's scales fill whole units and the
  // counts stay even (head_dim 256: two units per key), dwords otherwise
  static constexpr bool SX4 = D == 256;
  static constexpr int SPK = SX4 ? D / 128 : D / 32;    // scale copy units per key
  static constexpr int NSC = SK * SPK / kWave;          // scale copy instructions per stage and tensor
  static constexpr int NQ = NC + 2 * NSC;               // copy instructions per stage
  static constexpr int U = NQ / 4;                      // per wavefront when all four issue
  static constexpr int NS = D == 256 ? 3 : D == 128 ? 6 : 8;   // stages in flight: LDS and the vmcnt field
  static constexpr int VT = SK * Geo<D>::RB;            // decoded fp16 V tile
  static_assert(NQ % 4 == 0 && 2 * (NS - 1) * U <= 63, "copy counts");
  static_assert(UPR % 2 == 0 && NSC % 2 == 0, "a copy wave's instructions q = w + 2 j have the kind of 2 j");
  static constexpr int kind(int q) { return q < UPR ? 0 : q < 2 * UPR ? 1 : q < 2 * UPR + NSC ? 2 : 3; }
  static constexpr int first(int k) { return k == 0 ? 0 : k == 1 ? UPR : k == 2 ? 2 * UPR : 2 * UPR + NSC; }
  static constexpr int region(int k) { return k == 0 ? KC : k == 1 ? VC : k == 2 ? KS : VS; }
  static constexpr int UPK(int k) { return k < 2 ? UPR : SPK; }
  static constexpr int UB(int k) { return k < 2 || SX4 ? 16 : 4; }
  static constexpr int SWZ(int k) { return k == 0 ? SWC : 0; }
  static constexpr int ROWHEAD(int k) { return k < 2 ? D : D / 8; }   // bytes per (row, head) in HBM
  __device__ static const void *tensor(const QArgs &a, int k) { return k == 0 ? a.k : k == 1 ? a.v : k == 2 ? a.ks : a.vs; }
};

// bf16 K + Turbo4 V (head_dim 256): K bf16 [64][D] swizzled like the bf16
// kernel's K stages (the slot's K region is the stage's K tile), V indices
// [64][D/2], V scales [64][D/16] (E4M3 bytes, copied as dwords).  Kinds: 0 K,
// 1 V indices, 2 V scales.
template <int D>
struct B4Geo {
  static_assert(D == 256, "the bf16-K / Turbo4-V copies split evenly over four wavefronts at head_dim 256 only");
  static constexpr int SK = Geo<D>::SK;
  static constexpr int KB = SK * 2 * D, CB = SK * D / 2, SB = SK * D / 16;
  static constexpr int KC = 0, VC = KB, VS = KB + CB;
  static constexpr int SLOT = KB + CB + SB;
  static constexpr int NK = SK * (D / 8) / kWave, NV = SK * (D / 32) / kWave, NVS = SK * (D / 64) / kWave;
  static constexpr int NQ = NK + NV + NVS;
  static constexpr int U = NQ / 4;
  static constexpr int NS = 2;
  static constexpr int VT = SK * Geo<D>::RB;            // decoded bf16 V tile
  static_assert(NQ % 4 == 0 && 2 * (NS - 1) * U <= 63, "copy counts");
  static_assert(NK % 2 == 0 && NV % 2 == 0, "a copy wave's instructions q = w + 2 j have the kind of 2 j");
  static constexpr int kind(int q) { return q < NK ? 0 : q < NK + NV ? 1 : 2; }
  static constexpr int first(int k) { return k == 0 ? 0 : k == 1 ? NK : NK + NV; }
  static constexpr int region(int k) { return k == 0 ? KC : k == 1 ? VC : VS; }
  static constexpr int UPK(int k) { return k == 0 ? D / 8 : k == 1 ? D / 32 : D / 64; }
  static constexpr int UB(int k) { return k < 2 ? 16 : 4; }
  static constexpr int SWZ(int k) { return k == 0 ? Geo<D>::SW : 0; }
  static constexpr int ROWHEAD(int k) { return k == 0 ? 2 * D : k == 1 ? D / 2 : D / 16; }
  __device__ static const void *tensor(const QArgs &a, int k) { return k == 0 ? a.k : k == 1 ? a.v : a.vs; }
};

template <int D, int FMT>
using QGeo = typename std::conditional<FMT == kT8, T8Geo<D>, B4Geo<D>>::type;

// This lane's source offset for copy instruction q, in bytes from the stage's
// first key row (head kvh) of the tensor it copies; keys past `last` repeat it.
// rowb: bytes between consecutive keys of one head in that tensor.
template <class QG>
__device__ __forceinline__ unsigned copy_lane_off(int q, int lane, int last, unsigned rowb) {
  const int k = QG::kind(q), i = q - QG::first(k), s = kWave * i + lane;
  const int key = s / QG::UPK(k), pos = s % QG::UPK(k), gu = pos ^ (key & QG::SWZ(k));
  return (unsigned)min(key, last) * rowb + (unsigned)QG::UB(k) * (unsigned)gu;
}

// The score product's K operand straight from a raw stage: this lane's key
// row (16 wave + m16) and k-step ks hold 8 codes of scale group 2 ks + g4/2.
template <int D>
struct T8K {
  static constexpr int KST = D / 32;
  uint2 cw[KST];                                        // the codes of k-step ks
  uint32_t sb[KST];                                     // their scale (bf16 bits)
  __device__ __forceinline__ explicit T8K(const unsigned char *slot) {
    using T8 = T8Geo<D>;
    const int lane = threadIdx.x % kWave, g4 = lane >> 4, key = 16 * (threadIdx.x / kWave) + (lane & 15);
    const unsigned char *const row = slot + T8::KC + key * D;
    const int sw = key & T8::SWC;
    const uint16_t *const sr = (const uint16_t *)(slot + T8::KS) + key * T8::UPR + (g4 >> 1);
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const int u = 2 * ks + (g4 >> 1);
      cw[ks] = *(const uint2 *)(row + 16 * (u ^ sw) + 8 * (g4 & 1));
      sb[ks] = sr[2 * ks];
    }
  }
  __device__ __forceinline__ f16x8 operator()(const unsigned char *, int ks) const {
    return t8_decode8(cw[ks].x, cw[ks].y, T8Scale(sb[ks]));
  }
};

// One workgroup per (sequence, KV head, key chunk), the short-query route's
// geometry (rows r = l G + h - kvh G, at most 48).  Wavefronts 0-1 issue the
// first NS stages' copies; wavefronts 2-3 meanwhile build their (cos, sin)
// tables, normalise, rotate and WHT the query rows into fp16 operands and, in
// the workgroup that ends the sequence, prepare the new rows: with k_new given
// they are quantized as the append does and stored, otherwise read from the
// cache; either way decoded from the same codes.  Those are attended first,
// from fp16 tiles, while the cached stages land.  Each cached stage then
// decodes its V codes into the fp16 V tile and takes its K codes into
// registers, scores its keys from those codes (decoded per MFMA operand),
// refills its slot, and accumulates.
// At the end a chunk that is the whole sequence rotates its rows back
// through LDS and gates them; other chunks store their partials as they are,
// in the WHT basis, and the merge rotates the merged rows.
template <int D, int RTM, int FMT>
__global__ __launch_bounds__(kThreads) void quant_kernel(Params p, QArgs a) {
  using G = Geo<D>;
  using QG = QGeo<D, FMT>;
  using OT = typename std::conditional<FMT == kT8, f16_t, bf16_t>::type;   // MFMA operand type
  using OT8 = typename Op16<OT>::x8;
  constexpr int E = G::E, KST = G::KST, RB = G::RB, DBW = D / 64, SK = G::SK, NS = QG::NS, U = QG::U;
  constexpr int NG = D / 16, SLOT = QG::SLOT;
  constexpr int QBYTES = 16 * RTM * RB;
  constexpr int TABN = kMaxFusedTable;
  constexpr int PREP = QBYTES + 2 * TABN * 8;           // query rows, then one (cos, sin) table per prep wave
  constexpr int WORK = QG::VT + Xch::BYTES;             // V tile, then the stage exchange
  constexpr int ARENA = PREP > WORK ? PREP : WORK;
  constexpr int NPASS = 2 * RTM;
  constexpr int TJ = TABN / kWave;
  static_assert(16 * RTM * D * 4 + 16 * RTM * 4 <= NS * SLOT, "the epilogue tile fits in the ring");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NS * SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char arena[ARENA];
  unsigned char *const vtile = arena, *const xch = arena + QG::VT;
  // The Turbo4 levels, for per-lane lookups: copy 0 (written by wavefront 0)
  // for the stages, which come after workgroup barriers; copies 1 and 2 each
  // written and read by one prep wavefront alone, for the new rows it handles
  // before the first barrier.
  __shared__ float cbs_all[3][16];
  if constexpr (FMT == kB4) {
    const int wv = (int)threadIdx.x / kWave, ln = (int)threadIdx.x % kWave;
    if ((wv == 0 || wv >= 2) && ln < 16) cbs_all[wv == 0 ? 0 : wv - 1][ln] = a.cb[ln];
  }
  const float *const cbs = cbs_all[0];
  float thr[15];
#pragma unroll
  for (int i = 0; i < 15; ++i) thr[i] = a.thr[i];

  const int t = threadIdx.x, lane = t % kWave, g4 = lane >> 4, m16 = lane & 15, c16 = m16;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const bool copier = wave < 2;
  const int pw = wave - 2;
  // The KV heads of one (chunk, sequence) group run on one XCD (the workgroup
  // of block i runs on XCD i % 8), so the scale lines they share (D/8 bytes
  // per head of each key row) are fetched into one L2; groups go round the XCDs.
  const int hkv = p.Hkv;
  const int xj = blockIdx.x / 8, kvh = xj % hkv, grp = 8 * (xj / hkv) + blockIdx.x % 8;
  if (grp >= p.chunks * p.B) return;                    // the grid is rounded up to 8 groups
  const int chunk = grp / p.B, b = grp % p.B, slot = b * hkv + kvh;
  const int L = p.L, Gq = p.G, Hq = p.Hq, R = L * Gq, half = p.r / 2;
  const bf16_t *const q_gate = (const bf16_t *)p.q_gate;
  bf16_t *const outp = (bf16_t *)p.out;
  const int n = p.seq_lens[b];
  const int64_t off = p.seq_offset[b];
  const int cap = p.capacity ? p.capacity[b] : 0x7fffffff;

  // prep waves: query rows 8 k + 4 pw + g4 of pass k, the norm weights and the
  // positions of their table entries (in-range indices whatever n is)
  RawE<E> qraw[NPASS], wqraw, wkraw;
  int tpos[TJ], tpair[TJ];
  if (!copier) {
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
      const int r = min(8 * k + 4 * pw + g4, R - 1);
      const int l = r / Gq, h = kvh * Gq + r % Gq;
      qraw[k].load(q_gate + (((int64_t)b * L + l) * Hq + h) * 2 * D + E * c16);
    }
    wqraw.load((const bf16_t *)p.wq + E * c16);
    wkraw.load((const bf16_t *)p.wk + E * c16);
    const int hh = max(half, 1);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int e = lane + kWave * j, q = e / hh;
      tpos[j] = p.positions[(int64_t)b * L + min(q, L - 1)];
      tpair[j] = e - q * hh;
    }
  }

  const int64_t total = (int64_t)n + L;
  const bool in_range = n >= 0 && off >= 0 && total <= p.max_seq_len && off + total <= p.num_rows;
  const int nch = tile_chunk_count(total, p.even_split, p.chunks, p.chunk_keys);
  if (chunk >= nch) return;
  if (!in_range) {
    if (chunk == 0) {
      for (int e = t; e < R * D; e += kThreads) {
        const int r = e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        outp[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
      if (p.part_ml && t < R)
        *(float2 *)(p.part_ml + ((int64_t)slot * p.chunks * p.rows + t) * 2) =
            make_float2(__builtin_nanf(""), __builtin_nanf(""));
      if (t == 0) flag_error(p);
    }
    return;
  }
  const int64_t k0 = chunk_begin(total, p.even_split, nch, p.chunk_keys, chunk);
  const int64_t k1 = chunk == nch - 1 ? total : chunk_begin(total, p.even_split, nch, p.chunk_keys, chunk + 1);
  const bool tail = chunk == nch - 1, fuse_new = p.k_new != nullptr;
  const bool cap_ok = total <= (int64_t)cap;
  const int64_t cend = min(k1, (int64_t)n);
  const int nst = cend > k0 ? (int)((cend - k0 + SK - 1) / SK) : 0;

  // ---- copies.  Instruction q of a stage (0 <= q < NQ): K code rows (units
  // 64 q + lane), V code rows, K scale dwords, V scale dwords.  Wavefront w
  // has the list q = (w & 1) + 2 j (j < 2 U): a copy wave issues all of it in
  // the first fill, a refill takes every other entry (j even in the copy
  // waves, odd in the prep waves, so the four issue q = w + 4 j').  Its lane
  // offsets are computed once; only a chunk's last, partial stage (keys past
  // the chunk repeat its last) computes them again.
  const unsigned ring_lds = (unsigned)(uintptr_t)(lds_void *)ring;
  const int w1 = wave & 1;
  unsigned offA[2 * U];
  static_for<2 * U>([&](auto jc) {
    constexpr int j = decltype(jc)::value, k = QG::kind(2 * j);
    offA[j] = copy_lane_off<QG>(w1 + 2 * j, lane, SK - 1, (unsigned)(hkv * QG::ROWHEAD(k)));
  });
  auto issue = [&](int st, auto jc) {
    constexpr int j = decltype(jc)::value, k = QG::kind(2 * j);
    const int last = (int)min<int64_t>(SK - 1, cend - 1 - (k0 + (int64_t)SK * st));
    const unsigned lo =
        last == SK - 1 ? offA[j] : copy_lane_off<QG>(w1 + 2 * j, lane, last, (unsigned)(hkv * QG::ROWHEAD(k)));
    const int64_t r0 = (off + k0 + (int64_t)SK * st) * hkv + kvh;
    const unsigned dst =
        ring_lds + (st % NS) * SLOT + QG::region(k) + QG::UB(k) * kWave * (w1 + 2 * j - QG::first(k));
    const unsigned char *const src = (const unsigned char *)QG::tensor(a, k) + r0 * QG::ROWHEAD(k);
    if constexpr (QG::UB(k) == 16)
      dma16_sbase(src, lo, dst);
    else
      dma4_sbase(src, lo, dst);
  };

  // ---- prep waves: the new rows' loads (the second round trip: their
  // addresses depend on n), before any copy of theirs
  const int nr = 4 * (pw ^ 1) + g4;                     // new rows 8 k + nr go to the other prep wave
  // Turbo8: both rows as codes; bf16 K + Turbo4 V: K as a bf16 row (knraw), V as indices
  RawE<E> knraw[2], vnraw[2];
  Turbo8Row<D> qk[2], qv[2];
  Turbo4Row<D> q4[2];
  if (!copier && tail) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = min(8 * k + nr, L - 1);
      const int64_t crow = (off + n + l) * hkv + kvh;
      if (fuse_new) {
        const int64_t src = (((int64_t)b * L + l) * hkv + kvh) * D + E * c16;
        knraw[k].load((const bf16_t *)p.k_new + src);
        vnraw[k].load((const bf16_t *)p.v_new + src);
      } else if constexpr (FMT == kT8) {
#pragma unroll
        for (int c = 0; c < Turbo8Row<D>::CW; ++c) {
          qk[k].codes[c] = *(const uint32_t *)((const uint8_t *)a.k + crow * D + E * c16 + 4 * c);
          qv[k].codes[c] = *(const uint32_t *)((const uint8_t *)a.v + crow * D + E * c16 + 4 * c);
        }
        qk[k].scale = ((const bf16_t *)a.ks)[crow * NG + E * c16 / 16];
        qv[k].scale = ((const bf16_t *)a.vs)[crow * NG + E * c16 / 16];
      } else {
        knraw[k].load((const bf16_t *)a.k + crow * D + E * c16);
        const uint8_t *const cs4 = (const uint8_t *)a.v + crow * (D / 2) + E * c16 / 2;
#pragma unroll
        for (int c = 0; c < Turbo4Row<D>::CW; ++c)
          q4[k].codes[c] = E >= 8 ? *(const uint32_t *)(cs4 + 4 * c) : (uint32_t)*(const uint16_t *)cs4;
        q4[k].scale = ((const uint8_t *)a.vs)[crow * NG + E * c16 / 16];
      }
    }
  }
  if (copier) {
    for (int st = 0; st < min(NS, nst); ++st) static_for<2 * U>([&](auto jc) { issue(st, jc); });
  }

  float kx[2][E], vx[2][E];                             // decoded new rows 8 k + nr (prep waves, tail)
  if (!copier) {
    float2 *const tabw = (float2 *)(arena + QBYTES) + pw * TABN;
    const double step = p.rope_step;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int e = lane + kWave * j;
      if (kWave * j < L * half) {
        float c, sn;
        rope_angle_cs(tpos[j], rope_freq(step, tpair[j]), c, sn);
        if (e < L * half) tabw[e] = make_float2(c, sn);
      }
    }
    wave_lds_sync();
    float wq[E], wk[E];
    wqraw.to_float(wq);
    wkraw.to_float(wk);
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
      const int r = 8 * k + 4 * pw + g4;
      float x[E];
#pragma unroll
      for (int j = 0; j < E; ++j) x[j] = 0.f;           // rows >= R are zero
      if (8 * k + 4 * pw < R) {                         // the pass holds a row (wave-uniform)
        qraw[k].to_float(x);
        norm_rope<D>(x, wq, r < R, p.eps, p.r, tabw + (min(r, R - 1) / Gq) * half);
        if constexpr (FMT == kT8) row_wht<D>(x);        // the WHT(Q) bookend: K is rotated
      }
      put_row<D, OT>(arena, RB, r, E * c16, x);
    }
    if (tail) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int l = 8 * k + nr;
        if (8 * k + 4 * (pw ^ 1) < L) {                 // the pass holds a new row (wave-uniform)
          const int64_t crow = (off + n + l) * hkv + kvh;
          const bool store = fuse_new && l < L && cap_ok;   // the append: rows n + l
          if constexpr (FMT == kT8) {
            if (fuse_new) {
              knraw[k].to_float(kx[k]);
              vnraw[k].to_float(vx[k]);
              turbo8_new_row<D>(kx[k], true, wk, l < L, p.eps, p.r, tabw + min(l, L - 1) * half, qk[k]);
              turbo8_new_row<D>(vx[k], false, wk, l < L, p.eps, p.r, tabw + min(l, L - 1) * half, qv[k]);
              if (store) {
#pragma unroll
                for (int c = 0; c < Turbo8Row<D>::CW; ++c) {
                  *(uint32_t *)((uint8_t *)a.k + crow * D + E * c16 + 4 * c) = qk[k].codes[c];
                  *(uint32_t *)((uint8_t *)a.v + crow * D + E * c16 + 4 * c) = qv[k].codes[c];
                }
                if (c16 % Turbo8Row<D>::LPG == 0) {
                  ((bf16_t *)a.ks)[crow * NG + E * c16 / 16] = qk[k].scale;
                  ((bf16_t *)a.vs)[crow * NG + E * c16 / 16] = qv[k].scale;
                }
              }
            }
            qk[k].dequantize(kx[k]);
            qv[k].dequantize(vx[k]);
          } else {
            knraw[k].to_float(kx[k]);
            if (fuse_new) {
              // K: the bf16 cache's row (norm, rotation, rounded once); V: WHT, then Turbo4
              norm_rope<D>(kx[k], wk, l < L, p.eps, p.r, tabw + min(l, L - 1) * half);
              bf16_t kb[E];
#pragma unroll
              for (int j = 0; j < E; ++j) {
                kb[j] = (bf16_t)kx[k][j];
                kx[k][j] = (float)kb[j];
              }
              vnraw[k].to_float(vx[k]);
              row_wht<D>(vx[k]);
              q4[k].quantize(vx[k], cbs_all[1 + pw], thr);
              if (store) {
#pragma unroll
                for (int j = 0; j < E; ++j) ((bf16_t *)a.k)[crow * D + E * c16 + j] = kb[j];
                uint8_t *const cs4 = (uint8_t *)a.v + crow * (D / 2) + E * c16 / 2;
#pragma unroll
                for (int c = 0; c < Turbo4Row<D>::CW; ++c) {
                  if constexpr (E >= 8)
                    *(uint32_t *)(cs4 + 4 * c) = q4[k].codes[c];
                  else
                    *(uint16_t *)cs4 = (uint16_t)q4[k].codes[0];
                }
                if (c16 % Turbo4Row<D>::LPG == 0) ((uint8_t *)a.vs)[crow * NG + E * c16 / 16] = (uint8_t)q4[k].scale;
              }
            }
            q4[k].dequantize(vx[k], cbs_all[1 + pw]);
          }
        }
        if (!(8 * k + 4 * (pw ^ 1) < L) || l >= L) {
#pragma unroll
          for (int j = 0; j < E; ++j) kx[k][j] = vx[k][j] = 0.f;
        }
      }
    }
  }
  lds_barrier();                                        // query operands ready

  OT8 qf[RTM][KST];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt)
#pragma unroll
    for (int k = 0; k < KST; ++k) qf[rt][k] = *(const OT8 *)(arena + swz<G::SW>(16 * rt + m16, 4 * k + g4, RB));
  int lim[RTM];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) lim[rt] = n + (16 * rt + m16) / Gq;
  f32x4 O[RTM][DBW];
  float mrun[RTM], lrun[RTM];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    mrun[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int db = 0; db < DBW; ++db) O[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale_log2;

  // ---- the new rows first, from operand tiles in the V tile's place: V rows
  // 0 .. 31 (zero from L on), K rows 0 .. 15 at rows 32 .. 47
  if (tail) {
    lds_barrier();                                      // every wave holds its query operands
    if (!copier) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        put_row<D, OT>(vtile + 32 * RB, RB, 8 * k + nr, E * c16, kx[k]);
        put_row<D, OT>(vtile, RB, 8 * k + nr, E * c16, vx[k]);
      }
    } else {
      float z[E];
#pragma unroll
      for (int j = 0; j < E; ++j) z[j] = 0.f;
#pragma unroll
      for (int k = 0; k < 2; ++k) put_row<D, OT>(vtile, RB, 16 + 8 * k + 4 * wave + g4, E * c16, z);
    }
    lds_barrier();
    if (L == 1) {
      // One new key, visible to every row: attending it leaves each row's
      // reference max at its score, its sum at 1 (P = 2^0 exactly) and its
      // output at the value row, as a stage would; each wavefront sets that
      // state itself (the stage's score MFMAs, no exchange).
      const unsigned char *const kt = vtile + 32 * RB;
#pragma unroll
      for (int rt = 0; rt < RTM; ++rt) {
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KST; ++k) S = mfma_qk(*(const OT8 *)(kt + swz<G::SW>(m16, 4 * k + g4, RB)), qf[rt][k], S);
        mrun[rt] = rows4_max(g4 == 0 ? S[0] * sl2 : -INFINITY);   // key 0 sits in lane group 0
        lrun[rt] = 1.f;
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
          const int d = 16 * (DBW * wave + db) + 4 * g4;
          const typename Op16<OT>::x4 v4 = *(const typename Op16<OT>::x4 *)(vtile + swz<G::SW>(0, d / 8, RB) + 2 * (d % 8));
          O[rt][db] = f32x4{(float)v4[0], (float)v4[1], (float)v4[2], (float)v4[3]};
        }
      }
    } else {
      attend_stage<D, RTM, NoOp, OT>(vtile + 32 * RB, vtile, L, n, qf, O, mrun, lrun, lim, sl2, xch);
    }
  }

  // ---- cached stages
  for (int st = 0; st < nst; ++st) {
    // copies younger than stage st that this wave issued: of the ys later
    // stages in flight, f are of the first fill (2 U per copy wave, none in a
    // prep wave) and ys - f are refills (U per wave)
    const int ys = min(NS - 1, nst - 1 - st);
    const int f = max(0, min(NS, nst) - 1 - st);
    WaitUnits<U, 2 * (NS - 1)>::run(copier ? ys + f : ys - f);
    lds_barrier();
    const unsigned char *const sl = ring + (st % NS) * SLOT;
    // V -> the operand V tile: thread t decodes groups t + 256 i (key, group
    // of 16); every read is issued before the first decode
    constexpr int VG = SK * NG / kThreads;
    if constexpr (FMT == kT8) {
      uint4 vcw[VG];
      uint32_t vsb[VG];
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const int gi = t + kThreads * i, key = gi / NG, grp = gi % NG;
        vcw[i] = *(const uint4 *)(sl + QG::VC + key * D + 16 * grp);
        vsb[i] = *(const uint16_t *)(sl + QG::VS + 2 * (key * NG + grp));
      }
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const int gi = t + kThreads * i, key = gi / NG, grp = gi % NG;
        const T8Scale sc(vsb[i]);
        *(f16x8 *)(vtile + swz<G::SW>(key, 2 * grp, RB)) = t8_decode8(vcw[i].x, vcw[i].y, sc);
        *(f16x8 *)(vtile + swz<G::SW>(key, 2 * grp + 1, RB)) = t8_decode8(vcw[i].z, vcw[i].w, sc);
      }
    } else {
      // Turbo4: level x scale in fp32, rounded once to bf16
      uint2 vcw[VG];
      uint32_t vsb[VG];
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const int gi = t + kThreads * i, key = gi / NG, grp = gi % NG;
        vcw[i] = *(const uint2 *)(sl + QG::VC + key * (D / 2) + 8 * grp);
        vsb[i] = *(const uint8_t *)(sl + QG::VS + key * NG + grp);
      }
#pragma unroll
      for (int i = 0; i < VG; ++i) {
        const int gi = t + kThreads * i, key = gi / NG, grp = gi % NG;
        const float sc = unpk_fp8(vsb[i], false)[0];
        bf16x8 h[2];
#pragma unroll
        for (int e = 0; e < 16; ++e)
          h[e / 8][e % 8] = (bf16_t)(sc * cbs[((e < 8 ? vcw[i].x : vcw[i].y) >> (4 * (e % 8))) & 15u]);
        *(bf16x8 *)(vtile + swz<G::SW>(key, 2 * grp, RB)) = h[0];
        *(bf16x8 *)(vtile + swz<G::SW>(key, 2 * grp + 1, RB)) = h[1];
      }
    }
    const int sk0 = (int)(k0 + (int64_t)SK * st);
    const int nk_ = (int)min<int64_t>(SK, cend - sk0);
    // The slot is consumed once every wave has its scores (its V codes were
    // decoded and the K codes taken into registers before them): it is
    // refilled then.  (Refilling at once, behind one more barrier, measured
    // slower: the copies then wait in the memory pipeline ahead of the scores.)
    auto refill = [&]() {
      if (st + NS < nst) {
        static_for<U>([&](auto jc) {
          constexpr int j = 2 * decltype(jc)::value;
          if (copier)
            issue(st + NS, std::integral_constant<int, j>());
          else
            issue(st + NS, std::integral_constant<int, j + 1>());
        });
      }
    };
    if constexpr (FMT == kT8) {
      const T8K<D> kop(sl);                             // this wave's K codes, into registers
      attend_stage<D, RTM, decltype(refill), f16_t, T8K<D>>(nullptr, vtile, nk_, sk0, qf, O, mrun, lrun, lim, sl2,
                                                             xch, refill, kop);
    } else {
      // the slot's K region is the stage's bf16 K tile
      attend_stage<D, RTM, decltype(refill), bf16_t>(sl + QG::KC, vtile, nk_, sk0, qf, O, mrun, lrun, lim, sl2, xch,
                                                     refill);
    }
  }

  const bool single = nch == 1;
  const int64_t slot_rows = ((int64_t)slot * p.chunks + chunk) * p.rows;
  if (!single) {
    // ---- partials, still in the WHT basis (the merge rotates the merged
    // rows): each wavefront stores its own dims of every row from registers
    if (cap_ok) {
#pragma unroll
      for (int rt = 0; rt < RTM; ++rt) {
        const int r = 16 * rt + m16;
        if (r >= R) continue;
#pragma unroll
        for (int db = 0; db < DBW; ++db) {
          const int d = 16 * (DBW * wave + db) + 4 * g4;
          f32x4 *const dst = (f32x4 *)(p.part_o + (slot_rows + r) * D + d);
          // one row tile's partials (4 KB per workgroup at head_dim 256) stay in the
          // caches for the merge kernel; several tiles' are written past them (faster)
          if constexpr (RTM == 1) *dst = O[rt][db]; else __builtin_nontemporal_store(O[rt][db], dst);
        }
        if (wave == 0 && g4 == 0) *(float2 *)(p.part_ml + (slot_rows + r) * 2) = make_float2(mrun[rt], lrun[rt]);
      }
    } else if (chunk == 0) {
      for (int e = t; e < R * D; e += kThreads) {
        const int r = e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        outp[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
      if (t < R) *(float2 *)(p.part_ml + (slot_rows + t) * 2) = make_float2(__builtin_nanf(""), __builtin_nanf(""));
      if (t == 0) flag_error(p);
    }
    return;
  }

  // ---- a chunk that is the whole sequence: rotate the rows back (iWHT)
  // through LDS, 16 lanes per row, then the gate
  __syncthreads();                                      // every wave is done with the ring
  float *const otile = (float *)ring;                   // [16 RTM][D] fp32
  float *const linv = otile + 16 * RTM * D;             // [16 RTM] 1 / row sum
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt)
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      const int d = 16 * (DBW * wave + db) + 4 * g4;
      *(f32x4 *)(otile + (16 * rt + m16) * D + d) = O[rt][db];
    }
  if (wave == 0 && g4 == 0)
#pragma unroll
    for (int rt = 0; rt < RTM; ++rt) linv[16 * rt + m16] = 1.f / lrun[rt];
  __syncthreads();
  const int hr = t / 16;                                // this lane group's row slot (0 .. 15)
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    const int r = 16 * rt + hr;
    float x[E];
#pragma unroll
    for (int j = 0; j < E; ++j) x[j] = otile[r * D + E * c16 + j];
    row_wht<D>(x);
    if (r >= R) continue;
    const int l = r / Gq, h = kvh * Gq + r % Gq;
    const int64_t orow = ((int64_t)b * L + l) * Hq + h;
    RawE<E> zr;
    zr.load(q_gate + orow * 2 * D + D + E * c16);
    float z[E];
    zr.to_float(z);
    const float inv = linv[r];
    bf16_t *dst = outp + orow * D + E * c16;
#pragma unroll
    for (int j = 0; j < E; ++j) dst[j] = (bf16_t)(cap_ok ? x[j] * inv * sigmoid_f(z[j]) : __builtin_nanf(""));
  }
  if (!cap_ok && t == 0) flag_error(p);
}

static QArgs args_of(const QuantCache &c) {
  QArgs a;
  a.k = c.k;
  a.ks = c.ks;
  a.v = c.v;
  a.vs = c.vs;
  for (int i = 0; i < 16; ++i) a.cb[i] = c.cb[i];
  for (int i = 0; i < 15; ++i) a.thr[i] = c.thr[i];
  return a;
}

template <int D, int FMT>
static hipError_t launch_quant_d(const Params &p, const QArgs &a, hipStream_t s, const Timing &tm) {
  const int64_t groups = ((int64_t)p.B * p.chunks + 7) / 8 * 8;   // (chunk, sequence) groups, rounded up to 8
  const int64_t blocks = groups * p.Hkv;
  switch ((p.rows + 15) / 16) {
    case 1: launch_kernel(quant_kernel<D, 1, FMT>, blocks, s, tm, p, a); break;
    case 2: launch_kernel(quant_kernel<D, 2, FMT>, blocks, s, tm, p, a); break;
    case 3: launch_kernel(quant_kernel<D, 3, FMT>, blocks, s, tm, p, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_bf16(const Params &p, const QuantCache &c, hipStream_t s, const Timing &tm) {
  const QArgs a = args_of(c);
  if (c.fmt == kB4) return p.D == 256 ? launch_quant_d<256, kB4>(p, a, s, tm) : hipErrorInvalidValue;
  switch (p.D) {
    case 64: return launch_quant_d<64, kT8>(p, a, s, tm);
    case 128: return launch_quant_d<128, kT8>(p, a, s, tm);
    case 256: return launch_quant_d<256, kT8>(p, a, s, tm);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_append(const Params &p, const QuantCache &c, hipStream_t s) {
  const QArgs a = args_of(c);
  const dim3 grid((unsigned)((int64_t)p.B * p.L)), block(kThreads);
  if (c.fmt == kB4) {
    if (p.D != 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quant_append_kernel<256, kB4>), grid, block, 0, s, p, a);
    return hipGetLastError();
  }
  switch (p.D) {
    case 64: hipLaunchKernelGGL((quant_append_kernel<64, kT8>), grid, block, 0, s, p, a); break;
    case 128: hipLaunchKernelGGL((quant_append_kernel<128, kT8>), grid, block, 0, s, p, a); break;
    case 256: hipLaunchKernelGGL((quant_append_kernel<256, kT8>), grid, block, 0, s, p, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
