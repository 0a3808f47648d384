// qsa_prefill.hip -- bf16 gated grouped-query attention for long blocks of new
// rows (prefill chunks) on gfx950, after the prologue kernel has normalised and
// rotated the queries into the prepared buffer and appended the new keys and
// values to the cache (Atlas qwen3_5/mod.rs module doc: append, then attend).
//
// tile_kernel: one workgroup = (sequence b, KV head g, a range of keys of one
// tile of 256 query rows, or of a pair of tiles: see pair_ranges).  The rows
// are (new row l, head of group g) pairs in order r = l * G + (h - g * G)
// (DS4Server issue #113, Reproduction: query heads grouped within their KV
// group), so one K/V stream serves the whole group.  The keys of a segment
// (one tile's part of the range) stream through an HBM -> LDS ring of 32-key
// stages; eight
// wavefronts (two per SIMD, so one can issue while the other waits) each own
// two 16-row MFMA tiles (32 rows) and run their own online softmax over every
// stage:
// scores S^T = K Q^T on MFMA with the queries in registers, the running max and
// the probabilities in registers, then O^T += V^T P^T on MFMA.  The value
// product takes its keys in a permuted order that matches the layout the score
// product leaves the probabilities in, so P never goes through LDS; the
// transposing LDS reads fetch V^T in that same order.  One workgroup barrier
// per stage guards the ring slot.  A tile covered by one piece applies the gate
// attn * sigmoid(gate) (mlxd PR #99 Summary) and stores bf16; otherwise each
// piece writes its (max, sum, output / sum) for the merge kernel.
#include "qsa_device.h"

namespace qsa {

namespace {

constexpr int kTileThreads = kPrefillThreads;        // eight wavefronts
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kRowTiles = kPrefillRowTiles;          // 16-row MFMA tiles per wavefront
constexpr float kLazyMax = 8.f;                      // headroom of the running max, log2 units
constexpr int kReadAhead = 2;                        // ring operand reads in flight ahead of the products
constexpr int kPrefillRows = kPrefillTileRows;       // query rows per workgroup
static_assert(kPrefillRows == kTileWaves * 16 * kRowTiles, "row tiles of the wavefronts");

template <int D>
struct PGeo {
  static constexpr int RB = 2 * D;                      // bytes of one key row of one KV head
  static constexpr int OCT = D / 8;                     // 16-byte units per row
  static constexpr int SW = (OCT < 16 ? OCT : 16) - 1;  // K tile: unit u of row r sits at u ^ (r & SW)
  static constexpr int SWV = (OCT < 16 ? OCT : 16) / 2 - 1;   // V tile: at u ^ 2 (r & SWV)
  static constexpr int SK = 32;                         // keys per stage
  static constexpr int STAGE = SK * RB;                 // bytes per stage and tensor
  static constexpr int NS = 4;                          // ring slots per tensor
  static constexpr int NCP = SK * OCT;                  // 16-byte copies per stage and tensor
  static constexpr int LPS = (NCP + kTileThreads - 1) / kTileThreads;   // per thread (some idle when D = 64)
};

// Scores of one 32-key stage for this wavefront's RT row tiles (score steps
// of the tile kernel's stage loop): S[kb][rt][i] = S^T[key 16 kb + 4 g4 + i]
// [row m16 of tile rt], from the swizzled K stage tile and the query fragments
// in registers.  Unit 4 ks + g4 of key row 16 kb + m16 sits at unit
// (4 ks + g4) ^ (m16 & SW) = 4 (ks ^ c) + (g4 ^ (m16 & 3)) with
// c = (m16 & SW) >> 2.  The lane's part of the address for ks = 0 holds c in
// bits 6 and 7 (and the stage's LDS address has none of them), so every
// k-step's address is (stage + lane part) ^ 64 (ks & 3) plus an immediate:
// one register of lane offsets for every k-step.  This is that lane part: key
// row m16, unit g4 ^ (m16 & 3), plus c.
template <int D>
__device__ __forceinline__ unsigned qk_lane_offset() {
  using G = PGeo<D>;
  const int lane = threadIdx.x % kWave, g4 = lane >> 4, m16 = lane & 15;
  return (unsigned)(m16 * G::RB + 16 * (g4 ^ (m16 & 3)) + 64 * ((m16 & G::SW) >> 2));
}

// Online softmax of one stage's scores.  Keys key0 .. key0 + nkeys - 1; this
// lane's row sees key k when key0 + k <= lim (causal limit n_b + l).
// MASK = false when every key of the stage is visible to every row of the
// workgroup.  Leaves the bf16 probabilities in bp in the score layout: lane
// (g4, m16) holds keys 4 g4 + i and 16 + 4 g4 + i of row m16.  Returns whether
// the row's outputs (and its sum, kept as an output column) need rescaling by
// alpha.  scale_log2 > 0, so the max is taken on the raw scores.
template <bool MASK>
__device__ __forceinline__ bool stage_softmax(const f32x4 (&S)[2], int nkeys, int rel0, float &m, float &ls, int lim,
                                              float scale_log2, bf16x8 &bp, float &alpha) {
  const int g4 = (threadIdx.x % kWave) >> 4;
  float sc[8];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = S[kb][i];
      if constexpr (MASK) {
        const int k = 16 * kb + 4 * g4 + i;
        v = (k < nkeys && rel0 + k <= lim) ? v : -INFINITY;
      }
      sc[4 * kb + i] = v;
    }
  // maxima as NaN-propagating maximum (v_maximum3_f32), which takes its
  // operands as they are: fmaxf first quiets each operand with an instruction
  // of its own.  The scores are finite or -inf (masked).
  auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  float bm = mx(mx(mx(mx(sc[0], sc[1]), sc[2]), mx(mx(sc[3], sc[4]), sc[5])), mx(sc[6], sc[7]));
  {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = mx(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = mx(__uint_as_float(c[0]), __uint_as_float(c[1])) * scale_log2;
  }
  // The reference max moves only when the block max passes it by more than
  // kLazyMax (log2 units), so the probabilities stay <= 2^kLazyMax and the
  // output rarely needs rescaling; sums, outputs and the piece's (max, sum)
  // all refer to the same reference, which keeps the result exact.
  const bool up = bm > m + kLazyMax;
  const float mn = up ? bm : m;
  const float mu = mn == -INFINITY ? 0.f : mn;
  // v_exp_f32 directly: results below 2^-126 flush to zero, which is
  // negligible next to the reference's probability of at least 2^-kLazyMax
  alpha = __builtin_amdgcn_exp2f(m - mu);
  const bool rescale = up && m != -INFINITY;
  m = mn;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // the stage's share of the row sum adds the rounded probabilities, two at a
  // time, as a dot product with (1, 1) (v_dot2_f32_bf16)
  const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const f32x2 e = {__builtin_amdgcn_exp2f(__builtin_fmaf(sc[j], scale_log2, -mu)),
                     __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j + 1], scale_log2, -mu))};
    const bf16x2_t h = __builtin_convertvector(e, bf16x2_t);
    bp[j] = h[0];
    bp[j + 1] = h[1];
    ps = __builtin_amdgcn_fdot2_f32_bf16(h, ones, ps, false);
  }
  ls = ls * alpha + ps;
  return rescale;
}

// O^T[dim][row] += V^T[dim][key] P^T[key][row] over one 32-key stage for each
// row tile (value steps of the tile kernel's stage loop), with the MFMA's k
// index j of lane group g4 standing for key 4 g4 + j (j < 4) or
// 16 + 4 g4 + j - 4, the order the probabilities were left in; the
// transposing reads fetch those two 4-key runs of the swizzled V tile for dims
// 16 db + m16.  Unit 2 db + h (h = bit 1 of m16) of key row klo sits at unit
// 2 (db ^ s) + h, s = klo & SWV, = 2 ((db % E) ^ s) + 2 E (db / E) + h with
// E = SWV + 1; row klo + 16 has the same s.  The lane's part of the address
// for db = 0 holds s in bits 5 .. 4 + log2 E (and the stage's LDS address has
// none of them), so dim block db reads at (stage + lane part) ^ 32 (db % E)
// plus an immediate.  The swizzle leaves h alone, so the 32 lanes of rows
// klo = 0..7 (or 8..15) read 16 distinct units: no bank conflicts.  This is
// that lane part: key row klo = 4 g4 + m16 / 4, 8-byte half m16 & 1 of unit h,
// plus 32 s.
template <int D>
__device__ __forceinline__ unsigned pv_lane_offset() {
  using G = PGeo<D>;
  const int lane = threadIdx.x % kWave, g4 = lane >> 4, m16 = lane & 15;
  const int klo = 4 * g4 + (m16 >> 2);
  return (unsigned)(klo * G::RB + 16 * ((m16 >> 1) & 1) + 8 * (m16 & 1) + 32 * (klo & G::SWV));
}

}  // namespace

// Work items ((sequence, KV head) group, workgroup of the group) are numbered
// so that the workgroup of block i runs on XCD i % 8 and each XCD takes a
// contiguous range of items: the tiles that share a KV head share that XCD's
// L2.  With C > 1 chunks per tile the group's tiles t and T - 1 - t form a pair
// with 2 C workgroups (the middle tile of an odd count stands alone with C),
// and the pair's keys are cut into equal ranges (pair_ranges): causal rows see
// more keys the later their tile, and pairing the first tiles with the last
// gives every workgroup about the same number of keys.  A range that crosses
// the boundary between the pair's tiles runs as two segments, one per tile.
// Preloaded arguments: sequence metadata, the prepared queries and the grid shape.
template <int D>
__global__ __launch_bounds__(kTileThreads) void tile_kernel(const int32_t *__restrict__ seq_lens,
                                                        const int64_t *__restrict__ seq_offset,
                                                        const bf16_t *__restrict__ qt, int L, int Gq, int Hq,
                                                        int tiles, int nitems, Params p) {
  using G = PGeo<D>;
  constexpr int KST = D / 32, NDB = D / 16, NS = G::NS, LPS = G::LPS, SK = G::SK, RT = kRowTiles;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[2 * NS * G::STAGE];   // K ring | V ring
  unsigned char *const kring = ring, *const vring = ring + NS * G::STAGE;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int lane = t % kWave, g4 = lane >> 4, m16 = lane & 15;
  // XCD-contiguous item numbering
  const int per = nitems / 8, rem = nitems % 8, x = blockIdx.x % 8, j = blockIdx.x / 8;
  const int item = x * per + min(x, rem) + j;
  const int hkv = p.Hkv, pchunks = p.chunks;
  const int gw = tiles * pchunks;                       // workgroups per (sequence, KV head)
  const int bk = item / gw, wi = item % gw;
  const int b = bk / hkv, kvh = bk % hkv;
  // this workgroup's pair of tiles (ta, tc; ta == tc for a tile alone) and its
  // index v among the pair's wmax workgroups
  const int half = pchunks > 1 ? tiles / 2 : 0;         // pairs of two tiles
  int pair, v, wmax;
  if (wi < 2 * pchunks * half) {
    pair = wi / (2 * pchunks);
    v = wi % (2 * pchunks);
    wmax = 2 * pchunks;
  } else {
    pair = half + (wi - 2 * pchunks * half) / pchunks;
    v = (wi - 2 * pchunks * half) % pchunks;
    wmax = pchunks;
  }
  const int ta = pair, tc = pair < half ? tiles - 1 - pair : pair;
  const int R = L * Gq;                                 // rows of this KV head
  int wrow[RT], wr[RT];                                 // this lane's row in each of its row tiles
  bf16x8 qf[RT][KST];
  auto load_queries = [&](int tile) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      wrow[rt] = tile * kPrefillRows + 16 * (RT * wave + rt) + m16;
      wr[rt] = min(wrow[rt], R - 1);
      const int l = wr[rt] / Gq, h = kvh * Gq + wr[rt] % Gq;
      const bf16_t *src = qt + (((int64_t)b * L + l) * Hq + h) * D + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) qf[rt][ks] = __builtin_bit_cast(bf16x8, gld<uint4>(src + 32 * ks));
    }
  };
  auto queries_landed = [&]() {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < KST; ++ks) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qf[rt][ks])));
      }
  };

  // ------------------------------------------------------------ round trip 1: metadata
  const int n = seq_lens[b];
  const int64_t off = seq_offset[b];
  const int ck = p.chunk_keys, msl = p.max_seq_len;
  const int64_t nrows = p.num_rows;
  const bf16_t *const kc = (const bf16_t *)p.kc;
  const bf16_t *const vc = (const bf16_t *)p.vc;
  const int32_t *const capp = p.capacity;
  const float sl2 = p.scale_log2;
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"s"(n), "s"(off), "s"(ck), "s"(msl), "s"(nrows), "s"(kc), "s"(vc), "s"(capp), "s"(sl2));

  const int64_t total = (int64_t)n + L;
  const bool in_range = n >= 0 && off >= 0 && total <= msl && off + total <= nrows;
  const int cap = capp ? capp[b] : 0x7fffffff;
  auto nan_rows = [&](int tile) {                       // every output of the tile's rows
    const int r0 = tile * kPrefillRows, nr = min(r0 + kPrefillRows, R) - r0;
    for (int e = t; e < nr * D; e += kTileThreads) {
      const int r = r0 + e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
      ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
    }
  };
  if (!in_range) {
    if (v == 0) {
      nan_rows(ta);
      if (tc != ta) nan_rows(tc);
      if (t == 0) flag_error(p);
    }
    return;
  }
  const int64_t Ka = tile_keys(n, ta, kPrefillRows, R, Gq);
  const int64_t S = Ka + (tc != ta ? tile_keys(n, tc, kPrefillRows, R, Gq) : 0);
  const int nw = pair_ranges(S, wmax, ck);
  if (v >= nw) return;
  const int64_t x0 = range_start(v, S, nw), x1 = range_start(v + 1, S, nw);   // this workgroup's keys of the pair
  const int sg0 = x0 < Ka ? 0 : 1, sg1 = tc != ta && x1 > Ka ? 2 : 1;
  // The segments' facts go through LDS, so that none of them holds a scalar
  // register during the key stages: per segment (0: tile ta, 1: tile tc) the
  // tile, its keys [k0, k1), flags (the tile's only piece, its first piece,
  // within capacity) and this piece's partial slot.
  __shared__ int seg_info[2][5];
  if (t == 0) {
    const int lasta = range_of(Ka - 1, S, nw);          // the last range with keys of tile ta
    const int firstc = tc != ta ? range_of(Ka, S, nw) : nw;   // the first with keys of tile tc
    const int pslot = (bk * (tiles - half) + pair) * (2 * pchunks + 1);   // partial slots of the pair
    const int cap_ok = total <= (int64_t)cap;
    // the merge finds each split tile's pieces here: the workgroup holding a
    // tile's first piece writes them (pair-relative slots first | last << 16)
    if (p.tinfo) {
      if (v == 0) p.tinfo[bk * tiles + ta] = lasta << 16;
      if (tc != ta && v == firstc) p.tinfo[bk * tiles + tc] = (firstc + 1) | nw << 16;
    }
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const int64_t kb0 = sg ? Ka : 0;
      seg_info[sg][0] = sg ? tc : ta;
      seg_info[sg][1] = (int)(max(x0, kb0) - kb0);
      seg_info[sg][2] = (int)(min(x1, sg ? S : Ka) - kb0);
      seg_info[sg][3] = (sg ? firstc == nw - 1 : lasta == 0) | (sg ? v == firstc : v == 0) << 1 | cap_ok << 2;
      seg_info[sg][4] = pslot + v + sg;
    }
  }
  lds_barrier();
  auto opaque = [](unsigned x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  const unsigned kring_lds = (unsigned)(uintptr_t)(lds_void *)kring;
  const unsigned vring_lds = (unsigned)(uintptr_t)(lds_void *)vring;
  const unsigned rowb = (unsigned)(hkv * D * 2);       // bytes between consecutive keys of one KV head
  // the lanes' parts of the ring read addresses; opaque() at each stage keeps
  // the compiler from holding every k-step's or dim block's offset in a
  // register of its own across the stage loop
  const unsigned klane = qk_lane_offset<D>(), vlane = pv_lane_offset<D>();

#pragma clang loop unroll(disable)
  for (int sg = sg0; sg < sg1; ++sg) {
    // ---------------------------------------------------------- one segment: tile `tile`, keys [k0, k1)
    const int tile = __builtin_amdgcn_readfirstlane(seg_info[sg][0]);
    const int k0 = __builtin_amdgcn_readfirstlane(seg_info[sg][1]);
    const int k1 = __builtin_amdgcn_readfirstlane(seg_info[sg][2]);
    const int row0 = tile * kPrefillRows;
    // the segment's queries land before its first copies (no copy or store of
    // the segment before is outstanding then)
    load_queries(tile);
    queries_landed();
    if (sg != sg0) lds_barrier();                       // every wavefront is done with the ring
    const int nst = (int)((k1 - k0 + SK - 1) / SK);
    const int64_t kfull = min((int64_t)k1, (int64_t)n + row0 / Gq + 1);   // keys below this are visible to every row
    int lim[RT];                                        // causal limit of the lane's rows, relative to n_b
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lim[rt] = wr[rt] / Gq;

    // -------------------------------------------------------- key stages
    // This thread's copies of a stage: key row u / OCT of the stage, and the
    // 16-byte unit that the K (V) tile's swizzle puts at LDS position u % OCT
    // of that row; the source is that key's row of KV head kvh, addressed from
    // the stage's first key (wave-uniform) plus a lane offset.
    auto issue_stage = [&](int st) {   // keys k0 + SK st .. into ring slot st % NS
      const int64_t sk0 = k0 + (int64_t)SK * st;
      const int last = (int)min<int64_t>(SK - 1, k1 - 1 - sk0);   // keys past the segment repeat its last key
      const int64_t row = ((off + sk0) * hkv + kvh) * D;
      const bf16_t *kb = kc + row, *vb = vc + row;
#pragma unroll
      for (int i = 0; i < LPS; ++i) {
        const int u = t + kTileThreads * i, key = u / G::OCT, pos = u % G::OCT;
        const unsigned kr = (unsigned)min(key, last) * rowb;
        const unsigned dst = (st % NS) * G::STAGE + kTileThreads * 16 * i + wave * 1024;
        if (G::NCP % kTileThreads == 0 || kTileThreads * i + 64 * wave < G::NCP) {   // wave-uniform
          dma16_sbase(kb, kr + 16u * (unsigned)(pos ^ (key & G::SW)), kring_lds + dst);
          dma16_sbase(vb, kr + 16u * (unsigned)(pos ^ (2 * (key & G::SWV))), vring_lds + dst);
        }
      }
    };
    static_assert(NS >= 4, "stage copies overlap the two stages before");
#pragma unroll
    for (int st = 0; st < NS - 2; ++st)
      if (st < nst) issue_stage(st);

    f32x4 O[RT][NDB];
    float mrun[RT], lrun[RT];                           // lrun: this lane's share of the row sum
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      mrun[rt] = -INFINITY;
      lrun[rt] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Staggered wavefront pairs.  Every wavefront accumulates the values of
    // stage st - 1 (its probabilities kept from the iteration before), then
    // scores stage st and runs its softmax; the two wavefronts of a SIMD (w
    // and w + 4) meet the stage's barrier at different points of that
    // sequence: an early wavefront after the value product, a late one before
    // it.  So between two barriers an early wavefront scores, runs its softmax
    // and accumulates values, while its partner accumulates values, then
    // scores and runs its softmax: while one runs its softmax on the vector
    // ALUs, the other has products for the matrix cores.  One barrier per
    // stage: stage st is in LDS, the early wavefronts are done with stage
    // st - 1 and the late ones with stage st - 2, whose slot is refilled with
    // stage st + NS - 2 (stages st + 1 and st + 2 in flight while st - 1 and
    // st are in use).
    const bool late = wave >= kTileWaves / 2;
    bf16x8 bq[RT];                                      // probabilities of the stage before
    auto meet = [&](int st) {
      wait_stages<2 * LPS, NS>(min(NS - 3, nst - 1 - st));
      lds_barrier();
      if (st + NS - 2 < nst) issue_stage(st + NS - 2);  // into the slot of stage st - 2
    };
    // Ring reads (addresses: qk_lane_offset, pv_lane_offset): each is issued
    // kReadAhead steps before its products.  An iteration runs N = D / 16 value steps of stage st - 1
    // (dim block db), then N score steps of stage st (k-step i / 2, key block
    // i % 2); step j of those 2 N reads into x[j % NB].  A late wavefront has
    // passed the barrier of stage st before its value steps, so its first
    // score reads go out during its last value steps; an early one issues them
    // after the barrier.
    constexpr int N = D / 16, NB = kReadAhead + 1, RB = G::RB, E = G::SWV + 1;
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    bf16x8 x[NB];
    auto fetch_v = [&](unsigned va, int db) {
      const unsigned p0 = (va ^ (32u * (db % E))) + 32u * E * (db / E), p1 = p0 + 16u * RB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)p1);
      x[db % NB] = __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    auto fetch_k = [&](unsigned ka, int i) {
      const int ks = i / 2, kb = i % 2;
      const unsigned ad = (ka ^ (64u * (ks & 3))) + 256u * (ks >> 2) + 16u * RB * kb;
      x[(N + i) % NB] = *(const lds_bf16x8 *)(uintptr_t)ad;
    };
    // value steps of the stage at va; cross: the reads after them are the
    // first score reads of the stage at ka
    auto values = [&](unsigned va, unsigned ka, bool cross) {
#pragma unroll
      for (int db = 0; db < kReadAhead; ++db) fetch_v(va, db);
#pragma unroll
      for (int db = 0; db < N; ++db) {
        if (db + kReadAhead < N)
          fetch_v(va, db + kReadAhead);
        else if (cross)
          fetch_k(ka, db + kReadAhead - N);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) O[rt][db] = mfma_qk(x[db % NB], bq[rt], O[rt][db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int st = 0; st < nst; ++st) {
      const unsigned ka = kring_lds + (st % NS) * G::STAGE + opaque(klane);
      if (late) meet(st);
      if (st > 0) values(vring_lds + ((st - 1) % NS) * G::STAGE + opaque(vlane), ka, late);
      if (!late) meet(st);
      if (!late || st == 0) {
#pragma unroll
        for (int i = 0; i < kReadAhead; ++i) fetch_k(ka, i);
      }
      f32x4 Sc[2][RT];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) Sc[kb][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + kReadAhead < N) fetch_k(ka, i + kReadAhead);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) Sc[i % 2][rt] = mfma_qk(x[(N + i) % NB], qf[rt][i / 2], Sc[i % 2][rt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int64_t sk0 = k0 + (int64_t)SK * st;
      const int nk = (int)min<int64_t>(SK, k1 - sk0);
      float alpha[RT];
      bool r = false;
      if (sk0 + SK <= kfull) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const f32x4 st2[2] = {Sc[0][rt], Sc[1][rt]};
          r |= stage_softmax<false>(st2, nk, (int)(sk0 - n), mrun[rt], lrun[rt], lim[rt], sl2, bq[rt], alpha[rt]);
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const f32x4 st2[2] = {Sc[0][rt], Sc[1][rt]};
          r |= stage_softmax<true>(st2, nk, (int)(sk0 - n), mrun[rt], lrun[rt], lim[rt], sl2, bq[rt], alpha[rt]);
        }
      }
      if (__any(r)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int db = 0; db < NDB; ++db) O[rt][db] *= alpha[rt];
      }
    }
    if (nst > 0) values(vring_lds + ((nst - 1) % NS) * G::STAGE + vlane, 0u, false);   // no refill after the loop

    // -------------------------------------------------------- outputs
    // lane (g4, m16) holds dims 16 db + 4 g4 .. + 3 of row m16
    float lsum[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lsum[rt] = rows4_sum(lrun[rt]);
    const int flags = __builtin_amdgcn_readfirstlane(seg_info[sg][3]);
    const bool single = flags & 1, first_piece = flags & 2, cap_ok = flags & 4;
    if (single) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (wrow[rt] >= R) continue;
        const int l = wrow[rt] / Gq, h = kvh * Gq + wrow[rt] % Gq;
        const int64_t orow = ((int64_t)b * L + l) * Hq + h;
        const float inv = 1.f / lsum[rt];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = 16 * db + 4 * g4;
          RawE<4> zr;
          zr.load((const bf16_t *)p.q_gate + orow * 2 * D + D + d);
          float z[4];
          zr.to_float(z);
          bf16x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o4[i] = (bf16_t)(cap_ok ? O[rt][db][i] * inv * sigmoid_f(z[i]) : __builtin_nanf(""));
          *(bf16x4 *)((bf16_t *)p.out + orow * D + d) = o4;
        }
      }
    } else if (cap_ok) {
      // The piece's partial: its running max and sum, and its output divided
      // by the sum, in fp16 with the row scaled by a power of two s that puts
      // its largest magnitude in [1/2, 1) (s kept in fp32 beside the sum).
      // Each element keeps 11 significant bits, eight times finer than the
      // bf16 result.  A row that saw no key of the piece has sum 0 and stores
      // zeros (weight 0 in the merge).  Dim 16 db + 4 g4 + i of the row is
      // stored at 32 (db / 2) + 8 g4 + 4 (db % 2) + i: each lane writes
      // 16 bytes per store and the four lanes of a row 64 contiguous bytes.
      const int64_t slot_rows = (int64_t)__builtin_amdgcn_readfirstlane(seg_info[sg][4]) * p.rows;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float inv = lsum[rt] > 0.f ? 1.f / lsum[rt] : 0.f;
        float mx = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, __builtin_fabsf(O[rt][db][i]));
        mx = rows4_max(mx) * inv;                       // the four lane groups hold the row's dims
        const int e = mx > 0.f ? min(__builtin_amdgcn_frexp_expf(mx), 127) : 0;   // mx = f 2^e, f in [1/2, 1)
        if (wrow[rt] >= R) continue;
        const int rr = wrow[rt] - row0;
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        _Float16 *po = (_Float16 *)p.part_o + (slot_rows + rr) * D + 8 * g4;
#pragma unroll
        for (int db = 0; db < NDB; db += 2) {
          h8 hv;
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[i] = (_Float16)__builtin_ldexpf(O[rt][db + i / 4][i % 4] * inv, -e);
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, hv), (u32x4 *)(po + 16 * db));
        }
        if (g4 == 0)
          *(f32x4 *)(p.part_ml + (slot_rows + rr) * 4) = f32x4{mrun[rt], lsum[rt], __builtin_ldexpf(1.f, e), 0.f};
      }
    }
    if (!cap_ok && first_piece) {
      if (!single) nan_rows(tile);
      if (t == 0) flag_error(p);
    }
  }
}

template <int D>
static hipError_t launch_tile_d(const Params &p, hipStream_t s, const Timing &tm) {
  const int64_t nitems = (int64_t)p.B * p.Hkv * p.tiles * p.chunks;
  launch_kernel<kTileThreads>(tile_kernel<D>, nitems, s, tm, p.seq_lens, p.seq_offset, (const bf16_t *)p.qt, p.L, p.G, p.Hq,
                p.tiles, (int)nitems, p);
  return hipGetLastError();
}

hipError_t launch_tile_bf16(const Params &p, hipStream_t s, const Timing &tm) {
  if (p.rows != kPrefillRows && p.tiles != 1) return hipErrorInvalidValue;
  switch (p.D) {
    case 64: return launch_tile_d<64>(p, s, tm);
    case 128: return launch_tile_d<128>(p, s, tm);
    case 256: return launch_tile_d<256>(p, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
