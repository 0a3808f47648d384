// qsa_prefill.hip -- bf16 gated grouped-query attention for long blocks of new
// rows (prefill chunks) on gfx950, after the prologue kernel has normalised and
// rotated the queries into the prepared buffer and appended the new keys and
// values to the cache (Atlas qwen3_5/mod.rs module doc: append, then attend).
//
// tile_kernel: one workgroup = (sequence b, KV head g, tile of 64 query rows,
// key chunk).  The rows are (new row l, head of group g) pairs in order
// r = l * G + (h - g * G) (DS4Server issue #113, Reproduction: query heads
// grouped within their KV group).  The chunk's keys stream through the same
// HBM -> LDS ring of 64-key stages as the short-query kernel, and each stage
// goes through the same step: every wavefront scores its 16 keys against all
// 64 rows, the four agree on each row's running max and publish a bf16
// probability tile, and each accumulates its own D/4 output dims over the 64
// keys.  Per stage a wavefront reads 16 K rows and a quarter of the V tile from
// LDS for 64 x 64 x D x 4 flops of the workgroup, so the LDS stays well below
// its bandwidth while the MFMAs work.  A tile covered by one chunk applies the
// gate attn * sigmoid(gate) (mlxd PR #99 Summary) and stores bf16; otherwise
// it writes the chunk's (max, sum, unnormalised output) for the merge kernel.
#include "qsa_device.h"

namespace qsa {

namespace {

constexpr int kPrefillRows = kPrefillTileRows;   // query rows per workgroup: four 16-row MFMA tiles
static_assert(kPrefillRows == 64, "the stage step handles four row tiles");

}  // namespace

// Work items ((b, g, tile) slot, chunk) are numbered chunk-fastest; the
// workgroup of block i runs on XCD i % 8, and each XCD takes a contiguous range
// of items so that the tiles sharing a KV head share that XCD's L2.
// Preloaded arguments: sequence metadata, the prepared queries and the grid shape.
template <int D>
__global__ __launch_bounds__(kThreads) void tile_kernel(const int32_t *__restrict__ seq_lens,
                                                        const int64_t *__restrict__ seq_offset,
                                                        const bf16_t *__restrict__ qt, int L, int Gq, int Hq,
                                                        int tiles, int nitems, Params p) {
  using G = Geo<D>;
  constexpr int KST = D / 32, DBW = D / 64, NS = G::NS, LPS = G::LPS;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2 * G::RING];   // K ring | V ring
  __shared__ __attribute__((aligned(16))) unsigned char xch[Xch::BYTES];    // stage exchange
  unsigned char *const kring = ring, *const vring = ring + G::RING;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int lane = t % kWave, g4 = lane >> 4, m16 = lane & 15;
  // XCD-contiguous item numbering
  const int per = nitems / 8, rem = nitems % 8, x = blockIdx.x % 8, j = blockIdx.x / 8;
  const int item = x * per + min(x, rem) + j;
  const int hkv = p.Hkv, pchunks = p.chunks;
  const int chunk = item % pchunks, slot = item / pchunks;
  const int tile = slot % tiles, bk = slot / tiles;
  const int b = bk / hkv, kvh = bk % hkv;
  const int R = L * Gq;                                 // rows of this KV head
  const int row0 = tile * kPrefillRows;

  // ------------------------------------------------------------ round trip 1: metadata and queries
  const int n = seq_lens[b];
  const int64_t off = seq_offset[b];
  bf16x8 qf[4][KST];
  int64_t lim[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r = min(row0 + 16 * rt + m16, R - 1);
    const int l = r / Gq, h = kvh * Gq + r % Gq;
    const bf16_t *src = qt + (((int64_t)b * L + l) * Hq + h) * D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) qf[rt][ks] = __builtin_bit_cast(bf16x8, gld<uint4>(src + 32 * ks));
  }
  const int ck = p.chunk_keys, msl = p.max_seq_len;
  const int64_t nrows = p.num_rows;
  const bf16_t *const kc = (const bf16_t *)p.kc;
  const bf16_t *const vc = (const bf16_t *)p.vc;
  const int32_t *const capp = p.capacity;
  const float sl2 = p.scale_log2;
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"s"(n), "s"(off), "s"(ck), "s"(msl), "s"(nrows), "s"(kc), "s"(vc), "s"(capp), "s"(sl2));
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      asm volatile("" ::"v"(__builtin_bit_cast(u32x4, qf[rt][ks])));
    }

  const int64_t total = (int64_t)n + L;
  const bool in_range = n >= 0 && off >= 0 && total <= msl && off + total <= nrows;
  const int cap = capp ? capp[b] : 0x7fffffff;
  const int rlast = min(row0 + kPrefillRows, R) - 1;    // last row of the tile
  const int64_t kend = (int64_t)n + rlast / Gq + 1;     // keys the tile's rows can see
  const int nch = chunk_count(kend, ck);
  if (chunk >= nch) return;
  if (!in_range) {
    if (chunk == 0) {
      for (int e = t; e < (rlast - row0 + 1) * D; e += kThreads) {
        const int r = row0 + e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
      if (t == 0) flag_error(p);
    }
    return;
  }
  const int64_t k0 = (int64_t)chunk * ck;
  const int64_t k1 = chunk == nch - 1 ? kend : k0 + ck;
  const int nst = (int)((k1 - k0 + G::SK - 1) / G::SK);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) lim[rt] = (int64_t)n + (row0 + 16 * rt + m16) / Gq;

  // ------------------------------------------------------------ key stages
  const unsigned kring_lds = (unsigned)(uintptr_t)(lds_void *)kring;
  const unsigned vring_lds = (unsigned)(uintptr_t)(lds_void *)vring;
  auto issue_stage = [&](int st) {   // keys k0 + 64 st .. into ring slot st % NS
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int u = t + kThreads * i;
      const int key = u / G::OCT, pos = u % G::OCT, oct = pos ^ (key & G::SW);
      const int64_t kk = min(k0 + (int64_t)G::SK * st + key, k1 - 1);
      const int64_t e = ((off + kk) * hkv + kvh) * D + 8 * oct;
      const unsigned dst = (st % NS) * G::STAGE + kThreads * 16 * i + wave * 1024;
      dma16_asm(kc + e, kring_lds + dst);
      dma16_asm(vc + e, vring_lds + dst);
    }
  };
#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (st < nst) issue_stage(st);

  f32x4 O[4][DBW];
  float mrun[4], lrun[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    mrun[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int db = 0; db < DBW; ++db) O[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int st = 0; st < nst; ++st) {
    wait_stages<2 * LPS, NS>(min(NS - 1, nst - 1 - st));
    lds_barrier();
    const int so = (st % NS) * G::STAGE;
    const int64_t sk0 = k0 + (int64_t)G::SK * st;
    const int nk = (int)min<int64_t>(G::SK, k1 - sk0);
    attend_stage<D, 4>(kring + so, vring + so, nk, sk0, qf, O, mrun, lrun, lim, sl2, xch);
    lds_barrier();                                      // every wave is done with ring slot st % NS
    if (st + NS < nst) issue_stage(st + NS);
  }

  // ------------------------------------------------------------ outputs
  // every wavefront writes its own dims 16 (DBW wave + db) + 4 g4 .. + 3
  const bool cap_ok = total <= (int64_t)cap;
  const bool single = nch == 1;
  const int64_t slot_rows = ((int64_t)slot * pchunks + chunk) * p.rows;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r = row0 + 16 * rt + m16;
    if (r >= R) continue;
    const int l = r / Gq, h = kvh * Gq + r % Gq;
    const int64_t orow = ((int64_t)b * L + l) * Hq + h;
    if (single) {
      const float inv = 1.f / lrun[rt];
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const int d = 16 * (DBW * wave + db) + 4 * g4;
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
    } else if (cap_ok) {
      const int rr = r - row0;
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const int d = 16 * (DBW * wave + db) + 4 * g4;
        *(float4 *)(p.part_o + (slot_rows + rr) * D + d) = make_float4(O[rt][db][0], O[rt][db][1], O[rt][db][2], O[rt][db][3]);
      }
      if (wave == 0 && g4 == 0) *(float2 *)(p.part_ml + (slot_rows + rr) * 2) = make_float2(mrun[rt], lrun[rt]);
    }
  }
  if (!cap_ok && chunk == 0) {
    if (!single) {
      for (int e = t; e < (rlast - row0 + 1) * D; e += kThreads) {
        const int r = row0 + e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
    }
    if (t == 0) flag_error(p);
  }
}

template <int D>
static hipError_t launch_tile_d(const Params &p, hipStream_t s, const Timing &tm) {
  const int64_t nitems = (int64_t)p.B * p.Hkv * p.tiles * p.chunks;
  launch_kernel(tile_kernel<D>, nitems, s, tm, p.seq_lens, p.seq_offset, (const bf16_t *)p.qt, p.L, p.G, p.Hq,
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
