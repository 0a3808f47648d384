// qsa_tiles.hip -- bf16 gated grouped-query attention on MFMA (gfx950).
//
// split_kernel: one workgroup = (sequence b, KV head g, row tile, key chunk).
// The row tile holds up to 64 query rows: the G query heads that share KV head
// g times the new rows (DS4Server issue #113: query heads grouped within their
// KV group; Atlas Qwen35ForwardConfig: 16 query / 4 KV heads).  The chunk's
// keys stream through LDS 64 at a time with an online softmax (flash-decoding
// split-K).  A tile covered by one chunk is finished in place with the output
// gate attn * sigmoid(gate) (mlxd PR #99 Summary; Atlas sigmoid_gate);
// otherwise every chunk writes (max, sum, unnormalised output) and
// combine_kernel merges the chunks after the kernel boundary -- no device-wide
// fence or atomic is taken inside the streaming kernel.
//
// Fused mode (PREP = false, decode / verify): each workgroup derives its own
// queries from q_gate (split, RMS norm, partial rotation), and the workgroup
// whose chunk holds the new key slots n_b .. n_b+L-1 normalises, rotates and
// appends them (Atlas qwen3_5/mod.rs module doc: append at cache_pos, attend
// over cache_pos + 1 keys), patching them into its own LDS tile.  Prepared mode
// (PREP = true, long prefill): queries come from the prologue kernel's buffer
// and the cache already holds the new rows.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, lane l, g = l / 16, m = l % 16):
//   scores^T[key][row] = K[key][:] . Q[row][:]    A = K rows from LDS, B = Q
//   out^T[dim][row]   += V^T[dim][key] . P^T[key][row]
// Score block beta of a 32-key block maps MFMA row m to key 8(m/4) + 4 beta + m%4,
// so each lane ends up holding the 8 consecutive keys 8g .. 8g+7 of one query
// row: exactly the B operand the value product needs, with no lane shuffle.
// K and V are both staged row-major ([key][dim]) in LDS with 16-byte writes; the
// V^T operand (8 keys of one dim per lane) is read with the gfx950 transposing
// LDS load ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i%4 of the 8-byte rows addressed by lanes i/4 + 4j, j = 0..3.
#include <type_traits>

#include "qsa_internal.h"

namespace qsa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

// V^T operand of one 16x16x32 MFMA: dims dim0 + (l%16), keys key0 + 8(l/16) + 0..7,
// from a row-major [key][stride] bf16 tile, with two transposing 8-byte LDS loads.
__device__ __forceinline__ bf16x8 vt_operand(const bf16_t *tile, int stride, int key0, int dim0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const bf16_t *p0 = tile + (key0 + 8 * g + (i >> 2)) * stride + dim0 + 4 * (i & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p0 + 4 * stride));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Load through the global address space (never a flat access: flat loads also
// count against the LDS/scalar counter and stall unrelated LDS waits).
template <typename T> struct native_of { using type = T; };
template <> struct native_of<uint4> { using type = unsigned __attribute__((ext_vector_type(4))); };
template <> struct native_of<uint2> { using type = unsigned __attribute__((ext_vector_type(2))); };
template <typename T>
__device__ __forceinline__ T gload(const void *ptr) {
  using N = typename native_of<T>::type;
  return __builtin_bit_cast(T, *(const __attribute__((address_space(1))) N *)ptr);
}

// Raw 8- or 16-byte groups of bf16 <-> floats.
template <int N, typename R>
__device__ __forceinline__ void raw_to_float(const R &r, float *dst) {
  typedef __bf16 bfN __attribute__((ext_vector_type(N)));
  const bfN v = __builtin_bit_cast(bfN, r);
#pragma unroll
  for (int j = 0; j < N; ++j) dst[j] = (float)v[j];
}
template <int N, typename R>
__device__ __forceinline__ R float_to_raw(const float *src) {
  typedef __bf16 bfN __attribute__((ext_vector_type(N)));
  bfN v;
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = (bf16_t)src[j];
  return __builtin_bit_cast(R, v);
}

// Wave-local LDS ordering: every lane's earlier LDS writes are complete before
// any lane of the wave reads (LDS operations of one wave complete in order).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// RMS-normalise and rotate four head rows per wavefront, 16 lanes per row, each
// lane holding E = D/16 contiguous elements.  Partial sums of squares and the
// rotation partners (e +- r/2) go through LDS (red: [4][16], scr: [4][D] fp32
// for this wave), so there are no cross-lane shuffle chains.  cs: (cos, sin)
// of this row's position for the r/2 pairs.
template <int D>
__device__ __forceinline__ void norm_rope_rows16(float (&x)[D / 16], const float (&w)[D / 16],
                                                 const float2 *cs, int r, float eps, float *red,
                                                 float *scr) {
  constexpr int E = D / 16;
  const int lane = threadIdx.x % kWave, sub = lane >> 4, c16 = lane & 15;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) ss += x[j] * x[j];
  red[sub * 16 + c16] = ss;
  wave_lds_sync();
  ss = 0.f;
#pragma unroll
  for (int c = 0; c < 16; c += 4) {
    const float4 v = *(const float4 *)&red[sub * 16 + c];
    ss += (v.x + v.y) + (v.z + v.w);
  }
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int j = 0; j < E; ++j) x[j] = x[j] * inv * w[j];
  if (r == 0) return;
  float *row = scr + sub * D;
#pragma unroll
  for (int j = 0; j < E; ++j) row[c16 * E + j] = x[j];
  wave_lds_sync();
  const int h = r / 2;
  if (c16 * E < r) {                              // this lane holds rotated elements
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = c16 * E + j;
      const bool lo = e < h;
      const int pe = lo ? e + h : e - h;          // pair partner
      const float2 t = cs[lo ? e : e - h];        // (cos, sin)
      const float other = row[min(pe, D - 1)];
      const float y = lo ? x[j] * t.x - other * t.y : x[j] * t.x + other * t.y;
      x[j] = e < r ? y : x[j];
    }
  }
}

}  // namespace

template <int D, bool PREP, int RMAX>
__global__ __launch_bounds__(kThreads) void split_kernel(Params p) {
  constexpr int KST = D / 32;          // MFMA k-steps over head_dim
  constexpr int NDB = D / 16;          // 16-wide dim blocks of the output
  constexpr int KSTR = D + 8;          // K row stride in LDS (bf16)
  constexpr int OCT = D / 8;           // 16-byte units per key row
  constexpr int E = D / 16;            // elements per lane in the row routines (16 lanes per row)
  using Raw = typename std::conditional<(E >= 8), uint4, uint2>::type;  // never reads past a row
  constexpr int RE = E >= 8 ? 8 : 4;                    // elements per raw unit
  constexpr int EU = E / RE;                            // raw units per lane per row
  constexpr int KU = kTileKeys * OCT / kThreads;        // 16-byte K (and V) units per thread per stage
  constexpr int NEWR = PREP ? 1 : kMaxFusedNewRows;
  constexpr int QU = (RMAX * OCT + kThreads - 1) / kThreads;  // 16-byte query units per thread
  static_assert(KU >= 1 && E >= 4 && RMAX <= kTileRows, "head_dim too small for the tile");

  // fused mode keeps 32 spare rows so a chunk's new rows can join its last stage
  constexpr int TROWS = PREP ? kTileKeys : kTileKeys + 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[TROWS * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[TROWS * KSTR];   // V rows, same layout as K
  __shared__ __attribute__((aligned(16))) bf16_t newK[NEWR * D];
  __shared__ __attribute__((aligned(16))) bf16_t newV[NEWR * D];

  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int g4 = lane >> 4, m16 = lane & 15;
  const int sub = lane >> 4, c16 = lane & 15;      // row routines: 4 rows per wave, 16 lanes each

  // ---------------------------------------------------------------- work item
  int item = blockIdx.x;
  const int chunk = item % p.chunks;
  item /= p.chunks;
  const int tile = item % p.tiles;
  item /= p.tiles;
  const int kvh = item % p.Hkv;
  const int b = item / p.Hkv;
  const int slot = (b * p.Hkv + kvh) * p.tiles + tile;

  const int rows_total = p.L * p.G;
  const int row0 = tile * kTileRows;
  const int R = min(p.rows, rows_total - row0);
  const bf16_t *qg = (const bf16_t *)p.q_gate;
  const bool fuse_new = !PREP && p.k_new != nullptr;
  const int half = p.r / 2;

  // ---------------------------------------------------------------- phase A: small loads
  // Issued back to back with clamped (always valid) addresses.  The vector-memory
  // counter retires in order, so nothing that is issued after the K/V stage may be
  // waited on before the stage itself has landed.
  const int n = gload<int>(p.seq_lens + b);
  const int64_t off = gload<int64_t>(p.seq_offset + b);
  const int cap = p.capacity ? gload<int>(p.capacity + b) : 0x7fffffff;
  const int qunits = R * OCT;
  uint4 qreg[QU];
#pragma unroll
  for (int i = 0; i < QU; ++i) {
    const int e = min(t + kThreads * i, qunits - 1), rr = e / OCT, o = e % OCT;
    const int rg = row0 + rr, l = rg / p.G, h = kvh * p.G + rg % p.G;
    const bf16_t *src = PREP ? (const bf16_t *)p.qt + (((int64_t)b * p.L + l) * p.Hq + h) * D + 8 * o
                             : qg + (((int64_t)b * p.L + l) * p.Hq + h) * 2 * D + 8 * o;
    qreg[i] = gload<uint4>(src);
  }
  Raw wq_raw[EU], wk_raw[EU];
  const int tent = PREP ? 0 : p.L * half;             // rotation-table entries (new rows x pairs)
  int tpos = 0;
  double tinv = 0.0;
  if constexpr (!PREP) {
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      wq_raw[u] = gload<Raw>((const bf16_t *)p.wq + c16 * E + RE * u);
      wk_raw[u] = gload<Raw>((const bf16_t *)p.wk + c16 * E + RE * u);
    }
    // unconditional (clamped) so that no branch merge pulls a use of the loaded
    // value ahead of the K/V stage issue
    const int hh = max(half, 1), e = min(t, max(tent - 1, 0));
    tpos = gload<int>(p.positions + b * p.L + e / hh);
    tinv = p.inv_freq[e % hh];
  }

  // ---------------------------------------------------------------- bounds and chunk
  const int64_t total = (int64_t)n + p.L;
  if (!(n >= 0 && off >= 0 && total <= p.max_seq_len && off + total <= p.num_rows && total <= cap)) {
    if (chunk == 0) {
      for (int e = t; e < R * D; e += kThreads) {
        const int rg = row0 + e / D;
        const int l = rg / p.G, h = kvh * p.G + rg % p.G;
        ((bf16_t *)p.out)[(((int64_t)b * p.L + l) * p.Hq + h) * D + e % D] = (bf16_t)__builtin_nanf("");
      }
      if (t == 0) flag_error(p);
    }
    return;
  }
  const int lmax = (row0 + R - 1) / p.G;               // last new row in this tile
  const int64_t kend = (int64_t)n + lmax + 1;           // keys needed by the tile
  const int nch = chunk_count(kend, p.chunk_keys);
  if (chunk >= nch) return;
  const int64_t k0 = (int64_t)chunk * p.chunk_keys;
  const int64_t k1 = chunk == nch - 1 ? kend : k0 + p.chunk_keys;

  const int RT = (R + 15) / 16;              // 16-row MFMA tiles
  const int KS = RT <= 2 ? 2 : 1;            // waves splitting the keys of a stage
  const bool computes = wave < RT * KS;
  const int rt = wave % RT, ksub = wave / RT;

  // new rows n .. n+L-1 that fall in this chunk are produced here (fused mode)
  const int nlo = fuse_new ? (int)max((int64_t)0, min(k0 - n, (int64_t)p.L)) : 0;
  const int nhi = fuse_new ? (int)max((int64_t)nlo, min(k1 - n, (int64_t)p.L)) : 0;
  const int64_t patch_from = nhi > nlo ? (int64_t)n + nlo : INT64_MAX;  // keys >= this come from LDS

  // ---------------------------------------------------------------- phase B: new rows, then the stage
  const int nl = nlo + wave * 4 + sub;                  // new row handled by this lane group
  const bool has_nl = nl < nhi;
  Raw knew[EU], vnew[EU];
  if (nhi > nlo) {
    const int64_t src_row = ((int64_t)b * p.L + min(nl, nhi - 1)) * p.Hkv + kvh;
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      knew[u] = gload<Raw>((const bf16_t *)p.k_new + src_row * D + c16 * E + RE * u);
      vnew[u] = gload<Raw>((const bf16_t *)p.v_new + src_row * D + c16 * E + RE * u);
    }
  }

  const bf16_t *kc = (const bf16_t *)p.kc;
  const bf16_t *vc = (const bf16_t *)p.vc;
  // Loads always go to a clamped, valid row and land in registers untouched; the
  // validity of each unit is kept as a bit and applied when the stage is written
  // to LDS.  (Zeroing a load's destination register conditionally would make the
  // wave wait for that load right there, serialising the whole stage.)
  uint4 kreg[KU], vreg[KU];
  uint32_t ldmask = 0;
  auto load_stage = [&](int64_t sb) {
    ldmask = 0;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = t + kThreads * i, key = u / OCT, o = u % OCT;
      const int64_t ka = sb + key;
      const bool ld = ka < k1 && ka < patch_from;
      const int64_t src = ((off + (ld ? ka : k0)) * p.Hkv + kvh) * D + 8 * o;
      kreg[i] = gload<uint4>(kc + src);
      vreg[i] = gload<uint4>(vc + src);
      ldmask |= (uint32_t)ld << i;
    }
  };
  load_stage(k0);
  // Nothing that consumes an earlier load may be hoisted above the stage issue:
  // the vector-memory counter retires in order, so such a use would drain
  // every outstanding load before the K/V stage was even requested.
  __builtin_amdgcn_sched_barrier(0);

  // ---------------------------------------------------------------- queries (no global loads below)
  bf16_t *Qs = Ks;                                      // [64][KSTR], aliases the K stage
#pragma unroll
  for (int i = 0; i < QU; ++i) {
    const int e = t + kThreads * i;
    if (e < qunits) *(uint4 *)&Qs[(e / OCT) * KSTR + 8 * (e % OCT)] = qreg[i];
  }
  for (int e = t; e < (RT * 16 - R) * OCT; e += kThreads)
    *(uint4 *)&Qs[(R + e / OCT) * KSTR + 8 * (e % OCT)] = uint4{0, 0, 0, 0};
  if constexpr (!PREP) {
    // LDS scratch in the V stage region: rotation table [L][r/2] (64 D bytes),
    // per-wave fp32 rows [4][4][D] (64 D bytes), partial sums [4][4][16]
    float2 *cs = reinterpret_cast<float2 *>(Vt);
    float *scr = reinterpret_cast<float *>(Vt) + 16 * D + wave * 4 * D;
    float *red = reinterpret_cast<float *>(Vt) + 32 * D + wave * 64;
    auto put_cs = [&](int e, int pos, double inv) {
      const double a = (double)pos * inv;
      const double k = rint(a * 0.15915494309189535);  // 1 / (2 pi), reduction in double
      double rd = fma(-k, 6.283185307179586, a);
      rd = fma(-k, 2.4492935982947064e-16, rd);
      float c, sn;
      sincosf((float)rd, &sn, &c);
      cs[e] = make_float2(c, sn);
    };
    if (t < tent) put_cs(t, tpos, tinv);
    for (int e = t + kThreads; e < tent; e += kThreads)   // only when L * r/2 > 256
      put_cs(e, gload<int>(p.positions + b * p.L + e / half), p.inv_freq[e % half]);
    float wq[E], wk[E];
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      raw_to_float<RE>(wq_raw[u], wq + RE * u);
      raw_to_float<RE>(wk_raw[u], wk + RE * u);
    }
    __syncthreads();
    for (int base = 0; base < R; base += 16) {
      const int rr = base + wave * 4 + sub;
      const int rrc = min(rr, R - 1);
      float x[E];
      const bf16_t *src = Qs + rrc * KSTR + c16 * E;
#pragma unroll
      for (int j = 0; j < E; ++j) x[j] = (float)src[j];
      norm_rope_rows16<D>(x, wq, cs + ((row0 + rrc) / p.G) * half, p.r, p.eps, red, scr);
      wave_lds_sync();
      if (rr < R) {
        bf16_t *dst = Qs + rr * KSTR + c16 * E;
#pragma unroll
        for (int j = 0; j < E; ++j) dst[j] = (bf16_t)x[j];
      }
      wave_lds_sync();
    }
    if (nhi > nlo) {
      float x[E];
#pragma unroll
      for (int u = 0; u < EU; ++u) raw_to_float<RE>(knew[u], x + RE * u);
      norm_rope_rows16<D>(x, wk, cs + min(nl, nhi - 1) * half, p.r, p.eps, red, scr);
      if (has_nl) {
        const int64_t dst = ((off + n + nl) * p.Hkv + kvh) * D + c16 * E;
#pragma unroll
        for (int u = 0; u < EU; ++u) {
          const Raw kb = float_to_raw<RE, Raw>(x + RE * u);
          *(Raw *)((bf16_t *)p.kc + dst + RE * u) = kb;
          *(Raw *)((bf16_t *)p.vc + dst + RE * u) = vnew[u];
          *(Raw *)&newK[(nl - nlo) * D + c16 * E + RE * u] = kb;
          *(Raw *)&newV[(nl - nlo) * D + c16 * E + RE * u] = vnew[u];
        }
      }
    }
  }
  __syncthreads();  // Qs, newK, newV complete

  bf16x8 qf[KST];
  if (computes) {
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) qf[ks] = *(const bf16x8 *)&Qs[(rt * 16 + m16) * KSTR + 32 * ks + 8 * g4];
  }
  __syncthreads();  // Qs (aliasing Ks) and the prologue scratch (in Vt) are free again

  // ---------------------------------------------------------------- key loop
  f32x4 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  const int rowg = row0 + rt * 16 + m16;
  const int64_t lim = (int64_t)n + rowg / p.G;          // causal: row sees keys <= n + l

  int nst = (int)((k1 - k0 + kTileKeys - 1) / kTileKeys);
  if (TROWS > kTileKeys && nst >= 2) {
    // a final stage holding nothing but new rows (at most 32) joins the one before
    const int64_t last = k0 + (int64_t)(nst - 1) * kTileKeys;
    if (last >= patch_from && k1 - last <= TROWS - kTileKeys) --nst;
  }
  for (int st = 0; st < nst; ++st) {
    const int64_t sb = k0 + (int64_t)st * kTileKeys;
    const int64_t se = st == nst - 1 ? k1 : sb + kTileKeys;   // stage end (at most TROWS keys)
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = t + kThreads * i, key = u / OCT, o = u % OCT;
      const int64_t ka = sb + key;
      const bool ld = (ldmask >> i) & 1u;
      uint4 kv = ld ? kreg[i] : uint4{0, 0, 0, 0}, vv = ld ? vreg[i] : uint4{0, 0, 0, 0};
      if (ka >= patch_from && ka < k1) {
        kv = *(const uint4 *)&newK[(ka - n - nlo) * D + 8 * o];
        vv = *(const uint4 *)&newV[(ka - n - nlo) * D + 8 * o];
      }
      *(uint4 *)&Ks[key * KSTR + 8 * o] = kv;
      *(uint4 *)&Vt[key * KSTR + 8 * o] = vv;
    }
    if (TROWS > kTileKeys && se - sb > kTileKeys) {
      // spare rows: new rows from LDS, zeros past the chunk end
      for (int e = t; e < (TROWS - kTileKeys) * OCT; e += kThreads) {
        const int key = kTileKeys + e / OCT, o = e % OCT;
        const int64_t ka = sb + key;
        uint4 kv = uint4{0, 0, 0, 0}, vv = uint4{0, 0, 0, 0};
        if (ka >= patch_from && ka < k1) {
          kv = *(const uint4 *)&newK[(ka - n - nlo) * D + 8 * o];
          vv = *(const uint4 *)&newV[(ka - n - nlo) * D + 8 * o];
        }
        *(uint4 *)&Ks[key * KSTR + 8 * o] = kv;
        *(uint4 *)&Vt[key * KSTR + 8 * o] = vv;
      }
    }
    __syncthreads();
    if (st + 1 < nst) load_stage(sb + kTileKeys);
    __builtin_amdgcn_sched_barrier(0);

    if (computes) {
#pragma unroll
      for (int blk = 0; blk < TROWS / 32; ++blk) {
        if ((blk % KS) != ksub) continue;
        const int kb = 32 * blk;
        if (sb + kb >= se) continue;           // block entirely past the stage end
        f32x4 sacc[2];
#pragma unroll
        for (int beta = 0; beta < 2; ++beta) {
          sacc[beta] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int keyl = kb + 8 * (m16 >> 2) + 4 * beta + (m16 & 3);
#pragma unroll
          for (int ks = 0; ks < KST; ++ks) {
            const bf16x8 a = *(const bf16x8 *)&Ks[keyl * KSTR + 32 * ks + 8 * g4];
            sacc[beta] = mfma16(a, qf[ks], sacc[beta]);
          }
        }
        float sv[8];
        float mb = -INFINITY;
#pragma unroll
        for (int beta = 0; beta < 2; ++beta)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t ka = sb + kb + 8 * g4 + 4 * beta + i;
            const bool valid = ka < k1 && ka <= lim;
            const float v = valid ? sacc[beta][i] * p.scale_log2 : -INFINITY;
            sv[4 * beta + i] = v;
            mb = fmaxf(mb, v);
          }
        mb = fmaxf(mb, __shfl_xor(mb, 16, kWave));
        mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
        const float mn = fmaxf(m_run, mb);
        const float alpha = exp2f(m_run - mn);
        bf16x8 pf;
        float ps = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const bf16_t e = (bf16_t)exp2f(sv[k] - mn);
          pf[k] = e;
          ps += (float)e;
        }
        l_run = l_run * alpha + ps;
        m_run = mn;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          O[db] *= alpha;
          O[db] = mfma16(vt_operand(Vt, KSTR, kb, 16 * db, lane), pf, O[db]);
        }
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- merge key halves
  constexpr int XW = NDB * 4 + 2;
  float *xch = reinterpret_cast<float *>(Ks);   // [2][64][XW] fits exactly in Ks
  if (computes && KS == 2 && ksub == 1) {
    float *dst = xch + (rt * kWave + lane) * XW;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[db * 4 + i] = O[db][i];
    dst[NDB * 4] = m_run;
    dst[NDB * 4 + 1] = l_run;
  }
  __syncthreads();
  const bool owner = computes && ksub == 0;
  if (!owner) return;
  if (KS == 2) {
    const float *src = xch + (rt * kWave + lane) * XW;
    const float m1 = src[NDB * 4], l1 = src[NDB * 4 + 1];
    const float mn = fmaxf(m_run, m1);
    const float a0 = exp2f(m_run - mn), a1 = exp2f(m1 - mn);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[db][i] = O[db][i] * a0 + src[db * 4 + i] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = mn;
  }
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  const int rr = rt * 16 + m16;   // row within the tile held by this lane
  if (rr >= R) return;

  if (nch == 1) {
    // the whole tile in one chunk: normalise, gate and store here
    const int l = rowg / p.G, h = kvh * p.G + rowg % p.G;
    const int64_t o_base = (((int64_t)b * p.L + l) * p.Hq + h) * D;
    const bf16_t *z = qg + (((int64_t)b * p.L + l) * p.Hq + h) * 2 * D + D;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 16 * db + 4 * g4;
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16_t)(O[db][i] * inv * sigmoid(to_f(z[d + i])));
      *(bf16x4 *)((bf16_t *)p.out + o_base + d) = v;
    }
    return;
  }
  const int64_t ps_ = ((int64_t)slot * p.chunks + chunk) * p.rows + rr;
  float *po = p.part_o + ps_ * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) *(f32x4 *)(po + 16 * db + 4 * g4) = O[db];
  if (g4 == 0) {
    p.part_ml[ps_ * 2 + 0] = m_run;
    p.part_ml[ps_ * 2 + 1] = l_run;
  }
}

// Merge the key chunks of one (slot, row): weights 2^(m_c - M) / sum_c l_c 2^(m_c - M),
// weighted sum of the unnormalised chunk outputs, then the sigmoid gate.  Waves
// take interleaved chunks; lanes take EPL = D/64 dims.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(Params p) {
  constexpr int EPL = D / kWave;
  constexpr int kBatch = 16;                            // chunks in flight per wave
  __shared__ float wts[kMaxChunks];
  __shared__ float acc_x[kThreads / kWave][D];
  __shared__ float red[kThreads / kWave];
  __shared__ float s_inv;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int rr = blockIdx.x % p.rows;
  const int slot = blockIdx.x / p.rows;
  const int tile = slot % p.tiles;
  const int kvh = (slot / p.tiles) % p.Hkv;
  const int b = slot / (p.tiles * p.Hkv);
  const int rows_total = p.L * p.G;
  const int row0 = tile * kTileRows;
  const int R = min(p.rows, rows_total - row0);
  if (rr >= R) return;
  const int n = gload<int>(p.seq_lens + b);
  int64_t off;
  if (!seq_in_range(p, b, n, off)) return;              // the split kernel wrote NaN
  const int lmax = (row0 + R - 1) / p.G;
  const int nch = chunk_count((int64_t)n + lmax + 1, p.chunk_keys);
  if (nch == 1) return;                                 // finished by the split kernel

  // every load first: chunk statistics, the gate, the first batch of partial outputs
  const int64_t base = (int64_t)slot * p.chunks * p.rows + rr;   // + c * rows
  const int rg = row0 + rr, l = rg / p.G, h = kvh * p.G + rg % p.G;
  const bf16_t *zp = (const bf16_t *)p.q_gate + (((int64_t)b * p.L + l) * p.Hq + h) * 2 * D + D + lane * EPL;
  float z[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) z[j] = to_f(gload<bf16_t>(zp + j));
  const int cm = min(t, nch - 1);
  const float m_c = gload<float>(p.part_ml + (base + (int64_t)cm * p.rows) * 2);
  const float l_c = gload<float>(p.part_ml + (base + (int64_t)cm * p.rows) * 2 + 1);
  float v[kBatch][EPL];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int c = min(wave + k * (kThreads / kWave), nch - 1);
    const float *po = p.part_o + (base + (int64_t)c * p.rows) * D + lane * EPL;
#pragma unroll
    for (int j = 0; j < EPL; ++j) v[k][j] = gload<float>(po + j);
  }
  __builtin_amdgcn_sched_barrier(0);

  // weights w_c = 2^(m_c - M) / sum_c l_c 2^(m_c - M)   (chunks beyond 256 are rare)
  float mx = t < nch ? m_c : -INFINITY;
  for (int c = t + kThreads; c < nch; c += kThreads) mx = fmaxf(mx, p.part_ml[(base + (int64_t)c * p.rows) * 2]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float ls = 0.f;
  if (t < nch) {
    const float e = exp2f(m_c - M);
    wts[t] = e;
    ls = e * l_c;
  }
  for (int c = t + kThreads; c < nch; c += kThreads) {
    const float e = exp2f(p.part_ml[(base + (int64_t)c * p.rows) * 2] - M);
    wts[c] = e;
    ls += e * p.part_ml[(base + (int64_t)c * p.rows) * 2 + 1];
  }
  ls = wave_sum(ls);
  __syncthreads();
  if (lane == 0) red[wave] = ls;
  __syncthreads();
  if (t == 0) s_inv = 1.f / ((red[0] + red[1]) + (red[2] + red[3]));
  __syncthreads();

  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int c = wave + k * (kThreads / kWave);
    const float wc = c < nch ? wts[c] : 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] += wc * v[k][j];
  }
  for (int c0 = wave + kBatch * (kThreads / kWave); c0 < nch; c0 += kThreads / kWave) {
    const float wc = wts[c0];
    const float *po = p.part_o + (base + (int64_t)c0 * p.rows) * D + lane * EPL;
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] += wc * po[j];
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc_x[wave][lane * EPL + j] = acc[j];
  __syncthreads();
  if (wave != 0) return;
  const float inv = s_inv;
  bf16_t *out = (bf16_t *)p.out + (((int64_t)b * p.L + l) * p.Hq + h) * D;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int d = lane * EPL + j;
    const float o = ((acc_x[0][d] + acc_x[1][d]) + (acc_x[2][d] + acc_x[3][d])) * inv;
    out[d] = (bf16_t)(o * sigmoid(z[j]));
  }
}

template <int D>
static hipError_t launch_split_d(const Params &p, bool prep, hipStream_t s, const Timing &tm) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.tiles * p.chunks;
  if (prep)
    launch_kernel(split_kernel<D, true, kTileRows>, blocks, s, tm, p);
  else if (p.rows <= 16)
    launch_kernel(split_kernel<D, false, 16>, blocks, s, tm, p);
  else
    launch_kernel(split_kernel<D, false, kTileRows>, blocks, s, tm, p);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const Params &p, bool prepared_q, hipStream_t s, const Timing &tm) {
  switch (p.D) {
    case 64: return launch_split_d<64>(p, prepared_q, s, tm);
    case 128: return launch_split_d<128>(p, prepared_q, s, tm);
    case 256: return launch_split_d<256>(p, prepared_q, s, tm);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine_bf16(const Params &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.tiles * p.rows;
  switch (p.D) {
    case 64: hipLaunchKernelGGL((combine_kernel<64>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL((combine_kernel<128>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    case 256: hipLaunchKernelGGL((combine_kernel<256>), dim3(blocks), dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
