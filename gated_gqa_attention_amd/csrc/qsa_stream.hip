// qsa_stream.hip -- bf16 gated grouped-query attention for short query blocks
// (decode, speculative verify, ragged batched decode) on gfx950.
//
// stream_kernel: one workgroup = (sequence b, KV head g, key chunk).  Its rows
// are the G query heads of KV head g times the L new rows (DS4Server issue
// #113, Reproduction: query heads grouped within their KV group; Atlas
// Qwen35ForwardConfig: 16 query / 4 KV heads), at most 64, in order
// r = l * G + (h - g * G).
//
// Memory pipeline.  The chunk's cached keys stream through a ring of 64-key
// stages in LDS (64 KB for K and 64 KB for V at head_dim 256).  Stages are
// copied straight from HBM into LDS by global_load_lds_dwordx4 (no register
// staging); a stage's rows are XOR-swizzled in 16-byte units so that both the
// K operand reads (16 keys, one column) and the transposing V reads are free
// of bank conflicts.  While the first stages are in flight the workgroup
// splits q_gate, RMS-normalises and rotates its query rows (mlxd PR #99
// Summary and config audit table; Atlas FullAttentionLayer q_norm / k_norm,
// Qwen35ForwardConfig::rotary_dim), and the workgroup whose chunk ends the
// sequence normalises and rotates the new keys after the cached stages, keeps
// them in LDS as the last stage and appends them to the cache at the end (Atlas
// qwen3_5/mod.rs module doc: append at cache_pos, attend over cache_pos + 1 keys).
//
// Compute (the stage step in qsa_device.h).  Wavefront w scores keys
// 16 w .. 16 w + 15 of the stage against every row tile,
//   S^T[key][row] = K[key][:] . Q[row][:]            v_mfma_f32_16x16x32_bf16,
// the four wavefronts agree on each row's running max (log2 domain) through
// LDS and publish the stage's probabilities as one bf16 tile, and each
// wavefront then accumulates its own D/4 output dims over all keys of the stage,
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]   v_mfma_f32_16x16x32_bf16,
// with V^T read by gfx950's transposing LDS loads.  A chunk that covers the
// whole sequence applies the gate attn * sigmoid(gate) (mlxd PR #99 Summary)
// and stores bf16; otherwise it writes the chunk's (max, sum, unnormalised
// output) for the merge kernel.  The new keys become one more stage after the
// cached ones.
//
// Counters.  The copies are issued from inline assembly and waited for
// explicitly (s_waitcnt vmcnt with the number of younger copies): the compiler
// cannot count them, and any load it had to wait for after them would drain
// the whole ring.  So every small load the prologue needs lands before the
// first copy is issued, and later loads are consumed only after the stages.
#include "qsa_device.h"

namespace qsa {

namespace {

// RMS norm and partial rotation of one head row held by 16 lanes (E elements
// each, lane c16 holds elements E*c16 .. E*c16+E-1).  scr_row: this row's fp32
// scratch (D floats); cs: (cos, sin) of this row's position for pairs
// 0 .. r/2-1.  Every LDS read of a lane is issued before any is used.
template <int D>
__device__ __forceinline__ void norm_rope(float (&x)[D / 16], const float (&w)[D / 16], bool valid, float eps,
                                          int r, const float2 *cs, float *scr_row) {
  constexpr int E = D / 16;
  const int c16 = threadIdx.x & 15;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) ss += x[j] * x[j];
  ss = row16_sum(ss);
  const float inv = valid ? 1.0f / sqrtf(ss / (float)D + eps) : 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) x[j] = x[j] * inv * w[j];
  if (r == 0) return;
  const int half = r / 2;
#pragma unroll
  for (int j = 0; j < E; j += 4) *(float4 *)(scr_row + c16 * E + j) = make_float4(x[j], x[j + 1], x[j + 2], x[j + 3]);
  wave_lds_sync();
  if (c16 * E >= r) return;                             // no rotated element in this lane
  float xp[E], c[E], sn[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = c16 * E + j;
    const bool lo = e < half;
    xp[j] = scr_row[lo ? e + half : e - half];          // in range for every e < D
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = c16 * E + j;
    const int i = min(e < half ? e : e - half, half - 1);
    const float2 v = cs[i];
    c[j] = v.x;
    sn[j] = v.y;
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = c16 * E + j;
    const float lo_v = x[j] * c[j] - xp[j] * sn[j], hi_v = x[j] * c[j] + xp[j] * sn[j];
    x[j] = e < half ? lo_v : (e < r ? hi_v : x[j]);
  }
}

}  // namespace

// RTM: row tiles (16 rows each) of the workgroup, ceil(L * G / 16).
//
// The leading arguments are preloaded into SGPRs at wave launch, so the loads
// that need only them (sequence metadata, query rows, query norm weight,
// positions) are issued at once.  All of them are waited for before the first
// copy is issued: the vector-memory counter retires in order, and a load
// consumed after the copies would make its consumer wait for every copy.
// lgh packs L (bits 0-7), G (bits 8-15) and Hq (bits 16-31).
template <int D, int RTM>
__global__ __launch_bounds__(kThreads) void stream_kernel(const int32_t *__restrict__ seq_lens,
                                                          const int64_t *__restrict__ seq_offset,
                                                          const bf16_t *__restrict__ q_gate,
                                                          const bf16_t *__restrict__ wq_ptr,
                                                          const int32_t *__restrict__ positions, int nslot, int hkv,
                                                          int lgh, Params p) {
  using G = Geo<D>;
  constexpr int E = G::E, KST = G::KST, RB = G::RB, NS = G::NS, LPS = G::LPS, DBW = D / 64;
  constexpr int SCR = G::SCR > Xch::BYTES ? G::SCR : Xch::BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2 * G::RING];   // K ring | V ring
  unsigned char *const kring = ring, *const vring = ring + G::RING;
  __shared__ __attribute__((aligned(16))) float scr[SCR / 4];   // row scratch, then the stage exchange
  __shared__ __attribute__((aligned(16))) float2 tab[G::TAB_N];
  __shared__ int spos[kMaxFusedNewRows];
  unsigned char *const scrb = (unsigned char *)scr;

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int lane = t % kWave, g4 = lane >> 4, m16 = lane & 15;
  const int chunk = blockIdx.x / nslot, slot = blockIdx.x % nslot;
  const int b = slot / hkv, kvh = slot % hkv;
  const int L = lgh & 0xff, Gq = (lgh >> 8) & 0xff, Hq = lgh >> 16;
  const int R = L * Gq;

  // ------------------------------------------------------------ round trip 1: everything small
  const int n = seq_lens[b];
  const int64_t off = seq_offset[b];
  RawE<E> qraw[RTM];                                    // query half, row 16 rt + 4 wave + g4
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    const int r = min(16 * rt + 4 * wave + g4, R - 1);
    const int l = r / Gq, h = kvh * Gq + r % Gq;
    qraw[rt].load(q_gate + (((int64_t)b * L + l) * Hq + h) * 2 * D + E * m16);
  }
  RawE<E> wqraw;
  wqraw.load(wq_ptr + E * m16);
  const int tpos = positions[(int64_t)b * L + min(t, L - 1)];
  // arguments that live in memory, fetched in the same round trip
  const int ck = p.chunk_keys, msl = p.max_seq_len, rdim = p.r, pchunks = p.chunks, even = p.even_split;
  const int64_t nrows = p.num_rows;
  const bf16_t *const kc = (const bf16_t *)p.kc;
  const bf16_t *const vc = (const bf16_t *)p.vc;
  const bf16_t *const knew = (const bf16_t *)p.k_new;
  const double l2t = p.log2_theta;
  const float eps = p.eps, sl2 = p.scale_log2;
  __builtin_amdgcn_sched_barrier(0);                   // every load above is issued before any wait
  asm volatile("" ::"s"(n), "s"(off), "s"(ck), "s"(msl), "s"(rdim), "s"(pchunks), "s"(even), "s"(nrows), "s"(kc), "s"(vc),
               "s"(knew), "s"(l2t), "s"(eps), "s"(sl2));
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) qraw[rt].land();
  wqraw.land();
  asm volatile("" ::"v"(tpos));

  const int64_t total = (int64_t)n + L;
  const bool in_range = n >= 0 && off >= 0 && total <= msl && off + total <= nrows;
  // capacity only guards the writes at the end; its load is issued now so that
  // its round trip overlaps the stages
  const int32_t *const capp = p.capacity;
  const int cap = capp ? capp[b] : 0x7fffffff;
  const int64_t kend = total;
  const int nch = tile_chunk_count(kend, even, pchunks, ck);
  if (chunk >= nch) return;
  if (!in_range) {
    if (chunk == 0) {
      for (int e = t; e < R * D; e += kThreads) {
        const int r = e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
      if (t == 0) flag_error(p);
    }
    return;
  }
  const int64_t k0 = chunk_begin(kend, even, nch, ck, chunk);
  const int64_t k1 = chunk == nch - 1 ? kend : chunk_begin(kend, even, nch, ck, chunk + 1);
  const bool fuse_new = knew != nullptr;
  const bool tail = fuse_new && chunk == nch - 1;       // this workgroup holds the new keys
  const int64_t cend = fuse_new ? min(k1, (int64_t)n) : k1;   // cached keys [k0, cend)
  const int nst = cend > k0 ? (int)((cend - k0 + G::SK - 1) / G::SK) : 0;

  // ------------------------------------------------------------ ring fill
  const unsigned kring_lds = (unsigned)(uintptr_t)(lds_void *)kring;
  const unsigned vring_lds = (unsigned)(uintptr_t)(lds_void *)vring;
  // This thread's copies of a stage: key row u / OCT of the stage, and the
  // 16-byte unit that the swizzle puts at LDS position u % OCT of that row; the
  // source is addressed from the stage's first key (wave-uniform, in SGPRs)
  // plus a 32-bit lane offset shared by K and V.
  const unsigned rowb = (unsigned)(hkv * D * 2);       // bytes between consecutive keys of one KV head
  auto issue_half = [&](int st, bool is_k) {   // K or V of keys k0 + 64 st .. into ring slot st % NS
    const int64_t sk0 = k0 + (int64_t)G::SK * st;
    const int last = (int)min<int64_t>(G::SK - 1, cend - 1 - sk0);   // keys past the chunk repeat its last key
    const bf16_t *base = (is_k ? kc : vc) + ((off + sk0) * hkv + kvh) * D;
    const unsigned ring_lds = is_k ? kring_lds : vring_lds;
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int u = t + kThreads * i;
      const int key = u / G::OCT, pos = u % G::OCT, oct = pos ^ (key & G::SW);
      const unsigned voff = (unsigned)min(key, last) * rowb + 16u * (unsigned)oct;
      dma16_sbase(base, voff, ring_lds + (st % NS) * G::STAGE + kThreads * 16 * i + wave * 1024);
    }
  };
  auto issue_stage = [&](int st) {   // K and V of keys k0 + 64 st .. into ring slot st % NS, interleaved
    const int64_t sk0 = k0 + (int64_t)G::SK * st;
    const int last = (int)min<int64_t>(G::SK - 1, cend - 1 - sk0);
    const int64_t row = ((off + sk0) * hkv + kvh) * D;
    const bf16_t *kb = kc + row, *vb = vc + row;
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int u = t + kThreads * i;
      const int key = u / G::OCT, pos = u % G::OCT, oct = pos ^ (key & G::SW);
      const unsigned voff = (unsigned)min(key, last) * rowb + 16u * (unsigned)oct;
      const unsigned dst = (st % NS) * G::STAGE + kThreads * 16 * i + wave * 1024;
      dma16_sbase(kb, voff, kring_lds + dst);
      dma16_sbase(vb, voff, vring_lds + dst);
    }
  };
  // Whichever way a stage is issued, its 2 LPS copies stay contiguous in issue
  // order, so a stage is complete once at most 2 LPS copies per younger stage remain.
#pragma unroll
  for (int st = 0; st < NS; ++st)
    if (st < nst) issue_stage(st);

  // new keys and values (tail workgroup): consumed only after the key stages
  RawE<E> knraw, vnraw, wkraw;
  if (tail) {
    const int l = min(4 * wave + g4, L - 1);
    const int64_t src = (((int64_t)b * L + l) * hkv + kvh) * D + E * m16;
    knraw.load(knew + src);
    vnraw.load((const bf16_t *)p.v_new + src);
    wkraw.load((const bf16_t *)p.wk + E * m16);
  }

  // ------------------------------------------------------------ rotation table
  // L * r/2 <= TAB_N is a condition of this route
  const int half = rdim / 2;
  if (t < L) spos[t] = tpos;
  lds_barrier();
  for (int e = t; e < L * half; e += kThreads) {
    // theta^(-2i/r) = exp2(-(2i/r) log2 theta)
    const double inv = exp2(-2.0 * (double)(e % half) / (double)rdim * l2t);
    float c, s;
    rope_angle_cs(spos[e / half], inv, c, s);
    tab[e] = make_float2(c, s);
  }
  lds_barrier();

  // ------------------------------------------------------------ query rows -> MFMA operands
  float wq[E];
  wqraw.to_float(wq);
  bf16x8 qf[RTM][KST];
  int64_t lim[RTM];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) lim[rt] = (int64_t)n + (16 * rt + m16) / Gq;
  const int srow = 4 * wave + g4;                       // scratch row of this lane group
  auto prep_pass = [&](const int rt, const RawE<E> &raw) {
    const int r = 16 * rt + srow;
    const bool valid = r < R;
    const int l = min(r, R - 1) / Gq;
    float x[E];
    raw.to_float(x);
    norm_rope<D>(x, wq, valid, eps, rdim, tab + l * half, scr + srow * D);
    wave_lds_sync();
    // bf16 copy of the row into its own scratch row (stride 4D bytes, swizzled units)
    put_row_bf16<D>(scrb, 4 * D, srow, E * m16, x);
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) qf[rt][ks] = *(const bf16x8 *)(scrb + swz<G::SW>(m16, 4 * ks + g4, 4 * D));
    lds_barrier();
  };
  prep_pass(0, qraw[0]);
  if constexpr (RTM > 1) prep_pass(1, qraw[1]);
  if constexpr (RTM > 2) prep_pass(2, qraw[2]);
  if constexpr (RTM > 3) prep_pass(3, qraw[3]);

  // ------------------------------------------------------------ key stages
  f32x4 O[RTM][DBW];
  float mrun[RTM], lrun[RTM];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
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
    const int nk = (int)min<int64_t>(G::SK, cend - sk0);
    // the K half of the slot is refilled as soon as the scores are done, the V half after the stage
    attend_stage<D, RTM>(kring + so, vring + so, nk, sk0, qf, O, mrun, lrun, lim, sl2, scrb, [&]() {
      if (st + NS < nst) issue_half(st + NS, true);
    });
    lds_barrier();                                      // every wave is done with ring slot st % NS
    if (st + NS < nst) issue_half(st + NS, false);
  }

  // ------------------------------------------------------------ new keys (tail workgroup)
  // The new rows become one more stage in ring slot 0: K and V rows 0 .. 15
  // (rows >= L zero) and V rows 16 .. 31 zero (read by the value product).
  // The fp32 scratch of their norm sits in the K ring past slot 0.
  if (tail) {
    float wk[E], x[E], v[E];
    wkraw.to_float(wk);
    knraw.to_float(x);
    vnraw.to_float(v);
    const int l = srow;
    const bool valid = l < L;
    norm_rope<D>(x, wk, valid, eps, rdim, tab + min(l, L - 1) * half, (float *)(kring + G::STAGE) + srow * D);
    if (!valid) {
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = 0.f;
    }
    float zero[E];
#pragma unroll
    for (int j = 0; j < E; ++j) zero[j] = 0.f;
    put_row_bf16<D>(kring, RB, l, E * m16, x);
    put_row_bf16<D>(vring, RB, l, E * m16, v);          // v_new is bf16 already: exact
    put_row_bf16<D>(vring, RB, 16 + l, E * m16, zero);
    lds_barrier();
    attend_stage<D, RTM>(kring, vring, L, (int64_t)n, qf, O, mrun, lrun, lim, sl2, scrb);
  }

  // ------------------------------------------------------------ outputs
  // Every wavefront writes its own dims 16 (DBW wave + db) + 4 g4 .. + 3 of row
  // 16 rt + m16: the gated output when the chunk is the whole sequence, else
  // the chunk's unnormalised output and (max, sum) for the merge kernel.
  const bool cap_ok = total <= (int64_t)cap;
  const bool single = nch == 1;
  const int64_t slot_rows = ((int64_t)slot * pchunks + chunk) * p.rows;
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    const int r = 16 * rt + m16;
    if (r >= R) continue;
    const int l = r / Gq, h = kvh * Gq + r % Gq;
    const int64_t orow = ((int64_t)b * L + l) * Hq + h;
    if (single) {
      const float inv = 1.f / lrun[rt];
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const int d = 16 * (DBW * wave + db) + 4 * g4;
        RawE<4> zr;
        zr.load(q_gate + orow * 2 * D + D + d);
        float z[4];
        zr.to_float(z);
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o4[i] = (bf16_t)(cap_ok ? O[rt][db][i] * inv * sigmoid_f(z[i]) : __builtin_nanf(""));
        *(bf16x4 *)((bf16_t *)p.out + orow * D + d) = o4;
      }
    } else if (cap_ok) {
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const int d = 16 * (DBW * wave + db) + 4 * g4;
        *(float4 *)(p.part_o + (slot_rows + r) * D + d) = make_float4(O[rt][db][0], O[rt][db][1], O[rt][db][2], O[rt][db][3]);
      }
      if (wave == 0 && g4 == 0) *(float2 *)(p.part_ml + (slot_rows + r) * 2) = make_float2(mrun[rt], lrun[rt]);
    }
  }
  if (!cap_ok) {
    // the sequence's rows would pass its capacity: NaN outputs (written above when
    // the chunk is the whole sequence), no partials, no append, error bit set
    if (chunk == 0) {
      if (!single) {
        for (int e = t; e < R * D; e += kThreads) {
          const int r = e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
          ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
        }
      }
      if (t == 0) flag_error(p);
    }
    return;
  }

  // ------------------------------------------------------------ append the new rows to the cache
  if (tail) {
    for (int u = t; u < 16 * G::OCT; u += kThreads) {
      const int l = u / G::OCT, oct = u % G::OCT;
      if (l < L) {
        const int64_t dst = ((off + n + l) * hkv + kvh) * D + 8 * oct;
        *(uint4 *)((bf16_t *)p.kc + dst) = *(const uint4 *)(kring + swz<G::SW>(l, oct, RB));
        *(uint4 *)((bf16_t *)p.vc + dst) = *(const uint4 *)(vring + swz<G::SW>(l, oct, RB));
      }
    }
  }
}

template <int D, int RTM>
static void launch_stream_rt(const Params &p, hipStream_t s, const Timing &tm) {
  const int nslot = p.B * p.Hkv;
  const int64_t blocks = (int64_t)nslot * p.chunks;
  const int lgh = p.L | (p.G << 8) | (p.Hq << 16);
  launch_kernel(stream_kernel<D, RTM>, blocks, s, tm, p.seq_lens, p.seq_offset, (const bf16_t *)p.q_gate,
                (const bf16_t *)p.wq, p.positions, nslot, p.Hkv, lgh, p);
}

template <int D>
static hipError_t launch_stream_d(const Params &p, hipStream_t s, const Timing &tm) {
  switch ((p.rows + 15) / 16) {
    case 1: launch_stream_rt<D, 1>(p, s, tm); break;
    case 2: launch_stream_rt<D, 2>(p, s, tm); break;
    case 3: launch_stream_rt<D, 3>(p, s, tm); break;
    case 4: launch_stream_rt<D, 4>(p, s, tm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stream_bf16(const Params &p, hipStream_t s, const Timing &tm) {
  switch (p.D) {
    case 64: return launch_stream_d<64>(p, s, tm);
    case 128: return launch_stream_d<128>(p, s, tm);
    case 256: return launch_stream_d<256>(p, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
