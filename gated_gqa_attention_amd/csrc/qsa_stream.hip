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
// of bank conflicts.  Two wavefronts issue the first stages while the other
// two split q_gate, RMS-normalise and rotate the query rows (mlxd PR #99
// Summary and config audit table; Atlas FullAttentionLayer q_norm / k_norm,
// Qwen35ForwardConfig::rotary_dim) and, in the workgroup whose chunk ends the
// sequence, the new keys.  Those are attended before the cached stages, from
// a free ring slot or (several row tiles) from the arena, by each wavefront on
// its own; a single new key only sets the running state.  With one row tile
// and no free slot they follow the cached stages instead.  A call that is
// given k_new appends them to the cache at the end (Atlas qwen3_5/mod.rs
// module doc: append at cache_pos, attend over cache_pos + 1 keys); a call on
// rows already appended loads them from the cache into the same place and
// attends them the same way, so the two compute bitwise the same outputs.
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
// output) for the merge kernel, with non-temporal stores.
//
// Counters.  The copies are issued from inline assembly and waited for
// explicitly (s_waitcnt vmcnt with the number of younger copies): the compiler
// cannot count them, and any load it had to wait for after them would drain
// the whole ring.  So the wavefronts that issue the first stages load nothing
// but the sequence metadata before them, and later loads are consumed only
// after the stages.
#include "qsa_device.h"

namespace qsa {

// RTM: row tiles (16 rows each) of the workgroup, ceil(L * G / 16) <= 3.
//
// Two roles until the first stage.  Wavefronts 0-1 (the copy waves) load only
// the sequence metadata, then issue the K and V copies of the first stages;
// the memory system accepts copies at the rate it delivers, so those waves are
// held at the issue for most of the transfer.  A wave's vector-memory counter
// retires in order, so no wave consumes a load issued after its own copies:
// its consumer would wait for every copy.  Wavefronts 2-3 (the prep waves)
// issue no copy before the stages: they land all their own loads,
// each builds its own (cos, sin) table, the two normalise and rotate all query
// rows into bf16 MFMA operands in LDS, and, in the workgroup that holds the new
// keys, normalise and rotate those too.  Then all four wavefronts meet, take
// their query operands and run the stages together; refills of the ring are
// shared by all four.
// lgh packs L (bits 0-7), G (bits 8-15), r/2 (bits 16-23) and the rows of a row
// tile (bits 24-31).  nslot: sequences x KV heads.  PAGED: the
// cache rows go through a block table.
template <int D, int RTM, bool PAGED>
__global__ __launch_bounds__(kThreads) void stream_kernel(const int32_t *__restrict__ seq_lens,
                                                          const int64_t *__restrict__ seq_offset,
                                                          const bf16_t *__restrict__ q_gate,
                                                          const bf16_t *__restrict__ wq_ptr,
                                                          const int32_t *__restrict__ positions, int nslot, int hkv,
                                                          int lgh, Params p) {
  using G = Geo<D>;
  constexpr int E = G::E, KST = G::KST, RB = G::RB, NS = G::NS, LPS = G::LPS, DBW = D / 64;
  constexpr int QBYTES = 16 * RTM * RB;                 // prepared query rows, bf16, swizzled
  constexpr int TABN = kMaxFusedTable;                  // (cos, sin) entries per table copy
  constexpr int PREP = QBYTES + 2 * TABN * 8;
  // With several row tiles and no free ring slot, the new rows sit in the
  // arena after the stage exchange: V rows 0 .. 15 at NEWOFF, K rows 0 .. 15
  // right after them.  With one row tile they follow the cached stages in ring
  // slot 0 (a larger arena measured slower for decode).
  constexpr bool ARENA_NEW = RTM > 1;
  constexpr int NEWOFF = Xch::BYTES, NEWB = NEWOFF + 32 * RB;
  constexpr int ARENA = ARENA_NEW ? (PREP > NEWB ? PREP : NEWB) : (PREP > Xch::BYTES ? PREP : Xch::BYTES);
  static_assert(Xch::BYTES % 16 == 0, "arena layout");
  constexpr int NPASS = 2 * RTM;                        // query row passes per prep wave (8 rows each)
  static_assert(RTM <= 3, "query rows of the short-query route");
  __shared__ __attribute__((aligned(16))) unsigned char ring[2 * G::RING];   // K ring | V ring
  unsigned char *const kring = ring, *const vring = ring + G::RING;
  // query operands and the two (cos, sin) tables, then the stage exchange
  __shared__ __attribute__((aligned(16))) unsigned char arena[ARENA];

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int lane = t % kWave, g4 = lane >> 4, m16 = lane & 15;
  const bool copier = wave < 2;
  const int pw = wave - 2;                              // prep wave index (prep waves)
  const int L = lgh & 0xff, Gq = (lgh >> 8) & 0xff, half = (lgh >> 16) & 0xff, Hq = Gq * hkv;
  // Row tiles: a KV group's 33 .. 48 rows go in two tiles of 17 .. 24 rows (two
  // row tiles of 16), fewer rows in one.  Work item (chunk, sequence, KV head)
  // and row tile: the two tiles of one item run on one XCD (block i runs on XCD
  // i mod 8), one after the other in its order, so the second reads the item's
  // keys from that XCD's L2.  No division on the way to the first loads.
  const int trows = (unsigned)lgh >> 24;
  int tiles = 1, tile = 0, item = blockIdx.x;
  if constexpr (RTM == 2) {
    tiles = L * Gq > trows ? 2 : 1;
    const int xj = blockIdx.x / 8;
    tile = tiles == 2 ? xj & 1 : 0;
    item = 8 * (tiles == 2 ? xj >> 1 : xj) + blockIdx.x % 8;
  }
  // items past the grid's (padding) have chunk >= the chunk count, and return
  // with the chunks past a sequence's end
  const int chunk = (unsigned)item / (unsigned)nslot, bk = (unsigned)item % (unsigned)nslot;
  const int b = (unsigned)bk / (unsigned)hkv, kvh = (unsigned)bk % (unsigned)hkv, slot = bk * tiles + tile;
  constexpr bool paged = PAGED;                         // rows through a block table (seq_offset not read)
  // this workgroup's rows: row0 .. row0 + R - 1 of the KV group's L * G rows
  const int row0 = tile * trows, R = min(trows, L * Gq - row0);

  // ------------------------------------------------------------ round trip 1
  const int n = seq_lens[b];
  const int64_t off = paged ? 0 : seq_offset[b];
  const int ck = p.chunk_keys, msl = p.max_seq_len, pchunks = p.chunks, even = p.even_split;
  const int64_t nrows = p.num_rows;
  const bf16_t *const kc = (const bf16_t *)p.kc;
  const bf16_t *const vc = (const bf16_t *)p.vc;
  const bf16_t *const knew = (const bf16_t *)p.k_new;
  const bf16_t *const vnew = (const bf16_t *)p.v_new;
  const bf16_t *const wkp = (const bf16_t *)p.wk;
  const float eps = p.eps, sl2 = p.scale_log2;
  // prep waves: query rows 8 k + 4 pw + g4 of pass k, the norm weight, and the
  // position of table entries lane + 64 j; none of these addresses waits on an
  // argument loaded from memory
  RawE<E> qraw[NPASS], wqraw, knraw[2], vnraw[2], wkraw;
  constexpr int TJ = TABN / kWave;
  int tpos[TJ], tpair[TJ];
  if (!copier) {
#pragma unroll
    for (int k = 0; k < NPASS; ++k) {
      const int r = row0 + min(8 * k + 4 * pw + g4, R - 1);
      const int l = r / Gq, h = kvh * Gq + r % Gq;
      qraw[k].load(q_gate + (((int64_t)b * L + l) * Hq + h) * 2 * D + E * m16);
    }
    wqraw.load(wq_ptr + E * m16);
    // unconditional, with clamped (in-range) indices, so that every load is in
    // flight at once; entries past L * r/2 are not used
    const int hh = max(half, 1);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int e = lane + kWave * j, q = e / hh;
      tpos[j] = positions[(int64_t)b * L + min(q, L - 1)];
      tpair[j] = e - q * hh;
    }
    __builtin_amdgcn_sched_barrier(0);                 // every load above is issued before any wait
  }

  // The new-key pointers, which the workgroup holding the new keys loads from
  // before its copies, are used here so that their loads from the argument
  // segment are issued with the sequence length, not one round trip after it.
  asm volatile("" ::"s"(knew), "s"(vnew), "s"(wkp));
  const int64_t total = (int64_t)n + L;
  const int bsl = p.bs_log2, mblk = p.max_blocks;
  const bool in_range = n >= 0 && total <= msl &&
                        (paged ? total <= ((int64_t)mblk << bsl) : off >= 0 && off + total <= nrows);
  const int64_t kend = total;
  const int nch = tile_chunk_count(kend, even, pchunks, ck);
  if (chunk >= nch) return;
  if (!in_range) {
    // NaN outputs, and NaN chunk statistics for the merge kernel, which then
    // writes NaN too; no append; error bit set
    if (chunk == 0) {
      for (int e = t; e < R * D; e += kThreads) {
        const int r = row0 + e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
      if (p.part_ml && t < R)
        *(float2 *)(p.part_ml + ((int64_t)slot * pchunks * trows + t) * 2) =
            make_float2(__builtin_nanf(""), __builtin_nanf(""));
      if (t == 0) flag_error(p);
    }
    return;
  }
  const int64_t k0 = chunk_begin(kend, even, nch, ck, chunk);
  const int64_t k1 = chunk == nch - 1 ? kend : chunk_begin(kend, even, nch, ck, chunk + 1);
  // The new keys n .. n + L - 1 are attended by the last chunk's workgroup,
  // the same way whether this call appends them (k_new given) or they are
  // already in the cache: then its prep waves load the stored rows instead of
  // normalising and rotating k_new, and the call computes bitwise what it
  // computes when it appends them itself.
  const bool fuse_new = knew != nullptr;
  const bool tail = chunk == nch - 1;                   // this workgroup holds the new keys
  const int64_t cend = min(k1, (int64_t)n);             // cached keys [k0, cend)
  const int nst = cend > k0 ? (int)((cend - k0 + G::SK - 1) / G::SK) : 0;

  // Paged caches: the physical block of each logical block of this chunk's keys
  // [k0, k1) (its new rows too), block blk0 + i in lane i of bid0 (i < 64) or
  // of bid1 (i >= 64); the host keeps a chunk within 128 blocks.  A block id
  // outside the allocated rows makes this chunk's result NaN (its output, or
  // its statistics for the merge kernel) and nothing is read or written there.
  int bid0 = 0, bid1 = 0, blk0 = 0;
  if constexpr (PAGED) {
    const int32_t *const trow = p.btab + (int64_t)b * mblk;
    blk0 = (int)(k0 >> bsl);
    const int nblk = (int)(((max(k1, k0 + 1) - 1) >> bsl) - blk0 + 1);
    bid0 = trow[min(blk0 + lane, mblk - 1)];
    bid1 = trow[min(blk0 + kWave + lane, mblk - 1)];
    const int64_t nphys = nrows >> bsl;
    const bool bad = (lane < nblk && (bid0 < 0 || bid0 >= nphys)) ||
                     (lane + kWave < nblk && (bid1 < 0 || bid1 >= nphys));
    if (__any(bad)) {
      if (nch == 1) {
        for (int e = t; e < R * D; e += kThreads) {
          const int r = row0 + e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
          ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
        }
      } else if (t < R) {
        *(float2 *)(p.part_ml + (((int64_t)slot * pchunks + chunk) * trows + t) * 2) =
            make_float2(__builtin_nanf(""), __builtin_nanf(""));
      }
      if (t == 0) flag_error(p);
      return;
    }
  }
  // row of key tk (per lane) of this chunk in a paged cache
  auto paged_row = [&](int64_t tk) {
    const int i = (int)(tk >> bsl) - blk0;
    const int a0 = __builtin_amdgcn_ds_bpermute(4 * (i & (kWave - 1)), bid0);
    const int a1 = __builtin_amdgcn_ds_bpermute(4 * (i & (kWave - 1)), bid1);
    return ((int64_t)(i < kWave ? a0 : a1) << bsl) + (tk & ((1 << bsl) - 1));
  };

  // ------------------------------------------------------------ ring fill
  const unsigned kring_lds = (unsigned)(uintptr_t)(lds_void *)kring;
  const unsigned vring_lds = (unsigned)(uintptr_t)(lds_void *)vring;
  // A copy of unit u of a stage: key row u / OCT of the stage, and the 16-byte
  // unit that the swizzle puts at LDS position u % OCT of that row; the source
  // is addressed from the stage's first key (wave-uniform, in SGPRs) plus a
  // 32-bit lane offset shared by K and V.
  const unsigned rowb = (unsigned)(hkv * D * 2);       // bytes between consecutive keys of one KV head
  // ub: the wave's first unit (wave-uniform); the lane copies unit ub + lane.
  // In a paged cache the rows of one stage need not be contiguous: each lane
  // then addresses its own row (64-bit), and base is the tensor's.
  auto copy_unit = [&](const bf16_t *base, unsigned ring_lds, int st, int ub, int last) {
    const int u = ub + lane;
    const int key = u / G::OCT, pos = u % G::OCT, oct = pos ^ (key & G::SW);
    const unsigned lds = ring_lds + (st % NS) * G::STAGE + 16 * ub;
    if constexpr (PAGED) {
      // blocks hold at least one stage, so the stage's keys lie in its first
      // block or the next one: both ids by uniform lane reads, a select per lane
      const int64_t ts = k0 + (int64_t)G::SK * st, tk = ts + min(key, last);
      const int i0 = (int)(ts >> bsl) - blk0, i1 = i0 + 1;
      const int blo = __builtin_amdgcn_readlane(i0 < kWave ? bid0 : bid1, i0 & (kWave - 1));
      const int bhi = __builtin_amdgcn_readlane(i1 < kWave ? bid0 : bid1, i1 & (kWave - 1));
      const int64_t blk = (tk >> bsl) == (ts >> bsl) ? blo : bhi;
      const int64_t row = (blk << bsl) + (tk & ((1 << bsl) - 1));
      dma16_vaddr(base + (row * hkv + kvh) * D + 8 * oct, lds);
    } else {
      dma16_sbase(base, (unsigned)min(key, last) * rowb + 16u * (unsigned)oct, lds);
    }
  };
  auto stage_src = [&](int st, bool is_k) {
    if constexpr (PAGED) return is_k ? kc : vc;
    return (is_k ? kc : vc) + ((off + k0 + (int64_t)G::SK * st) * hkv + kvh) * D;
  };
  auto stage_last = [&](int st) {   // keys past the chunk repeat its last key
    return (int)min<int64_t>(G::SK - 1, cend - 1 - (k0 + (int64_t)G::SK * st));
  };
  // refills: K or V of stage st, 2 LPS units per thread over all four waves
  auto issue_half = [&](int st, bool is_k) {
    const int last = stage_last(st);
    const bf16_t *base = stage_src(st, is_k);
#pragma unroll
    for (int i = 0; i < LPS; ++i) copy_unit(base, is_k ? kring_lds : vring_lds, st, kWave * wave + kThreads * i, last);
  };
  // The first stages: the copy waves issue both halves of each, in stage
  // order, so the copies younger than a stage of the first fill are 4 LPS per
  // thread per later stage in a copy wave (K and V) and none in a prep wave.
  auto issue_first_half = [&](int st, bool is_k, int w2) {
    const int last = stage_last(st);
    const bf16_t *base = stage_src(st, is_k);
#pragma unroll
    for (int i = 0; i < 2 * LPS; ++i)
      copy_unit(base, is_k ? kring_lds : vring_lds, st, kWave * w2 + (kThreads / 2) * i, last);
  };
  // The new keys become one more stage.  When the cached stages leave a ring
  // slot unused, the new keys take it and are attended first, while the cached
  // stages are still in flight; otherwise, with several row tiles, they are put
  // in the arena once every wave has its query operands and attended first all
  // the same, and with one row tile they follow the cached stages in slot 0.
  const bool early_new = tail && nst < NS;
  const int new_slot = (early_new ? nst : 0) * G::STAGE;
  const int nr = 4 * (pw ^ 1) + g4;
  // New key and value rows 8 k + nr of the tail workgroup (prep waves).  They
  // go to the other prep wave than query rows 8 k + 4 pw + g4, so that with
  // few rows (decode: one query group, one new row) each prep wave has one pass.
  // Their pointers come from the argument segment, so they are a second round
  // trip; they are issued before any copy of the workgroup (the barrier below),
  // since a load behind the copies in the CU's memory pipeline lands only after
  // them.  No copy of the prep waves precedes their consumer, the key preparation.
  if (!copier && tail) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = min(8 * k + nr, L - 1);
      if (fuse_new) {
        const int64_t src = (((int64_t)b * L + l) * hkv + kvh) * D + E * m16;
        knraw[k].load(knew + src);
        vnraw[k].load(vnew + src);
      } else {                                          // rows n + l of the cache (in range: checked above)
        const int64_t row = paged ? paged_row((int64_t)n + l) : off + n + l;
        const int64_t src = (row * hkv + kvh) * D + E * m16;
        knraw[k].load(kc + src);
        vnraw[k].load(vc + src);
      }
    }
    if (fuse_new) wkraw.load(wkp + E * m16);
  }
  lds_barrier();
  // passes of prep wave w (rows 8 k + 4 w .. + 3 of pass k) that hold a query row
  auto passes = [&](int w) { return min(NPASS, (R - 4 * w + 7) / 8); };
  if (copier) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st < nst) {
        issue_first_half(st, true, wave);
        issue_first_half(st, false, wave);
      }
    }
    // The query rows of the passes that hold none (all >= R) are zero: the copy
    // waves write them while their copies are in flight, so the prep waves only
    // take the passes with rows to prepare.
    const int z0 = 4 * (NPASS - passes(0)), zrows = z0 + 4 * (NPASS - passes(1));
    for (int u = t; u < zrows * G::OCT; u += 2 * kWave) {
      const int i = u / G::OCT, w = i < z0 ? 0 : 1, j = i < z0 ? i : i - z0;
      const int row = 8 * (passes(w) + j / 4) + 4 * w + j % 4;
      *(uint4 *)(arena + row * RB + 16 * (u % G::OCT)) = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // capacity only guards the writes at the end; its pointer comes from the
  // argument segment, so it is loaded behind the copies, and as a vector load
  // (its index is a lane value, an opaque zero), which lands after them and is
  // awaited only at the outputs: a scalar load would hold up the next barrier,
  // which waits for every outstanding scalar and LDS operation
  const int32_t *const capp = p.capacity;
  int cap = 0x7fffffff;
  if (capp) {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    cap = gld<int>(capp + b + z);
  }

  // ------------------------------------------------------------ prep waves
  float2 *const tabw = (float2 *)(arena + QBYTES) + (copier ? 0 : pw) * TABN;
  float kx[2][E];                                       // new key rows 8 k + nr (prep waves)
  // The new rows, written by the prep waves: K and V rows 0 .. 15 (rows >= L
  // zero), into ring slot new_slot or into the arena.
  unsigned char *const nkb = early_new || !ARENA_NEW ? kring + new_slot : arena + NEWOFF + 16 * RB;
  unsigned char *const nvb = early_new || !ARENA_NEW ? vring + new_slot : arena + NEWOFF;
  // A single new key is read only from row 0 (its score and its value row set
  // the state directly); otherwise rows L .. 15 are zero for the products.
  auto put_new_rows = [&]() {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int l = 8 * k + nr;
      if (L == 1 && early_new && l > 0) continue;
      float v[E];
      vnraw[k].to_float(v);
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (l >= L) v[j] = 0.f;
      put_row_bf16<D>(nkb, RB, l, E * m16, kx[k]);
      put_row_bf16<D>(nvb, RB, l, E * m16, v);        // v_new is bf16 already: exact
    }
  };
  if (!copier) {
    // every load of this wave lands before its copies are issued
#pragma unroll
    for (int k = 0; k < NPASS; ++k) qraw[k].land();
    wqraw.land();
#pragma unroll
    for (int j = 0; j < TJ; ++j) asm volatile("" ::"v"(tpos[j]));
    // this wave's (cos, sin) table: entry l * r/2 + i for new row l, pair i
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
    float wq[E];
    wqraw.to_float(wq);
    // The raw rows wait in their LDS slots and one loop (not unrolled: its code
    // stays in the instruction cache from the first pass on) prepares them in place.
    const int npass = passes(pw);                       // later passes' rows are zero (the copy waves')
#pragma unroll
    for (int k = 0; k < NPASS; ++k)
      if (k < npass) qraw[k].template store_lds<G::SW>(arena, RB, 8 * k + 4 * pw + g4, E * m16);
#pragma unroll 1
    for (int k = 0; k < npass; ++k) {
      const int r = 8 * k + 4 * pw + g4;
      float x[E];
      RawE<E> raw;
      raw.template load_lds<G::SW>(arena, RB, r, E * m16);
      raw.to_float(x);
      norm_rope<D>(x, wq, r < R, eps, 2 * half, tabw + ((row0 + min(r, R - 1)) / Gq) * half);   // rows >= R become zero
      put_row_bf16<D>(arena, RB, r, E * m16, x);
    }
    if (tail) {
      float wk[E];
      if (fuse_new) wkraw.to_float(wk);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int l = 8 * k + nr;
        if (8 * k + 4 * (pw ^ 1) < L) {                 // the pass holds a new row (wave-uniform)
          knraw[k].to_float(kx[k]);
          if (fuse_new) {
            norm_rope<D>(kx[k], wk, l < L, eps, 2 * half, tabw + min(l, L - 1) * half);   // rows >= L become zero
          } else if (l >= L) {
#pragma unroll
            for (int j = 0; j < E; ++j) kx[k][j] = 0.f;
          }
        } else {
#pragma unroll
          for (int j = 0; j < E; ++j) kx[k][j] = 0.f;
        }
      }
    }
    if (early_new) put_new_rows();
  }
  lds_barrier();                                        // query operands ready; first stages issued

  // ------------------------------------------------------------ query rows -> MFMA operands
  bf16x8 qf[RTM][KST];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt)
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) qf[rt][ks] = *(const bf16x8 *)(arena + swz<G::SW>(16 * rt + m16, 4 * ks + g4, RB));
  // key positions and causal limits fit in 32 bits: n + L <= max_seq_len <= 2^30
  int lim[RTM];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) lim[rt] = n + (row0 + 16 * rt + m16) / Gq;

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
  // The new keys are attended first, while the cached stages are in flight:
  // from the free ring slot, where the prep waves put them before the barrier
  // above, or from the arena, once every wave has its query operands.
  if (early_new && L == 1) {
    // One new key, visible to every row: attending it leaves each row's
    // reference max at its score, its sum at 1 (P = 2^0) and its output at the
    // value row.  Each wavefront sets that state itself from the rows in the
    // free slot (written before the barrier above): the same MFMA score as a
    // stage, with no exchange.
#pragma unroll
    for (int rt = 0; rt < RTM; ++rt) {
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
        S = mfma_qk(*(const bf16x8 *)(nkb + swz<G::SW>(m16, 4 * ks + g4, RB)), qf[rt][ks], S);
      mrun[rt] = rows4_max(g4 == 0 ? S[0] * sl2 : -INFINITY);   // key 0 sits in lane group 0
      lrun[rt] = 1.f;
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const int d = 16 * (DBW * wave + db) + 4 * g4;
        const bf16x4 v4 = *(const bf16x4 *)(nvb + swz<G::SW>(0, d / 8, RB) + 2 * (d % 8));
        O[rt][db] = f32x4{(float)v4[0], (float)v4[1], (float)v4[2], (float)v4[3]};
      }
    }
  } else if (tail && (early_new || ARENA_NEW)) {
    if (!early_new) {
      lds_barrier();                                    // every wave has its query operands (the new rows reuse the arena)
      if (!copier) put_new_rows();
      lds_barrier();
    }
    attend_new_rows<D, RTM>(nkb, nvb, L, n, qf, O, mrun, lrun, lim, sl2);
  }
  for (int st = 0; st < nst; ++st) {
    // copies younger than stage st that this wave issued: of the ys later
    // stages in flight, f are of the first fill (4 LPS per thread in a copy
    // wave, K and V halves; none in a prep wave) and ys - f are refills (2 LPS
    // per thread in every wave)
    const int ys = min(NS - 1, nst - 1 - st);
    const int f = max(0, min(NS, nst) - 1 - st);
    WaitUnits<LPS, 4 * (NS - 1)>::run(copier ? 2 * (ys + f) : 2 * (ys - f));
    lds_barrier();
    const int so = (st % NS) * G::STAGE;
    const int sk0 = (int)k0 + G::SK * st;
    const int nk = min(G::SK, (int)cend - sk0);
    // the K half of the slot is refilled as soon as the scores are done, the V half after the stage
    attend_stage<D, RTM>(kring + so, vring + so, nk, sk0, qf, O, mrun, lrun, lim, sl2, arena, [&]() {
      if (st + NS < nst) issue_half(st + NS, true);
    });
    lds_barrier();                                      // every wave is done with ring slot st % NS
    if (st + NS < nst) issue_half(st + NS, false);
  }

  // ------------------------------------------------------------ new keys, one row tile, no free slot
  // The new rows become one more stage in ring slot 0: K and V rows 0 .. 15
  // (rows >= L zero) from the prep waves, V rows 16 .. 31 zero (read by the
  // value product) from the copy waves.
  if (!ARENA_NEW && tail && !early_new) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float v[E];
      if (!copier) {
        const int l = 8 * k + nr;
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = 0.f;
        vnraw[k].to_float(v);
        if (l >= L) {
#pragma unroll
          for (int j = 0; j < E; ++j) v[j] = 0.f;
        }
        put_row_bf16<D>(kring, RB, l, E * m16, kx[k]);
        put_row_bf16<D>(vring, RB, l, E * m16, v);      // v_new is bf16 already: exact
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = 0.f;
        put_row_bf16<D>(vring, RB, 16 + 8 * k + 4 * wave + g4, E * m16, v);
      }
    }
    lds_barrier();
    attend_stage<D, RTM>(kring, vring, L, n, qf, O, mrun, lrun, lim, sl2, arena);
  }

  // ------------------------------------------------------------ outputs
  // Every wavefront writes its own dims 16 (DBW wave + db) + 4 g4 .. + 3 of row
  // 16 rt + m16: the gated output when the chunk is the whole sequence, else
  // the chunk's unnormalised output and (max, sum) for the merge kernel.
  asm volatile("" : "+v"(cap));                       // consumed only here, after every stage
  const bool cap_ok = total <= (int64_t)cap;
  const bool single = nch == 1;
  const int64_t slot_rows = ((int64_t)slot * pchunks + chunk) * trows;
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    const int r = 16 * rt + m16;
    if (r >= R) continue;
    const int l = (row0 + r) / Gq, h = kvh * Gq + (row0 + r) % Gq;
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
        f32x4 *const dst = (f32x4 *)(p.part_o + (slot_rows + r) * D + d);
        // one row tile's partials (4 KB per workgroup at head_dim 256) stay in the
        // caches for the merge kernel; several tiles' are written past them (faster)
        if constexpr (RTM == 1) *dst = O[rt][db]; else __builtin_nontemporal_store(O[rt][db], dst);
      }
      if (wave == 0 && g4 == 0) *(float2 *)(p.part_ml + (slot_rows + r) * 2) = make_float2(mrun[rt], lrun[rt]);
    }
  }
  if (!cap_ok) {
    // the sequence's rows would pass its capacity: NaN outputs (written above when
    // the chunk is the whole sequence), NaN chunk statistics in place of the
    // partials (so the merge kernel writes NaN too), no append, error bit set
    if (chunk == 0) {
      if (!single) {
        for (int e = t; e < R * D; e += kThreads) {
          const int r = row0 + e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
          ((bf16_t *)p.out)[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
        }
        if (t < R) *(float2 *)(p.part_ml + (slot_rows + t) * 2) = make_float2(__builtin_nanf(""), __builtin_nanf(""));
      }
      if (t == 0) flag_error(p);
    }
    return;
  }

  // ------------------------------------------------------------ append the new rows to the cache
  // (the workgroup holding the new keys in every row tile prepares and
  // attends them; the first tile's stores them)
  if (tail && fuse_new && tile == 0) {
    for (int u = t; u < 16 * G::OCT; u += kThreads) {
      const int l = u / G::OCT, oct = u % G::OCT;
      const int64_t row = paged ? paged_row((int64_t)n + min(l, L - 1)) : off + n + l;
      if (l < L) {
        const int64_t dst = (row * hkv + kvh) * D + 8 * oct;
        *(uint4 *)((bf16_t *)p.kc + dst) = *(const uint4 *)(nkb + swz<G::SW>(l, oct, RB));
        *(uint4 *)((bf16_t *)p.vc + dst) = *(const uint4 *)(nvb + swz<G::SW>(l, oct, RB));
      }
    }
  }
}

template <int D, int RTM, bool PAGED>
static void launch_stream_rt(const Params &p, hipStream_t s, const Timing &tm) {
  const int nslot = p.B * p.Hkv;
  const int64_t items = (int64_t)nslot * p.chunks;
  const int64_t blocks = (items + 7) / 8 * 8 * p.tiles;   // items in groups of 8 (one per XCD), times the row tiles
  const int lgh = p.L | (p.G << 8) | ((p.r / 2) << 16) | (p.rows << 24);
  launch_kernel(stream_kernel<D, RTM, PAGED>, blocks, s, tm, p.seq_lens, p.seq_offset, (const bf16_t *)p.q_gate,
                (const bf16_t *)p.wq, p.positions, nslot, p.Hkv, lgh, p);
}

template <int D, bool PAGED>
static hipError_t launch_stream_dp(const Params &p, hipStream_t s, const Timing &tm) {
  switch ((p.rows + 15) / 16) {
    case 1: launch_stream_rt<D, 1, PAGED>(p, s, tm); break;
    case 2: launch_stream_rt<D, 2, PAGED>(p, s, tm); break;
    case 3: launch_stream_rt<D, 3, PAGED>(p, s, tm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_stream_d(const Params &p, hipStream_t s, const Timing &tm) {
  return p.btab ? launch_stream_dp<D, true>(p, s, tm) : launch_stream_dp<D, false>(p, s, tm);
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
