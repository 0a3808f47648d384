// qsa_merge.hip -- merge of split-K partials (gfx950).
//
// The attention kernels cut the keys of a (sequence, KV head, row tile) into
// chunks when one workgroup per tile would leave the chip idle (flash-decoding
// split-K).  Each chunk leaves its running max (log2 domain), sum and
// unnormalised output; this kernel combines them with log-sum-exp weights and
// applies the output gate attn * sigmoid(gate) (mlxd PR #99 Summary; Atlas
// sigmoid_gate).  It runs after the attention kernel on the same stream, so
// the kernel boundary orders the partials' stores before these loads.
#include "qsa_device.h"

namespace qsa {

// Merge the key chunks of one (slot, row): weights 2^(m_c - M) / sum_c l_c 2^(m_c - M),
// weighted sum of the unnormalised chunk outputs, then the sigmoid gate.  For
// the short-query route (one row tile per sequence and KV head), whose rows can
// have thousands of chunks: one wavefront per (slot, row, 64-dim slice), with
// no LDS and no barrier; the slices spread the partials' bytes over D/64 times
// more CUs.  Chunks go in batches of 64: lane c holds chunk c's statistics and
// the batch max and sums are wavefront reductions.  Lane (q, c16) reads 16-byte
// pieces (dims 4 c16 .. + 3 of the slice) of chunks q, q + 4, ..., so a batch is
// 16 wide loads per lane; it fetches each of those chunks' weight from the lane
// holding its statistics, and the four lane groups are summed at the end.
//
// The leading arguments are preloaded into SGPRs, so the first batch's loads
// (taken for the grid's chunk count, before the sequence length is known) and
// the length itself form one round trip.  A sequence out of range has NaN
// statistics in chunk 0 (written by the attention kernel), so its merged rows
// are NaN.  lg packs L (bits 0-7), the row tiles per KV head, one or two (bits
// 8-15), and G (bits 16-31).
//
// ROT: the partials are in the Walsh-Hadamard basis (the Turbo8 cache's), so
// the merged row is rotated back (the iWHT(out) bookend) before the gate; the
// merge is linear, so rotating the merged row is rotating every chunk's.  Then
// one workgroup takes the D/64 slices of a row, one wavefront each, and the
// merged row goes through LDS to wavefront 0, which holds it whole (D/64
// dims per lane) for the rotation.
template <int D, bool ROT>
__global__ __launch_bounds__(ROT ? D : kWave) void combine_kernel(const int32_t *__restrict__ seq_lens,
                                                                  const float *__restrict__ part_ml,
                                                                  const float *__restrict__ part_o,
                                                                  const bf16_t *__restrict__ q_gate, int rows,
                                                                  int chunks, int hkv, int lg, Params p) {
  constexpr int NSL = D / kWave;                        // 64-dim slices per row
  constexpr int CPL = kWave / 4;                        // chunks per lane and batch
  // lane (q, c16) holds dims 4 c16 .. 4 c16 + 3 of the slice for chunks q, q + 4, ...
  const int lane = ROT ? threadIdx.x % kWave : threadIdx.x, q = lane >> 4, c16 = lane & 15;
  const int slice = ROT ? __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) : blockIdx.x % NSL;
  const int rowid = ROT ? blockIdx.x : blockIdx.x / NSL;
  const int d = kWave * slice + 4 * c16;
  const int L = lg & 0xff, two = ((lg >> 8) & 0xff) == 2 ? 1 : 0, G = lg >> 16, Hq = G * hkv;
  const int rr = rowid % rows;
  const int slot = rowid / rows;                        // (sequence, KV head, row tile)
  const int kvh = (unsigned)(slot >> two) % (unsigned)hkv, b = (unsigned)(slot >> two) / (unsigned)hkv;
  const int gr = (slot & two) * rows + rr;              // the row within the KV group
  const int l = gr / G, h = kvh * G + gr % G;
  if (gr >= L * G) return;
  const int64_t base = (int64_t)slot * chunks * rows + rr;   // + c * rows
  const int n = seq_lens[b];
  RawE<4> zr;
  zr.load(q_gate + (((int64_t)b * L + l) * Hq + h) * 2 * D + D + d);
  float2 ml = gld<float2>(part_ml + (base + (int64_t)min(lane, chunks - 1) * rows) * 2);
  float4 v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * j < chunks) v[j] = gld<float4>(part_o + (base + (int64_t)min(q + 4 * j, chunks - 1) * rows) * D + d);
  }
  __builtin_amdgcn_sched_barrier(0);                   // every load above is issued before any wait

  // chunks of this sequence (the grid's count at most, whatever the length says)
  const int nch = min(chunks, tile_chunk_count((int64_t)n + (L * G - 1) / G + 1, p.even_split, chunks, p.chunk_keys));
  if (nch == 1) return;                                 // finished by the attention kernel
  float M = -INFINITY, lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nch; c0 += kWave) {
    if (c0 > 0) {
      ml = gld<float2>(part_ml + (base + (int64_t)min(c0 + lane, nch - 1) * rows) * 2);
#pragma unroll
      for (int j = 0; j < CPL; ++j) v[j] = gld<float4>(part_o + (base + (int64_t)min(c0 + q + 4 * j, nch - 1) * rows) * D + d);
    }
    const bool own = c0 + lane < nch;                   // lane c holds chunk c0 + c's statistics
    const float mc = own ? ml.x : -INFINITY;
    const float Mn = fmaxf(M, rows4_max(row16_max(mc)));
    const float mu = Mn == -INFINITY ? 0.f : Mn;        // a chunk whose rows saw no key has m = -inf: weight 0
    const float alpha = __builtin_amdgcn_exp2f(M - mu);
    const float wc = own ? __builtin_amdgcn_exp2f(mc - mu) : 0.f;
    lsum = lsum * alpha + rows4_sum(row16_sum(wc * (own ? ml.y : 0.f)));
    acc.x *= alpha;
    acc.y *= alpha;
    acc.z *= alpha;
    acc.w *= alpha;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      // the weight of chunk c0 + q + 4 j, from the lane that holds its statistics;
      // chunks past the sequence's count were loaded at a clamped index (or, in the
      // first batch, before the count was known) and are left out by a select, not
      // by a zero weight, so that whatever an earlier call left there cannot reach
      // the sum (0 * inf is NaN)
      const float w = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (q + 4 * j), __float_as_int(wc)));
      if (c0 + q + 4 * j < nch) {
        acc.x += w * v[j].x;
        acc.y += w * v[j].y;
        acc.z += w * v[j].z;
        acc.w += w * v[j].w;
      }
    }
    M = Mn;
  }
  // the four lane groups hold disjoint chunk sets of the same dims
  acc.x = rows4_sum(acc.x);
  acc.y = rows4_sum(acc.y);
  acc.z = rows4_sum(acc.z);
  acc.w = rows4_sum(acc.w);
  if constexpr (ROT) {
    __shared__ __attribute__((aligned(16))) float mrow[D];
    if (q == 0) *(float4 *)(mrow + d) = acc;
    __syncthreads();
    if (slice == 0) {
      constexpr int EPL = D / kWave;                    // dims EPL lane .. + EPL - 1
      float x[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) x[j] = mrow[EPL * lane + j];
#pragma unroll
      for (int hb = 1; hb < EPL; hb <<= 1)
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (!(j & hb)) {
            const float a = x[j], c = x[j + hb];
            x[j] = a + c;
            x[j + hb] = a - c;
          }
#pragma unroll
      for (int lh = 1; lh < kWave; lh <<= 1) {
        const bool up = lane & lh;                      // this lane holds the second of each pair
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
          const float o = __shfl_xor(x[j], lh, kWave);
          x[j] = up ? o - x[j] : x[j] + o;
        }
      }
      const float norm = 1.0f / sqrtf((float)D);
#pragma unroll
      for (int j = 0; j < EPL; ++j) mrow[EPL * lane + j] = x[j] * norm;
    }
    __syncthreads();
    acc = *(const float4 *)(mrow + d);
  }
  if (q == 0) {
    float z[4];
    zr.to_float(z);
    const float inv = 1.f / lsum;
    bf16x4 o4;
    o4[0] = (bf16_t)(acc.x * inv * sigmoid_f(z[0]));
    o4[1] = (bf16_t)(acc.y * inv * sigmoid_f(z[1]));
    o4[2] = (bf16_t)(acc.z * inv * sigmoid_f(z[2]));
    o4[3] = (bf16_t)(acc.w * inv * sigmoid_f(z[3]));
    *(bf16x4 *)((bf16_t *)p.out + (((int64_t)b * L + l) * Hq + h) * D + d) = o4;
  }
}

// The tile route's merge: one wavefront per (slot, row), lane c holding dims
// EPL c .. + EPL - 1.  The pieces of a tile are the key ranges of its pair
// that hold its keys (pair_ranges): slots 0 .. of the pair for its first tile,
// .. 2 chunks for its second, as the attention kernel recorded them in tinfo.
// A piece's row holds (max, sum, scale) in fp32 and its output divided by the
// sum and the scale in fp16.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_rows_kernel(Params p) {
  constexpr int EPL = D / kWave;
  const int prows = p.rows, ptiles = p.tiles, hkv = p.Hkv, L = p.L, Gq = p.G, Hq = p.Hq, pch = p.chunks;
  const int msl = p.max_seq_len;
  const int64_t nrows = p.num_rows;
  const int32_t *const seq_lens = p.seq_lens, *const capp = p.capacity;
  const int64_t *const seq_offset = p.seq_offset;
  const bf16_t *const q_gate = (const bf16_t *)p.q_gate;
  const float *const part_ml = p.part_ml, *const part_o = p.part_o;
  bf16_t *const outp = (bf16_t *)p.out;
  asm volatile("" ::"s"(prows), "s"(ptiles), "s"(hkv), "s"(L), "s"(Gq), "s"(Hq), "s"(pch), "s"(msl),
               "s"(nrows), "s"(seq_lens), "s"(capp), "s"(seq_offset), "s"(q_gate), "s"(part_ml), "s"(part_o),
               "s"(outp));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  // (slot, row) pair; the planner keeps B L Hq below 2^31, so 32-bit unsigned
  // divisions (a few instructions, where 64-bit ones are a long sequence)
  const unsigned id = blockIdx.x * (unsigned)(kThreads / kWave) + (unsigned)wave;
  const unsigned nslots = (unsigned)p.B * (unsigned)hkv * (unsigned)ptiles;
  if (id >= nslots * (unsigned)prows) return;
  const int rr = (int)(id % (unsigned)prows);
  const unsigned slot = id / (unsigned)prows;
  const int tile = (int)(slot % (unsigned)ptiles);
  const int64_t bk = slot / (unsigned)ptiles;
  const int kvh = (int)((unsigned)bk % (unsigned)hkv);
  const int b = (int)((unsigned)bk / (unsigned)hkv);
  const int row0 = tile * prows;
  const int Rk = L * Gq, R = min(prows, Rk - row0);
  if (rr >= R) return;
  // the tile's pair (this merge runs with more than one chunk per tile)
  const int half = ptiles / 2, pair = min(tile, ptiles - 1 - tile);
  const bool second = tile > ptiles - 1 - tile;
  const int top = 2 * pch;                              // the pair's last slot
  const int64_t base = ((bk * (ptiles - half) + pair) * (top + 1)) * prows + rr;   // + slot * rows
  // Every load whose address does not wait on the sequence length goes out
  // first, in the round trip of the length itself: the gate and the
  // statistics and outputs of up to PF slots where the tile's pieces usually
  // are (slots 0 .. chunks - 1 of a first tile or a tile alone, chunks .. 2
  // chunks of a second; slots past those are clamped to the last, so no other
  // tile's partials are fetched, and any outside the tile's actual pieces are
  // read but not used).
  constexpr int PF = 4;
  const int g0 = second ? pch : 0, hi = second ? 2 * pch : pch - 1;
  const int info = p.tinfo[slot];                       // this tile's piece slots in the pair
  const int rg = row0 + rr, l = rg / Gq, h = kvh * Gq + rg % Gq;
  const bf16_t *zp = q_gate + (((int64_t)b * L + l) * Hq + h) * 2 * D + D + lane * EPL;
  float z[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) z[j] = (float)zp[j];
  // unconditional, at clamped (in-range) slots, and held in place by an empty
  // asm with a memory clobber, so that the compiler issues them all here
  // a piece's row: (max, sum, scale, 0) in part_ml and its output divided by
  // the sum and by the scale in fp16 in part_o, dim 16 db + 4 g + i at
  // 32 (db / 2) + 8 g + 4 (db % 2) + i (the attention kernel's store order);
  // this lane's EPL dims are contiguous there
  typedef _Float16 hE __attribute__((ext_vector_type(EPL)));
  const int d0 = lane * EPL, dpos = (d0 >> 5) * 32 + ((d0 >> 2) & 3) * 8 + ((d0 >> 4) & 1) * 4 + (d0 & 3);
  const _Float16 *const po16 = (const _Float16 *)part_o + dpos;
  f32x4 pml[PF];
  hE pv[PF];
#pragma unroll
  for (int c = 0; c < PF; ++c) {
    const int cc = min(g0 + c, hi);
    pml[c] = *(const f32x4 *)(part_ml + (base + (int64_t)cc * prows) * 4);
    pv[c] = *(const hE *)(po16 + (base + (int64_t)cc * prows) * D);
  }
  asm volatile("" ::: "memory");
  const int n = seq_lens[b];
  const int64_t off = seq_offset[b];
  const int cap = capp ? capp[b] : 0x7fffffff;
  const int64_t total = (int64_t)n + L;
  if (!(n >= 0 && off >= 0 && total <= msl && off + total <= nrows && total <= (int64_t)cap))
    return;                                             // the attention kernel wrote NaN
  const int first = info & 0xffff, last = info >> 16;   // the tile's pieces: slots first .. last
  if (first == last) return;                            // finished by the attention kernel
  auto fetched = [&](int c) { return c >= g0 && c < g0 + PF && c <= hi; };   // slot c is in registers
  auto held = [&](int j) { return g0 + j >= first && g0 + j <= last && fetched(g0 + j); };
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < PF; ++c)
    if (held(c)) M = fmaxf(M, pml[c][0]);
  for (int c = first; c <= last; ++c)
    if (!fetched(c)) M = fmaxf(M, part_ml[(base + (int64_t)c * prows) * 4]);
  // out = sum_c w_c l_c s_c x_c / sum_c w_c l_c, w_c = 2^(m_c - M)
  float lsum = 0.f, acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int c = 0; c < PF; ++c) {
    if (held(c)) {
      const float wl = exp2f(pml[c][0] - M) * pml[c][1];   // a piece whose rows saw no key has m = -inf: weight 0
      lsum += wl;
      const float f = wl * pml[c][2];
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[j] += f * (float)pv[c][j];
    }
  }
  for (int c = first; c <= last; ++c) {
    if (fetched(c)) continue;
    const f32x4 ml = *(const f32x4 *)(part_ml + (base + (int64_t)c * prows) * 4);
    const float wl = exp2f(ml[0] - M) * ml[1];
    lsum += wl;
    const float f = wl * ml[2];
    const hE x = *(const hE *)(po16 + (base + (int64_t)c * prows) * D);
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] += f * (float)x[j];
  }
  const float inv = 1.f / lsum;
  bf16_t *out = outp + (((int64_t)b * L + l) * Hq + h) * D + lane * EPL;
#pragma unroll
  for (int j = 0; j < EPL; ++j) out[j] = (bf16_t)(acc[j] * inv * sigmoid_f(z[j]));
}

hipError_t launch_combine_bf16(const Params &p, hipStream_t s, bool per_row) {
  if (per_row) {
    const int64_t pairs = (int64_t)p.B * p.Hkv * p.tiles * p.rows;
    const int64_t blocks = (pairs + kThreads / kWave - 1) / (kThreads / kWave);
    switch (p.D) {
      case 64: hipLaunchKernelGGL((combine_rows_kernel<64>), dim3(blocks), dim3(kThreads), 0, s, p); break;
      case 128: hipLaunchKernelGGL((combine_rows_kernel<128>), dim3(blocks), dim3(kThreads), 0, s, p); break;
      case 256: hipLaunchKernelGGL((combine_rows_kernel<256>), dim3(blocks), dim3(kThreads), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.tiles * p.rows * (p.D / kWave);   // tiles == 1 on this route
  const int lg = p.L | (p.tiles << 8) | (p.G << 16);
  const bf16_t *qg = (const bf16_t *)p.q_gate;
  switch (p.D) {
    case 64:
      hipLaunchKernelGGL((combine_kernel<64, false>), dim3(blocks), dim3(kWave), 0, s, p.seq_lens, p.part_ml, p.part_o,
                         qg, p.rows, p.chunks, p.Hkv, lg, p);
      break;
    case 128:
      hipLaunchKernelGGL((combine_kernel<128, false>), dim3(blocks), dim3(kWave), 0, s, p.seq_lens, p.part_ml,
                         p.part_o, qg, p.rows, p.chunks, p.Hkv, lg, p);
      break;
    case 256:
      hipLaunchKernelGGL((combine_kernel<256, false>), dim3(blocks), dim3(kWave), 0, s, p.seq_lens, p.part_ml,
                         p.part_o, qg, p.rows, p.chunks, p.Hkv, lg, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine_wht_bf16(const Params &p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.rows;
  const int lg = p.L | (p.tiles << 8) | (p.G << 16);
  const bf16_t *qg = (const bf16_t *)p.q_gate;
  switch (p.D) {
    case 64:
      hipLaunchKernelGGL((combine_kernel<64, true>), dim3(blocks), dim3(64), 0, s, p.seq_lens, p.part_ml, p.part_o, qg,
                         p.rows, p.chunks, p.Hkv, lg, p);
      break;
    case 128:
      hipLaunchKernelGGL((combine_kernel<128, true>), dim3(blocks), dim3(128), 0, s, p.seq_lens, p.part_ml, p.part_o,
                         qg, p.rows, p.chunks, p.Hkv, lg, p);
      break;
    case 256:
      hipLaunchKernelGGL((combine_kernel<256, true>), dim3(blocks), dim3(256), 0, s, p.seq_lens, p.part_ml, p.part_o,
                         qg, p.rows, p.chunks, p.Hkv, lg, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
