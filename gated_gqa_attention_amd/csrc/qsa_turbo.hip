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
// bookend: (H q).(H k) = q.k) and rounded to fp16 MFMA operands.  Each 64-key
// stage's codes and scales are loaded into registers (the next stage's while
// the current one is attended), decoded to codes x scales (12 significant bits,
// which fp16's 11 keep better than bf16's 8), rounded to fp16 and written into
// the same swizzled LDS tiles as the bf16 kernel's copies, so the stage step is
// the bf16 kernel's (attend_stage), on fp16 MFMAs.  The workgroup holding the
// sequence's end quantizes the new rows as the append does (when k_new is
// given: and stores them), decodes them and attends them as a last stage.  At
// the end the accumulated rows, still in the rotated basis, go through LDS and
// are rotated back (the iWHT(out) bookend) before the gate (a whole sequence
// in one chunk) or before they are stored as the chunk's partials for the
// merge kernel (the merge is linear, so rotating each chunk is rotating the
// sum).
#include "qsa_device.h"

namespace qsa {

namespace {

// (cos, sin) of the rotary angles of the L new rows of sequence b, entry
// l * half + i, in LDS (half = rotary_dim / 2 pairs).
__device__ __forceinline__ void rope_table(float2 *tab, const int32_t *positions, int b, int L, int half,
                                           double step) {
  for (int e = threadIdx.x; e < L * half; e += kThreads) {
    float c, s;
    rope_angle_cs(positions[(int64_t)b * L + e / half], rope_freq(step, e % half), c, s);
    tab[e] = make_float2(c, s);
  }
}

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

// ------------------------------------------------------------------ append
template <int D>
__global__ __launch_bounds__(kThreads) void turbo8_append_kernel(Params p, const bf16_t *__restrict__ k_new,
                                                                 const bf16_t *__restrict__ v_new,
                                                                 uint8_t *__restrict__ kq, bf16_t *__restrict__ ks,
                                                                 uint8_t *__restrict__ vq, bf16_t *__restrict__ vs) {
  constexpr int E = D / 16, ROWS = kThreads / 16;
  __shared__ __attribute__((aligned(16))) float2 cs[kMaxPairs];
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
    Turbo8Row<D> q;
    turbo8_new_row<D>(x, is_k, w, valid, p.eps, p.r, cs, q);
    if (!valid || !ok) continue;
    const int64_t row = (off + n + l) * p.Hkv + head;
    uint8_t *codes = (is_k ? kq : vq) + row * D + E * c16;
#pragma unroll
    for (int c = 0; c < Turbo8Row<D>::CW; ++c) {
      if constexpr (E >= 4) *(uint32_t *)(codes + 4 * c) = q.codes[c];
    }
    if (c16 % Turbo8Row<D>::LPG == 0) (is_k ? ks : vs)[row * (D / 16) + E * c16 / 16] = q.scale;
  }
}

// ------------------------------------------------------------------ attention
template <int D, int RTM>
__global__ __launch_bounds__(kThreads) void turbo8_kernel(Params p, const uint8_t *__restrict__ kq,
                                                          const bf16_t *__restrict__ ks,
                                                          const uint8_t *__restrict__ vq,
                                                          const bf16_t *__restrict__ vs, uint8_t *__restrict__ kq_w,
                                                          bf16_t *__restrict__ ks_w, uint8_t *__restrict__ vq_w,
                                                          bf16_t *__restrict__ vs_w) {
  using G = Geo<D>;
  constexpr int E = G::E, KST = G::KST, RB = G::RB, DBW = D / 64, SK = G::SK;
  constexpr int NG = D / 16;                            // groups per row
  constexpr int GPT = SK * NG / kThreads;               // groups per thread and stage (per tensor)
  constexpr int QBYTES = 16 * RTM * RB;
  constexpr int TABN = kMaxFusedTable;
  constexpr int PREP = QBYTES + TABN * 8;
  constexpr int ARENA = PREP > Xch::BYTES ? PREP : Xch::BYTES;
  constexpr int SLOT = SK * RB;                         // one stage of one tensor
  static_assert(2 * 2 * SLOT >= 16 * RTM * D * 4 + 16 * RTM * 4, "the epilogue tile fits in the ring");
  __shared__ __attribute__((aligned(16))) unsigned char ring[4 * SLOT];   // K slot 0 | K slot 1 | V slot 0 | V slot 1
  __shared__ __attribute__((aligned(16))) unsigned char arena[ARENA];

  const int t = threadIdx.x, lane = t % kWave, g4 = lane >> 4, m16 = lane & 15, c16 = m16;
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int nslot = p.B * p.Hkv;
  const int chunk = blockIdx.x / nslot, slot = blockIdx.x % nslot;
  const int hkv = p.Hkv, b = slot / hkv, kvh = slot % hkv;
  const int L = p.L, Gq = p.G, Hq = p.Hq, R = L * Gq, half = p.r / 2;
  const int n = p.seq_lens[b];
  const int64_t off = p.seq_offset[b];
  const int64_t total = (int64_t)n + L;
  const bool in_range = n >= 0 && off >= 0 && total <= p.max_seq_len && off + total <= p.num_rows;
  const int nch = tile_chunk_count(total, p.even_split, p.chunks, p.chunk_keys);
  if (chunk >= nch) return;
  const bf16_t *const q_gate = (const bf16_t *)p.q_gate;
  bf16_t *const outp = (bf16_t *)p.out;
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
  const int64_t cend = min(k1, (int64_t)n);
  const int nst = cend > k0 ? (int)((cend - k0 + SK - 1) / SK) : 0;

  // ---- one stage's codes and scales in registers: thread t holds groups
  // t + 256 i of the stage (key = group / NG, 16-code group = group % NG)
  uint4 kc[GPT], vc[GPT];
  bf16_t ksc[GPT], vsc[GPT];
  auto load_stage = [&](int st) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int gi = t + kThreads * i, key = gi / NG, grp = gi % NG;
      const int64_t tk = min(k0 + (int64_t)SK * st + key, cend - 1);   // keys past the chunk repeat its last
      const int64_t row = (off + tk) * hkv + kvh;
      if constexpr (NG >= 1) {
        kc[i] = gld<uint4>(kq + row * D + 16 * grp);
        vc[i] = gld<uint4>(vq + row * D + 16 * grp);
        ksc[i] = ks[row * NG + grp];
        vsc[i] = vs[row * NG + grp];
      }
    }
  };
  // decode the registers' groups into the swizzled bf16 tiles of ring slot sl
  auto store_stage = [&](int sl) {
    unsigned char *kt = ring + sl * SLOT, *vt = ring + (2 + sl) * SLOT;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int gi = t + kThreads * i, key = gi / NG, grp = gi % NG;
#pragma unroll
      for (int tensor = 0; tensor < 2; ++tensor) {
        const uint4 c = tensor ? vc[i] : kc[i];
        const float s = (float)(tensor ? vsc[i] : ksc[i]);
        const uint32_t w4[4] = {c.x, c.y, c.z, c.w};
        f16x8 h[2];
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const f32x2_t f = unpk_fp8(w4[j / 4], (j % 4) != 0);
          h[j / 8][j % 8] = (f16_t)(f[0] * s);
          h[j / 8][j % 8 + 1] = (f16_t)(f[1] * s);
        }
        unsigned char *tile = tensor ? vt : kt;
        *(f16x8 *)(tile + swz<G::SW>(key, 2 * grp, RB)) = h[0];
        *(f16x8 *)(tile + swz<G::SW>(key, 2 * grp + 1, RB)) = h[1];
      }
    }
  };
  if (nst > 0) load_stage(0);

  // ---- query rows: norm, rotation, WHT, bf16 operands (16 lanes per row)
  float2 *const tab = (float2 *)(arena + QBYTES);
  rope_table(tab, p.positions, b, L, half, p.rope_step);
  __syncthreads();
  float wq[E], wk[E];
  {
    RawE<E> a, c;
    a.load((const bf16_t *)p.wq + E * c16);
    c.load((const bf16_t *)p.wk + E * c16);
    a.to_float(wq);
    c.to_float(wk);
  }
  const int hr = t / 16;                                // this lane group's row slot (0 .. 15)
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    const int r = 16 * rt + hr, rc = min(r, R - 1);
    const int l = rc / Gq, h = kvh * Gq + rc % Gq;
    RawE<E> raw;
    raw.load(q_gate + (((int64_t)b * L + l) * Hq + h) * 2 * D + E * c16);
    float x[E];
    raw.to_float(x);
    norm_rope<D>(x, wq, r < R, p.eps, p.r, tab + l * half);
    row_wht<D>(x);
    put_row<D, f16_t>(arena, RB, r, E * c16, x);
  }
  // ---- the new rows (tail): quantized as the append does; stored when this
  // call appends them, read back from the cache otherwise; kept decoded
  float nk[E], nv[E];
  Turbo8Row<D> qk, qv;
  const int nl = hr;                                    // new row of this lane group
  if (tail) {
    const int lc = min(nl, L - 1);
    const int64_t crow = (off + n + lc) * hkv + kvh;
    if (fuse_new) {
      RawE<E> a, c;
      a.load((const bf16_t *)p.k_new + (((int64_t)b * L + lc) * hkv + kvh) * D + E * c16);
      c.load((const bf16_t *)p.v_new + (((int64_t)b * L + lc) * hkv + kvh) * D + E * c16);
      a.to_float(nk);
      c.to_float(nv);
      turbo8_new_row<D>(nk, true, wk, nl < L, p.eps, p.r, tab + lc * half, qk);
      turbo8_new_row<D>(nv, false, wk, nl < L, p.eps, p.r, tab + lc * half, qv);
    } else {
#pragma unroll
      for (int c = 0; c < Turbo8Row<D>::CW; ++c) {
        qk.codes[c] = *(const uint32_t *)(kq + crow * D + E * c16 + 4 * c);
        qv.codes[c] = *(const uint32_t *)(vq + crow * D + E * c16 + 4 * c);
      }
      qk.scale = ks[crow * NG + E * c16 / 16];
      qv.scale = vs[crow * NG + E * c16 / 16];
    }
    qk.dequantize(nk);
    qv.dequantize(nv);
    if (nl >= L) {
#pragma unroll
      for (int j = 0; j < E; ++j) nk[j] = nv[j] = 0.f;
    }
  }
  __syncthreads();
  f16x8 qf[RTM][KST];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt)
#pragma unroll
    for (int k = 0; k < KST; ++k) qf[rt][k] = *(const f16x8 *)(arena + swz<G::SW>(16 * rt + m16, 4 * k + g4, RB));
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
  __syncthreads();                                      // every wave holds its operands: the arena is the exchange now

  // ---- cached stages
  for (int st = 0; st < nst; ++st) {
    store_stage(st & 1);
    if (st + 1 < nst) load_stage(st + 1);
    __syncthreads();
    const int sk0 = (int)(k0 + (int64_t)SK * st);
    const int nk_ = (int)min<int64_t>(SK, cend - sk0);
    attend_stage<D, RTM, NoOp, f16_t>(ring + (st & 1) * SLOT, ring + (2 + (st & 1)) * SLOT, nk_, sk0, qf, O, mrun,
                                      lrun, lim, sl2, arena);
  }
  // ---- the new rows as a last stage: K and V rows 0 .. 15 (zero past L), V
  // rows 16 .. 31 zero (read by the value product)
  if (tail) {
    const int sl = nst & 1;
    unsigned char *kt = ring + sl * SLOT, *vt = ring + (2 + sl) * SLOT;
    put_row<D, f16_t>(kt, RB, nl, E * c16, nk);
    put_row<D, f16_t>(vt, RB, nl, E * c16, nv);
    float z[E];
#pragma unroll
    for (int j = 0; j < E; ++j) z[j] = 0.f;
    put_row<D, f16_t>(vt, RB, 16 + nl, E * c16, z);
    __syncthreads();
    attend_stage<D, RTM, NoOp, f16_t>(kt, vt, L, n, qf, O, mrun, lrun, lim, sl2, arena);
  }

  // ---- append (the fused call's new rows)
  const int32_t *const capp = p.capacity;
  const bool cap_ok = !capp || total <= (int64_t)capp[b];
  if (tail && fuse_new && cap_ok && nl < L) {
    const int64_t crow = (off + n + nl) * hkv + kvh;
#pragma unroll
    for (int c = 0; c < Turbo8Row<D>::CW; ++c) {
      *(uint32_t *)(kq_w + crow * D + E * c16 + 4 * c) = qk.codes[c];
      *(uint32_t *)(vq_w + crow * D + E * c16 + 4 * c) = qv.codes[c];
    }
    if (c16 % Turbo8Row<D>::LPG == 0) {
      ks_w[crow * NG + E * c16 / 16] = qk.scale;
      vs_w[crow * NG + E * c16 / 16] = qv.scale;
    }
  }

  // ---- rotate the rows back (iWHT) through LDS, then gate or store partials
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
  const bool single = nch == 1;
  const int64_t slot_rows = ((int64_t)slot * p.chunks + chunk) * p.rows;
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
    if (single) {
      RawE<E> zr;
      zr.load(q_gate + orow * 2 * D + D + E * c16);
      float z[E];
      zr.to_float(z);
      const float inv = linv[r];
      float o[E];
#pragma unroll
      for (int j = 0; j < E; ++j) o[j] = cap_ok ? x[j] * inv * sigmoid_f(z[j]) : __builtin_nanf("");
      bf16_t *dst = outp + orow * D + E * c16;
#pragma unroll
      for (int j = 0; j < E; ++j) dst[j] = (bf16_t)o[j];
    } else if (cap_ok) {
      float *po = p.part_o + (slot_rows + r) * D + E * c16;
#pragma unroll
      for (int j = 0; j < E; j += 4) *(f32x4 *)(po + j) = f32x4{x[j], x[j + 1], x[j + 2], x[j + 3]};
    }
  }
  if (!single && cap_ok && wave == 0 && g4 == 0) {
#pragma unroll
    for (int rt = 0; rt < RTM; ++rt)
      if (16 * rt + m16 < R)
        *(float2 *)(p.part_ml + (slot_rows + 16 * rt + m16) * 2) = make_float2(mrun[rt], lrun[rt]);
  }
  if (!cap_ok && chunk == 0) {
    if (!single) {
      for (int e = t; e < R * D; e += kThreads) {
        const int r = e / D, d = e % D, l = r / Gq, h = kvh * Gq + r % Gq;
        outp[(((int64_t)b * L + l) * Hq + h) * D + d] = (bf16_t)__builtin_nanf("");
      }
      if (t < R) *(float2 *)(p.part_ml + (slot_rows + t) * 2) = make_float2(__builtin_nanf(""), __builtin_nanf(""));
    }
    if (t == 0) flag_error(p);
  }
}

template <int D>
static hipError_t launch_turbo8_d(const Params &p, const Turbo8Cache &c, hipStream_t s, const Timing &tm) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.chunks;
  switch ((p.rows + 15) / 16) {
    case 1: launch_kernel(turbo8_kernel<D, 1>, blocks, s, tm, p, c.kq, c.ks, c.vq, c.vs, c.kq, c.ks, c.vq, c.vs); break;
    case 2: launch_kernel(turbo8_kernel<D, 2>, blocks, s, tm, p, c.kq, c.ks, c.vq, c.vs, c.kq, c.ks, c.vq, c.vs); break;
    case 3: launch_kernel(turbo8_kernel<D, 3>, blocks, s, tm, p, c.kq, c.ks, c.vq, c.vs, c.kq, c.ks, c.vq, c.vs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_turbo8_bf16(const Params &p, const Turbo8Cache &c, hipStream_t s, const Timing &tm) {
  switch (p.D) {
    case 64: return launch_turbo8_d<64>(p, c, s, tm);
    case 128: return launch_turbo8_d<128>(p, c, s, tm);
    case 256: return launch_turbo8_d<256>(p, c, s, tm);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_turbo8_append(const Params &p, const Turbo8Cache &c, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.L;
  const bf16_t *kn = (const bf16_t *)p.k_new, *vn = (const bf16_t *)p.v_new;
  switch (p.D) {
    case 64: hipLaunchKernelGGL(turbo8_append_kernel<64>, dim3(blocks), dim3(kThreads), 0, s, p, kn, vn, c.kq, c.ks, c.vq, c.vs); break;
    case 128: hipLaunchKernelGGL(turbo8_append_kernel<128>, dim3(blocks), dim3(kThreads), 0, s, p, kn, vn, c.kq, c.ks, c.vq, c.vs); break;
    case 256: hipLaunchKernelGGL(turbo8_append_kernel<256>, dim3(blocks), dim3(kThreads), 0, s, p, kn, vn, c.kq, c.ks, c.vq, c.vs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
