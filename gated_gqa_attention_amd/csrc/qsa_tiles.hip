// qsa_tiles.hip -- bf16 gated grouped-query attention on MFMA (gfx950).
//
// One workgroup = (sequence b, KV head g, row tile, key chunk).  The row tile
// holds up to 64 query rows: the G query heads that share KV head g times the
// new rows (DS4Server issue #113: query heads grouped within their KV group;
// Atlas Qwen35ForwardConfig: 16 query / 4 KV heads).  Keys of the chunk are
// streamed through LDS 64 at a time; softmax is online (flash-decoding
// split-K); chunks of one tile are merged by the last workgroup to arrive,
// which also applies the output gate attn * sigmoid(gate) (mlxd PR #99
// Summary; Atlas sigmoid_gate).
//
// Fused mode (PREP = false, decode / verify): every workgroup derives its own
// queries from q_gate (split, RMS norm, partial rotation), and the workgroup
// whose chunk holds the new key slots n_b .. n_b+L-1 normalises, rotates and
// appends them (Atlas qwen3_5/mod.rs module doc: append at cache_pos, attend
// over cache_pos + 1 keys).  Prepared mode (PREP = true, long prefill): queries
// come from the prologue kernel's buffer and the cache already holds the rows.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, lane l, g = l / 16, m = l % 16):
//   scores^T[key][row] = K[key][:] . Q[row][:]    A = K rows from LDS, B = Q
//   out^T[dim][row]   += V^T[dim][key] . P^T[key][row]
// Score block beta of a 32-key block maps MFMA row m to key 8(m/4) + 4 beta + m%4,
// so each lane ends up holding the 8 consecutive keys 8g .. 8g+7 of one query
// row: exactly the B operand the value product needs, with no lane shuffle.
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kVStride = kTileKeys + 8;  // V^T row stride (bf16): conflict-free 16-byte reads

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// RMS-normalise and rotate one head row with a whole wavefront.  Every wave of
// the workgroup must call this the same number of times (it uses barriers);
// `active` selects whether this wave's row is real.  x holds EPL = D/64
// contiguous elements per lane on entry and the result on exit.
template <int D>
__device__ __forceinline__ void norm_rope_rows(float (&x)[D / kWave], const bf16_t *w, bool active,
                                               int pos, const Params &p, float *scratch) {
  constexpr int EPL = D / kWave;
  const int lane = threadIdx.x % kWave;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) ss += x[j] * x[j];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D + p.eps);
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    x[j] = active ? x[j] * inv * to_f(w[lane * EPL + j]) : 0.f;
    scratch[lane * EPL + j] = x[j];
  }
  __syncthreads();
  if (active && p.r > 0) {
    const int half = p.r / 2;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane * EPL + j;
      if (e < p.r) {
        const int i = e < half ? e : e - half;
        float c, s;
        rope_cs(pos, i, p.r, p.theta, c, s);
        const float other = scratch[e < half ? e + half : e - half];
        x[j] = e < half ? x[j] * c - other * s : x[j] * c + other * s;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

}  // namespace

template <int D, bool PREP>
__global__ __launch_bounds__(kThreads) void tiles_bf16_kernel(Params p) {
  constexpr int EPL = D / kWave;
  constexpr int KST = D / 32;          // MFMA k-steps over head_dim
  constexpr int NDB = D / 16;          // 16-wide dim blocks of the output
  constexpr int KSTR = D + 8;          // K row stride in LDS (bf16)
  constexpr int OCT = D / 8;           // 16-byte units per key row
  constexpr int KU = kTileKeys * OCT / kThreads;        // K units per thread per stage
  constexpr int VU = (kTileKeys / 2) * OCT / kThreads;  // V (key pair, unit) per thread per stage
  static_assert(KU >= 1 && VU >= 1, "head_dim too small for the tile");

  __shared__ __attribute__((aligned(16))) bf16_t Ks[kTileKeys * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * kVStride];
  __shared__ int s_ticket;

  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int g4 = lane >> 4, m16 = lane & 15;

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
  const int n = p.seq_lens[b];
  int64_t off;
  if (!seq_in_range(p, b, n, off)) {
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
  const int nch = (int)((kend + p.chunk_keys - 1) / p.chunk_keys);
  if (chunk >= nch) return;
  const int64_t k0 = (int64_t)chunk * p.chunk_keys;
  const int64_t k1 = min(kend, k0 + (int64_t)p.chunk_keys);

  const int RT = (R + 15) / 16;              // 16-row MFMA tiles
  const int KS = RT <= 2 ? 2 : 1;            // waves splitting the keys of a stage
  const bool computes = wave < RT * KS;
  const int rt = wave % RT, ksub = wave / RT;

  const bf16_t *kc = (const bf16_t *)p.kc;
  const bf16_t *vc = (const bf16_t *)p.vc;
  const bf16_t *qg = (const bf16_t *)p.q_gate;

  // ---------------------------------------------------------------- queries
  bf16_t *Qs = Ks;                                      // [64][KSTR], aliases the K stage
  float *scratch = reinterpret_cast<float *>(Vt) + wave * D;
  for (int e = t; e < (RT * 16 - R) * OCT; e += kThreads) {
    const int rr = R + e / OCT, o = e % OCT;
    *(bf16x8 *)&Qs[rr * KSTR + 8 * o] = bf16x8{};
  }
  if constexpr (PREP) {
    for (int e = t; e < R * OCT; e += kThreads) {
      const int rr = e / OCT, o = e % OCT;
      const int rg = row0 + rr, l = rg / p.G, h = kvh * p.G + rg % p.G;
      *(bf16x8 *)&Qs[rr * KSTR + 8 * o] =
          *(const bf16x8 *)((const bf16_t *)p.qt + (((int64_t)b * p.L + l) * p.Hq + h) * D + 8 * o);
    }
  } else {
    for (int base = 0; base < R; base += kThreads / kWave) {
      const int rr = base + wave;
      const bool act = rr < R;
      const int rg = row0 + rr, l = rg / p.G, h = kvh * p.G + rg % p.G;
      float x[EPL];
      const bf16_t *src = qg + (((int64_t)b * p.L + l) * p.Hq + h) * 2 * D;   // query half
#pragma unroll
      for (int j = 0; j < EPL; ++j) x[j] = act ? to_f(src[lane * EPL + j]) : 0.f;
      norm_rope_rows<D>(x, (const bf16_t *)p.wq, act, act ? p.positions[b * p.L + l] : 0, p, scratch);
      if (act) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) Qs[rr * KSTR + lane * EPL + j] = (bf16_t)x[j];
      }
    }
    // new key/value rows that fall in this chunk: normalise, rotate, append
    if (p.k_new) {
      const int64_t lo64 = max(k0 - n, (int64_t)0), hi64 = min(k1 - n, (int64_t)p.L);
      const int lo = (int)lo64, hi = (int)max(hi64, lo64);
      for (int base = lo; base < hi; base += kThreads / kWave) {
        const int l = base + wave;
        const bool act = l < hi;
        const int64_t src_row = ((int64_t)b * p.L + (act ? l : lo)) * p.Hkv + kvh;
        const bf16_t *ks = (const bf16_t *)p.k_new + src_row * D;
        float x[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) x[j] = act ? to_f(ks[lane * EPL + j]) : 0.f;
        norm_rope_rows<D>(x, (const bf16_t *)p.wk, act, act ? p.positions[b * p.L + l] : 0, p, scratch);
        if (act) {
          const int64_t dst = ((off + n + l) * p.Hkv + kvh) * D;
          const bf16_t *vs = (const bf16_t *)p.v_new + src_row * D;
#pragma unroll
          for (int j = 0; j < EPL; ++j) {
            ((bf16_t *)p.kc)[dst + lane * EPL + j] = (bf16_t)x[j];
            ((bf16_t *)p.vc)[dst + lane * EPL + j] = vs[lane * EPL + j];
          }
        }
      }
    }
  }
  __syncthreads();  // Qs complete; appended rows visible to this workgroup

  bf16x8 qf[KST];
  if (computes) {
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) qf[ks] = *(const bf16x8 *)&Qs[(rt * 16 + m16) * KSTR + 32 * ks + 8 * g4];
  }
  __syncthreads();  // Qs (aliasing Ks) is free again

  // ---------------------------------------------------------------- key loop
  f32x4 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f, l_run = 0.f;
  const int rowg = row0 + rt * 16 + m16;
  const int64_t lim = (int64_t)n + rowg / p.G;          // causal: row sees keys <= n + l

  uint4 kreg[KU];
  uint4 vreg[VU][2];
  auto load_stage = [&](int64_t sb) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = t + kThreads * i, key = u / OCT, o = u % OCT;
      const int64_t ka = sb + key;
      kreg[i] = ka < k1 ? *(const uint4 *)(kc + ((off + ka) * p.Hkv + kvh) * D + 8 * o) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = t + kThreads * i, kp = u % (kTileKeys / 2), o = u / (kTileKeys / 2);
      const int64_t ka = sb + 2 * kp;
      vreg[i][0] = ka < k1 ? *(const uint4 *)(vc + ((off + ka) * p.Hkv + kvh) * D + 8 * o) : uint4{0, 0, 0, 0};
      vreg[i][1] = ka + 1 < k1 ? *(const uint4 *)(vc + ((off + ka + 1) * p.Hkv + kvh) * D + 8 * o)
                               : uint4{0, 0, 0, 0};
    }
  };

  const int nst = (int)((k1 - k0 + kTileKeys - 1) / kTileKeys);
  load_stage(k0);
  for (int st = 0; st < nst; ++st) {
    const int64_t sb = k0 + (int64_t)st * kTileKeys;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int u = t + kThreads * i, key = u / OCT, o = u % OCT;
      *(uint4 *)&Ks[key * KSTR + 8 * o] = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VU; ++i) {
      const int u = t + kThreads * i, kp = u % (kTileKeys / 2), o = u / (kTileKeys / 2);
      const uint32_t a[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
      const uint32_t c[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
      uint32_t *vrow = reinterpret_cast<uint32_t *>(Vt);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 8o+2w (low halves) and 8o+2w+1 (high halves); keys 2kp (low) and 2kp+1 (high)
        vrow[((8 * o + 2 * w) * kVStride) / 2 + kp] = (a[w] & 0xffffu) | (c[w] << 16);
        vrow[((8 * o + 2 * w + 1) * kVStride) / 2 + kp] = (a[w] >> 16) | (c[w] & 0xffff0000u);
      }
    }
    __syncthreads();
    if (st + 1 < nst) load_stage(sb + kTileKeys);

    if (computes) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        if ((blk % KS) != ksub) continue;
        const int kb = 32 * blk;
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
          const bf16x8 a = *(const bf16x8 *)&Vt[(16 * db + m16) * kVStride + kb + 8 * g4];
          O[db] = mfma16(a, pf, O[db]);
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
  if (owner && KS == 2) {
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
  if (owner) {
    l_run += __shfl_xor(l_run, 16, kWave);
    l_run += __shfl_xor(l_run, 32, kWave);
  }
  const int rr = rt * 16 + m16;   // row within the tile held by this lane

  // ---------------------------------------------------------------- single chunk: finish here
  if (nch == 1) {
    if (owner && rr < R) {
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
    }
    return;
  }

  // ---------------------------------------------------------------- partial + last-arrival combine
  const int64_t pslot = (int64_t)slot * p.chunks;
  if (owner && rr < R) {
    float *po = p.part_o + ((pslot + chunk) * p.rows + rr) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) *(f32x4 *)(po + 16 * db + 4 * g4) = O[db];
    if (g4 == 0) {
      p.part_ml[((pslot + chunk) * p.rows + rr) * 2 + 0] = m_run;
      p.part_ml[((pslot + chunk) * p.rows + rr) * 2 + 1] = l_run;
    }
  }
  __threadfence();
  __syncthreads();
  if (t == 0) s_ticket = atomicAdd(&p.counters[slot], 1);
  __syncthreads();
  if (s_ticket != nch - 1) return;
  __threadfence();

  // weights w[c][row] = 2^(m_c - M_row) / sum_c l_c 2^(m_c - M_row), staged in LDS
  float *wts = reinterpret_cast<float *>(Ks);          // [nch][R], then [R] for 1/L
  float *mls = reinterpret_cast<float *>(Vt);          // [nch][R] raw l
  for (int e = t; e < nch * R; e += kThreads) {
    const int c = e / R, r2 = e % R;
    const float *ml = p.part_ml + ((pslot + c) * p.rows + r2) * 2;
    wts[e] = ml[0];
    mls[e] = ml[1];
  }
  __syncthreads();
  if (t < R) {
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, wts[c * R + t]);
    float Ls = 0.f;
    for (int c = 0; c < nch; ++c) Ls += mls[c * R + t] * exp2f(wts[c * R + t] - M);
    const float inv = 1.f / Ls;
    for (int c = 0; c < nch; ++c) wts[c * R + t] = exp2f(wts[c * R + t] - M) * inv;
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  for (int e = t; e < R * D4; e += kThreads) {
    const int r2 = e / D4, d = 4 * (e % D4);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const float *po = p.part_o + (pslot * p.rows + r2) * D + d;
    const int64_t cstride = (int64_t)p.rows * D;
#pragma unroll 8
    for (int c = 0; c < nch; ++c) acc += wts[c * R + r2] * *(const f32x4 *)(po + c * cstride);
    const int rg = row0 + r2, l = rg / p.G, h = kvh * p.G + rg % p.G;
    const bf16_t *z = qg + (((int64_t)b * p.L + l) * p.Hq + h) * 2 * D + D + d;
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16_t)(acc[i] * sigmoid(to_f(z[i])));
    *(bf16x4 *)((bf16_t *)p.out + (((int64_t)b * p.L + l) * p.Hq + h) * D + d) = v;
  }
  if (t == 0) p.counters[slot] = 0;   // ready for the next call on this workspace
}

template <int D>
static hipError_t launch_d(const Params &p, bool prep, hipStream_t s) {
  const int64_t blocks = (int64_t)p.B * p.Hkv * p.tiles * p.chunks;
  if (prep)
    hipLaunchKernelGGL((tiles_bf16_kernel<D, true>), dim3(blocks), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((tiles_bf16_kernel<D, false>), dim3(blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_tiles_bf16(const Params &p, bool prepared_q, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_d<64>(p, prepared_q, s);
    case 128: return launch_d<128>(p, prepared_q, s);
    case 256: return launch_d<256>(p, prepared_q, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
