// qsa_rows.hip -- row-wise kernels: the prologue (norm + partial rotation of new
// keys and/or queries, KV append) and the fp32 attention path.
//
// Norm: x * w / sqrt(mean(x^2) + eps) per head (mlxd PR #99 config audit,
// has_qk_norm; Atlas FullAttentionLayer q_norm / k_norm).  Rotation: first
// rotary_dim dims, dim i paired with i + rotary_dim/2 (mlxd PR #99 Summary,
// partial_rotary_factor; Atlas Qwen35ForwardConfig::rotary_dim).  Append at
// slot seq_lens[b] + l (Atlas qwen3_5/mod.rs module doc).
#include "qsa_device.h"

namespace qsa {

// One workgroup per new row (b, l).  It tabulates the (cos, sin) of the row's
// position once; then every 16 lanes take one head row, lane c16 holding the
// E = D/16 contiguous elements E c16 .., so that a wavefront works on four head
// rows at a time.  Heads [0, nk) are key heads: normalised, rotated, rounded
// and written with the matching value row to the cache.  Heads [nk, nk+nq) are
// query heads: normalised and rotated into the prepared-query buffer p.qt
// (element type TQ).  The norm and the rotation are norm_rope, the routine the
// short-query kernel runs on the new keys of a fused call, with the same table
// and the same reduction order, so the cache rows written here are bitwise the
// rows that a fused call writes.  A rotation whose halves do not start on a
// lane boundary (r/2 not a multiple of E, which the short-query route never
// takes) goes through an LDS copy of the row instead.
template <typename T, typename TQ, int D>
__global__ __launch_bounds__(kThreads) void prologue_kernel(Params p, int do_q, int do_kv) {
  constexpr int E = D / 16, ROWS = kThreads / 16;
  __shared__ float scratch[ROWS][D];
  __shared__ __attribute__((aligned(16))) float2 cs[kMaxPairs];
  const int m16 = threadIdx.x & 15, hr = threadIdx.x / 16;   // head-row slot of these 16 lanes
  const int64_t bl = blockIdx.x;                        // new row (b, l)
  const int b = (int)(blockIdx.x / (unsigned)p.L), l = (int)(blockIdx.x % (unsigned)p.L);
  const int nk = do_kv ? p.Hkv : 0, nq = do_q ? p.Hq : 0, njobs = nk + nq;
  const int r = p.r, half = r / 2;
  const bool whole = half % E == 0;
  if (r > 0) {
    const int pos = p.positions[bl];
    for (int i = threadIdx.x; i < half; i += kThreads) {
      float c, sn;
      rope_angle_cs(pos, rope_freq(p.rope_step, i), c, sn);
      cs[i] = make_float2(c, sn);
    }
  }
  __syncthreads();
  int n = 0;
  int64_t off = 0, row = 0;
  bool kv_ok = true;
  if (nk) {
    kv_ok = seq_in_range(p, b, n = p.seq_lens[b], off);
    if (kv_ok) kv_ok = (row = cache_row(p, b, off, (int64_t)n + l)) >= 0;   // the row this new token goes to
  }
  if (!kv_ok && threadIdx.x == 0) flag_error(p);

  // every lane runs every pass (the rotation permutes across lanes); rows past
  // the last job take a clamped row and are not stored
  for (int j0 = 0; j0 < njobs; j0 += ROWS) {
    const int job = j0 + hr;
    const bool valid = job < njobs;
    const int jb = valid ? job : njobs - 1;
    const bool is_k = jb < nk;
    const int head = is_k ? jb : jb - nk;
    const T *src = is_k ? (const T *)p.k_new + (bl * p.Hkv + head) * D
                        : (const T *)p.q_gate + (bl * p.Hq + head) * 2 * D;   // query half of [q | gate]
    const T *wp = is_k ? (const T *)p.wk : (const T *)p.wq;
    float x[E], w[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      x[j] = to_f(src[E * m16 + j]);
      w[j] = to_f(wp[E * m16 + j]);
    }
    if (whole) {
      norm_rope<D>(x, w, valid, p.eps, r, cs);
    } else {
      row_norm<D>(x, w, valid, p.eps);
      // partner i +- r/2 of each rotated element, through this row's scratch copy
#pragma unroll
      for (int j = 0; j < E; ++j) scratch[hr][E * m16 + j] = x[j];
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int e = E * m16 + j;
        if (e < r) {
          const bool lo = e < half;
          const float2 v = cs[lo ? e : e - half];
          const float other = scratch[hr][lo ? e + half : e - half];
          x[j] = lo ? x[j] * v.x - other * v.y : x[j] * v.x + other * v.y;
        }
      }
      wave_lds_sync();                                  // the next pass rewrites the scratch row
    }
    if (!valid) continue;
    if (is_k) {
      if (!kv_ok) continue;
      const int64_t dst = (row * p.Hkv + head) * D + E * m16;
      const T *vsrc = (const T *)p.v_new + (bl * p.Hkv + head) * D + E * m16;
      // the lane's E contiguous values in 16-byte pieces (8-byte when that is
      // all of them), so that the K and V rows go out in whole vectors
      using V = typename std::conditional<(E * sizeof(T) >= 16), uint4, uint2>::type;
      constexpr int PER = (int)(sizeof(V) / sizeof(T)), NV = E / PER;
      static_assert(NV * PER == E, "whole pieces");
      V vv[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) vv[i] = gld<V>(vsrc + PER * i);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        T k8[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) k8[j] = from_f<T>(x[PER * i + j]);
        *(V *)((T *)p.kc + dst + PER * i) = __builtin_bit_cast(V, k8);
        *(V *)((T *)p.vc + dst + PER * i) = vv[i];
      }
    } else {
      TQ *dst = (TQ *)p.qt + (bl * p.Hq + head) * D + E * m16;
#pragma unroll
      for (int j = 0; j < E; ++j) dst[j] = from_f<TQ>(x[j]);
    }
  }
}

// fp32 attention: one workgroup per query row (b, l, h), plain two-pass softmax
// over keys 0 .. n_b + l of KV head h / G, reading the prepared query from p.qt.
template <int D>
__global__ __launch_bounds__(kThreads) void rows_f32_kernel(Params p) {
  __shared__ float q[D];
  __shared__ float pbuf[kThreads];
  __shared__ float red_m[kThreads / kWave], red_s[kThreads / kWave];
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int64_t f = blockIdx.x;
  const int h = (int)(f % p.Hq);
  const int64_t bl = f / p.Hq;
  const int l = (int)(bl % p.L), b = (int)(bl / p.L);
  const int g = h / p.G;
  float *out = (float *)p.out + f * D;
  const int n = p.seq_lens[b];
  int64_t off;
  if (!seq_in_range(p, b, n, off)) {
    if (t < D) out[t] = __builtin_nanf("");
    if (t == 0) flag_error(p);
    return;
  }
  if (t < D) q[t] = ((const float *)p.qt)[f * D + t];
  __syncthreads();
  const float *K = (const float *)p.kc;
  const float *V = (const float *)p.vc;
  const int64_t total = (int64_t)n + l + 1;

  auto score = [&](int64_t j) {
    const float *kr = K + ((off + j) * p.Hkv + g) * D;
    float acc = 0.f;
    for (int d = 0; d < D; ++d) acc += q[d] * kr[d];
    return acc * p.scale;
  };

  // pass 1: max and normaliser
  float m = -INFINITY, s = 0.f;
  for (int64_t j = t; j < total; j += kThreads) {
    const float sc = score(j);
    if (sc > m) {
      s = s * expf(m - sc) + 1.f;
      m = sc;
    } else {
      s += expf(sc - m);
    }
  }
  const float mw = wave_max(m);
  s = (s > 0.f) ? s * expf(m - mw) : 0.f;
  s = wave_sum(s);
  if (lane == 0) {
    red_m[wave] = mw;
    red_s[wave] = s;
  }
  __syncthreads();
  float M = red_m[0];
  for (int w = 1; w < kThreads / kWave; ++w) M = fmaxf(M, red_m[w]);
  float S = 0.f;
  for (int w = 0; w < kThreads / kWave; ++w)
    if (red_s[w] > 0.f) S += red_s[w] * expf(red_m[w] - M);

  // pass 2: weighted values
  float acc = 0.f;
  for (int64_t base = 0; base < total; base += kThreads) {
    const int64_t j = base + t;
    pbuf[t] = j < total ? expf(score(j) - M) / S : 0.f;
    __syncthreads();
    if (t < D) {
      const int64_t cnt = min((int64_t)kThreads, total - base);
      for (int64_t k = 0; k < cnt; ++k) acc += pbuf[k] * V[((off + base + k) * p.Hkv + g) * D + t];
    }
    __syncthreads();
  }
  if (t < D) {
    const float z = ((const float *)p.q_gate)[f * 2 * D + D + t];
    out[t] = acc / (1.f + expf(-z));
  }
}

template <typename T, typename TQ>
static hipError_t prologue_for(const Params &p, bool do_q, bool do_kv, hipStream_t s) {
  if (!do_q && !do_kv) return hipSuccess;
  const int64_t blocks = (int64_t)p.B * p.L;            // one workgroup per new row
  switch (p.D) {
    case 64:
      hipLaunchKernelGGL((prologue_kernel<T, TQ, 64>), dim3(blocks), dim3(kThreads), 0, s, p, (int)do_q, (int)do_kv);
      break;
    case 128:
      hipLaunchKernelGGL((prologue_kernel<T, TQ, 128>), dim3(blocks), dim3(kThreads), 0, s, p, (int)do_q, (int)do_kv);
      break;
    case 256:
      hipLaunchKernelGGL((prologue_kernel<T, TQ, 256>), dim3(blocks), dim3(kThreads), 0, s, p, (int)do_q, (int)do_kv);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prologue(const Params &p, int dtype, bool do_q, bool do_kv, hipStream_t s) {
  // bf16 path prepares bf16 queries (MFMA operands); fp32 path keeps fp32
  return dtype == 0 ? prologue_for<bf16_t, bf16_t>(p, do_q, do_kv, s)
                    : prologue_for<float, float>(p, do_q, do_kv, s);
}

hipError_t launch_rows_f32(const Params &p, hipStream_t s, const Timing &tm) {
  const int64_t blocks = (int64_t)p.B * p.L * p.Hq;
  switch (p.D) {
    case 64: launch_kernel(rows_f32_kernel<64>, blocks, s, tm, p); break;
    case 128: launch_kernel(rows_f32_kernel<128>, blocks, s, tm, p); break;
    case 256: launch_kernel(rows_f32_kernel<256>, blocks, s, tm, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
