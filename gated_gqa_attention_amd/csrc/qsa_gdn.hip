// qsa_gdn.hip -- one GatedDeltaNet decode step (gfx950): the linear-attention
// layer of hybrid Qwen3.5 (Atlas docs, spark_model/forward/qwen3_5/mod.rs:
// LinearAttentionLayer / LinearAttentionState / LinearAttentionScratch,
// Qwen35ForwardConfig GDN sizes, Qwen35Kernels causal_conv1d_update_l2norm,
// gdn_compute_gate, sigmoid_bf16_to_f32, gated_delta_rule_decode), fused into
// one kernel.  The update rule is the published gated delta rule:
//
//   conv:   state row of channel c <- [older inputs .., x_c]; u_c = silu(w_c . row)
//   q, k:   l2-normalised per key head (x / sqrt(sum x^2 + 1e-6)); q / sqrt(Dk)
//   gate:   g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)
//   state:  S <- exp(g) S;  S <- S + beta k (v - S^T k)^T;  o = S^T q
//   output: y = o / sqrt(mean(o^2) + eps) * norm_weight * silu(z)
//
// with value head h reading key head h / (Hv / Hk).
//
// One workgroup (512 threads) per (sequence, key head) takes that key head's
// R = Hv / Hk value heads, so the convolution of all the channels it reads
// (the key head's query and key channels, its value heads' value channels) and
// the in-place update of their conv state happen once, in one place.  Each
// value head's state S [Dk = 128][Dv = 128] fp32 is held in registers by 512/R
// threads: thread (rg, c4) holds rows rg * 8R .. + 8R - 1, columns 4 c4 .. + 3
// (float4 rows, so a wavefront's loads and stores are 512-byte runs).  The
// state is read once and written once: S^T k and S^T q of the old state are
// reduced together (lanes, then wavefronts through LDS), and since
//   kv = exp(g) S^T k,  delta = beta (v - kv),
//   o  = exp(g) S^T q + delta (k . q),  S' = exp(g) S + k delta^T,
// the output needs no second pass over the updated state.  The state loads
// are issued right after the conv inputs' and land while the convolution and
// the norms run.  Everything is fp32; y is rounded to bf16 once.
#include "qsa_device.h"

namespace qsa {

namespace {

constexpr int kGdnD = 128;                              // key and value head dims taken
constexpr int kGdnThreads = 512;

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + __expf(-x)); }

// log(1 + e^x) without overflow
__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x + log1pf(__expf(-x)) : log1pf(__expf(x)); }

}  // namespace

template <int R>
__global__ __launch_bounds__(kGdnThreads) void gdn_decode_kernel(GdnParams p) {
  constexpr int D = kGdnD, T = kGdnThreads, TPH = T / R, RG = TPH / 32, RPT = D / RG, WPH = TPH / kWave;
  constexpr int NCH = (2 + R) * D;                      // channels convolved here: q | k | R value heads
  constexpr int CPT = (NCH + T - 1) / T;
  __shared__ __attribute__((aligned(16))) float cbuf[NCH];
  __shared__ __attribute__((aligned(16))) float red[R][WPH][2][D];
  __shared__ float hsc[2 * R + 1];                      // exp(g), beta per value head; k . q

  const int t = threadIdx.x, lane = t % kWave;
  const int Hk = p.Hk, Hv = p.Hv, K = p.K, C = p.C;
  const int kh = blockIdx.x % Hk, b = blockIdx.x / Hk;
  const int j = t / TPH, lt = t % TPH, c4 = lt % 32, rg = lt / 32, hw = lt / kWave;
  const int h = kh * R + j;

  // ---- conv inputs: channel ci of this workgroup -> global channel
  float xin[CPT], st[CPT][4], w[CPT][4];
  int cgl[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ci = min(t + T * i, NCH - 1);
    const int cg = ci < D ? kh * D + ci : ci < 2 * D ? Hk * D + kh * D + (ci - D) : 2 * Hk * D + kh * R * D + (ci - 2 * D);
    cgl[i] = cg;
    xin[i] = (float)p.qkv[(int64_t)b * C + cg];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      st[i][jj] = jj < K ? p.conv_state[((int64_t)b * C + cg) * K + jj] : 0.f;
      w[i][jj] = jj < K ? (float)p.conv_w[(int64_t)cg * K + jj] : 0.f;
    }
  }
  // the output's gate and norm weight (the lanes that write y), the head scalars
  bf16x4 zr = {}, wn = {};
  if (rg == 0) {
    zr = *(const bf16x4 *)(p.z + ((int64_t)b * Hv + h) * D + 4 * c4);
    wn = *(const bf16x4 *)(p.norm_w + 4 * c4);
  }
  float ga = 0.f, gb = 0.f, alog = 0.f, dtb = 0.f;
  const int sj = t - kWave;                             // wavefront 1 computes the head scalars
  if (sj >= 0 && sj < R) {
    const int hh = kh * R + sj;
    ga = (float)p.a[(int64_t)b * Hv + hh];
    gb = (float)p.b[(int64_t)b * Hv + hh];
    alog = p.a_log[hh];
    dtb = (float)p.dt_bias[hh];
  }
  // ---- this thread's state rows
  float *const srow = p.state + (((int64_t)b * Hv + h) * D + rg * RPT) * D + 4 * c4;
  f32x4 S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = *(const f32x4 *)(srow + (int64_t)i * D);

  // ---- convolution: shift the new input in, taps, SiLU; conv state written back
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    if (t + T * i >= NCH) continue;
    float ns[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) ns[jj] = jj + 1 < K ? st[i][jj + 1] : xin[i];
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (jj < K) acc = fmaf(w[i][jj], ns[jj], acc);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (jj < K) p.conv_state[((int64_t)b * C + cgl[i]) * K + jj] = ns[jj];
    cbuf[t + T * i] = silu_f(acc);
  }
  __syncthreads();

  // ---- wavefront 0: l2 norms of q and k (q also / sqrt(Dk)) and k . q;
  // wavefront 1: exp(g) and beta of the value heads
  if (t < kWave) {
    const float2 q2 = *(const float2 *)(cbuf + 2 * lane), k2 = *(const float2 *)(cbuf + D + 2 * lane);
    float sq = q2.x * q2.x + q2.y * q2.y, sk = k2.x * k2.x + k2.y * k2.y, skq = k2.x * q2.x + k2.y * q2.y;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      sq += __shfl_xor(sq, m, kWave);
      sk += __shfl_xor(sk, m, kWave);
      skq += __shfl_xor(skq, m, kWave);
    }
    const float rq = 1.f / (sqrtf(sq + 1e-6f) * sqrtf((float)D)), rk = 1.f / sqrtf(sk + 1e-6f);
    *(float2 *)(cbuf + 2 * lane) = make_float2(q2.x * rq, q2.y * rq);
    *(float2 *)(cbuf + D + 2 * lane) = make_float2(k2.x * rk, k2.y * rk);
    if (lane == 0) hsc[2 * R] = skq * rq * rk;
  } else if (sj < R) {
    const float g = -expf(alog) * softplus_f(ga + dtb);
    hsc[2 * sj] = expf(g);
    hsc[2 * sj + 1] = 1.f / (1.f + expf(-gb));
  }
  __syncthreads();

  // ---- S^T k and S^T q of this thread's rows, then over the head's threads
  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float qr = cbuf[rg * RPT + i], kr = cbuf[D + rg * RPT + i];
    pk += S[i] * kr;
    pq += S[i] * qr;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {                         // lanes l and l + 32 hold row groups 2 m and 2 m + 1
    pk[e] += __shfl_xor(pk[e], 32, kWave);
    pq[e] += __shfl_xor(pq[e], 32, kWave);
  }
  if (lane < 32) {
    *(f32x4 *)&red[j][hw][0][4 * c4] = pk;
    *(f32x4 *)&red[j][hw][1][4 * c4] = pq;
  }
  __syncthreads();
  f32x4 sk4 = {0.f, 0.f, 0.f, 0.f}, sq4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ww = 0; ww < WPH; ++ww) {
    sk4 += *(const f32x4 *)&red[j][ww][0][4 * c4];
    sq4 += *(const f32x4 *)&red[j][ww][1][4 * c4];
  }
  const float eg = hsc[2 * j], bt = hsc[2 * j + 1], kq = hsc[2 * R];
  const f32x4 v = *(const f32x4 *)(cbuf + 2 * D + j * D + 4 * c4);
  const f32x4 delta = (v - eg * sk4) * bt;
  const f32x4 o = eg * sq4 + delta * kq;

  // ---- the updated state (written once, not read again here: non-temporal)
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float kr = cbuf[D + rg * RPT + i];
    __builtin_nontemporal_store(eg * S[i] + kr * delta, (f32x4 *)(srow + (int64_t)i * D));
  }

  // ---- gated RMS norm over the value head's D outputs (lanes 0-31 of its first wavefront)
  if (rg == 0) {
    float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m, kWave);
    const float inv = 1.f / sqrtf(ss / (float)D + p.eps);
    bf16x4 y4;
#pragma unroll
    for (int e = 0; e < 4; ++e) y4[e] = (bf16_t)(o[e] * inv * (float)wn[e] * silu_f((float)zr[e]));
    *(bf16x4 *)(p.y + ((int64_t)b * Hv + h) * D + 4 * c4) = y4;
  }
}

hipError_t launch_gdn_decode(const GdnParams &p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)p.B * p.Hk)), block(kGdnThreads);
  switch (p.Hv / p.Hk) {
    case 1: hipLaunchKernelGGL(gdn_decode_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(gdn_decode_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(gdn_decode_kernel<4>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qsa
