// qsa_linear.hip -- the projections on either side of the attention core, for
// the few rows of decode and speculative verify (gfx950).
//
// qkv: q_gate | k_new | v_new = x W_qkv^T, W_qkv = [q_proj; k_proj; v_proj],
//      with q_proj's rows per head ordered [query(D) | gate(D)], so the split
//      of the doubled q_proj output into queries and gate (mlxd PR #99
//      Summary; Atlas Qwen35Kernels qkv_split) is where each output feature is
//      stored: features [0, 2 Hq D) go to q_gate [rows][Hq][2D], the next Hkv D
//      to k_new, the last Hkv D to v_new (Atlas FullAttentionLayer q_proj /
//      k_proj / v_proj).
// o:   y = attn W_o^T, attn being the gated attention output [rows][Hq D]
//      (mlxd PR #99 Summary: o_proj(attn * sigmoid(gate))).
//
// Both are y[m][n] = sum_k x[m][k] W[n][k] with W row-major [N][K] in bf16 and
// few rows m: the weights stream once from HBM and set the time.  Up to four
// rows go through gemv_kernel (below).  More rows: one workgroup per 16 output
// features; its wavefronts split K into equal
// contiguous ranges and each accumulates C^T[n][m] = W[n][:] . x[m][:] with
// v_mfma_f32_16x16x32_bf16 (A = 16 weight rows x 32 k, read straight from HBM
// as 16-byte pieces; B = 32 k x 16 rows of x, which stays in L2), up to 64 rows
// as four 16-row tiles.  The wavefronts' partial sums meet in LDS, in a fixed
// order, and the fp32 sum is rounded once to bf16.
#include "qsa_device.h"

namespace qsa {

namespace {

// MT: 16-row tiles of x (rows <= 16 MT).  WAVES: wavefronts splitting K.
template <int MT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void linear_kernel(const bf16_t *__restrict__ x,
                                                               const bf16_t *__restrict__ w, int M, int N, int K,
                                                               bf16_t *__restrict__ y0, int n0_end, int ld0,
                                                               bf16_t *__restrict__ y1, int n1_end, int ld1,
                                                               bf16_t *__restrict__ y2, int ld2) {
  __shared__ f32x4 red[WAVES][MT][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, g4 = lane >> 4, m16 = lane & 15;
  const int nb = blockIdx.x * 16;                       // first output feature of the workgroup
  const int kw = K / WAVES;                             // this wavefront's K range: [wave kw, wave kw + kw)
  const bf16_t *wr = w + (int64_t)(nb + m16) * K + wave * kw + 8 * g4;
  const bf16_t *xr[MT];
  bool xv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + m16;
    xv[mt] = m < M;
    xr[mt] = x + (int64_t)(xv[mt] ? m : 0) * K + wave * kw + 8 * g4;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Batches of U k-steps, double-buffered: the loads of the next batch are in
  // flight while the current one goes through the MFMAs.
  constexpr int U = MT <= 1 ? 8 : 4;
  const int steps = kw / 32;
  auto load = [&](int s0, bf16x8(&a)[U], bf16x8(&b)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < steps) {
        a[u] = __builtin_bit_cast(bf16x8, gld<uint4>(wr + 32 * (s0 + u)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          b[u][mt] = xv[mt] ? __builtin_bit_cast(bf16x8, gld<uint4>(xr[mt] + 32 * (s0 + u))) : bf16x8{};
      }
    }
  };
  auto compute = [&](int s0, const bf16x8(&a)[U], const bf16x8(&b)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < steps) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_qk(a[u], b[u][mt], acc[mt]);
      }
  };
  bf16x8 a0[U], b0[U][MT], a1[U], b1[U][MT];
  load(0, a0, b0);
  for (int s0 = 0; s0 < steps; s0 += 2 * U) {
    if (s0 + U < steps) load(s0 + U, a1, b1);
    compute(s0, a0, b0);
    if (s0 + 2 * U < steps) load(s0 + 2 * U, a0, b0);
    if (s0 + U < steps) compute(s0 + U, a1, b1);
  }
  // lane (g4, m16) holds C^T[4 g4 + i][m16]: features nb + 4 g4 + i of row 16 mt + m16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x4 s = red[0][mt][lane];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) s += red[v][mt][lane];
    const int m = 16 * mt + m16;
    if (m >= M) continue;
    const int n = nb + 4 * g4;                          // four consecutive features, all in one output
    bf16x4 o4;
#pragma unroll
    for (int i = 0; i < 4; ++i) o4[i] = (bf16_t)s[i];
    bf16_t *dst = n < n0_end ? y0 + (int64_t)m * ld0 + n
                             : n < n1_end ? y1 + (int64_t)m * ld1 + (n - n0_end) : y2 + (int64_t)m * ld2 + (n - n1_end);
    *(bf16x4 *)dst = o4;
  }
}

// Few rows (MR <= 4): one output feature per wavefront, no MFMA.  Lane l
// holds elements 8 l .. 8 l + 7 of every 512-wide piece of the weight row, so
// each load instruction reads 1 KB of one contiguous row, and all of a row's
// pieces are in flight at once; x's matching pieces (L2-resident) are loaded
// alongside.  The fp32 products are summed over the lane's pieces, then over
// the 64 lanes (a fixed tree of lane swaps), and lane 0 rounds and stores.
// PMAX: the largest piece count the registers are sized for (K <= 512 PMAX);
// sized to the call, so that short rows leave room for more wavefronts per
// SIMD and so more loads in flight per CU.
constexpr int kGemvMaxPieces = 16;                      // K <= 16 * 512
template <int MR, int PMAX>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const bf16_t *__restrict__ x, const bf16_t *__restrict__ w,
                                                        int N, int K, bf16_t *__restrict__ y0, int n0_end, int ld0,
                                                        bf16_t *__restrict__ y1, int n1_end, int ld1,
                                                        bf16_t *__restrict__ y2, int ld2) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int n = blockIdx.x * (kThreads / kWave) + wave;
  if (n >= N) return;
  const int pieces = K / 512;
  const bf16_t *wr = w + (int64_t)n * K + 8 * lane;
  uint4 wv[PMAX], xv[MR][PMAX];
#pragma unroll
  for (int j = 0; j < PMAX; ++j)
    if (j < pieces) {
      wv[j] = gld<uint4>(wr + 512 * j);
#pragma unroll
      for (int m = 0; m < MR; ++m) xv[m][j] = gld<uint4>(x + (int64_t)m * K + 8 * lane + 512 * j);
    }
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll
  for (int j = 0; j < PMAX; ++j)
    if (j < pieces) {
      const bf16x8 wb = __builtin_bit_cast(bf16x8, wv[j]);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const bf16x8 xb = __builtin_bit_cast(bf16x8, xv[m][j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[m] = fmaf((float)xb[i], (float)wb[i], acc[m]);
      }
    }
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = rows4_sum(row16_sum(acc[m]));
  if (lane != 0) return;
  bf16_t *dst = n < n0_end ? y0 + n : n < n1_end ? y1 + (n - n0_end) : y2 + (n - n1_end);
  const int ld = n < n0_end ? ld0 : n < n1_end ? ld1 : ld2;
#pragma unroll
  for (int m = 0; m < MR; ++m) dst[(int64_t)m * ld] = (bf16_t)acc[m];
}

template <int MR>
hipError_t launch_gemv_mr(const bf16_t *x, const bf16_t *w, int N, int K, bf16_t *y0, int n0_end, int ld0, bf16_t *y1,
                          int n1_end, int ld1, bf16_t *y2, int ld2, hipStream_t s) {
  const dim3 grid((N + kThreads / kWave - 1) / (kThreads / kWave));
  const int pieces = K / 512;
  if (pieces <= 4)
    hipLaunchKernelGGL((gemv_kernel<MR, 4>), grid, dim3(kThreads), 0, s, x, w, N, K, y0, n0_end, ld0, y1, n1_end,
                       ld1, y2, ld2);
  else if (pieces <= 8)
    hipLaunchKernelGGL((gemv_kernel<MR, 8>), grid, dim3(kThreads), 0, s, x, w, N, K, y0, n0_end, ld0, y1, n1_end,
                       ld1, y2, ld2);
  else
    hipLaunchKernelGGL((gemv_kernel<MR, kGemvMaxPieces>), grid, dim3(kThreads), 0, s, x, w, N, K, y0, n0_end, ld0,
                       y1, n1_end, ld1, y2, ld2);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_linear_mt(const bf16_t *x, const bf16_t *w, int M, int N, int K, bf16_t *y0, int n0_end, int ld0,
                            bf16_t *y1, int n1_end, int ld1, bf16_t *y2, int ld2, int waves, hipStream_t s) {
  const dim3 grid(N / 16);
  if (waves == 8)
    hipLaunchKernelGGL((linear_kernel<MT, 8>), grid, dim3(8 * kWave), 0, s, x, w, M, N, K, y0, n0_end, ld0, y1,
                       n1_end, ld1, y2, ld2);
  else
    hipLaunchKernelGGL((linear_kernel<MT, 4>), grid, dim3(4 * kWave), 0, s, x, w, M, N, K, y0, n0_end, ld0, y1,
                       n1_end, ld1, y2, ld2);
  return hipGetLastError();
}

}  // namespace

// y0 takes features [0, n0_end), y1 [n0_end, n1_end), y2 the rest; ld*: row
// strides in elements.  Requires N % 16 == 0, K % (32 waves) == 0, the three
// boundaries on multiples of 4, M <= 64.  Eight wavefronts split K when there
// are too few 16-feature tiles to give every CU a workgroup with four.
hipError_t launch_linear_bf16(const void *x, const void *w, int M, int N, int K, void *y0, int n0_end, int ld0,
                              void *y1, int n1_end, int ld1, void *y2, int ld2, hipStream_t s) {
  const int waves = (N / 16 < 384 && K % (32 * 8) == 0) ? 8 : 4;
  const bf16_t *xb = (const bf16_t *)x, *wb = (const bf16_t *)w;
  bf16_t *a = (bf16_t *)y0, *b = (bf16_t *)y1, *c = (bf16_t *)y2;
  if (M <= 4 && K % 512 == 0 && K <= 512 * kGemvMaxPieces) {
    switch (M) {
      case 1: return launch_gemv_mr<1>(xb, wb, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, s);
      case 2: return launch_gemv_mr<2>(xb, wb, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, s);
      case 3: return launch_gemv_mr<3>(xb, wb, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, s);
      default: return launch_gemv_mr<4>(xb, wb, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, s);
    }
  }
  switch ((M + 15) / 16) {
    case 1: return launch_linear_mt<1>(xb, wb, M, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, waves, s);
    case 2: return launch_linear_mt<2>(xb, wb, M, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, waves, s);
    case 3:
    case 4: return launch_linear_mt<4>(xb, wb, M, N, K, a, n0_end, ld0, b, n1_end, ld1, c, ld2, waves, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qsa
