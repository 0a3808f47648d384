// qsa_device.h -- device helpers shared by the streaming and tile kernels
// (gfx950): stage geometry of the HBM -> LDS key ring, the copies and their
// explicit counter waits, the XOR row swizzle, cross-lane reductions without
// LDS traffic, and global loads that stay in the global address space.
#pragma once

#include <type_traits>

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct Geo {
  static constexpr int RB = 2 * D;                      // bytes of one key row of one KV head
  static constexpr int OCT = D / 8;                     // 16-byte units per row
  static constexpr int SW = (OCT < 16 ? OCT : 16) - 1;  // XOR swizzle mask over units
  static constexpr int SK = 64;                         // keys per stage
  static constexpr int STAGE = SK * RB;                 // bytes per stage and tensor
  static constexpr int RING = 65536;                    // bytes per tensor ring
  static constexpr int NS = RING / STAGE;               // stages in flight
  static constexpr int LPS = SK * OCT / kThreads;       // 16-byte copies per thread, stage and tensor
  static constexpr int KST = D / 32;                    // k-steps of the score product
  static constexpr int NDB = D / 16;                    // 16-dim blocks of the value product
  static constexpr int E = D / 16;                      // elements per lane in row work (16 lanes per row)
};

__device__ __forceinline__ f32x4 mfma_qk(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_qk(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16-bit MFMA operand types: bf16 (the bf16 cache's own values) or fp16 (values
// that need more than bf16's 8 significant bits, such as decoded Turbo8 codes).
template <typename T> struct Op16;
template <> struct Op16<bf16_t> { using x8 = bf16x8; using x4 = bf16x4; };
template <> struct Op16<f16_t> { using x8 = f16x8; using x4 = f16x4; };

__device__ __forceinline__ float sigmoid_f(float z) { return 1.f / (1.f + __expf(-z)); }

// max of two floats as NaN-propagating maximum (v_maximum3_f32), which takes
// its operands as they are: fmaxf has the compiler quiet each operand first
// with an instruction of its own.  Scores and maxima here are finite or -inf.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// Cross-lane reductions without LDS traffic.  Each step combines a lane with
// one partner symmetrically (a + b == b + a), so every lane of a group ends
// with the bitwise same value.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {   // DPP move (row_ror / quad_perm), all lanes valid
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// sum over the 16 lanes of a row
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0x128>(v);   // row_ror:8
  v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  return v;
}
// max over the 16 lanes of a row
__device__ __forceinline__ float row16_max(float v) {
  v = fmax_nan(v, dpp<0x128>(v));   // row_ror:8
  v = fmax_nan(v, dpp<0x124>(v));   // row_ror:4
  v = fmax_nan(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmax_nan(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  return v;
}
// combine lanes i, i^16, i^32, i^48 (the four rows) with gfx950's lane swaps
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax_nan(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Waits for this wave's LDS operations, then for every wave of the workgroup.
// Vector-memory copies still in flight are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte HBM -> LDS copies, one per lane: lane i writes LDS bytes lds + 16 i.
// The LDS address must be uniform over the wave (it goes through M0).
// The source is a wave-uniform base address (SGPRs) plus a 32-bit byte
// offset per lane.
__device__ __forceinline__ void dma16_sbase(const void *base, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// The same copy from a 64-bit address per lane (paged caches, whose rows of
// one stage need not be contiguous).
__device__ __forceinline__ void dma16_vaddr(const void *src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// The same copy of one dword per lane: lane i writes LDS bytes lds + 4 i.
__device__ __forceinline__ void dma4_sbase(const void *base, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// f(std::integral_constant<int, j>) for j = 0 .. N-1, in order (a loop whose
// index is a compile-time constant in the body).
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>());
  }
}

// Waits until at most u * PER vector-memory operations of this wave are
// outstanding (u wave-uniform, 0 <= u <= MAXU).
template <int PER, int MAXU>
struct WaitUnits {
  static_assert(PER * MAXU <= 63, "vmcnt field");
  __device__ static __forceinline__ void run(int u) {
    if (u == MAXU) {
      wait_vm<MAXU * PER>();
      return;
    }
    WaitUnits<PER, MAXU - 1>::run(u);
  }
};
template <int PER>
struct WaitUnits<PER, 0> {
  __device__ static __forceinline__ void run(int) { wait_vm<0>(); }
};

// Wait until at most `younger` stages (2 * LPS copies each) are outstanding.
template <int LPS2, int NS>
__device__ __forceinline__ void wait_stages(int younger) {
  static_assert((NS - 1) * LPS2 <= 63, "vmcnt field");
  switch (younger) {
    case 0: wait_vm<0>(); break;
    case 1: if constexpr (NS > 1) wait_vm<1 * LPS2>(); break;
    case 2: if constexpr (NS > 2) wait_vm<2 * LPS2>(); break;
    case 3: if constexpr (NS > 3) wait_vm<3 * LPS2>(); break;
    case 4: if constexpr (NS > 4) wait_vm<4 * LPS2>(); break;
    case 5: if constexpr (NS > 5) wait_vm<5 * LPS2>(); break;
    case 6: if constexpr (NS > 6) wait_vm<6 * LPS2>(); break;
    default: if constexpr (NS > 7) wait_vm<7 * LPS2>(); break;
  }
}

// Global loads through the global address space (never flat).
template <typename T> struct nat { using type = T; };
template <> struct nat<uint4> { using type = unsigned __attribute__((ext_vector_type(4))); };
template <> struct nat<uint2> { using type = unsigned __attribute__((ext_vector_type(2))); };
template <> struct nat<float2> { using type = float __attribute__((ext_vector_type(2))); };
template <> struct nat<float4> { using type = float __attribute__((ext_vector_type(4))); };
template <typename T>
__device__ __forceinline__ T gld(const void *ptr) {
  using N = typename nat<T>::type;
  return __builtin_bit_cast(T, *(const __attribute__((address_space(1))) N *)ptr);
}

// E consecutive bf16 values as raw 16- or 8-byte pieces.
template <int E>
struct RawE {
  static constexpr int NV = E >= 8 ? E / 8 : 1;
  using V = typename std::conditional<E >= 8, uint4, uint2>::type;
  V v[NV];
  __device__ __forceinline__ void load(const bf16_t *src) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = gld<V>(src + i * (E >= 8 ? 8 : 4));
  }
  // Make the compiler wait for the load here (an empty use of the registers).
  __device__ __forceinline__ void land() const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const typename nat<V>::type r = __builtin_bit_cast(typename nat<V>::type, v[i]);
      asm volatile("" ::"v"(r));
    }
  }
  // Byte offset of piece i (elements [e0 + 8 i, ..) for E >= 8, or the half
  // unit holding [e0, e0 + 4) for E == 4) in a tile of rb-byte rows whose
  // 16-byte units are XOR-swizzled by the row (the layout of put_row_bf16).
  template <int SW>
  __device__ __forceinline__ static int lds_off(int rb, int row, int e0, int i) {
    return E >= 8 ? row * rb + 16 * ((e0 / 8 + i) ^ (row & SW)) : row * rb + 16 * ((e0 / 8) ^ (row & SW)) + 8 * ((e0 / 4) & 1);
  }
  template <int SW>
  __device__ __forceinline__ void store_lds(unsigned char *tile, int rb, int row, int e0) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) *(V *)(tile + lds_off<SW>(rb, row, e0, i)) = v[i];
  }
  template <int SW>
  __device__ __forceinline__ void load_lds(const unsigned char *tile, int rb, int row, int e0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = *(const V *)(tile + lds_off<SW>(rb, row, e0, i));
  }
  __device__ __forceinline__ void to_float(float *x) const {
    constexpr int PER = E >= 8 ? 8 : 4;
    typedef __bf16 bfP __attribute__((ext_vector_type(PER)));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bfP b = __builtin_bit_cast(bfP, v[i]);
#pragma unroll
      for (int j = 0; j < PER; ++j) x[i * PER + j] = (float)b[j];
    }
  }
};

// Byte offset of (row, 16-byte unit) in a swizzled tile of `rb`-byte rows.
template <int SW>
__device__ __forceinline__ int swz(int row, int unit, int rb) {
  return row * rb + 16 * (unit ^ (row & SW));
}

// Store E floats (rounded to the 16-bit type T, nearest even) of one row at
// elements [e0, e0 + E) of a swizzled tile.
template <int D, typename T = bf16_t>
__device__ __forceinline__ void put_row(unsigned char *tile, int rb, int row, int e0, const float *x) {
  using G = Geo<D>;
  using V8 = typename Op16<T>::x8;
  using V4 = typename Op16<T>::x4;
  constexpr int E = G::E;
  if constexpr (E >= 8) {
#pragma unroll
    for (int u = 0; u < E / 8; ++u) {
      V8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (T)x[8 * u + j];
      *(V8 *)(tile + swz<G::SW>(row, e0 / 8 + u, rb)) = v;
    }
  } else {
    V4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (T)x[j];
    *(V4 *)(tile + swz<G::SW>(row, e0 / 8, rb) + 8 * ((e0 / 4) & 1)) = v;
  }
}
template <int D>
__device__ __forceinline__ void put_row_bf16(unsigned char *tile, int rb, int row, int e0, const float *x) {
  put_row<D, bf16_t>(tile, rb, row, e0, x);
}


// RMS norm of one head row held by 16 lanes (E = D/16 elements each, lane
// c16 holding elements E c16 .. E c16 + E - 1): x * w / sqrt(mean(x^2) + eps)
// (mlxd PR #99, config audit table, has_qk_norm; Atlas FullAttentionLayer
// q_norm / k_norm).  A row that is not valid becomes zero.
template <int D>
__device__ __forceinline__ void row_norm(float (&x)[D / 16], const float (&w)[D / 16], bool valid, float eps) {
  constexpr int E = D / 16;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) ss += x[j] * x[j];
  ss = row16_sum(ss);
  const float inv = valid ? 1.0f / sqrtf(ss / (float)D + eps) : 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) x[j] = x[j] * inv * w[j];
}

// row_norm, then the partial rotation of the first r dims, dim i paired with
// dim i + r/2 (mlxd PR #99 Summary, partial_rotary_factor; Atlas
// Qwen35ForwardConfig::rotary_dim).  cs: (cos, sin) of this row's position for
// pairs 0 .. r/2-1, 16-byte aligned.  Only rotary dims with r/2 a multiple of
// E are taken here, so every rotated lane holds E elements of one half, its
// partner lane is r/(2E) lanes away in the same row, and its pairs are the E
// consecutive pairs from i0: the partner values come over by lane permutes and
// the pair table is read as whole vectors.  Every lane of the wavefront must
// take part.  This is the one routine that normalises and rotates new keys
// before they are stored, whichever entry point stores them.
template <int D>
__device__ __forceinline__ void norm_rope(float (&x)[D / 16], const float (&w)[D / 16], bool valid, float eps,
                                          int r, const float2 *cs) {
  constexpr int E = D / 16;
  const int lane = threadIdx.x % kWave, c16 = lane & 15;
  row_norm<D>(x, w, valid, eps);
  if (r == 0) return;
  const int half = r / 2, e0 = c16 * E, nl = half / E;
  const bool lo = e0 < half, rot = e0 < r;
  const int src = rot ? (lo ? lane + nl : lane - nl) : lane;
  float xp[E];
#pragma unroll
  for (int j = 0; j < E; ++j) xp[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(x[j])));
  if (!rot) return;
  const int i0 = lo ? e0 : e0 - half;
  float4 cs4[E / 2];
#pragma unroll
  for (int j = 0; j < E / 2; ++j) cs4[j] = *(const float4 *)(cs + i0 + 2 * j);
  const float sg = lo ? -1.f : 1.f;                     // lo: x c - x' s; hi: x c + x' s
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float cj = j % 2 == 0 ? cs4[j / 2].x : cs4[j / 2].z;
    const float sj = j % 2 == 0 ? cs4[j / 2].y : cs4[j / 2].w;
    x[j] = fmaf(sg * xp[j], sj, x[j] * cj);
  }
}

// Orthonormal Walsh-Hadamard transform of one head row held by 16 lanes
// (lane c16 holds elements E c16 .. E c16 + E - 1): butterflies (a, b) ->
// (a + b, a - b) over every bit of the element index, the low log2(E) bits
// inside the lane and the four lane bits across lanes, then a scale of
// 1/sqrt(D).  Sylvester order, its own inverse (Atlas Qwen35Kernels
// wht_bf16_inplace / wht_bf16_inplace_inv: the rotation bookends of the Turbo
// KV formats).  Every lane of the wavefront must take part.
template <int D>
__device__ __forceinline__ void row_wht(float (&x)[D / 16]) {
  constexpr int E = D / 16;
  const int c16 = threadIdx.x & 15;
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (!(j & h)) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
#pragma unroll
  for (int lh = 1; lh < 16; lh <<= 1) {
    const bool up = c16 & lh;                           // this lane holds the b of each pair
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float o = __shfl_xor(x[j], lh, kWave);
      x[j] = up ? o - x[j] : x[j] + o;
    }
  }
  const float norm = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int j = 0; j < E; ++j) x[j] *= norm;
}

// Two floats to E4M3 codes in the low (hi = false) or high half of a dword, and
// two codes from a dword's low or high half to floats (gfx950's conversions:
// round to nearest even, the OCP E4M3 format; the halves must be constants).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_fp8(float a, float b, uint32_t old, bool hi) {
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}
__device__ __forceinline__ f32x2_t unpk_fp8(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// Turbo8 groups of 16 consecutive elements (Atlas MetalKvDtype::Turbo8: FP8
// E4M3 codes with a bf16 scale per 16 elements).  A group spans 16 / E lanes
// of a 16-lane row (one lane for D = 256).  The scale is the group's largest
// magnitude over 448 (the largest E4M3 value), rounded to bf16; a code is
// x / scale rounded to nearest E4M3, ties to even, after clamping to +-448
// (the hardware conversion turns larger values into NaN rather than
// saturating); a zero group has a zero scale and zero codes.  All in fp32.
template <int D>
struct Turbo8Row {
  static constexpr int E = D / 16;
  static constexpr int LPG = 16 / E < 1 ? 1 : 16 / E;   // lanes per group
  static constexpr int CW = (E + 3) / 4;                // dwords of codes per lane
  uint32_t codes[CW];                                   // E codes, byte j of element j
  bf16_t scale;                                         // this lane's group scale
  __device__ __forceinline__ void quantize(const float (&x)[E]) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
    for (int lh = 1; lh < LPG; lh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, lh, kWave));
    scale = (bf16_t)(amax / 448.0f);
    const float s = (float)scale;
#pragma unroll
    for (int w = 0; w < CW; ++w) codes[w] = 0;
    if (s == 0.f) return;
#pragma unroll
    for (int j = 0; j < E; j += 2) {
      const float a = fminf(fmaxf(x[j] / s, -448.f), 448.f);
      const float b = fminf(fmaxf(x[j + 1] / s, -448.f), 448.f);
      codes[j / 4] = pk_fp8(a, b, codes[j / 4], (j % 4) != 0);
    }
  }
  // codes x scale in fp32 (exact: 4 x 8 significant bits)
  __device__ __forceinline__ void dequantize(float (&x)[E]) const {
    const float s = (float)scale;
#pragma unroll
    for (int j = 0; j < E; j += 2) {
      const f32x2_t f = unpk_fp8(codes[j / 4], (j % 4) != 0);
      x[j] = f[0] * s;
      x[j + 1] = f[1] * s;
    }
  }
};

// Turbo4 groups of 16 consecutive elements (the V side of Atlas
// MetalKvDtype::Bf16KTurbo4V): 4-bit indices into a 16-level codebook and one
// E4M3 scale per group.  A group's indices are the levels nearest to x / sigma
// (sigma the group's RMS; the count of decision thresholds below it, so the
// lower level on a tie) and its scale is sqrt(sum x^2 / sum level^2) in E4M3
// (round to nearest even, after a clamp at 448), so that the decoded group
// keeps the group's L2 norm; a zero group has scale 0 and index 0.  Indices
// pack two per byte, element 2i in the low nibble.  cb: the 16 levels in LDS;
// thr: the 15 thresholds.  fp32 throughout.  A group spans 16 / E lanes of a
// 16-lane row.
template <int D>
struct Turbo4Row {
  static constexpr int E = D / 16;
  static constexpr int LPG = 16 / E < 1 ? 1 : 16 / E;   // lanes per group
  static constexpr int CW = (E / 2 + 3) / 4;            // dwords of packed indices per lane
  uint32_t codes[CW];
  uint32_t scale;                                       // E4M3 bits (byte 0)
  __device__ __forceinline__ void quantize(const float (&x)[E], const float *cb, const float (&thr)[15]) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) ss = fmaf(x[j], x[j], ss);
#pragma unroll
    for (int lh = 1; lh < LPG; lh <<= 1) ss += __shfl_xor(ss, lh, kWave);
#pragma unroll
    for (int w = 0; w < CW; ++w) codes[w] = 0;
    scale = 0;
    const float sigma = sqrtf(ss / 16.f);
    float cc = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float u = ss > 0.f ? x[j] / sigma : 0.f;
      int idx = 0;
#pragma unroll
      for (int t = 0; t < 15; ++t) idx += thr[t] < u ? 1 : 0;
      if (ss == 0.f) idx = 0;
      const float c = cb[idx];
      cc = fmaf(c, c, cc);
      codes[j / 8] |= (uint32_t)idx << (4 * (j % 8));
    }
#pragma unroll
    for (int lh = 1; lh < LPG; lh <<= 1) cc += __shfl_xor(cc, lh, kWave);
    if (ss > 0.f) scale = pk_fp8(fminf(sqrtf(ss / cc), 448.f), 0.f, 0u, false) & 0xffu;
  }
  // level x scale in fp32
  __device__ __forceinline__ void dequantize(float (&x)[E], const float *cb) const {
    const float s = unpk_fp8(scale, false)[0];
#pragma unroll
    for (int j = 0; j < E; ++j) x[j] = s * cb[(codes[j / 8] >> (4 * (j % 8))) & 15u];
  }
};

// Turbo8 codes to fp16 MFMA operands, code x scale rounded once to nearest
// even (exact in fp32: 4 x 8 significant bits).  gfx950's scaled conversion
// takes only the exponent of its fp32 scale, so it gives code x 2^e exactly
// (the scale being 1.m x 2^e); one packed fp16 multiply by 1.m (exact in fp16)
// then rounds the product.  Values that fall below fp16's normal range (2^-14)
// keep fewer bits, and values past 65504 overflow.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
struct T8Scale {
  float e;                                              // the scale itself: its exponent is used
  f16x2_t m;                                            // (1.m, 1.m)
  __device__ __forceinline__ explicit T8Scale(uint32_t bf16_bits) {
    const uint32_t bits = bf16_bits << 16;
    e = __uint_as_float(bits);
    const _Float16 h = (_Float16)__uint_as_float((bits & 0x007F0000u) | 0x3F800000u);
    m = f16x2_t{h, h};
  }
};
// codes 0-3 of w (byte j = code j) decoded into fp16
__device__ __forceinline__ f16x4 t8_decode4(uint32_t w, const T8Scale &s) {
  const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s.e, false) * s.m;
  const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s.e, true) * s.m;
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ f16x8 t8_decode8(uint32_t w0, uint32_t w1, const T8Scale &s) {
  const f16x4 a = t8_decode4(w0, s), b = t8_decode4(w1, s);
  return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Exchange area of one stage: the probability tile P[row tile][row][key] in
// bf16 (row stride padded to 144 bytes, conflict-free for the 16-byte reads
// of the value product) and each wavefront's block maxima and sums per row.
struct Xch {
  static constexpr int PSTRIDE = 64 * 2 + 16;
  static constexpr int PBYTES = 4 * 16 * PSTRIDE;
  static constexpr int FLAGS = PBYTES + 2 * 4 * 64 * 4;    // after the block maxima and sums
  static constexpr int BYTES = FLAGS + 16;
};

// One stage of up to 64 keys (global indices key0 ..) held in swizzled LDS
// tiles kt / vt of RB-byte rows.  Wavefront w scores keys 16w .. 16w+15 against
// every row tile; the four wavefronts agree on each row's new running max
// through LDS and publish their probabilities as one bf16 tile; then each
// wavefront accumulates its own D/4 output dims over all keys of the stage.
// Key k is visible to row r when k < nkeys and key0 + k <= lim[r] (causal
// limit n_b + l_r).  When every row already has a reference max, each wave
// publishes its probabilities against it at once, with a flag if one of its
// block maxima passes it by more than kMaxLead; only then is the stage
// published again from the agreed maxima.  So a stage holds one workgroup
// barrier, two on its first keys or when the reference moves; on_k_free runs
// after the first, when no wave reads the K tile any more.
constexpr float kMaxLead = 8.f;

struct NoOp {
  __device__ void operator()() const {}
};

// The score product's K operand of k-step ks for this lane (key m16 of the
// wavefront's block kb, dims 8 (4 ks + g4) .. + 7) from a swizzled tile of
// 16-bit values.
template <int D, typename T>
struct TileK {
  __device__ __forceinline__ typename Op16<T>::x8 operator()(const unsigned char *kb, int ks) const {
    const int lane = threadIdx.x % kWave;
    return *(const typename Op16<T>::x8 *)(kb + swz<Geo<D>::SW>(lane & 15, 4 * ks + (lane >> 4), Geo<D>::RB));
  }
};

template <int D, int RTM, typename KFree = NoOp, typename T = bf16_t, typename KOp = TileK<D, T>>
__device__ __forceinline__ void attend_stage(const unsigned char *kt, const unsigned char *vt, int nkeys, int key0,
                                             const typename Op16<T>::x8 (&qf)[RTM][D / 32], f32x4 (&O)[RTM][D / 64],
                                             float (&m)[RTM], float (&lsum)[RTM], const int (&lim)[RTM],
                                             float scale_log2, unsigned char *xch, KFree on_k_free = KFree(),
                                             const KOp &kop = KOp()) {
  using G = Geo<D>;
  using V8 = typename Op16<T>::x8;
  using V4 = typename Op16<T>::x4;
  constexpr int KST = D / 32, DBW = D / 64, RB = G::RB;
  const int lane = threadIdx.x % kWave, g4 = lane >> 4, m16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  float *const wmax = (float *)(xch + Xch::PBYTES);     // [4 waves][64 rows]
  float *const wsum = wmax + 4 * 64;
  const int nvalid = max(0, min(16, nkeys - 16 * wave));

  // scores of this wavefront's 16 keys
  f32x4 S[RTM];
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) S[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nvalid > 0) {
    // Every K operand is read before the first product, so the reads overlap
    // one another instead of each product waiting out its own read's latency.
    // One row tile accumulates in two chains (even and odd column blocks),
    // which halves the chain of dependent products; they are summed at the end.
    const unsigned char *kb = kt + 16 * wave * RB;
    V8 a[KST];
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) a[ks] = kop(kb, ks);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RTM == 1) {
      f32x4 S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KST; ks += 2) {
        S[0] = mfma_qk(a[ks], qf[0][ks], S[0]);
        S1 = mfma_qk(a[ks + 1], qf[0][ks + 1], S1);
      }
      S[0] += S1;
    } else {
#pragma unroll
      for (int ks = 0; ks < KST; ++ks)
#pragma unroll
        for (int rt = 0; rt < RTM; ++rt) S[rt] = mfma_qk(a[ks], qf[rt][ks], S[rt]);
    }
  }
  float sc[RTM][4];
  bool fresh = false, lifts = false;
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    // keys j of this wavefront with j < vis are visible to the lane's row
    const int vis = min(lim[rt] - key0 - 16 * wave + 1, nvalid);
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * g4 + i;
      sc[rt][i] = j < vis ? S[rt][i] * scale_log2 : -INFINITY;
      bm = fmax_nan(bm, sc[rt][i]);
    }
    bm = rows4_max(bm);
    if (g4 == 0) wmax[wave * 64 + 16 * rt + m16] = bm;
    fresh |= m[rt] == -INFINITY;
    lifts |= bm > m[rt] + kMaxLead;
  }
  // every wave holds the same reference max per row, so fresh is the same in all
  fresh = __any(fresh);
  int *const wflag = (int *)(xch + Xch::FLAGS);

  // reference max of each row, probabilities, block sums.  The reference max
  // moves only when the stage max passes it by more than kMaxLead (log2
  // units), so probabilities stay <= 2^kMaxLead and the output rescale is rare;
  // sums and outputs always refer to the current reference, which is what the
  // merge receives.  exp2 is v_exp_f32 (results below 2^-126 flush to zero).
  float alpha[RTM];
  bool rescale = false;
  auto publish = [&](bool agreed) {                     // agreed: from the four block maxima
#pragma unroll
    for (int rt = 0; rt < RTM; ++rt) {
      const int row = 16 * rt + m16;
      float mu = m[rt];
      alpha[rt] = 1.f;
      if (agreed) {
        const float M = fmax_nan(fmax_nan(wmax[row], wmax[64 + row]), fmax_nan(wmax[128 + row], wmax[192 + row]));
        const bool grow = M > m[rt] + kMaxLead;         // also when m is -inf and M is finite
        const float mn = grow ? M : m[rt];
        mu = mn == -INFINITY ? 0.f : mn;
        alpha[rt] = __builtin_amdgcn_exp2f(m[rt] - mu);
        rescale |= grow && m[rt] != -INFINITY;
        m[rt] = mn;
      }
      float ps = 0.f;
      V4 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = (T)__builtin_amdgcn_exp2f(sc[rt][i] - mu);
        ps += (float)pv[i];
      }
      *(V4 *)(xch + (16 * rt + m16) * Xch::PSTRIDE + 2 * (16 * wave + 4 * g4)) = pv;
      ps = rows4_sum(ps);
      if (g4 == 0) wsum[wave * 64 + row] = ps;
    }
  };
  if (fresh) {
    lds_barrier();
    on_k_free();                                        // every wave is done with the K tile
    publish(true);
    lds_barrier();
  } else {
    // against the current reference (alpha = 1, the same values as publish(true)
    // gives when no row's reference moves)
    if (lane == 0) wflag[wave] = __any(lifts) ? 1 : 0;
    publish(false);
    lds_barrier();
    on_k_free();
    if (wflag[0] | wflag[1] | wflag[2] | wflag[3]) {    // the same in every wave
      publish(true);                                    // each wave rewrites only its own columns and sums
      lds_barrier();
    }
  }
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    const int row = 16 * rt + m16;
    lsum[rt] = lsum[rt] * alpha[rt] + ((wsum[row] + wsum[64 + row]) + (wsum[128 + row] + wsum[192 + row]));
  }
  if (__any(rescale)) {
#pragma unroll
    for (int rt = 0; rt < RTM; ++rt)
#pragma unroll
      for (int db = 0; db < DBW; ++db) O[rt][db] *= alpha[rt];
  }

  // value product over this wavefront's dims: O^T[dim][row] += V^T[dim][key] P^T[key][row].
  // V^T operand (dims dim0 + m16, keys kb + 8 g4 .. + 7) from two transposing
  // reads; lane (g4, i) addresses the 8-byte piece (key kb + 8 g4 + i/4 (+4),
  // dims dim0 + 4 (i%4) ..) of the swizzled V tile.
  // Both 32-key halves' operands are read before the first product (the
  // second half only when the stage has keys there).
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const bool two = nkeys > 32;
  V8 bp[2][RTM], va[2][DBW];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks == 1 && !two) break;
#pragma unroll
    for (int rt = 0; rt < RTM; ++rt)
      bp[ks][rt] = *(const V8 *)(xch + (16 * rt + m16) * Xch::PSTRIDE + 2 * (32 * ks + 8 * g4));
    const int vk = 32 * ks + 8 * g4 + (m16 >> 2), q4 = m16 & 3;
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      const int unit = 2 * (DBW * wave + db) + (q4 >> 1);
      const unsigned char *p0 = vt + swz<G::SW>(vk, unit, RB) + 8 * (q4 & 1);
      const unsigned char *p1 = vt + swz<G::SW>(vk + 4, unit, RB) + 8 * (q4 & 1);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
      const s16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      va[ks][db] = __builtin_bit_cast(V8, v8);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks == 1 && !two) break;
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int rt = 0; rt < RTM; ++rt) O[rt][db] = mfma_qk(va[ks][db], bp[ks][rt], O[rt][db]);
  }
}

// The new rows attended by each wavefront on its own, as the first keys of the
// chunk (m = -inf, sums and outputs zero): at most 16 keys, K and V rows 0 ..
// 15 at kt and vt (rows >= nkeys finite).  All of them lie in one 16-key block,
// so every wavefront scores that block against every row tile (the same MFMA
// as a stage), takes the causal mask, reference max and sums within itself,
// and runs the value product over its own dims from 16x16x16 MFMAs, whose B
// operand is the score tile's own layout (lane group g4: keys 4 g4 .. 4 g4 + 3).
template <int D, int RTM>
__device__ __forceinline__ void attend_new_rows(const unsigned char *kt, const unsigned char *vt, int nkeys, int key0,
                                                const bf16x8 (&qf)[RTM][D / 32], f32x4 (&O)[RTM][D / 64],
                                                float (&m)[RTM], float (&lsum)[RTM], const int (&lim)[RTM],
                                                float scale_log2) {
  using G = Geo<D>;
  constexpr int KST = D / 32, DBW = D / 64, RB = G::RB;
  const int lane = threadIdx.x % kWave, g4 = lane >> 4, m16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int vk = 4 * g4 + (m16 >> 2), q4 = m16 & 3;
#pragma unroll
  for (int rt = 0; rt < RTM; ++rt) {
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) S = mfma_qk(*(const bf16x8 *)(kt + swz<G::SW>(m16, 4 * ks + g4, RB)), qf[rt][ks], S);
    const int vis = min(lim[rt] - key0 + 1, nkeys);
    float sc[4], bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = 4 * g4 + i < vis ? S[i] * scale_log2 : -INFINITY;
      bm = fmax_nan(bm, sc[i]);
    }
    const float M = rows4_max(bm);                      // the reference: m was -inf
    const float mu = M == -INFINITY ? 0.f : M;
    m[rt] = M;
    bf16x4 pv;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = (bf16_t)__builtin_amdgcn_exp2f(sc[i] - mu);
      ps += (float)pv[i];
    }
    lsum[rt] = rows4_sum(ps);
    const s16x4 pb = __builtin_bit_cast(s16x4, pv);
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      // lane (g4, i) addresses the 8-byte piece (key 4 g4 + i/4, dims 16 (DBW w + db) + 4 (i%4) ..)
      const unsigned char *pa = vt + swz<G::SW>(vk, 2 * (DBW * wave + db) + (q4 >> 1), RB) + 8 * (q4 & 1);
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)pa);
      O[rt][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, O[rt][db], 0, 0, 0);
    }
  }
}

}  // namespace
}  // namespace qsa
