// Device helpers shared by the libdsa kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// MFMA operand / accumulator types for v_mfma_f32_16x16x32_bf16.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bf16 (low half = lo), round to nearest even: one
// v_cvt_pk_bf16_f32.  Matches f32_to_bf16_rne on every non-NaN input.
typedef __bf16 bf16x2_vec __attribute__((ext_vector_type(2)));
typedef float f32x2_vec __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_vec v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_vec));
}

// Word i of a uint4 (i a compile-time constant after unrolling).
__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Order-preserving map of a finite float to an unsigned key (larger float ->
// larger key): 2^31 plus the value's magnitude bits, negated for a negative
// value, so -0 and +0 share the key 2^31 and no finite value (nor -inf) maps
// to 0.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  const uint32_t u = __float_as_uint(f), m = u & 0x7fffffffu;
  return (u & 0x80000000u) ? 0x80000000u - m : 0x80000000u + m;
}

// ---- cross-lane primitives at ALU latency (DPP and gfx950 permlane swaps) ----
// Lane l of v_permlane32_swap(x, x) receives {x[l % 32], x[l % 32 + 32]};
// lane l of v_permlane16_swap(x, x) receives {x[even row], x[odd row]} of its
// pair of 16-lane rows.  Combining the two halves in that fixed order gives
// bit-identical results in both lanes of each pair.

template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = true>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // i <-> 15-i within 16 lanes

// (x[lo], x[hi]) of the lane pairs l, l^16 and l, l^32.
__device__ __forceinline__ void pair16(float v, float& lo, float& hi) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(p[0]);
  hi = __uint_as_float(p[1]);
}
__device__ __forceinline__ void pair32(float v, float& lo, float& hi) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(p[0]);
  hi = __uint_as_float(p[1]);
}
// Value held by lane l ^ 16 / l ^ 32.
__device__ __forceinline__ float xor16(float v) {
  float lo, hi;
  pair16(v, lo, hi);
  return ((threadIdx.x >> 4) & 1) ? lo : hi;
}
__device__ __forceinline__ float xor32(float v) {
  float lo, hi;
  pair32(v, lo, hi);
  return ((threadIdx.x >> 5) & 1) ? lo : hi;
}
__device__ __forceinline__ int xor16_i(int v) {
  const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)(((threadIdx.x >> 4) & 1) ? p[0] : p[1]);
}
__device__ __forceinline__ int xor32_i(int v) {
  const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)(((threadIdx.x >> 5) & 1) ? p[0] : p[1]);
}
// Sum / max over the four 16-lane rows (lanes with the same l % 16).
__device__ __forceinline__ float rows_sum(float v) {
  float lo, hi;
  pair16(v, lo, hi);
  v = lo + hi;
  pair32(v, lo, hi);
  return lo + hi;
}
__device__ __forceinline__ float rows_max(float v) {
  float lo, hi;
  pair16(v, lo, hi);
  v = fmaxf(lo, hi);
  pair32(v, lo, hi);
  return fmaxf(lo, hi);
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111>(x);                 // row_shr:1
  x += dpp_i<0x112>(x);                 // row_shr:2
  x += dpp_i<0x114>(x);                 // row_shr:4
  x += dpp_i<0x118>(x);                 // row_shr:8
  x += dpp_i<0x142, 0xA, false>(x);     // row_bcast:15 into rows 1 and 3
  x += dpp_i<0x143, 0xC, false>(x);     // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<kDppXor1>((int)x));
  x = max(x, (uint32_t)dpp_i<kDppXor2>((int)x));
  x = max(x, (uint32_t)dpp_i<kDppHalfMirror>((int)x));
  x = max(x, (uint32_t)dpp_i<kDppMirror>((int)x));
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max((uint32_t)p[0], (uint32_t)p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}

// Sum over aligned groups of W lanes (W a power of two), the same bits in
// every lane of a group.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if (W >= 2) v += dpp_f<kDppXor1>(v);
  if (W >= 4) v += dpp_f<kDppXor2>(v);
  if (W >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (W >= 16) v += dpp_f<kDppMirror>(v);
  if (W >= 32) {
    float lo, hi;
    pair16(v, lo, hi);
    v = lo + hi;
  }
  if (W >= 64) {
    float lo, hi;
    pair32(v, lo, hi);
    v = lo + hi;
  }
  return v;
}

// k_norm (LayerNorm with bias, biased variance) of a row of W*8 channels held
// 8 per lane over an aligned group of W lanes; returns this lane's 8 outputs
// as bf16 (round to nearest even).
template <int W>
__device__ __forceinline__ uint4 layer_norm8_bf16(const float (&x)[8], const float (&lw)[8],
                                                  const float (&lb)[8], float eps) {
  constexpr int D = W * 8;
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) sum += x[c];
  const float mean = group_sum<W>(sum) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float d = x[c] - mean;
    sq = fmaf(d, d, sq);
  }
  const float rstd = 1.0f / sqrtf(group_sum<W>(sq) / (float)D + eps);
  uint32_t pk[4];
#pragma unroll
  for (int c = 0; c < 8; c += 2)
    pk[c >> 1] = pack_bf16x2((x[c] - mean) * rstd * lw[c] + lb[c],
                             (x[c + 1] - mean) * rstd * lw[c + 1] + lb[c + 1]);
  return make_uint4(pk[0], pk[1], pk[2], pk[3]);
}

// The 8 bf16 values of a 16-byte word as floats (exact).
__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float (&x)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t w = u4_word(v, c >> 1);
    x[c] = bf16_to_f32((c & 1) ? (w >> 16) : (w & 0xffffu));
  }
}

}  // namespace dsa
