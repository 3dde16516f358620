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

// Word i of a uint4 (i a compile-time constant after unrolling).
__device__ __forceinline__ uint32_t u4_word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// OCP fp8 E4M3FN code -> bf16 bits, exact (every E4M3 value, subnormals
// included, is a bf16 value).  Normal codes move their exponent from bias 7 to
// bias 127; subnormal codes m * 2^-9 are formed as 2^-6 * (1 + m/8) - 2^-6.
__device__ __forceinline__ uint32_t fp8e4m3_to_bf16(uint32_t code) {
  uint32_t em = code & 0x7fu;
  bool sub = em < 8u;
  uint32_t bits = (em << 20) + ((sub ? 121u : 120u) << 23);
  float f = __uint_as_float(bits) - (sub ? 0.015625f : 0.0f);
  return (__float_as_uint(f) >> 16) | ((code & 0x80u) << 8);
}

// Order-preserving map of a finite float to an unsigned key (larger float ->
// larger key); -0 is mapped like +0.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum_xor(float v, int width_mask) {
  // butterfly over lanes l ^ 1, 2, 4, ... up to width_mask (a power of two - 1)
  for (int o = 1; o <= width_mask; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace dsa
