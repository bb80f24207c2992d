// Device helpers shared by the gfx950 kernels: number-format codecs, lane reductions, vector types.
//
// Formats follow "MXFP vs NVFP4" (tqpw.cn 81738) sections 2.1-2.2 and the format table of
// "General notes on quantization" (zdszero): E2M1 (1-2-1, bias 1, values {0,.5,1,1.5,2,3,4,6}),
// E4M3 (1-4-3, bias 7, OCP fn: largest finite 448), E8M0 (pure exponent byte, bias 127).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa4 {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------- E2M1
// Nearest E2M1 code of v (ties to the even mantissa, saturating at +-6); the sign bit is v's sign
// bit. The thresholds are the midpoints of neighbouring grid values: a midpoint goes down when
// the lower neighbour has an even mantissa (0, 1, 2, 4) and up otherwise.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 8u);
}

// E2M1 code -> float (exact).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
  const float mag = (m < 4u) ? 0.5f * (float)m : (float)(2u << ((m - 4u) >> 1)) * ((m & 1u) ? 1.5f : 1.0f);
  return (c & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------------------------------- E4M3
// Hardware conversion: round to nearest even, sign kept; finite for |x| < 480 (448 < |x| < 480
// gives 448). Callers only pass magnitudes <= 448 * (1 + 2^-23).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}
__device__ __forceinline__ uint32_t e4m3_encode2(float lo, float hi) {  // two codes in bits 15:0
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false) & 0xffffu;
}
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// ---------------------------------------------------------------------------------------- E8M0
// Smallest e with 6 * 2^e >= amax (amax >= 0 finite), clamped to [-127, 127]; -127 for amax = 0.
// With amax = 1.m * 2^(E-127) (E the biased exponent), amax = f * 2^(E-126), f = 0.5 + m/2^24;
// e = E-126-3 if f <= 0.75 (m <= 2^22) else E-126-2. Subnormal amax gives e < -127 -> -127.
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xffu);
  const uint32_t m = b & 0x7fffffu;
  if (E == 0) return -127;
  int e = (m <= 0x400000u) ? E - 129 : E - 128;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// MXFP8 (E4M3 elements): smallest e with 448 * 2^e >= amax, clamped, -127 for amax = 0. With f as above
// and 448 = 0.875 * 2^9: e = E-126-9 if f <= 0.875 (m <= 0x600000) else E-126-8.
__device__ __forceinline__ int mx8_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xffu);
  const uint32_t m = b & 0x7fffffu;
  if (E == 0) return -127;
  int e = (m <= 0x600000u) ? E - 135 : E - 134;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^-e as a float for e in [-127, 126] (exact; 2^-126 is the smallest normal).
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }
// float -> bf16 bits, nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------------------- lanes
// Lane exchange within a wave (xor pattern), via ds_swizzle / DPP chosen by the compiler.
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, 64); }

}  // namespace fa4
