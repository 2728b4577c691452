// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ee.h"

namespace ee {

typedef _Float16 f16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes

constexpr int kWave = 64;

constexpr float kLog2e = 1.4426950408889634f;

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26:
// erf(x) = 1 - (a1 t + ... + a5 t^5) exp(-x^2), t = 1 / (1 + p x), x >= 0,
// absolute error <= 1.5e-7; odd extension for x < 0.  Straight-line code on the
// hardware exp2 / reciprocal, so it inlines into GEMM epilogues without calls.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float y = 1.0f - poly * __builtin_amdgcn_exp2f(-ax * ax * kLog2e);
  return copysignf(y, x);
}

// GeLU of the add-bias + activation step.
//   tanh form: 0.5 u (1 + tanh(z)), z = sqrt(2/pi) (u + 0.044715 u^3), evaluated
//              as u / (1 + exp(-2 z)) since 0.5 (1 + tanh z) = 1 / (1 + e^{-2z});
//              exp(-2z) -> +inf gives u * 0 = 0 and exp -> 0 gives u (the limits);
//   erf form:  0.5 u (1 + erf(u / sqrt 2)).
__device__ __forceinline__ float gelu_f(float u, int form) {
  if (form == EE_GELU_TANH) {
    // exp(-2z) = 2^(u (c1 + c3 u^2)): the constants folded, so two multiplies
    // and one fma before the exp2 (the GEMM epilogue runs this per element)
    constexpr float c1 = -2.0f * kLog2e * 0.7978845608028654f;  // sqrt(2/pi)
    constexpr float c3 = c1 * 0.044715f;
    const float e = __builtin_amdgcn_exp2f(u * __builtin_fmaf(c3, u * u, c1));
    return u * __builtin_amdgcn_rcpf(1.0f + e);
  }
  return 0.5f * u * (1.0f + erf_as(u * 0.7071067811865476f));  // 1/sqrt(2)
}

// Storage <-> fp32.  fp32 -> fp16 conversion rounds to nearest even.
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ f16 from_f32<f16>(float v) { return (f16)v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

}  // namespace ee
