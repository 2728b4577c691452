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

constexpr int kWave = 64;

// GeLU of the add-bias + activation step.  tanh form:
// 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))); erf form: 0.5 u (1 + erf(u / sqrt 2)).
// tanhf / erff are the ROCm device library's.
__device__ __forceinline__ float gelu_f(float u, int form) {
  if (form == EE_GELU_TANH) {
    const float k = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * u * (1.0f + tanhf(k * (u + 0.044715f * u * u * u)));
  }
  return 0.5f * u * (1.0f + erff(u * 0.7071067811865476f));  // 1/sqrt(2)
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
