// Standalone add bias + GeLU, g[r, c] = gelu(u[r, c] + bias[c]) (the
// add-bias + activation step of the announcement article's "Ease of use"
// listing).  The layer normally fuses this step into the FC1 GEMM epilogue;
// this kernel is the unfused form.  HBM-bound elementwise pass: 16-byte
// vectors, each workgroup walks a band of rows so the bias vector stays in
// registers/L1 across the band.  Rows are ld elements apart.  u and g may be
// the same buffer (each element is read and then written by one thread).
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kGeluThreads = 256;

template <typename T, typename V, int E>
__global__ __launch_bounds__(kGeluThreads) void bias_gelu_kernel(const T* u, const T* __restrict__ bias,
                                                                 int64_t rows, int cols, int ld, int form,
                                                                 T* g) {
  const int vpr = cols / E;
  const V* bv = reinterpret_cast<const V*>(bias);
  for (int c = blockIdx.x * kGeluThreads + threadIdx.x; c < vpr; c += gridDim.x * kGeluThreads) {
    const V b = bv[c];
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
      const V a = __builtin_nontemporal_load(reinterpret_cast<const V*>(u + r * ld) + c);
      V o;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = from_f32<T>(gelu_f(to_f32(a[e]) + to_f32(b[e]), form));
      reinterpret_cast<V*>(g + r * ld)[c] = o;
    }
  }
}

}  // namespace

hipError_t launch_bias_gelu(ee_dtype dt, const void* u, const void* bias, int64_t rows, int cols, int ld,
                            ee_gelu form, void* g, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int E = dt == EE_F16 ? 8 : 4;
  const int vpr = cols / E;
  const unsigned gx = (unsigned)((vpr + kGeluThreads - 1) / kGeluThreads);
  const unsigned gy = (unsigned)(rows < 1024 ? rows : 1024);
  if (dt == EE_F16)
    hipLaunchKernelGGL((bias_gelu_kernel<f16, half8, 8>), dim3(gx, gy), dim3(kGeluThreads), 0, s,
                       static_cast<const f16*>(u), static_cast<const f16*>(bias), rows, cols, ld, (int)form,
                       static_cast<f16*>(g));
  else
    hipLaunchKernelGGL((bias_gelu_kernel<float, floatx4, 4>), dim3(gx, gy), dim3(kGeluThreads), 0, s,
                       static_cast<const float*>(u), static_cast<const float*>(bias), rows, cols, ld, (int)form,
                       static_cast<float*>(g));
  return hipGetLastError();
}

}  // namespace ee
