// Dense contractions with fp32 FMA on the vector ALUs: the fp32 layer (and any
// fp16 shape the MFMA kernel does not take, K % 64 != 0).
//   C[M, N] = epilogue(A[M, K] . W[N, K]^T), fp32 arithmetic.
// 64 x 64 tile, K step 16, 256 threads each owning a 4 x 4 block; both
// operand tiles are stored K-major in LDS (+1 padding against bank conflicts).
// Every dimension is guarded, so any M, N, K >= 1 works.  Rows are read and
// written at the given pitches (lda, ldw, ldc >= K, K, N elements).
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kT = 64, kKS = 16, kVThreads = 256;

template <typename T, int EPI>
__global__ __launch_bounds__(kVThreads) void gemm_valu_kernel(const T* __restrict__ A, const T* __restrict__ W,
                                                              const T* __restrict__ bias, const T* __restrict__ R,
                                                              T* __restrict__ C, int M, int N, int K, int lda,
                                                              int ldw, int ldc, int gelu_form) {
  __shared__ float sA[kKS][kT + 1];
  __shared__ float sW[kKS][kT + 1];
  const int t = threadIdx.x;
  const int tx = t & 15, ty = t >> 4;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += kKS) {
    // 64 rows x 16 k per operand: 4 elements per thread, k fastest (coalesced)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = t + q * kVThreads;
      const int r = idx / kKS, k = idx % kKS;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + k;
      sA[k][r] = (gm < M && gk < K) ? to_f32(A[(int64_t)gm * lda + gk]) : 0.f;
      sW[k][r] = (gn < N && gk < K) ? to_f32(W[(int64_t)gn * ldw + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKS; ++k) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = sW[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float v = acc[i][j];
      if (EPI != EE_EPI_NONE) v += to_f32(bias[col]);
      if (EPI == EE_EPI_BIAS_RESIDUAL) v += to_f32(R[(int64_t)row * ldc + col]);
      if (EPI == EE_EPI_BIAS_GELU) v = gelu_f(v, gelu_form);
      C[(int64_t)row * ldc + col] = from_f32<T>(v);
    }
  }
}

template <typename T>
hipError_t launch_t(const void* A, const void* W, const void* bias, const void* R, int M, int N, int K,
                    const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C, hipStream_t s) {
  const dim3 grid((unsigned)((N + kT - 1) / kT), (unsigned)((M + kT - 1) / kT)), block(kVThreads);
  const T* a = static_cast<const T*>(A);
  const T* w = static_cast<const T*>(W);
  const T* b = static_cast<const T*>(bias);
  const T* r = static_cast<const T*>(R);
  T* c = static_cast<T*>(C);
#define EE_VALU_LAUNCH(E)                                                                                \
  hipLaunchKernelGGL((gemm_valu_kernel<T, E>), grid, block, 0, s, a, w, b, r, c, M, N, K, ld.a, ld.w, ld.c, \
                     (int)form)
  switch (epi) {
    case EE_EPI_NONE: EE_VALU_LAUNCH(EE_EPI_NONE); break;
    case EE_EPI_BIAS: EE_VALU_LAUNCH(EE_EPI_BIAS); break;
    case EE_EPI_BIAS_RESIDUAL: EE_VALU_LAUNCH(EE_EPI_BIAS_RESIDUAL); break;
    case EE_EPI_BIAS_GELU: EE_VALU_LAUNCH(EE_EPI_BIAS_GELU); break;
  }
#undef EE_VALU_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_valu(ee_dtype dt, const void* A, const void* W, const void* bias, const void* R, int64_t M,
                            int N, int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                            hipStream_t s) {
  if (M <= 0) return hipSuccess;
  return dt == EE_F16 ? launch_t<f16>(A, W, bias, R, (int)M, N, K, ld, epi, form, C, s)
                      : launch_t<float>(A, W, bias, R, (int)M, N, K, ld, epi, form, C, s);
}

}  // namespace ee
