// Dense contractions of the layer in fp16 on the CDNA4 matrix cores:
//   C[M, N] = epilogue(A[M, K] . W[N, K]^T),  fp32 accumulation,
// with the epilogues the layer needs fused into the store: + bias (QKV),
// + bias + residual (out-projection, FC2), gelu(+ bias) (FC1).  M = T, the
// number of valid tokens, so the GEMMs do no work on padding; the announcement
// article's "Runtime" section notes that these GEMMs dominate as models grow.
//
// Design (gfx950, wave64):
//   * Both operands are K-contiguous, which is the layout the MFMA operand
//     registers want: every lane reads 8 consecutive K values (16 bytes).
//   * Workgroup tile BM x BN x 64 with 4 waves in a 2 x 2 grid; a wave owns a
//     (BM/2) x (BN/2) block of 32 x 32 v_mfma_f32_32x32x16_f16 fragments.
//   * Two LDS stages (BM=BN=256: 2 x 64 KiB of the 160 KiB per CU); the next
//     K tile is fetched into registers while the current one feeds the MFMAs,
//     then stored to the other stage: one barrier per K tile.
//   * LDS rows are 128 bytes (8 chunks of 16 B); chunk c of row r is stored at
//     chunk c ^ f(r), f(r) = ((r >> 1) & 7) ^ ((r & 1) << 2), so the 16 rows
//     read by a quarter-wave land on distinct banks whether the LDS serves
//     8 or 16 lanes of a 128-bit read per cycle.
//   * Tile order: the hardware deals consecutive workgroup ids round-robin to
//     the 8 XCDs, so ids are remapped to give each XCD a contiguous range, and
//     that range walks tiles in groups of 4 M-tiles, so the workgroups that
//     share an XCD's L2 share A and W panels.
//   * Ragged M (and N): out-of-range rows load a clamped in-range row, and
//     their results are never stored.  K must be a multiple of 64.
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

__device__ __forceinline__ int lds_swizzle(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_f16_mfma_kernel(const f16* __restrict__ A, const f16* __restrict__ W,
                                                                 const f16* __restrict__ bias,
                                                                 const f16* __restrict__ R, f16* __restrict__ C,
                                                                 int M, int N, int K, int gelu_form, int tiles_m,
                                                                 int tiles_n) {
  constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int AL = BM / 32, BL = BN / 32;  // 16-byte loads per thread per K tile
  constexpr int STAGE = (BM + BN) * kBK;     // halves per LDS stage
  __shared__ __attribute__((aligned(16))) f16 smem[2 * STAGE];

  // ---- tile assignment: XCD-contiguous ranges, grouped 4 M-tiles at a time
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int ig = bid - group * per_group;
  const int m0 = (first_m + ig % gm) * BM;
  const int n0 = (ig / gm) * BN;

  // ---- global -> register -> LDS mapping: 32 rows x 8 chunks per pass
  const int t = threadIdx.x;
  const int lrow = t >> 3, lch = t & 7;
  const f16* ag[AL];
  const f16* bg[BL];
#pragma unroll
  for (int i = 0; i < AL; ++i) ag[i] = A + (int64_t)min(m0 + lrow + 32 * i, M - 1) * K + lch * 8;
#pragma unroll
  for (int j = 0; j < BL; ++j) bg[j] = W + (int64_t)min(n0 + lrow + 32 * j, N - 1) * K + lch * 8;
  const int soff = lrow * kBK + ((lch ^ lds_swizzle(lrow)) * 8);
  half8 ra[AL], rb[BL];

  // ---- wave / lane roles for the MFMA fragments
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int hk = lane >> 5;  // which 8-wide K half of a 16-wide MFMA step this lane feeds
  const int rsw = lds_swizzle(lane & 15);
  const int abase = (wm * WTM + (lane & 31)) * kBK;
  const int bbase = (wn * WTN + (lane & 31)) * kBK;

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = K / kBK;
#pragma unroll
  for (int i = 0; i < AL; ++i) ra[i] = *reinterpret_cast<const half8*>(ag[i]);
#pragma unroll
  for (int j = 0; j < BL; ++j) rb[j] = *reinterpret_cast<const half8*>(bg[j]);
  {
    f16* sa = smem;
    f16* sb = smem + BM * kBK;
#pragma unroll
    for (int i = 0; i < AL; ++i) *reinterpret_cast<half8*>(sa + soff + i * 32 * kBK) = ra[i];
#pragma unroll
    for (int j = 0; j < BL; ++j) *reinterpret_cast<half8*>(sb + soff + j * 32 * kBK) = rb[j];
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = (kt + 1) * kBK;
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] = *reinterpret_cast<const half8*>(ag[i] + k0);
#pragma unroll
      for (int j = 0; j < BL; ++j) rb[j] = *reinterpret_cast<const half8*>(bg[j] + k0);
    }
    const f16* sa = smem + cur * STAGE;
    const f16* sb = sa + BM * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = ((kk * 2 + hk) ^ rsw) * 8;
      half8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const half8*>(sa + abase + i * 32 * kBK + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = *reinterpret_cast<const half8*>(sb + bbase + j * 32 * kBK + ch);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      f16* da = smem + (cur ^ 1) * STAGE;
      f16* db = da + BM * kBK;
#pragma unroll
      for (int i = 0; i < AL; ++i) *reinterpret_cast<half8*>(da + soff + i * 32 * kBK) = ra[i];
#pragma unroll
      for (int j = 0; j < BL; ++j) *reinterpret_cast<half8*>(db + soff + j * 32 * kBK) = rb[j];
    }
    __syncthreads();
  }

  // ---- epilogue.  Fragment element e of lane l is row (e/4)*8 + (l/32)*4 + e%4,
  // column l%32 of its 32 x 32 block.
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = n0 + wn * WTN + j * 32 + (lane & 31);
    if (col >= N) continue;
    const float bcol = (EPI != EE_EPI_NONE) ? (float)bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rbase = m0 + wm * WTM + i * 32 + hk * 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = rbase + (e >> 2) * 8 + (e & 3);
        if (row < M) {
          float v = acc[i][j][e] + bcol;
          if (EPI == EE_EPI_BIAS_RESIDUAL) v += (float)R[(int64_t)row * N + col];
          if (EPI == EE_EPI_BIAS_GELU) v = gelu_f(v, gelu_form);
          C[(int64_t)row * N + col] = (f16)v;
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch_cfg(const void* A, const void* W, const void* bias, const void* R, int M, int N, int K,
                      ee_epilogue epi, ee_gelu form, void* C, hipStream_t s) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const dim3 grid((unsigned)(tm * tn)), block(kThreads);
  const f16* a = static_cast<const f16*>(A);
  const f16* w = static_cast<const f16*>(W);
  const f16* b = static_cast<const f16*>(bias);
  const f16* r = static_cast<const f16*>(R);
  f16* c = static_cast<f16*>(C);
  switch (epi) {
    case EE_EPI_NONE:
      hipLaunchKernelGGL((gemm_f16_mfma_kernel<BM, BN, EE_EPI_NONE>), grid, block, 0, s, a, w, b, r, c, M, N, K,
                         (int)form, tm, tn);
      break;
    case EE_EPI_BIAS:
      hipLaunchKernelGGL((gemm_f16_mfma_kernel<BM, BN, EE_EPI_BIAS>), grid, block, 0, s, a, w, b, r, c, M, N, K,
                         (int)form, tm, tn);
      break;
    case EE_EPI_BIAS_RESIDUAL:
      hipLaunchKernelGGL((gemm_f16_mfma_kernel<BM, BN, EE_EPI_BIAS_RESIDUAL>), grid, block, 0, s, a, w, b, r, c, M,
                         N, K, (int)form, tm, tn);
      break;
    case EE_EPI_BIAS_GELU:
      hipLaunchKernelGGL((gemm_f16_mfma_kernel<BM, BN, EE_EPI_BIAS_GELU>), grid, block, 0, s, a, w, b, r, c, M, N,
                         K, (int)form, tm, tn);
      break;
  }
  return hipGetLastError();
}

}  // namespace

bool gemm_f16_mfma_ok(int64_t M, int N, int K) {
  return M >= 1 && M <= (1 << 30) && N >= 1 && K >= kBK && K % kBK == 0;
}

hipError_t launch_gemm_f16_mfma(const void* A, const void* W, const void* bias, const void* R, int64_t M, int N,
                                int K, ee_epilogue epi, ee_gelu form, void* C, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int64_t tiles_big = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles_big >= 256) return launch_cfg<256, 256>(A, W, bias, R, (int)M, N, K, epi, form, C, s);
  return launch_cfg<128, 128>(A, W, bias, R, (int)M, N, K, epi, form, C, s);
}

}  // namespace ee
