// fp16 GEMMs with few rows of A, C[M, N] = epilogue(A[M, K] . W[N, K]^T) for
// M <= 32: the step of incremental decoding, where A holds one new token per
// sequence.  Such a product does 2*M flops per weight element, far below the
// MFMA/HBM ridge, so its time is the time to read W once: the kernel is a W
// streamer with the matrix cores attached.
//
// Decomposition: stream-K (Osama, Merrill, Cecka, Garland and Owens,
// "Stream-K: Work-centric Parallel Decomposition for Dense Matrix-Matrix
// Multiplication", PPoPP 2023).  The (N tile, K tile) iteration space, N tile
// major, is cut into equal contiguous ranges, one per workgroup, so every CU
// streams the same number of W bytes whatever the number of N tiles (a
// split-K grid of whole tiles leaves part of the last round of workgroups
// idle).  With at least as many workgroups as N tiles, a range covers pieces
// of at most two tiles.  A workgroup writes the fp32 sums of each piece to its
// own slot, slot = workgroup + tile (unique because both grow along the
// range), and a second kernel adds the pieces of every tile in K order (a
// fixed order: the result does not depend on timing) and applies the epilogue.
//
// Loads: a K tile is 64 wide; W tiles are 256 rows (32 KiB) and the A tile is
// 32 rows (4 KiB), both moved by 16-byte direct-to-LDS buffer loads, 8 rows of
// 128 bytes per wave instruction, with the same XOR chunk swizzle as the large
// GEMM.  The ring has 4 stages (144 KiB, one workgroup per CU), so while a K
// tile is multiplied the next three are in flight: ~108 KiB per CU, ~27 MiB
// over 256 CUs, several times bandwidth x latency of HBM.  One barrier per K
// tile both publishes tile f (each wave first waits for its own loads of it)
// and frees the stage of tile f-1, which then receives tile f+3.
//
// Ragged M and N: the A descriptor ends at row M and the W descriptor at row
// N, so rows past them load zeros; the reduce stores only rows < M and
// columns < N.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kBK = 64;       // K per stage (128-byte LDS rows)
constexpr int kSkBM = 32;     // rows of A: all of M
constexpr int kSkBN = 256;    // rows of W per N tile
constexpr int kSkDepth = 4;   // stages in the LDS ring
constexpr int kSkWaves = 4;
constexpr int kSkMinPerWg = 8;  // K tiles per workgroup below which the ring cannot fill

// chunk c of LDS row r is stored at chunk c ^ f(r); a fragment read by 16
// consecutive rows then spreads over the banks (f depends on r & 15 only)
__device__ __forceinline__ int sk_swizzle(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

__device__ __forceinline__ void sk_load_lds16(__amdgpu_buffer_rsrc_t rsrc, f16* lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0,
                                           0);
}

// Word 3 of a raw (unformatted, stride 0) buffer descriptor on gfx9-family GPUs.
constexpr int kSkBufferFlags = 0x00020000;

// Waits until at most N of this wave's vector memory operations are pending
// and its LDS reads are done, then joins the workgroup barrier.  Direct-to-LDS
// loads complete in issue order among themselves, so with the newest N
// allowed to fly every older load has written LDS.  (The compiler does not
// count a direct-to-LDS load as an LDS write, and __syncthreads would wait
// for every load.)
template <int N>
__device__ __forceinline__ void sk_barrier_after_loads() {
  static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void sk_wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 32x32x16 fragment geometry: element e of lane l of the accumulator sits at
// row (e/4)*8 + (l/32)*4 + e%4 (from A) and column l%32 (from W); an operand
// lane supplies row l%32 with the 8 K values of group l/32.
__device__ __forceinline__ int sk_acc_row(int lane, int e) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Partial sums of workgroup g: its range of flat K tiles [g*per_wg, ...) of
// the tiles_n x kt space; slot g + tile holds [kSkBM][kSkBN] fp32.
__global__ __launch_bounds__(64 * kSkWaves) void gemm_streamk_kernel(const f16* __restrict__ A, int lda,
                                                                   const f16* __restrict__ W, int ldw, int M, int N,
                                                                   int kt, int tiles_n, int per_wg,
                                                                   float* __restrict__ P) {
  constexpr int BM = kSkBM, BN = kSkBN, D = kSkDepth, NW = kSkWaves;
  constexpr int STAGE = (BM + BN) * kBK;  // halves: A rows, then W rows
  constexpr int WTN = BN / NW;            // W rows (columns of C) per wave
  constexpr int FN = WTN / 32;            // 32 x 32 accumulator blocks per wave
  constexpr int NLW = WTN / 8;            // W loads per wave per K tile
  constexpr int NL = 1 + NLW;             // and one A load (8 of the 32 rows)
  static_assert(BM == 8 * NW, "one A load per wave");
  __shared__ __attribute__((aligned(16))) f16 smem[D * STAGE];

  const int g = blockIdx.x;
  const int total = kt * tiles_n;
  const int f0 = g * per_wg, f1 = min(total, f0 + per_wg);  // the launch keeps f0 < total
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // this lane's 16-byte chunk of each load: row lr of the load's 8, physical
  // chunk lp, which holds the logical chunk lp ^ f(row)
  const int lr = lane >> 3, lp = lane & 7;
  const int ra = 8 * wave + lr;
  const int aoff = (ra * lda + ((lp ^ sk_swizzle(ra)) * 8)) * 2;
  int woff[NLW];
#pragma unroll
  for (int q = 0; q < NLW; ++q) {
    const int rw = wave * WTN + 8 * q + lr;
    woff[q] = (rw * ldw + ((lp ^ sk_swizzle(rw)) * 8)) * 2;
  }
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, M * lda * 2, kSkBufferFlags);

  // loads of flat K tile f (tile f / kt, K offset f % kt) into a stage
  auto issue = [&](int stage, int f) {
    const int tile = f / kt;
    const int k2 = (f - tile * kt) * kBK * 2;  // byte offset of the K tile
    const int n0 = tile * BN;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)n0 * ldw), (short)0, min(BN, N - n0) * ldw * 2, kSkBufferFlags);
    f16* st = smem + stage * STAGE;
    sk_load_lds16(arsrc, st + 8 * wave * kBK, aoff, k2);
#pragma unroll
    for (int q = 0; q < NLW; ++q) sk_load_lds16(wrsrc, st + (BM + wave * WTN + 8 * q) * kBK, woff[q], k2);
  };

  floatx16 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

  const int kg = lane >> 5, rsw = sk_swizzle(lane & 15);
  const int a_row = (lane & 31) * kBK;
  const int w_row = (BM + wave * WTN + (lane & 31)) * kBK;
  auto multiply = [&](int stage) {
    const f16* st = smem + stage * STAGE;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = ((kk * 2 + kg) ^ rsw) * 8;
      const half8 a = *reinterpret_cast<const half8*>(st + a_row + ch);
      half8 b[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const half8*>(st + w_row + j * 32 * kBK + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[j], acc[j], 0, 0, 0);
    }
  };

  // the fp32 sums of the finished piece of `tile` to slot g + tile (rows < M)
  auto store_piece = [&](int tile) {
    float* dst = P + (int64_t)(g + tile) * BM * BN;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = wave * WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = sk_acc_row(lane, e);
        if (row < M) dst[row * BN + col] = acc[j][e];
        acc[j][e] = 0.f;
      }
    }
  };

  // prologue: K tiles f0 .. f0+D-2 (clamped to the range) into stages 0..D-2
#pragma unroll
  for (int i = 0; i < D - 1; ++i) issue(i, min(f0 + i, f1 - 1));
  int tile = f0 / kt;
  int piece_end = min(f1, (tile + 1) * kt);
  for (int f = f0; f < f1; ++f) {
    const int i = f - f0;
    // tile f has landed for every wave; every wave is done with the stage of f-1
    sk_barrier_after_loads<(D - 2) * NL>();
    // f+D-1 goes to the stage of f-1; past the range, the last tile is loaded
    // again into a stage nobody reads (keeps the per-wave load count fixed)
    issue((i + D - 1) % D, min(f + D - 1, f1 - 1));
    multiply(i % D);
    if (f + 1 == piece_end) {
      store_piece(tile);
      ++tile;
      piece_end = min(f1, piece_end + kt);
    }
  }
  sk_wait_all_loads();  // no load may still be writing LDS when the workgroup retires
}

// C[m, n] = epilogue(sum over the pieces of tile n / kSkBN, in K order).
template <int EPI, int V>
__global__ __launch_bounds__(256) void streamk_reduce_kernel(const float* __restrict__ P, int M, int N, int kt,
                                                             int per_wg, const f16* __restrict__ bias,
                                                             const f16* __restrict__ R, f16* __restrict__ C, int ldc,
                                                             int gelu_form) {
  constexpr bool kBias = EPI == EE_EPI_BIAS || EPI == EE_EPI_BIAS_RESIDUAL || EPI == EE_EPI_BIAS_GELU;
  const int per_row = N / V;
  const int64_t items = (int64_t)M * per_row;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < items; i += (int64_t)gridDim.x * 256) {
    const int row = (int)(i / per_row);
    const int col = (int)(i - (int64_t)row * per_row) * V;
    const int tile = col / kSkBN, nl = col - tile * kSkBN;
    const int g_first = (int)((int64_t)tile * kt / per_wg);
    const int g_last = (int)((((int64_t)tile + 1) * kt - 1) / per_wg);
    float v[V];
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = 0.f;
    for (int g = g_first; g <= g_last; ++g) {
      const float* src = P + ((int64_t)(g + tile) * kSkBM + row) * kSkBN + nl;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] += src[k];
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
      float x = v[k] + (kBias ? (float)bias[col + k] : 0.f);
      if (EPI == EE_EPI_BIAS_RESIDUAL) x += (float)R[(int64_t)row * ldc + col + k];
      if (EPI == EE_EPI_BIAS_GELU) x = gelu_f(x, gelu_form);
      C[(int64_t)row * ldc + col + k] = (f16)x;
    }
  }
}

template <int EPI>
hipError_t launch_sk_reduce(const float* P, int M, int N, int kt, int per_wg, const void* bias, const void* R,
                            void* C, int ldc, ee_gelu form, hipStream_t s) {
  const bool vec = N % 8 == 0 && ldc % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(C) | reinterpret_cast<uintptr_t>(R)) & 15) == 0;
  const int64_t items = (int64_t)M * (vec ? N / 8 : N);
  const unsigned grid = (unsigned)std::min<int64_t>((items + 255) / 256, 4096);
  const f16* b = static_cast<const f16*>(bias);
  const f16* r = static_cast<const f16*>(R);
  f16* c = static_cast<f16*>(C);
  if (vec)
    hipLaunchKernelGGL((streamk_reduce_kernel<EPI, 8>), dim3(grid), dim3(256), 0, s, P, M, N, kt, per_wg, b, r, c, ldc,
                       (int)form);
  else
    hipLaunchKernelGGL((streamk_reduce_kernel<EPI, 1>), dim3(grid), dim3(256), 0, s, P, M, N, kt, per_wg, b, r, c, ldc,
                       (int)form);
  return hipGetLastError();
}

// Compute units of the current device, cached per device.
int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace

StreamKPlan gemm_f16_streamk_plan(int64_t M, int N, int K, const GemmPitch& ld) {
  StreamKPlan p{};
  const int cus = cu_count();
  if (M < 1 || M > kSkBM || N < 1 || K < kBK || K % kBK != 0) return p;
  if (ld.a < K || ld.w < K || ld.c < N || ld.a % 8 != 0 || ld.w % 8 != 0) return p;
  // 32-bit buffer offsets: the A range and one W tile
  if ((int64_t)kSkBM * ld.a * 2 >= (1ll << 31) || (int64_t)kSkBN * ld.w * 2 >= (1ll << 31)) return p;
  const int64_t kt = K / kBK, tiles_n = (N + kSkBN - 1) / kSkBN, total = kt * tiles_n;
  if (total >= (1ll << 31)) return p;
  // at least one workgroup per N tile (so a range meets at most two tiles),
  // a whole number of workgroups per CU
  const int64_t wgs = (int64_t)cus * ((tiles_n + cus - 1) / cus);
  const int64_t per_wg = (total + wgs - 1) / wgs;
  if (per_wg < kSkMinPerWg) return p;
  p.kt = (int)kt;
  p.tiles_n = (int)tiles_n;
  p.per_wg = (int)per_wg;
  p.workgroups = (int)((total + per_wg - 1) / per_wg);
  p.scratch_bytes = (size_t)(p.workgroups + p.tiles_n) * kSkBM * kSkBN * sizeof(float);
  return p;
}

hipError_t launch_gemm_f16_streamk(const StreamKPlan& p, const void* A, const void* W, const void* bias, const void* R,
                                   int64_t M, int N, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                                   void* scratch, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (p.workgroups < 1) return hipErrorInvalidValue;
  float* P = static_cast<float*>(scratch);
  hipLaunchKernelGGL(gemm_streamk_kernel, dim3((unsigned)p.workgroups), dim3(64 * kSkWaves), 0, s,
                     static_cast<const f16*>(A), ld.a, static_cast<const f16*>(W), ld.w, (int)M, N, p.kt, p.tiles_n,
                     p.per_wg, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (epi) {
    case EE_EPI_NONE: return launch_sk_reduce<EE_EPI_NONE>(P, (int)M, N, p.kt, p.per_wg, bias, R, C, ld.c, form, s);
    case EE_EPI_BIAS: return launch_sk_reduce<EE_EPI_BIAS>(P, (int)M, N, p.kt, p.per_wg, bias, R, C, ld.c, form, s);
    case EE_EPI_BIAS_RESIDUAL:
      return launch_sk_reduce<EE_EPI_BIAS_RESIDUAL>(P, (int)M, N, p.kt, p.per_wg, bias, R, C, ld.c, form, s);
    case EE_EPI_BIAS_GELU:
      return launch_sk_reduce<EE_EPI_BIAS_GELU>(P, (int)M, N, p.kt, p.per_wg, bias, R, C, ld.c, form, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ee
