// fp16 GEMMs with few rows of A, C[M, N] = epilogue(A[M, K] . W[N, K]^T) for
// M <= 128: the step of incremental decoding, where A holds one new token per
// sequence.  Such a product does 2*M flops per weight element, below the
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
// Loads: a K tile is 64 wide; W tiles are 256 rows (32 KiB) and the A tile
// 32, 64 or 128 rows (the smallest that holds M), both moved by 16-byte
// direct-to-LDS buffer loads, 8 rows of 128 bytes per wave instruction, with
// the same XOR chunk swizzle as the large GEMM.  The ring has as many stages
// as fit the LDS, at most 4 (one workgroup per CU), so while a K tile is
// multiplied the next two or three are in flight: ~100 KiB per CU, ~25 MiB
// over 256 CUs, several times bandwidth x latency of HBM.  One barrier per K
// tile both publishes tile f (each wave first waits for its own loads of it)
// and frees the stage of tile f-1, which then receives tile f+D-1.
//
// Ragged M and N: the A descriptor ends at row M and the W descriptor at row
// N, so rows past them load zeros; only rows < M reach the partial sums and
// only columns < N the output.
#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "lds_dma.h"

namespace ee {
namespace {

constexpr int kBK = 64;         // K per stage (128-byte LDS rows, 8 chunks of 16 bytes)
constexpr int kSkBN = 256;      // rows of W per N tile
constexpr int kSkWaves = 4;
constexpr int kSkMinPerWg = 8;  // K tiles per workgroup below which the ring cannot fill
constexpr int kSkLds = 160 * 1024;

// Ring stages for an A tile of BM rows: as many as fit the LDS, at most 4
// (32 rows: 4 x 36 KiB; 64: 4 x 40 KiB; 128: 3 x 48 KiB).
template <int BM>
constexpr int sk_depth() {
  return kSkLds / ((BM + kSkBN) * kBK * 2) < 4 ? kSkLds / ((BM + kSkBN) * kBK * 2) : 4;
}

// 32x32x16 fragment geometry: element e of lane l of the accumulator sits at
// row (e/4)*8 + (l/32)*4 + e%4 (from A) and column l%32 (from W); an operand
// lane supplies row l%32 with the 8 K values of group l/32.
__device__ __forceinline__ int sk_acc_row(int lane, int e) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Workgroup g sums its range of flat K tiles [g*per_wg, ...) of the
// tiles_n x kt space; the sums of its piece of `tile` go to slot g + tile of
// P, [M][kSkBN] fp32 per slot.  A tile of BM >= M rows; the 4 waves split the
// tile's 256 W rows, each multiplying all BM rows of A by its 64.
template <int BM>
__global__ __launch_bounds__(64 * kSkWaves) void gemm_streamk_kernel(const f16* __restrict__ A, int lda,
                                                                   const f16* __restrict__ W, int ldw, int M, int N,
                                                                   int kt, int tiles_n, int per_wg,
                                                                   float* __restrict__ P) {
  constexpr int BN = kSkBN, D = sk_depth<BM>(), NW = kSkWaves;
  constexpr int STAGE = (BM + BN) * kBK;  // halves: A rows, then W rows
  constexpr int WTN = BN / NW;            // W rows (columns of C) per wave
  constexpr int FM = BM / 32, FN = WTN / 32;  // 32 x 32 accumulator blocks per wave
  constexpr int NLA = BM / NW / 8;        // A loads (8 rows each) per wave per K tile
  constexpr int NLW = WTN / 8;            // W loads per wave per K tile
  constexpr int NL = NLA + NLW;
  static_assert(BM % 32 == 0 && D >= 3, "whole fragments, at least two K tiles in flight");
  __shared__ __attribute__((aligned(16))) f16 smem[D * STAGE];

  const int g = blockIdx.x;
  const int total = kt * tiles_n;
  const int f0 = g * per_wg, f1 = min(total, f0 + per_wg);  // the launch keeps f0 < total
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // this lane's 16-byte chunk of each load: row lr of the load's 8, physical
  // chunk lp, which holds the logical chunk lp ^ lds_swizzle(row)
  const int lr = lane >> 3, lp = lane & 7;
  int aoff[NLA], woff[NLW];
#pragma unroll
  for (int q = 0; q < NLA; ++q) {
    const int ra = wave * (BM / NW) + 8 * q + lr;
    aoff[q] = (ra * lda + ((lp ^ lds_swizzle(ra)) * 8)) * 2;
  }
#pragma unroll
  for (int q = 0; q < NLW; ++q) {
    const int rw = wave * WTN + 8 * q + lr;
    woff[q] = (rw * ldw + ((lp ^ lds_swizzle(rw)) * 8)) * 2;
  }
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, M * lda * 2, kBufferFlags);

  // The next K tile to load, (lt, lk), walks the range in order; once the
  // range's last tile is issued it stays there, so the loads past the range
  // fetch that tile again into a stage nobody reads (the per-wave load count
  // per K tile stays fixed, which the barrier's count relies on).
  // (The division's reciprocal is computed on the vector unit; readfirstlane
  // keeps the position in scalar registers, else every load that takes it as
  // its scalar offset becomes a loop over lanes.)
  int lt = __builtin_amdgcn_readfirstlane(f0 / kt);
  int lk = __builtin_amdgcn_readfirstlane(f0 - lt * kt), unissued = f1 - f0;
  auto issue_next = [&](int stage) {
    const int n0 = lt * BN;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)n0 * ldw), (short)0, min(BN, N - n0) * ldw * 2, kBufferFlags);
    const int k2 = lk * kBK * 2;  // byte offset of the K tile
    f16* st = smem + stage * STAGE;
#pragma unroll
    for (int q = 0; q < NLA; ++q) buffer_load_lds16(arsrc, st + (wave * (BM / NW) + 8 * q) * kBK, aoff[q], k2);
#pragma unroll
    for (int q = 0; q < NLW; ++q) buffer_load_lds16(wrsrc, st + (BM + wave * WTN + 8 * q) * kBK, woff[q], k2);
    if (--unissued > 0 && ++lk == kt) {
      lk = 0;
      ++lt;
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int kg = lane >> 5, rsw = lds_swizzle(lane & 15);
  const int a_row = (lane & 31) * kBK;
  const int w_row = (BM + wave * WTN + (lane & 31)) * kBK;
  auto multiply = [&](int stage) {
    const f16* st = smem + stage * STAGE;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int ch = ((kk * 2 + kg) ^ rsw) * 8;
      half8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const half8*>(st + a_row + i * 32 * kBK + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const half8*>(st + w_row + j * 32 * kBK + ch);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // the fp32 sums of the finished piece of `tile` to slot g + tile (rows < M)
  auto store_piece = [&](int tile) {
    float* dst = P + (int64_t)(g + tile) * M * BN;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wave * WTN + j * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = i * 32 + sk_acc_row(lane, e);
          if (row < M) dst[row * BN + col] = acc[i][j][e];
          acc[i][j][e] = 0.f;
        }
      }
  };

  // K tiles [fa, fb) of the range; the loads run D-1 tiles ahead across pieces.
  // Stage rs holds tile f; ws, the stage of tile f-1, receives tile f+D-1.
  int rs = 0, ws = D - 1;
  auto run = [&](int fa, int fb) {
    for (int f = fa; f < fb; ++f) {
      // tile f has landed for every wave; every wave is done with the stage of f-1
      barrier_after_loads<(D - 2) * NL>();
      issue_next(ws);
      multiply(rs);
      rs = rs + 1 == D ? 0 : rs + 1;
      ws = ws + 1 == D ? 0 : ws + 1;
    }
  };

  // prologue: K tiles f0 .. f0+D-2 into stages 0..D-2
#pragma unroll
  for (int i = 0; i < D - 1; ++i) issue_next(i);
  // the range holds a piece of one tile, or the end of one and the start of
  // the next; each piece is stored after its own loop (stores inside one loop
  // over the range make the compiler keep every store address in registers)
  const int tile = __builtin_amdgcn_readfirstlane(f0 / kt);
  const int split = min(f1, (tile + 1) * kt);
  run(f0, split);
  store_piece(tile);
  if (split < f1) {
    run(split, f1);
    store_piece(tile + 1);
  }
  wait_dma();  // no load may still be writing LDS when the workgroup retires
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
      const float* src = P + ((int64_t)(g + tile) * M + row) * kSkBN + nl;
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

// A-tile rows for M rows of A (0: more than the kernel takes).
int sk_tile_rows(int64_t M) { return M <= 32 ? 32 : M <= 64 ? 64 : M <= kStreamKMaxRows ? 128 : 0; }

}  // namespace

StreamKPlan gemm_f16_streamk_plan(int64_t M, int N, int K, const GemmPitch& ld) {
  StreamKPlan p{};
  const int bm = sk_tile_rows(M);
  if (M < 1 || bm == 0 || N < 1 || K < kBK || K % kBK != 0) return p;
  if (ld.a < K || ld.w < K || ld.c < N || ld.a % 8 != 0 || ld.w % 8 != 0) return p;
  // 32-bit buffer offsets: the A range and one W tile
  if ((int64_t)bm * ld.a * 2 >= (1ll << 31) || (int64_t)kSkBN * ld.w * 2 >= (1ll << 31)) return p;
  const int64_t kt = K / kBK, tiles_n = (N + kSkBN - 1) / kSkBN, total = kt * tiles_n;
  if (total >= (1ll << 31)) return p;
  // at least one workgroup per N tile (so a range meets at most two tiles),
  // a whole number of rounds of one workgroup per CU (the ring fills the LDS)
  const int cus = device_cu_count();
  const int64_t wgs = (int64_t)cus * ((tiles_n + cus - 1) / cus);
  const int64_t per_wg = (total + wgs - 1) / wgs;
  if (per_wg < kSkMinPerWg) return p;
  p.tile_rows = bm;
  p.kt = (int)kt;
  p.tiles_n = (int)tiles_n;
  p.per_wg = (int)per_wg;
  p.workgroups = (int)((total + per_wg - 1) / per_wg);
  p.scratch_bytes = (size_t)(p.workgroups + p.tiles_n) * (size_t)M * kSkBN * sizeof(float);
  return p;
}

hipError_t launch_gemm_f16_streamk(const StreamKPlan& p, const void* A, const void* W, const void* bias, const void* R,
                                   int64_t M, int N, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                                   void* scratch, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (p.workgroups < 1 || sk_tile_rows(M) != p.tile_rows) return hipErrorInvalidValue;
  float* P = static_cast<float*>(scratch);
  const f16* a = static_cast<const f16*>(A);
  const f16* w = static_cast<const f16*>(W);
  const dim3 grid((unsigned)p.workgroups), block(64 * kSkWaves);
  switch (p.tile_rows) {
    case 32:
      hipLaunchKernelGGL(gemm_streamk_kernel<32>, grid, block, 0, s, a, ld.a, w, ld.w, (int)M, N, p.kt, p.tiles_n,
                         p.per_wg, P);
      break;
    case 64:
      hipLaunchKernelGGL(gemm_streamk_kernel<64>, grid, block, 0, s, a, ld.a, w, ld.w, (int)M, N, p.kt, p.tiles_n,
                         p.per_wg, P);
      break;
    default:
      hipLaunchKernelGGL(gemm_streamk_kernel<128>, grid, block, 0, s, a, ld.a, w, ld.w, (int)M, N, p.kt, p.tiles_n,
                         p.per_wg, P);
      break;
  }
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
