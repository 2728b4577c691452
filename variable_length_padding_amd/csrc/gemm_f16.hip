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
//   * Large problems: workgroup tile 256 x 256 x 64, 2 x 2 waves (one per
//     SIMD), each wave a 128 x 128 block of v_mfma_f32_16x16x32_f16 fragments
//     (256 fp32 accumulators per lane, in AGPRs).  Small problems: 128 x 128
//     tiles, 2 x 2 waves of 32 x 32 x 16 fragments.  The 128 x 128 wave block
//     reads 2/3 of the LDS bytes per flop that a 128 x 64 block (two waves per
//     SIMD) does; the chip is power-limited under this load and ran ~15% higher
//     clocks with it (1.8 vs 1.5 GHz on the FC1 shape).
//   * An LDS ring of 2 A stages and 2 W stages (4 x 32 KiB of the 160 KiB per
//     CU) filled by 16-byte direct-to-LDS buffer loads (buffer_load_dwordx4
//     ... lds): no register staging and no LDS store instructions.  Tile kt+2
//     is requested right after the barrier that retires tile kt's stages, one
//     load per four MFMAs (bunching them stalls MFMA issue), so a load has
//     about a K tile of MFMA work to land; one barrier per K tile.  From
//     K = 32768 the large tile keeps 3 W stages (the ring fills the 160 KiB)
//     and requests W two K tiles ahead: there both operands stream from HBM.
//   * MFMA fragments are double-buffered in registers: the LDS reads of K step
//     kk+1 are in flight while the MFMAs of step kk issue.
//   * LDS rows are 128 bytes (8 chunks of 16 B); chunk c of row r is stored at
//     chunk c ^ f(r), f(r) = ((r >> 1) & 7) ^ ((r & 1) << 2), so the 16 rows
//     read by a quarter-wave land on distinct banks whether the LDS serves
//     8 or 16 lanes of a 128-bit read per cycle.
//   * Tile order: the hardware deals consecutive workgroup ids round-robin to
//     the 8 XCDs, so ids are remapped to give each XCD a contiguous range, and
//     that range walks tiles in groups of 4 M-tiles, so the workgroups that
//     share an XCD's L2 share A and W panels.
//   * A 256 x 256 tile count just past a multiple of the CU count runs whole
//     rounds of 256-row tiles and the remaining rows as 128 x 128 tiles (a
//     second launch), when that is estimated to end sooner (gemm_big_rows).
//   * Epilogues go through LDS so C and the residual move in 16-byte vectors
//     (store_tile_staged); a direct per-element store covers N % 8 != 0.
//   * Ragged M (and N): the buffer descriptors end at the last valid row, so
//     out-of-range rows load zeros; their results are never stored.  K must be
//     a multiple of 64, and 256 rows at the operand's row pitch must fit
//     32-bit offsets.
//   * Row pitches (lda, ldw, ldc, in elements) may exceed the row lengths.
//     A row stride that is a multiple of 32 KiB puts every row of a panel on
//     the same few HBM channels: at K = 49152 (96 KiB rows) this kernel ran
//     7% slower than with 128 bytes of padding per row of A and W.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "lds_dma.h"

namespace ee {
namespace {

// Large-problem configuration: MFMA shape and wave grid of the 256 x 256 tile.
#ifndef EE_GEMM_WGM
#define EE_GEMM_WGM 2
#define EE_GEMM_WGN 2
#endif
#ifndef EE_GEMM_MF
#define EE_GEMM_MF 16
#endif
// Large problems: one workgroup per CU looping over tiles (1), or one per tile (0).
#ifndef EE_GEMM_PERSIST
#define EE_GEMM_PERSIST 1
#endif
// Large problems: K ranges from this length on use three W stages in the LDS
// ring (W requested two K tiles ahead, A one), shorter ones two (both one
// ahead).  Three measured 1.7% faster on FC2 (K = 49152, where both operands
// stream from HBM) and 1.6% slower on the QKV GEMM (K = 12288).
#ifndef EE_GEMM_DEEP_W_K
#define EE_GEMM_DEEP_W_K 32768
#endif

constexpr int kBK = 64;
// Split-K partial store (internal): fp32 sums of one K range, no epilogue.
constexpr int kEpiPartial = 4;
template <int EPI>
constexpr bool kHasBias = EPI == EE_EPI_BIAS || EPI == EE_EPI_BIAS_RESIDUAL || EPI == EE_EPI_BIAS_GELU;

// Tile origin of this workgroup: XCD-contiguous ranges of workgroup ids,
// walked in groups of 4 M-tiles (see the file comment).
template <int BM, int BN>
__device__ __forceinline__ void tile_origin(int tile, int n_tiles, int tiles_m, int tiles_n, int& m0, int& n0) {
  int bid = tile;
  const int nblk = n_tiles;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  constexpr int GM = 4;
  const int per_group = GM * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int ig = bid - group * per_group;
  m0 = (first_m + ig % gm) * BM;
  n0 = (ig / gm) * BN;
}

// Fragment geometry of the two MFMA shapes used here.  Element e of lane l
// of a fragment sits at (row(l, e), col(l)) of its MF x MF block:
//   32x32x16: row (e/4)*8 + (l/32)*4 + e%4, column l%32 (16 fp32 per lane);
//   16x16x32: row (l/16)*4 + e,             column l%16 (4 fp32 per lane).
// A lane feeds the row l%MF of an operand fragment with 8 consecutive K values
// from K group l/MF.
template <int MF>
struct Frag;
template <>
struct Frag<32> {
  using acc_t = floatx16;
  static constexpr int kElems = 16, kK = 16, kPad = 8;
  __device__ static int row(int lane, int e) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }
  __device__ static acc_t mfma(half8 a, half8 b, acc_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};
template <>
struct Frag<16> {
  using acc_t = floatx4;
  static constexpr int kElems = 4, kK = 32, kPad = 4;
  __device__ static int row(int lane, int e) { return (lane >> 4) * 4 + e; }
  __device__ static acc_t mfma(half8 a, half8 b, acc_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
};

// Row-major epilogue through LDS: the MFMA result layout gives a lane one
// column of several rows, so storing from it writes 2 bytes per lane and
// short row pieces.  Instead each wave writes one band of its block (one
// fragment row: 32 or 16 rows; bias and GeLU applied, still fp32) to its own
// slice of the LDS,
// then reads it back as 8 consecutive columns per lane, so C (and the residual
// R) move in 16-byte vectors and whole row segments.  The rounding is the
// same as a direct store: (acc + bias) + R in fp32, one fp16 rounding.
// Needs N % 8 == 0 and 16-byte aligned C and R.  The row pitch WTN + kPad
// puts the rows one lane group writes at once on disjoint banks.
template <int MF, int FN>
struct StagedEpilogue {
  static constexpr int WTN = FN * MF;
  static constexpr int kLd = WTN + Frag<MF>::kPad;
  static constexpr int kBandRows = MF;               // one fragment row per band
  static constexpr int kFloats = kBandRows * kLd;    // per wave
  static constexpr int kLanesPerRow = WTN / 8;
  static constexpr int kRowsPerPass = 64 / kLanesPerRow;
};

template <int MF, int FM, int FN, int EPI>
__device__ __forceinline__ void store_tile_staged(const typename Frag<MF>::acc_t (&acc)[FM][FN], float* __restrict__ stage,
                                                  int row0, int col0, int lane, const f16* __restrict__ bias,
                                                  const f16* __restrict__ R, f16* __restrict__ C, int M, int N,
                                                  int ldc, int gelu_form, float* __restrict__ Pp) {
  using SE = StagedEpilogue<MF, FN>;
  constexpr int FPB = 1;  // fragment rows per band
  constexpr int PASSES = SE::kBandRows / SE::kRowsPerPass;
  const int c8 = lane % SE::kLanesPerRow, rsub = lane / SE::kLanesPerRow;
  const int col = col0 + c8 * 8;
  float bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cj = col0 + j * MF + lane % MF;
    bcol[j] = (kHasBias<EPI> && cj < N) ? (float)bias[cj] : 0.f;
  }
#pragma unroll
  for (int band = 0; band < FM / FPB; ++band) {
    // the residual of this band is requested before the band goes through LDS
    half8 rv[PASSES];
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int row = row0 + band * SE::kBandRows + it * SE::kRowsPerPass + rsub;
      if (EPI == EE_EPI_BIAS_RESIDUAL && row < M && col < N)
        rv[it] = *reinterpret_cast<const half8*>(R + (int64_t)row * ldc + col);
    }
#pragma unroll
    for (int ii = 0; ii < FPB; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < Frag<MF>::kElems; ++e) {
          float v = acc[band * FPB + ii][j][e] + bcol[j];
          if (EPI == EE_EPI_BIAS_GELU) v = gelu_f(v, gelu_form);
          stage[(ii * MF + Frag<MF>::row(lane, e)) * SE::kLd + j * MF + lane % MF] = v;
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int r = it * SE::kRowsPerPass + rsub;
      const int row = row0 + band * SE::kBandRows + r;
      const float4 lo = *reinterpret_cast<const float4*>(stage + r * SE::kLd + c8 * 8);
      const float4 hi = *reinterpret_cast<const float4*>(stage + r * SE::kLd + c8 * 8 + 4);
      if (EPI == kEpiPartial) {
        if (row < M && col < N) {
          *reinterpret_cast<float4*>(Pp + (int64_t)row * N + col) = lo;
          *reinterpret_cast<float4*>(Pp + (int64_t)row * N + col + 4) = hi;
        }
      } else if (row < M && col < N) {
        const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        half8 out;
#pragma unroll
        for (int k = 0; k < 8; ++k) out[k] = (f16)(EPI == EE_EPI_BIAS_RESIDUAL ? v[k] + (float)rv[it][k] : v[k]);
        *reinterpret_cast<half8*>(C + (int64_t)row * ldc + col) = out;
      }
    }
    __syncthreads();  // the next band overwrites this wave's slice
  }
}

// Direct per-element epilogue of a wave's FM x FN block of fragments whose
// top-left output element is (row0, col0); used when N % 8 != 0.
template <int MF, int FM, int FN, int EPI>
__device__ __forceinline__ void store_tile(const typename Frag<MF>::acc_t (&acc)[FM][FN], int row0, int col0, int lane,
                                           const f16* __restrict__ bias, const f16* __restrict__ R,
                                           f16* __restrict__ C, int M, int N, int ldc, int gelu_form,
                                           float* __restrict__ Pp) {
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int col = col0 + j * MF + lane % MF;
    if (col >= N) continue;
    const float bcol = kHasBias<EPI> ? (float)bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int e = 0; e < Frag<MF>::kElems; ++e) {
        const int row = row0 + i * MF + Frag<MF>::row(lane, e);
        if (row < M && EPI == kEpiPartial) {
          Pp[(int64_t)row * N + col] = acc[i][j][e];
        } else if (row < M) {
          float v = acc[i][j][e] + bcol;
          if (EPI == EE_EPI_BIAS_RESIDUAL) v += (float)R[(int64_t)row * ldc + col];
          if (EPI == EE_EPI_BIAS_GELU) v = gelu_f(v, gelu_form);
          C[(int64_t)row * ldc + col] = (f16)v;
        }
      }
    }
  }
}

template <int MF, int BM, int BN, int WGM, int WGN, int EPI, int WDEPTH>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f16_mfma_kernel(const f16* __restrict__ A, int lda,
                                                                 const f16* __restrict__ W, int ldw,
                                                                 const f16* __restrict__ bias,
                                                                 const f16* __restrict__ R, f16* __restrict__ C,
                                                                 int ldc, int M, int N, int K, int gelu_form,
                                                                 int tiles_m, int tiles_n, float* __restrict__ P) {
  using FR = Frag<MF>;
  using acc_t = typename FR::acc_t;
  constexpr int NW = WGM * WGN;                // waves: WGM x WGN grid over the tile
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int NSTEP = kBK / FR::kK;          // MFMA K steps per K tile (4 or 2)
  constexpr int AJ = BM / (8 * NW), BJ = BN / (8 * NW);  // direct-to-LDS loads per wave per K tile (8 rows each)
  constexpr int ASZ = BM * kBK, WSZ = BN * kBK;  // halves per A / W stage
  static_assert(NSTEP == 2 || NSTEP == 4, "two or four K steps per K tile");
  // LDS ring: 2 A stages and WD W stages.  WD == 2: [A0 W0 | A1 W1].  WD == 3:
  // [A0 | W0 | W1 | A1 | W2], so that A1 and W2 are adjacent: the epilogue
  // stages through them while the next tile's A0, W0 and W1 load.
  constexpr int WD = (BM == 256 && BN == 256 && BJ == 8) ? WDEPTH : 2;
  static_assert(WD == 2 || WD == 3, "two or three W stages");
  constexpr int RING = 2 * ASZ + WD * WSZ;
  __shared__ __attribute__((aligned(16))) f16 smem[RING];
  auto a_off = [](int st) { return WD == 2 ? st * (ASZ + WSZ) : (st ? ASZ + 2 * WSZ : 0); };
  auto w_off = [](int st) { return WD == 2 ? st * (ASZ + WSZ) + ASZ : (st == 2 ? 2 * ASZ + 2 * WSZ : ASZ + st * WSZ); };

  // split-K: workgroup row y of the grid sums the y-th of gridDim.y equal K ranges
  const int k_len = K / (int)gridDim.y, kbeg = (int)blockIdx.y * k_len;
  const int n_tiles = tiles_m * tiles_n;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: keeps LDS bases scalar

  // ---- global -> LDS: each wave fills rows [wave*BM/NW, (wave+1)*BM/NW) of the A
  // tile (and likewise of W) with 16-byte direct-to-LDS buffer loads.  One load
  // of a wave writes 1 KiB of LDS = 8 rows; lane l lands in row l/8, physical
  // chunk l%8, so it fetches the logical chunk (l%8) ^ f(row).  The buffer
  // descriptors start at the tile's first row and end at the last valid row
  // (M or N), so rows past the end read as zeros and offsets stay 32-bit.
  const int lr = lane >> 3, lp = lane & 7;
  int aoff[AJ], boff[BJ];  // byte offsets of this lane's 16-byte chunk, K tile 0
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int r = wave * (BM / NW) + 8 * j + lr;
    aoff[j] = (r * lda + ((lp ^ lds_swizzle(r)) * 8)) * 2;
  }
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    const int r = wave * (BN / NW) + 8 * j + lr;
    boff[j] = (r * ldw + ((lp ^ lds_swizzle(r)) * 8)) * 2;
  }
  __amdgpu_buffer_rsrc_t arsrc, wrsrc;
  int m0 = 0, n0 = 0;
  auto set_tile = [&](int tile) {
    tile_origin<BM, BN>(tile, n_tiles, tiles_m, tiles_n, m0, n0);
    arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * lda), (short)0, min(BM, M - m0) * lda * 2,
                                              kBufferFlags);
    wrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)n0 * ldw), (short)0, min(BN, N - n0) * ldw * 2,
                                              kBufferFlags);
  };
  // load q of a tile's A rows (q < AJ, K offset ka into A stage as) or of its
  // W rows (K offset kw into W stage ws); A loads are issued before W loads
  auto dma_one = [&](int as, int ka, int ws, int kw, int q) {
    if (q < AJ) {
      f16* sa = smem + a_off(as) + (wave * (BM / NW) + 8 * q) * kBK;
      buffer_load_lds16(arsrc, sa, aoff[q], (kbeg + ka) * 2);
    } else {
      f16* sb = smem + w_off(ws) + (wave * (BN / NW) + 8 * (q - AJ)) * kBK;
      buffer_load_lds16(wrsrc, sb, boff[q - AJ], (kbeg + kw) * 2);
    }
  };
  auto dma_a = [&](int as, int ka) {
#pragma unroll
    for (int q = 0; q < AJ; ++q) dma_one(as, ka, 0, 0, q);
  };
  auto dma_w = [&](int ws, int kw) {
#pragma unroll
    for (int q = AJ; q < AJ + BJ; ++q) dma_one(0, 0, ws, kw, q);
  };

  // ---- wave / lane roles for the MFMA fragments.  Fragment rows are
  // lane % MF (+ MF per fragment), so f(row) = f(lane % 16) for both shapes.
  const int wm = wave / WGN, wn = wave % WGN;
  const int kg = lane / MF;  // which 8-wide K group of an MFMA step this lane feeds
  const int rsw = lds_swizzle(lane & 15);
  const int abase = (wm * WTM + lane % MF) * kBK;
  const int bbase = (wn * WTN + lane % MF) * kBK;
  // Reads are issued in the order the MFMAs below consume them (a0, b0..bN, a1..aM),
  // so each MFMA waits only for its own operands.
  auto frag_one = [&](int as, int ws, int kk, int r, half8 (&af)[FM], half8 (&bf)[FN]) {
    const f16* sa = smem + a_off(as);
    const f16* sw = smem + w_off(ws);
    const int ch = ((kk * (FR::kK / 8) + kg) ^ rsw) * 8;
    if (r == 0)
      af[0] = *reinterpret_cast<const half8*>(sa + abase + ch);
    else if (r <= FN)
      bf[r - 1] = *reinterpret_cast<const half8*>(sw + bbase + (r - 1) * MF * kBK + ch);
    else
      af[r - FN] = *reinterpret_cast<const half8*>(sa + abase + (r - FN) * MF * kBK + ch);
  };
  auto frags = [&](int as, int ws, int kk, half8 (&af)[FM], half8 (&bf)[FN]) {
#pragma unroll
    for (int r = 0; r < FM + FN; ++r) frag_one(as, ws, kk, r, af, bf);
  };

  acc_t acc[FM][FN];
  auto mfmas = [&](const half8 (&af)[FM], const half8 (&bf)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = FR::mfma(af[i], bf[j], acc[i][j]);
  };

  // ---- main loop.  A stage kt%2 and W stage kt%WD hold K tile kt.  The
  // barrier at the end of tile kt both publishes tile kt+1 (each wave waited
  // for its own loads of it) and retires every read of those stages, which
  // then receive A of tile kt+2 and W of tile kt+WD (clamped to the last tile:
  // a redundant load into a stage nobody reads again keeps the loop body free
  // of branches).  With WD == 3 a W load has two K tiles of MFMAs to land: W
  // streams from HBM, while A (the activations) mostly hits in the caches.
  // The MFMAs of the tile's last K step issue after the barrier, from
  // fragments already in registers, while the next tile's first fragments
  // and the new loads are in flight.
  //
  // Within a K step the order is written out and fenced with sched_barrier:
  // the LDS reads of the next step are spread evenly over the MFMAs (reads in
  // consumption order: a0, b0.., a1..) and, after the barrier, so are the
  // tile's direct-to-LDS loads.  LDS demand stays even (no bursts) and each
  // operand is requested well before its first use.
  constexpr int NF = FM + FN;  // LDS reads per K step
  constexpr int NM = FM * FN;  // MFMAs per K step
  constexpr int NL = AJ + BJ;  // direct-to-LDS loads per K tile
  // MFMAs of step X interleaved with the reads of step rkk from stages
  // (ras, rws) into Y, and (with_dma, a compile-time flag so the step stays
  // one basic block) with the loads of A offset dka into stage das and of W
  // offset dkw into stage dws.
  auto step = [&](auto with_dma, const half8 (&xa)[FM], const half8 (&xb)[FN], int ras, int rws, int rkk,
                  half8 (&ya)[FM], half8 (&yb)[FN], int das, int dka, int dws, int dkw) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (decltype(with_dma)::value) {
#pragma unroll
        for (int q = m * NL / NM; q < (m + 1) * NL / NM; ++q) dma_one(das, dka, dws, dkw, q);
      }
#pragma unroll
      for (int r = m * NF / NM; r < (m + 1) * NF / NM; ++r) frag_one(ras, rws, rkk, r, ya, yb);
      const int i = m / FN, j = m % FN;
      acc[i][j] = FR::mfma(xa[i], xb[j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int nk = k_len / kBK;
  half8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  const std::integral_constant<bool, false> no_dma;
  const std::integral_constant<bool, true> with_dma;
  // the K steps of a tile before its barrier (all but the last); NSTEP is even,
  // so the last step's fragments are always in fa1/fb1
  auto steps_before_barrier = [&](int as, int ws) {
    step(no_dma, fa0, fb0, as, ws, 1, fa1, fb1, 0, 0, 0, 0);
    if constexpr (NSTEP == 4) {
      step(no_dma, fa1, fb1, as, ws, 2, fa0, fb0, 0, 0, 0, 0);
      step(no_dma, fa0, fb0, as, ws, 3, fa1, fb1, 0, 0, 0, 0);
    }
  };

  // ---- tiles: one per workgroup, or several (a persistent launch, fewer
  // workgroups than tiles).  When the epilogue's staging fits in the ring's
  // second half (A1 and the last W stage), the next tile's first K tiles are
  // loaded into the first half while this tile's results are stored.
  using SE = StagedEpilogue<MF, FN>;
  constexpr int kStageAt = a_off(1), kStageRoom = RING - kStageAt;  // halves
  constexpr bool kOverlap = NW * SE::kFloats * 4 <= kStageRoom * 2;
  static_assert(NW * SE::kFloats * 4 <= RING * 2, "epilogue staging exceeds the LDS ring");
  const bool vec_ok = (N & 7) == 0 && (ldc & 7) == 0 &&
                      ((reinterpret_cast<uintptr_t>(C) | reinterpret_cast<uintptr_t>(R)) & 15) == 0;
  float* const stage_base = reinterpret_cast<float*>(kOverlap ? smem + kStageAt : smem);
  // the loads of a tile's first K tile (A0, W0), which do not touch the
  // staging area; the rest follow at the tile's start (the epilogue's
  // barriers wait for every load in flight, so it gets no more than these)
  auto early_loads = [&]() {
    dma_a(0, 0);
    dma_w(0, 0);
  };
  int tile = blockIdx.x;
  if (tile >= n_tiles) return;
  set_tile(tile);
  early_loads();
  for (;;) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < FR::kElems; ++e) acc[i][j][e] = 0.f;
    // A0 and W0 are in flight (issued above, or during the previous epilogue)
    dma_a(1, min(1, nk - 1) * kBK);
    if constexpr (WD == 3) dma_w(1, min(1, nk - 1) * kBK);
    dma_w(WD - 1, min(WD - 1, nk - 1) * kBK);
    wait_dma();
    __syncthreads();
    frags(0, 0, 0, fa0, fb0);
    int ca = 0, cw = 0;  // stages of K tile kt
    for (int kt = 0; kt + 1 < nk; ++kt) {
      steps_before_barrier(ca, cw);
      if constexpr (WD == 3) {
        // A of tile kt+1 and W of tile kt+1 landed; W of tile kt+2 may still fly
        barrier_after_loads<BJ>();
      } else {
        wait_dma();
        __syncthreads();
      }
      const int na = ca ^ 1, nw = cw + 1 == WD ? 0 : cw + 1;
      step(with_dma, fa1, fb1, na, nw, 0, fa0, fb0, ca, min(kt + 2, nk - 1) * kBK, cw,
           min(kt + WD, nk - 1) * kBK);
      ca = na;
      cw = nw;
    }
    steps_before_barrier(ca, cw);
    mfmas(fa1, fb1);
    wait_dma();  // no load may still be writing LDS when it is reused or the workgroup retires

    const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN;
    const int next = tile + (int)gridDim.x;
    __syncthreads();  // every wave is done reading the ring
    if (kOverlap && next < n_tiles) {
      set_tile(next);
      early_loads();
    }
    float* const Pp = P + (int64_t)blockIdx.y * M * N;
    if (vec_ok)
      store_tile_staged<MF, FM, FN, EPI>(acc, stage_base + wave * SE::kFloats, row0, col0, lane, bias, R, C, M, N,
                                         ldc, gelu_form, Pp);
    else
      store_tile<MF, FM, FN, EPI>(acc, row0, col0, lane, bias, R, C, M, N, ldc, gelu_form, Pp);
    if (next >= n_tiles) break;
    tile = next;
    __syncthreads();  // every wave's staging is done before the ring is loaded again
    if (!kOverlap) {
      set_tile(tile);
      early_loads();
    }
  }
}

// max_wgs > 0: at most that many workgroups, each looping over tiles
template <int MF, int BM, int BN, int WGM, int WGN, int WDEPTH = 2>
hipError_t launch_cfg(const void* A, const void* W, const void* bias, const void* R, int M, int N, int K,
                      const GemmPitch& ld, int epi, ee_gelu form, void* C, int splits, float* P, hipStream_t s,
                      int max_wgs = 0) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int wgs = max_wgs > 0 ? std::min(tm * tn, max_wgs) : tm * tn;
  const dim3 grid((unsigned)wgs, (unsigned)splits), block(64 * WGM * WGN);
  const f16* a = static_cast<const f16*>(A);
  const f16* w = static_cast<const f16*>(W);
  const f16* b = static_cast<const f16*>(bias);
  const f16* r = static_cast<const f16*>(R);
  f16* c = static_cast<f16*>(C);
#define EE_GEMM_LAUNCH(E)                                                                                        \
  hipLaunchKernelGGL((gemm_f16_mfma_kernel<MF, BM, BN, WGM, WGN, E, WDEPTH>), grid, block, 0, s, a, ld.a, w, ld.w, b, r, \
                     c, ld.c, M, N, K, (int)form, tm, tn, P)
  switch (epi) {
    case EE_EPI_NONE: EE_GEMM_LAUNCH(EE_EPI_NONE); break;
    case EE_EPI_BIAS: EE_GEMM_LAUNCH(EE_EPI_BIAS); break;
    case EE_EPI_BIAS_RESIDUAL: EE_GEMM_LAUNCH(EE_EPI_BIAS_RESIDUAL); break;
    case EE_EPI_BIAS_GELU: EE_GEMM_LAUNCH(EE_EPI_BIAS_GELU); break;
    case kEpiPartial: EE_GEMM_LAUNCH(kEpiPartial); break;
  }
#undef EE_GEMM_LAUNCH
  return hipGetLastError();
}

// C = epilogue(sum over the splits of P[split]): the partial sums added in
// split order in fp32, then bias, GeLU or residual and one fp16 rounding, as
// the unsplit store does.  8 columns per thread (N % 8 == 0) or 1.
template <int EPI, int V>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int splits, int64_t M, int N,
                                                          const f16* __restrict__ bias, const f16* __restrict__ R,
                                                          f16* __restrict__ C, int ldc, int gelu_form) {
  const int64_t per_row = N / V, total = M * per_row;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row;
    const int col = (int)(i - row * per_row) * V;
    float v[V];
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = 0.f;
    for (int sp = 0; sp < splits; ++sp) {
      const float* src = P + ((int64_t)sp * M + row) * N + col;
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] += src[k];
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
      float x = v[k] + (kHasBias<EPI> ? (float)bias[col + k] : 0.f);
      if (EPI == EE_EPI_BIAS_RESIDUAL) x += (float)R[row * ldc + col + k];
      if (EPI == EE_EPI_BIAS_GELU) x = gelu_f(x, gelu_form);
      C[row * ldc + col + k] = (f16)x;
    }
  }
}

template <int EPI>
hipError_t launch_reduce(const float* P, int splits, int64_t M, int N, const void* bias, const void* R, void* C,
                         int ldc, ee_gelu form, hipStream_t s) {
  const bool vec = N % 8 == 0 && ldc % 8 == 0;
  const int64_t items = M * (vec ? N / 8 : N);
  const unsigned grid = (unsigned)std::min<int64_t>((items + 255) / 256, 4096);
  if (vec)
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI, 8>), dim3(grid), dim3(256), 0, s, P, splits, M, N,
                       static_cast<const f16*>(bias), static_cast<const f16*>(R), static_cast<f16*>(C), ldc, (int)form);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI, 1>), dim3(grid), dim3(256), 0, s, P, splits, M, N,
                       static_cast<const f16*>(bias), static_cast<const f16*>(R), static_cast<f16*>(C), ldc, (int)form);
  return hipGetLastError();
}

}  // namespace

int device_cu_count() {
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

bool gemm_f16_mfma_ok(int64_t M, int N, int K, const GemmPitch& ld, const void* A, const void* W) {
  const bool pitches = ld.a >= K && ld.w >= K && ld.c >= N && ld.a % 8 == 0 && ld.w % 8 == 0 &&
                       (int64_t)256 * std::max(ld.a, ld.w) * 2 < (1ll << 31);
  const bool aligned = ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(W)) & 15) == 0;
  return M >= 1 && M <= (1 << 30) && N >= 1 && K >= kBK && K % kBK == 0 && pitches && aligned;
}

// Time of a 128 x 128 tile relative to a 256 x 256 tile of the same K (a
// quarter of the work at a lower MFMA rate).
constexpr double kSmallTileCost = 0.36;

// Rows [0, m_big) of a large problem go to the 256 x 256 kernel and the rest
// to 128 x 128 tiles.  A tile count just past a multiple of the CU count
// leaves most CUs idle in the last round of 256 x 256 tiles; running only
// whole rounds of 256-row tiles there and the remaining rows as 128 x 128
// tiles ends sooner.  Both kernels add an element's K tiles in the same order;
// their MFMA shapes differ (16x16x32 and 32x32x16), and on gfx950 they give
// the same bits for every element (tested on random data against GEMMs run
// on each 256-row block alone), so the split changes no results.
int64_t gemm_big_rows(int64_t M, int N, int cus) {
  const int64_t tn = (N + 255) / 256, tiles = ((M + 255) / 256) * tn;
  const int64_t whole = tiles / cus * cus;
  if (whole == tiles) return M;
  const int64_t m_tiles = whole / tn;  // 256-row tiles that fit in the whole rounds
  const int64_t rest = M - m_tiles * 256;
  if (m_tiles <= 0 || rest <= 0) return M;
  const int64_t small = ((rest + 127) / 128) * ((N + 127) / 128);
  const double t_plain = (double)((tiles + cus - 1) / cus);
  const double t_split = (double)((m_tiles * tn + cus - 1) / cus) + kSmallTileCost * (double)((small + cus - 1) / cus);
  return t_split < t_plain ? m_tiles * 256 : M;
}

hipError_t launch_gemm_f16_mfma(const void* A, const void* W, const void* bias, const void* R, int64_t M, int N,
                                int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int64_t tiles_big = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles_big >= 256) {
    const int cus = device_cu_count();
    const int wgs = EE_GEMM_PERSIST ? cus : 0;
    const int64_t m_big = gemm_big_rows(M, N, cus);
    hipError_t e;
    if (K >= EE_GEMM_DEEP_W_K)
      e = launch_cfg<EE_GEMM_MF, 256, 256, EE_GEMM_WGM, EE_GEMM_WGN, 3>(A, W, bias, R, (int)m_big, N, K, ld, epi, form,
                                                                        C, 1, nullptr, s, wgs);
    else
      e = launch_cfg<EE_GEMM_MF, 256, 256, EE_GEMM_WGM, EE_GEMM_WGN, 2>(A, W, bias, R, (int)m_big, N, K, ld, epi, form,
                                                                        C, 1, nullptr, s, wgs);
    if (e != hipSuccess || m_big == M) return e;
    // the remaining rows: A, C and the residual from row m_big on
    const f16* a = static_cast<const f16*>(A) + m_big * ld.a;
    const f16* r = R ? static_cast<const f16*>(R) + m_big * ld.c : nullptr;
    f16* c = static_cast<f16*>(C) + m_big * ld.c;
    const int64_t rest = M - m_big;
    // Few remaining rows stream all of W through few tiles: 128 x 64 tiles
    // (the same MFMA shape) put twice as many CUs on it.
    if (((rest + 127) / 128) * ((N + 127) / 128) * 2 <= cus)
      return launch_cfg<32, 128, 64, 2, 2>(a, W, bias, r, (int)rest, N, K, ld, epi, form, c, 1, nullptr, s);
    return launch_cfg<32, 128, 128, 2, 2>(a, W, bias, r, (int)rest, N, K, ld, epi, form, c, 1, nullptr, s);
  }
  return launch_cfg<32, 128, 128, 2, 2>(A, W, bias, R, (int)M, N, K, ld, epi, form, C, 1, nullptr, s);
}

// Measured at M = 32 on the GPT-3 decode shapes (weights streamed once): four
// K ranges were best on all four (QKV 201 vs 217 us unsplit, FC1 232 vs 238,
// FC2 237 vs 632, out 67 vs 171); two were slower than none wherever the
// unsplit grid already had a workgroup per CU.
int gemm_f16_splitk_choice(int64_t M, int N, int K, size_t scratch_bytes) {
  if (M > 128) return 1;
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  for (int splits = 4; splits >= 2; splits /= 2) {
    const bool fits = K % (kBK * splits) == 0 && K / splits >= 4 * kBK &&
                      (size_t)splits * (size_t)M * (size_t)N * 4 <= scratch_bytes;
    if (fits && (splits == 4 || tiles < 256)) return splits;
  }
  return 1;
}

size_t gemm_f16_splitk_bytes(int64_t M, int N, int splits) { return (size_t)splits * (size_t)M * (size_t)N * 4; }

hipError_t launch_gemm_f16_splitk(const void* A, const void* W, const void* bias, const void* R, int64_t M, int N,
                                  int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C, int splits,
                                  void* scratch, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  float* P = static_cast<float*>(scratch);
  // the partial sums are dense [splits][M][N]
  const GemmPitch pld{ld.a, ld.w, N};
  hipError_t e = launch_cfg<32, 128, 128, 2, 2>(A, W, nullptr, nullptr, (int)M, N, K, pld, kEpiPartial, form,
                                                nullptr, splits, P, s);
  if (e != hipSuccess) return e;
  switch (epi) {
    case EE_EPI_NONE: return launch_reduce<EE_EPI_NONE>(P, splits, M, N, bias, R, C, ld.c, form, s);
    case EE_EPI_BIAS: return launch_reduce<EE_EPI_BIAS>(P, splits, M, N, bias, R, C, ld.c, form, s);
    case EE_EPI_BIAS_RESIDUAL:
      return launch_reduce<EE_EPI_BIAS_RESIDUAL>(P, splits, M, N, bias, R, C, ld.c, form, s);
    case EE_EPI_BIAS_GELU: return launch_reduce<EE_EPI_BIAS_GELU>(P, splits, M, N, bias, R, C, ld.c, form, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ee
