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
//   * Tile order (gemm_tile_order.h): the hardware deals consecutive workgroup
//     ids round-robin to the 8 XCDs; each XCD walks its share of the tiles in
//     groups of 4 M-tiles, so the workgroups that share an XCD's L2 share A and
//     W panels, and pairs of XCDs split the N range of the same groups.
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
#include <atomic>
#include <chrono>
#include <numeric>
#include <random>
#include <type_traits>

#include "device_common.h"
#include "gemm_ordered_split.h"
#include "gemm_plan.h"
#include "gemm_tile_order.h"
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
#ifndef EE_GEMM_WIDE
#define EE_GEMM_WIDE 1
#endif
#ifndef EE_GEMM_WIDE_LB
#define EE_GEMM_WIDE_LB 5
#endif
#ifndef EE_GEMM_WIDE_Q1
#define EE_GEMM_WIDE_Q1 6
#endif
#ifndef EE_GEMM_WIDE_FOLD
#define EE_GEMM_WIDE_FOLD 0
#endif
#ifndef EE_GEMM_WIDE_GAP1
#define EE_GEMM_WIDE_GAP1 5
#endif
// Bands of the residual requested ahead in the staged epilogue: 3 on 256 x
// 256 tiles (the TP-shard out projection, K = 3072, 2-3% faster; no change at
// K = 12288 and 49152); none on 256 x 384, whose register file has no room
// (one band ahead added spills and no speed).
#ifndef EE_GEMM_RES_AHEAD
#define EE_GEMM_RES_AHEAD 3
#endif
#ifndef EE_GEMM_RES_AHEAD_WIDE
#define EE_GEMM_RES_AHEAD_WIDE 0
#endif
#ifndef EE_GEMM_DEEP_W_K
#define EE_GEMM_DEEP_W_K 32768
#endif

constexpr int kBK = 64;
// Cache policy bit (sc1) of a buffer access: device scope, so a store is
// written through to memory and a load is served from it, not from a line
// this XCD's L2 may hold.
constexpr int kCacheDevice = 16;
// Split-K partial store (internal): fp32 sums of one K range, no epilogue.
constexpr int kEpiPartial = 4;
template <int EPI>
constexpr bool kHasBias = EPI == EE_EPI_BIAS || EPI == EE_EPI_BIAS_RESIDUAL || EPI == EE_EPI_BIAS_GELU;

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

// f(std::integral_constant<int, I>) for I = I0 .. N - 1, unrolled by the
// compiler's front end (a loop of inline asm blocks is not always unrolled).
template <int I0, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, N>(f);
  }
}

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

//
// With RAW and a `raw` target, the same path stores the tile's plain fp32
// sums instead (no bias, GeLU or residual): row-major at a pitch of raw_ld
// elements from the tile origin (rm0, rn0) over raw_rows rows, written through to memory
// (device-scope stores) for a workgroup on another XCD.  One consumer of the
// accumulators for both results: a second store path beside this one made the
// register allocator spill in the persistent kernel.
template <int MF, int FM, int FN, int EPI, bool RAW = false>
__device__ __forceinline__ void store_tile_staged(const typename Frag<MF>::acc_t (&acc)[FM][FN], float* __restrict__ stage,
                                                  int row0, int col0, int lane, const f16* __restrict__ bias,
                                                  const f16* __restrict__ R, f16* __restrict__ C, int M, int N,
                                                  int ldc, int gelu_form, float* __restrict__ Pp,
                                                  float* __restrict__ raw = nullptr, int raw_rows = 0,
                                                  int raw_ld = 0, int rm0 = 0, int rn0 = 0) {
  const bool to_raw = RAW && raw != nullptr;
  using SE = StagedEpilogue<MF, FN>;
  constexpr int FPB = 1;  // fragment rows per band
  constexpr int PASSES = SE::kBandRows / SE::kRowsPerPass;
  const int c8 = lane % SE::kLanesPerRow, rsub = lane / SE::kLanesPerRow;
  // a 192-column wave tile has 24 lanes per row: lanes 48-63 stay idle
  const bool lane_on = SE::kRowsPerPass * SE::kLanesPerRow == 64 || rsub < SE::kRowsPerPass;
  const int col = col0 + c8 * 8;
  float bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cj = col0 + j * MF + lane % MF;
    bcol[j] = (kHasBias<EPI> && cj < N) ? (float)bias[cj] : 0.f;
  }
  // The residual rows of band b are requested RA bands ahead, while band
  // b - RA goes through LDS: the registers that held the main loop's operand
  // fragments are free here, and a request issued at its own band waited
  // out most of its latency.
  constexpr int NB = FM / FPB;
  constexpr int RA = EPI == EE_EPI_BIAS_RESIDUAL ? (FN > 8 ? EE_GEMM_RES_AHEAD_WIDE : EE_GEMM_RES_AHEAD) : 0;
  constexpr int RS = (RA < NB ? RA : NB - 1) + 1;  // residual band buffers
  half8 rvb[RS][PASSES];
  auto load_rv = [&](auto BAND) __attribute__((always_inline)) {
    constexpr int band = decltype(BAND)::value;
    if constexpr (EPI == EE_EPI_BIAS_RESIDUAL && band < NB) {
#pragma unroll
      for (int it = 0; it < PASSES; ++it) {
        const int row = row0 + band * SE::kBandRows + it * SE::kRowsPerPass + rsub;
        if (!to_raw && lane_on && row < M && col < N)
          rvb[band % RS][it] = *reinterpret_cast<const half8*>(R + (int64_t)row * ldc + col);
      }
    }
  };
  static_for<0, RS - 1>([&](auto B) __attribute__((always_inline)) { load_rv(B); });
  // bands unrolled by the front end: with GeLU a 12-fragment band is too long
  // for the loop unroller, and an indexed band would put acc in memory
  static_for<0, NB>([&](auto BAND) __attribute__((always_inline)) {
    constexpr int band = decltype(BAND)::value;
    load_rv(std::integral_constant<int, band + RS - 1>{});
    half8 (&rv)[PASSES] = rvb[band % RS];
#pragma unroll
    for (int ii = 0; ii < FPB; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < Frag<MF>::kElems; ++e) {
          const float a = acc[band * FPB + ii][j][e];
          float v = a + bcol[j];
          if (EPI == EE_EPI_BIAS_GELU) v = gelu_f(v, gelu_form);
          stage[(ii * MF + Frag<MF>::row(lane, e)) * SE::kLd + j * MF + lane % MF] = to_raw ? a : v;
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < PASSES; ++it) {
      const int r = it * SE::kRowsPerPass + rsub;
      const int row = row0 + band * SE::kBandRows + r;
      if (!lane_on) continue;
      const float4 lo = *reinterpret_cast<const float4*>(stage + r * SE::kLd + c8 * 8);
      const float4 hi = *reinterpret_cast<const float4*>(stage + r * SE::kLd + c8 * 8 + 4);
      if (to_raw) {
        // bounded by the tile: a store outside it is dropped
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(raw, (short)0, raw_rows * raw_ld * 4, kBufferFlags);
        const int off = ((row - rm0) * raw_ld + (col - rn0)) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), rs, off, 0, kCacheDevice);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), rs, off + 16, 0, kCacheDevice);
      } else if (EPI == kEpiPartial) {
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
  });
}

// Direct per-element epilogue of a wave's FM x FN block of fragments whose
// top-left output element is (row0, col0); used when N % 8 != 0.
template <int MF, int FM, int FN, int EPI>
__device__ __forceinline__ void store_tile(const typename Frag<MF>::acc_t (&acc)[FM][FN], int row0, int col0, int lane,
                                           const f16* __restrict__ bias, const f16* __restrict__ R,
                                           f16* __restrict__ C, int M, int N, int ldc, int gelu_form,
                                           float* __restrict__ Pp) {
  static_for<0, FN>([&](auto J) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    const int col = col0 + j * MF + lane % MF;
    if (col >= N) return;
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
  });
}

// In-order stream-K of a persistent launch's partial last round.  After
// `rounds` whole rounds of tiles (tile = blockIdx.x + r * gridDim.x), the
// `extra` tiles left are cut into `wgs` equal contiguous ranges of their
// (tile, K tile) steps, one range per workgroup.  A piece that starts inside
// a tile continues from the fp32 sums that the previous workgroup (whose range
// ends there) stored in its slot of `partial`, once that workgroup's flag
// holds this launch's `tag`: every element still adds its K tiles in one
// chain, in order, so the bits are those of the tile computed whole.  A piece
// runs after about as many of its workgroup's whole tiles as its first K tile
// is far into the tile, so its predecessor (an earlier slot) is done by then.
// extra == 0: whole tiles only (the last round partial).
struct OrderedSplit {
  unsigned long long* flags;  // [wgs]; then, kOrderedFlagBytes on, [wgs][BM * BN] fp32 partial tiles
  unsigned long long tag;     // unique per launch
  int rounds, extra, wgs;
};
// Polls of a predecessor's flag (about 0.25 us apart) before a piece gives up
// and recomputes its tile from K tile 0: only if the predecessor never ran,
// which a launch of at most one workgroup per CU, alone on the device, rules out.
constexpr int kOrderedSpin = 1 << 16;

template <int MF, int BM, int BN, int WGM, int WGN, int EPI, int WDEPTH, bool ORD>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f16_mfma_kernel(const f16* __restrict__ A, int lda,
                                                                 const f16* __restrict__ W, int ldw,
                                                                 const f16* __restrict__ bias,
                                                                 const f16* __restrict__ R, f16* __restrict__ C,
                                                                 int ldc, int M, int N, int K, int gelu_form,
                                                                 int tiles_m, int tiles_n, float* __restrict__ P,
                                                                 OrderedSplit os) {
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
  int kb = kbeg;  // K offset of the current work item's first K tile
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
    gemm_tile_origin(tile, n_tiles, tiles_m, tiles_n, BM, BN, m0, n0);
    arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * lda), (short)0, min(BM, M - m0) * lda * 2,
                                              kBufferFlags);
    wrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)n0 * ldw), (short)0, min(BN, N - n0) * ldw * 2,
                                              kBufferFlags);
  };
  // load q of a tile's A rows (q < AJ, K offset ka into A stage as) or of its
  // W rows (K offset kw into W stage ws); A loads are issued before W loads
  // Rows 16 apart have the same swizzle, so a 256 x 384 tile (whose register
  // file has no room for an offset per load) keeps the offsets of loads 0
  // and 1 and adds 16 rows per further pair in the loop itself; the row
  // offset stays in the lane offset, which the descriptor's range check sees.
  auto lane_off = [&](const int* off, int q, int ld) {
    if constexpr (BN == 384 && EE_GEMM_WIDE_FOLD) {
      int o = off[q & 1];
      asm volatile("" : "+v"(o));
      return o + (q >> 1) * 32 * ld;
    } else {
      return off[q];
    }
  };
  auto dma_one = [&](int as, int ka, int ws, int kw, int q) {
    if (q < AJ) {
      f16* sa = smem + a_off(as) + (wave * (BM / NW) + 8 * q) * kBK;
      buffer_load_lds16(arsrc, sa, lane_off(aoff, q, lda), (kb + ka) * 2);
    } else {
      f16* sb = smem + w_off(ws) + (wave * (BN / NW) + 8 * (q - AJ)) * kBK;
      buffer_load_lds16(wrsrc, sb, lane_off(boff, q - AJ, ldw), (kb + kw) * 2);
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
  // ---- one tile's (or piece's) K loop over nk K tiles from K offset kb,
  // after its first K tile's loads (A0, W0) were issued
  auto k_loop = [&](int nk) {
    // A0 and W0 are in flight (issued before, or during the previous epilogue)
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
  };
  // ---- the K loop of a 256 x 384 tile (wave tile 128 x 192: 384 accumulators
  // per lane).  Both operands' fragments for a whole K step, double-buffered
  // as above, would not fit beside them, so the A fragments alone are
  // double-buffered and the W (B) fragments stream through a ring of NBR
  // registers: the MFMAs go column by column (column j's FM MFMAs take B
  // fragment j and the resident A fragments) and B fragment j + LB is read at
  // the start of column j.  Step 1 of K tile kt reads its last B fragment
  // (column FN - 1) at column PB - 1; the tile's one barrier sits before
  // column PB.  It waits for this wave's loads of tile kt + 1 and for its LDS
  // reads, so after it the next tile's A fragments and first B fragments are
  // read from the other stage, and the loads of tile kt + 2 go into this one:
  // loads [0, Q1) after the barrier, the rest in step 0 of tile kt + 1.
  //
  // The compiler gives every MFMA accumulator the AGPR class, and 384 do not
  // fit in the 256 AGPRs: columns [0, kWideA) use the builtin (AGPRs), the
  // rest inline asm with VGPR accumulators.  The compiler knows nothing of
  // the asm MFMAs' latency, which matters only for their results (an MFMA
  // reads its A and B operands at issue, so a ring slot may be refilled right
  // after): each accumulator's MFMAs are a K step apart, and the s_nops after
  // the last step wait out the last ones before anything reads them.
  constexpr bool kWide = BN == 384;
  constexpr int LB = EE_GEMM_WIDE_LB, NBR = LB + 1, PB = FN - LB, Q1 = EE_GEMM_WIDE_Q1, kWideA = 8;
  constexpr int kPostSlots = (FN - PB) * FM;            // MFMA slots after the barrier
  constexpr int kAPer = (FM + (FN - PB) - 1) / (FN - PB);  // next-tile A reads per column there
  constexpr int kDmaGap2 = kPostSlots / (Q1 > 0 ? Q1 : 1);  // slots between loads there
  constexpr int kDmaGap1 = EE_GEMM_WIDE_GAP1;               // slots between step 0's loads
  static_assert(!kWide || (MF == 16 && NSTEP == 2 && WD == 2 && FN % NBR == 0 && PB > 0 && kAPer < FM &&
                           kDmaGap1 * (NL - Q1) <= FN * FM && kDmaGap2 >= 2 && FM * kWideA * 4 == 256),
                "the wide K loop's schedule");
  auto read_a = [&](int st, int kk, int i) {
    const int ch = ((kk * (FR::kK / 8) + kg) ^ rsw) * 8;
    return *reinterpret_cast<const half8*>(smem + a_off(st) + abase + i * MF * kBK + ch);
  };
  auto read_b = [&](int st, int kk, int j) {
    const int ch = ((kk * (FR::kK / 8) + kg) ^ rsw) * 8;
    return *reinterpret_cast<const half8*>(smem + w_off(st) + bbase + j * MF * kBK + ch);
  };
  half8 br[NBR];
  // One K step of a wide tile from stage c: S is the step (0 or 1); NX (step
  // 1) whether a next K tile follows; DM which loads go out: 1 = loads
  // [Q1, NL) of the tile at K offset dk into stage c ^ 1 (step 0), 2 = loads
  // [0, Q1) of it into stage c, after the barrier (step 1).
  auto wide_step = [&](auto S, auto NX, auto DM, auto Z, const half8 (&xa)[FM], half8 (&ya)[FM], int c,
                       int dk) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value, dm = decltype(DM)::value;
    constexpr bool nx = decltype(NX)::value, z = decltype(Z)::value;
    static_for<0, FN * FM>([&](auto M) __attribute__((always_inline)) {
      constexpr int m = decltype(M)::value, j = m / FM, i = m % FM;
      if constexpr (s == 1 && nx && m == PB * FM) barrier_after_loads<0>();
      if constexpr (i == 0) {
        constexpr int jb = j + LB;
        if constexpr (jb < FN)
          br[jb % NBR] = read_b(c, s, jb);
        else if constexpr (s == 0)
          br[jb % NBR] = read_b(c, 1, jb - FN);
        else if constexpr (nx)
          br[jb % NBR] = read_b(c ^ 1, 0, jb - FN);
      }
      if constexpr (s == 0 && i == FM / 2 && j < FM) ya[j] = read_a(c, 1, j);
      if constexpr (s == 1 && nx && j >= PB && i % (FM / kAPer) == 1) {
        constexpr int ia = (j - PB) * kAPer + i / (FM / kAPer);
        if constexpr (ia < FM) ya[ia] = read_a(c ^ 1, 0, ia);
      }
      if constexpr (dm == 1 && m >= 2 && (m - 2) % kDmaGap1 == 0 && (m - 2) / kDmaGap1 < NL - Q1)
        dma_one(c ^ 1, dk, c ^ 1, dk, Q1 + (m - 2) / kDmaGap1);
      if constexpr (dm == 2 && m > PB * FM && (m - PB * FM - 1) % kDmaGap2 == 0 && (m - PB * FM - 1) / kDmaGap2 < Q1)
        dma_one(c, dk, c, dk, (m - PB * FM - 1) / kDmaGap2);
      if constexpr (z && j < kWideA)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(acc[i][j]) : "v"(xa[i]), "v"(br[j % NBR]));
      else if constexpr (z)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=v"(acc[i][j]) : "v"(xa[i]), "v"(br[j % NBR]));
      else if constexpr (j < kWideA)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(xa[i]), "v"(br[j % NBR]));
      else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc[i][j]) : "v"(xa[i]), "v"(br[j % NBR]));
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // nk >= 1: a K loop of one K tile loads tile 0 twice (stage 1 is read by no step)
  auto k_loop_wide = [&](int nk, auto Z0) __attribute__((always_inline)) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    // K tile 0 (stage 0) is in flight; loads [0, Q1) of K tile 1 go into
    // stage 1 now, the rest in step 0 below, as for every later K tile
#pragma unroll
    for (int q = 0; q < Q1; ++q) dma_one(1, min(1, nk - 1) * kBK, 1, min(1, nk - 1) * kBK, q);
    barrier_after_loads<Q1>();
    br[0] = read_b(0, 0, 0);
#pragma unroll
    for (int i = 0; i < FM; ++i) fa0[i] = read_a(0, 0, i);
#pragma unroll
    for (int j = 1; j < LB; ++j) br[j] = read_b(0, 0, j);
    // step 0 of K tile 0 starts the sums from 0 (Z0: an inline constant, so
    // the accumulators are never written by VALU instructions, whose results
    // the asm MFMAs would not wait for) or from acc as prepared; then step 1
    // of K tile kt and step 0 of K tile kt + 1 per iteration
    wide_step(I0{}, F{}, I1{}, Z0, fa0, fa1, 0, min(1, nk - 1) * kBK);
    int kt = 0;
    for (; kt + 1 < nk; ++kt) {
      wide_step(I1{}, T{}, I2{}, F{}, fa1, fa0, kt & 1, min(kt + 2, nk - 1) * kBK);
      wide_step(I0{}, F{}, I1{}, F{}, fa0, fa1, (kt + 1) & 1, min(kt + 2, nk - 1) * kBK);
    }
    wide_step(I1{}, F{}, I0{}, F{}, fa1, fa0, kt & 1, 0);
    // the last MFMAs' results are written before anything reads them (24
    // wait states: more than a 16-pass MFMA needs)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    wait_dma();  // no load may still be writing LDS when it is reused or the workgroup retires
  };
  auto run_k_loop = [&](int nk) {
    if constexpr (kWide)
      k_loop_wide(nk, std::integral_constant<bool, !ORD>{});
    else
      k_loop(nk);
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < FR::kElems; ++e) acc[i][j][e] = 0.f;
  };
  auto epilogue = [&](int row0, int col0) {
    float* const Pp = P + (int64_t)blockIdx.y * M * N;
    if (vec_ok)
      store_tile_staged<MF, FM, FN, EPI>(acc, stage_base + wave * SE::kFloats, row0, col0, lane, bias, R, C, M, N,
                                         ldc, gelu_form, Pp);
    else
      store_tile<MF, FM, FN, EPI>(acc, row0, col0, lane, bias, R, C, M, N, ldc, gelu_form, Pp);
  };

  if constexpr (!ORD) {
    // ---- whole tiles: blockIdx.x, then every gridDim.x-th
    int tile = blockIdx.x;
    if (tile >= n_tiles) return;
    set_tile(tile);
    early_loads();
    for (;;) {
      zero_acc();
      run_k_loop(k_len / kBK);
      const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN;
      const int next = tile + (int)gridDim.x;
      __syncthreads();  // every wave is done reading the ring
      if (kOverlap && next < n_tiles) {
        set_tile(next);
        early_loads();
      }
      epilogue(row0, col0);
      if (next >= n_tiles) break;
      tile = next;
      __syncthreads();  // every wave's staging is done before the ring is loaded again
      if (!kOverlap) {
        set_tile(tile);
        early_loads();
      }
    }
  } else {
    // ---- in-order stream-K (gemm_ordered_split.h): whole tiles, and up to
    // two pieces of this workgroup's K range over the extra tiles.  The sums
    // a piece leaves, and the flag that publishes them, move by device-scope
    // coherent accesses (sc1: written through to memory, read past this XCD's
    // L2) ordered by waiting for the stores' completion, instead of fences,
    // which write back or invalidate the whole L2 of the XCD.
    const int b = blockIdx.x, G = gridDim.x, KT = k_len / kBK;
    // Item c, and the item count, recomputed where needed from the split's
    // three numbers: the register allocator is at its limit here, and values
    // kept live across the K loop would spill.  The empty asm hides the
    // inputs' provenance, so the computation stays where it is written.
    struct ItemAt {
      OrderedItem it;
      int n;
    };
    auto item_at = [&](int c) {
      int rounds = os.rounds, extra = os.extra, wgs = os.wgs;
      asm volatile("" : "+s"(rounds), "+s"(extra), "+s"(wgs));
      const OrderedWork w = ordered_work(b, G, n_tiles, KT, rounds, extra, wgs);
      return ItemAt{ordered_item(w, b, G, KT, c), ordered_items(w)};
    };
    const ItemAt first = item_at(0);
    if (first.n == 0) return;
    int c = 0;
    OrderedItem it = first.it;
    set_tile(it.tile);
    kb = kbeg + it.k0 * kBK;
    early_loads();
    for (;;) {
      zero_acc();
      if (it.pred >= 0) {
        // thread 0 polls the predecessor's flag; then every wave reads its sums
        int* const note = reinterpret_cast<int*>(smem + a_off(1));  // stage 1: not loaded yet
        if (t == 0) {
          int ok = 0;
          for (int n = 0; n < kOrderedSpin; ++n) {
            if (__hip_atomic_load(os.flags + it.pred, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == os.tag) {
              ok = 1;
              break;
            }
            __builtin_amdgcn_s_sleep(8);
          }
          *note = ok;
        }
        __syncthreads();
        const int ok = __builtin_amdgcn_readfirstlane(*note);
        __syncthreads();  // every wave has read `note` before stage 1 is loaded
        if (ok) {
          // the predecessor's sums, row-major in the tile (store_tile_staged's raw form)
          const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
              reinterpret_cast<char*>(os.flags) + kOrderedFlagBytes + (size_t)it.pred * BM * BN * 4, (short)0,
              BM * BN * 4, kBufferFlags);
          const int voff = ((wm * WTM + FR::row(lane, 0)) * BN + wn * WTN + lane % MF) * 4;
          static_for<0, FM * FN>([&](auto IJ) __attribute__((always_inline)) {
            constexpr int i = decltype(IJ)::value / FN, j = decltype(IJ)::value % FN;
#pragma unroll
            for (int e = 0; e < FR::kElems; ++e)
              acc[i][j][e] = __builtin_bit_cast(
                  float, __builtin_amdgcn_raw_buffer_load_b32(
                             src, voff, ((i * MF + FR::row(0, e) - FR::row(0, 0)) * BN + j * MF) * 4, kCacheDevice));
          });
        } else {
          // never published: compute the tile from its first K tile instead
          wait_dma();
          __syncthreads();
          it.k0 = 0;
          kb = kbeg;
          early_loads();
        }
      }
      if constexpr (kWide) {
        // the wide K loop's asm MFMAs take acc as it stands (zeros or a
        // predecessor's sums): each value is placed in its MFMA's register
        // class here, and the s_nops let those writes complete first
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < kWideA; ++j) asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
          for (int j = kWideA; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
        }
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
      }
      run_k_loop(it.k1 - it.k0);
      const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN;
      const int tile_m0 = m0, tile_n0 = n0;  // set_tile below moves m0, n0 to the next item
      const ItemAt nxa = item_at(c + 1);
      const bool more = c + 1 < nxa.n;
      const OrderedItem nx = nxa.it;
      __syncthreads();  // every wave is done reading the ring
      if (kOverlap && more) {
        set_tile(nx.tile);
        kb = kbeg + nx.k0 * kBK;
        early_loads();
      }
      // a piece that ends inside its tile leaves its sums for workgroup b + 1
      // (raw fp32, row-major in the tile), through the same staged store
      float* const raw = it.partial ? reinterpret_cast<float*>(reinterpret_cast<char*>(os.flags) + kOrderedFlagBytes) +
                                          (size_t)b * BM * BN
                                    : nullptr;
      if (vec_ok) {
        float* const Pp = P + (int64_t)blockIdx.y * M * N;
        store_tile_staged<MF, FM, FN, EPI, true>(acc, stage_base + wave * SE::kFloats, row0, col0, lane, bias, R, C,
                                                 M, N, ldc, gelu_form, Pp, raw, BM, BN, tile_m0, tile_n0);
      } else {
        epilogue(row0, col0);  // never with a partial piece: the host splits only where vec_ok holds
      }
      if (it.partial) {
        wait_dma();       // this wave's written-through stores have completed
        __syncthreads();  // ... and every other wave's
        if (t == 0) __hip_atomic_store(os.flags + b, os.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (!more) break;
      it = nx;
      ++c;
      __syncthreads();  // every wave's staging is done before the ring is loaded again
      if (!kOverlap) {
        set_tile(it.tile);
        kb = kbeg + it.k0 * kBK;
        early_loads();
      }
    }
  }
}

// max_wgs > 0: at most that many workgroups, each looping over tiles
template <int MF, int BM, int BN, int WGM, int WGN, int WDEPTH = 2>
hipError_t launch_cfg(const void* A, const void* W, const void* bias, const void* R, int M, int N, int K,
                      const GemmPitch& ld, int epi, ee_gelu form, void* C, int splits, float* P, hipStream_t s,
                      int max_wgs = 0, const OrderedSplit& os = OrderedSplit{}) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int wgs = max_wgs > 0 ? std::min(tm * tn, max_wgs) : tm * tn;
  const dim3 grid((unsigned)wgs, (unsigned)splits), block(64 * WGM * WGN);
  const f16* a = static_cast<const f16*>(A);
  const f16* w = static_cast<const f16*>(W);
  const f16* b = static_cast<const f16*>(bias);
  const f16* r = static_cast<const f16*>(R);
  f16* c = static_cast<f16*>(C);
  // the in-order stream-K form exists for the persistent 256 x 256 and 256 x 384 tiles only
  constexpr bool kCanOrder = BM == 256 && (BN == 256 || BN == 384);
#define EE_GEMM_LAUNCH(E)                                                                                       \
  if (kCanOrder && os.extra > 0)                                                                                \
    hipLaunchKernelGGL((gemm_f16_mfma_kernel<MF, BM, BN, WGM, WGN, E, WDEPTH, kCanOrder>), grid, block, 0, s, a, \
                       ld.a, w, ld.w, b, r, c, ld.c, M, N, K, (int)form, tm, tn, P, os);                         \
  else                                                                                                          \
    hipLaunchKernelGGL((gemm_f16_mfma_kernel<MF, BM, BN, WGM, WGN, E, WDEPTH, false>), grid, block, 0, s, a, ld.a, w, \
                       ld.w, b, r, c, ld.c, M, N, K, (int)form, tm, tn, P, os)
  switch (epi) {
    case EE_EPI_NONE: EE_GEMM_LAUNCH(EE_EPI_NONE); break;
    case EE_EPI_BIAS: EE_GEMM_LAUNCH(EE_EPI_BIAS); break;
    case EE_EPI_BIAS_RESIDUAL: EE_GEMM_LAUNCH(EE_EPI_BIAS_RESIDUAL); break;
    case EE_EPI_BIAS_GELU: EE_GEMM_LAUNCH(EE_EPI_BIAS_GELU); break;
    case kEpiPartial:  // split-K partial sums (128 x 128 tiles only): never with an ordered split
      if constexpr (BN != 384)
        hipLaunchKernelGGL((gemm_f16_mfma_kernel<MF, BM, BN, WGM, WGN, kEpiPartial, WDEPTH, false>), grid, block, 0, s,
                           a, ld.a, w, ld.w, b, r, c, ld.c, M, N, K, (int)form, tm, tn, P, os);
      else
        return hipErrorInvalidValue;
      break;
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

namespace {
// A tag no earlier launch of this process used, nor (but with probability
// 2^-64) one of another process that left flags in the same memory.
unsigned long long next_ordered_tag() {
  static std::atomic<unsigned long long> ctr{[] {
    std::random_device rd;
    const unsigned long long t = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    return (((unsigned long long)rd() << 32) ^ rd() ^ (t * 0x9e3779b97f4a7c15ull));
  }()};
  unsigned long long v;
  do v = ++ctr;
  while (v == 0);
  return v;
}

OrderedSplit ordered_split(int64_t M, int N, int K, int wgs, void* scratch, size_t bytes, int bn) {
  OrderedSplit os{};
  const int64_t p = scratch ? ordered_wgs(M, N, K, wgs, bytes, bn) : 0;
  if (p == 0) return os;
  const int64_t n_tiles = ((M + 255) / 256) * ((N + bn - 1) / bn);
  const int64_t rounds = n_tiles / wgs, extra = n_tiles - rounds * wgs;
  os.flags = static_cast<unsigned long long*>(scratch);
  os.tag = next_ordered_tag();
  os.rounds = (int)rounds;
  os.extra = (int)extra;
  os.wgs = (int)p;
  return os;
}
}  // namespace

size_t gemm_f16_ordered_bytes() { return kOrderedFlagBytes + (size_t)kOrderedMaxWgs * kOrderedTileBytes; }

int gemm_f16_parts(int64_t M, int N, int K, GemmPart (&parts)[kGemmMaxParts], size_t ordered_bytes,
                   bool vec_stores) {
  return gemm_plan_parts(M, N, K, parts, ordered_bytes, vec_stores,
                         GemmPlanOpts{device_cu_count(), EE_GEMM_PERSIST != 0, EE_GEMM_WIDE != 0, EE_GEMM_DEEP_W_K});
}

hipError_t launch_gemm_f16_part(const GemmPart& p, const void* A, const void* W, const void* bias, const void* R,
                                int N, int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                                hipStream_t s, void* ordered, size_t ordered_bytes) {
  if (p.rows <= 0) return hipSuccess;
  // the part's rows of A, C and the residual
  const f16* a = static_cast<const f16*>(A) + p.row0 * ld.a;
  const f16* r = R ? static_cast<const f16*>(R) + p.row0 * ld.c : nullptr;
  f16* c = static_cast<f16*>(C) + p.row0 * ld.c;
  const int M = (int)p.rows;
  const int wgs = EE_GEMM_PERSIST ? device_cu_count() : 0;
  const int bn = p.cfg == kGemmWide ? 384 : 256;
  const int64_t tiles = ((int64_t)(M + 255) / 256) * ((N + bn - 1) / bn);
  const OrderedSplit os = p.ordered && wgs > 0
                              ? ordered_split(M, N, K, (int)std::min<int64_t>(tiles, wgs), ordered, ordered_bytes, bn)
                              : OrderedSplit{};
  switch (p.cfg) {
    case kGemmBig2:
      return launch_cfg<EE_GEMM_MF, 256, 256, EE_GEMM_WGM, EE_GEMM_WGN, 2>(a, W, bias, r, M, N, K, ld, epi, form, c, 1,
                                                                          nullptr, s, wgs, os);
    case kGemmBig3:
      return launch_cfg<EE_GEMM_MF, 256, 256, EE_GEMM_WGM, EE_GEMM_WGN, 3>(a, W, bias, r, M, N, K, ld, epi, form, c, 1,
                                                                          nullptr, s, wgs, os);
    case kGemmWide:
      return launch_cfg<16, 256, 384, 2, 2, 2>(a, W, bias, r, M, N, K, ld, epi, form, c, 1, nullptr, s, wgs, os);
    case kGemm128x64: return launch_cfg<32, 128, 64, 2, 2>(a, W, bias, r, M, N, K, ld, epi, form, c, 1, nullptr, s);
    case kGemm128x128: return launch_cfg<32, 128, 128, 2, 2>(a, W, bias, r, M, N, K, ld, epi, form, c, 1, nullptr, s);
  }
  return hipErrorInvalidValue;
}

const char* gemm_f16_kernel_label(int cfg, ee_epilogue epi, bool ordered) {
  // gemm_f16_mfma_kernel's template arguments <MF, BM, BN, WGM, WGN, EPI, WDEPTH, ORD>
  static const char* const labels[5][4] = {
#define EE_L(cfg) {"gemm_f16_mfma_kernel<" cfg ", 0, 2, false>", "gemm_f16_mfma_kernel<" cfg ", 1, 2, false>", \
                   "gemm_f16_mfma_kernel<" cfg ", 2, 2, false>", "gemm_f16_mfma_kernel<" cfg ", 3, 2, false>"}
      EE_L("16, 256, 256, 2, 2"),
      {"gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 0, 3, false>", "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 1, 3, false>",
       "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 2, 3, false>", "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 3, 3, false>"},
      EE_L("32, 128, 128, 2, 2"),
      EE_L("32, 128, 64, 2, 2"),
      EE_L("16, 256, 384, 2, 2"),
#undef EE_L
  };
  static const char* const ordered_labels[3][4] = {
      {"gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 0, 2, true>", "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 1, 2, true>",
       "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 2, 2, true>", "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 3, 2, true>"},
      {"gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 0, 3, true>", "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 1, 3, true>",
       "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 2, 3, true>", "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 3, 3, true>"},
      {"gemm_f16_mfma_kernel<16, 256, 384, 2, 2, 0, 2, true>", "gemm_f16_mfma_kernel<16, 256, 384, 2, 2, 1, 2, true>",
       "gemm_f16_mfma_kernel<16, 256, 384, 2, 2, 2, 2, true>", "gemm_f16_mfma_kernel<16, 256, 384, 2, 2, 3, 2, true>"},
  };
  const int e = (int)epi;
  if (cfg < 0 || cfg > kGemmWide || e < 0 || e > 3) return "gemm_f16_mfma_kernel";
  if (ordered && cfg <= kGemmBig3) return ordered_labels[cfg][e];
  return ordered && cfg == kGemmWide ? ordered_labels[2][e] : labels[cfg][e];
}


hipError_t launch_gemm_f16_mfma(const void* A, const void* W, const void* bias, const void* R, int64_t M, int N,
                                int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C, hipStream_t s) {
  GemmPart parts[kGemmMaxParts];
  const int n = gemm_f16_parts(M, N, K, parts, 0, false);
  for (int i = 0; i < n; ++i) {
    const hipError_t e = launch_gemm_f16_part(parts[i], A, W, bias, R, N, K, ld, epi, form, C, s, nullptr, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
