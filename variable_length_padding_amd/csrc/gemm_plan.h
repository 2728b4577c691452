// Host-side plan of a large fp16 GEMM: which tile configuration runs which
// rows, and whether a persistent launch runs its partial last round as
// in-order stream-K pieces (gemm_ordered_split.h).  Plain C++ with no HIP
// dependency, so that a host compiler can check the plans on their own.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <numeric>

#include "gemm_ordered_split.h"

namespace ee {

// Tile configurations: 256 x 256 with two or three W stages, 128 x 128,
// 128 x 64, and 256 x 384.
enum { kGemmBig2 = 0, kGemmBig3 = 1, kGemm128x128 = 2, kGemm128x64 = 3, kGemmWide = 4 };
struct GemmPart {
  int64_t row0, rows;
  int cfg;
  bool ordered;  // its partial last round as in-order stream-K pieces
};
constexpr int kGemmMaxParts = 3;

// What the plan depends on besides the problem: the device's CU count (the
// persistent launch's workgroups) and the build's choices.
struct GemmPlanOpts {
  int cus;
  bool persist;   // large problems as one persistent launch
  bool wide;      // 256 x 384 tiles where N % 384 == 0
  int deep_w_k;   // from this K on the 256 x 256 tile uses three W stages
};

constexpr int kPlanBK = 64;  // K tile of the large kernels

// In-order stream-K scratch: 4 KiB of flags, then one partial tile of fp32
// sums (256 rows of the tile's width) per workgroup taking part.
constexpr size_t kOrderedFlagBytes = 4096;
constexpr int kOrderedMaxWgs = 256;
constexpr size_t ordered_tile_bytes(int bn) { return (size_t)256 * bn * 4; }
constexpr size_t kOrderedTileBytes = ordered_tile_bytes(384);  // the widest tile
// The fewest K tiles in a piece (2048 of K): a shorter one spends much of its
// time on its prologue and on storing or loading partial sums (the TP-shard
// out projection, K = 3072, ran 5% slower split into pieces of 18 K tiles).
constexpr int kOrderedMinPiece = 32;

// Estimated times, in rounds of 256 x 256 tiles of the same K:
// a 128 x 128 tile (a quarter of the work at a lower MFMA rate);
constexpr double kSmallTileCost = 0.36;
// a round of 128 x 64 tiles over a few rows, which streams all of W through
// the CUs (109 rows of the TP-shard FC1 and FC2: 0.155 ms against 0.30 ms
// per round of 256 x 256 tiles);
constexpr double kNarrowRoundCost = 0.52;
// a 256 x 384 tile: 1.5 times the work at 4.5% less time per flop (FC1, QKV
// and out GEMMs at 8192 rows, same process), and at K >= deep_w_k, against
// the three-W-stage 256 x 256 kernel, 10% less (FC2 at 4096 to 8192 rows);
// below kWideMinGainK no less (the TP-shard out projection, K = 3072: its
// whole wide rounds took as long as the same rows' 256 x 256 rounds);
constexpr double kWideRoundCost = 1.43;
constexpr double kWideRoundCostLongK = 1.35;
constexpr double kWideRoundCostShortK = 1.5;
constexpr int kWideMinGainK = 8192;
// a launch beyond its rounds (its first and last tiles' loads and stores
// overlap no other tile's MFMAs; a split's partial sums).
constexpr double kLaunchCost = 0.05;
// the 256 x 256 plan of the rows left after whole rounds of 256 x 384 tiles,
// per estimated round: few M tiles, whose leftover tiles the tile order cannot
// deal to the XCDs in step (the request stream's QKV GEMM at 7889 rows: its
// last 1745 rows at 1076 TFLOP/s against 1430 for the wide rounds; 256 x 384
// tiles on every row, the last round 62% full, ran 3.4% faster than the two
// launches that the estimate without this factor chose).
constexpr double kWideRestSquareCost = 1.25;

// Workgroups among which a persistent launch of `wgs` workgroups over tiles
// 256 rows by bn columns shares its partial last round, or 0 (no split:
// whole rounds only, too little scratch, or a split that would not pay).
inline int64_t ordered_wgs(int64_t M, int N, int K, int wgs, size_t bytes, int bn = 256) {
  if (bytes < kOrderedFlagBytes + 2 * ordered_tile_bytes(bn) || wgs > kOrderedMaxWgs) return 0;
  const int64_t n_tiles = ((M + 255) / 256) * ((N + bn - 1) / bn);
  const int slots = (int)std::min<size_t>((bytes - kOrderedFlagBytes) / ordered_tile_bytes(bn), kOrderedMaxWgs);
  return ordered_split_wgs(n_tiles, wgs, K / kPlanBK, slots, kOrderedMinPiece);
}

// Rows [0, m_big) of a large problem go to the 256 x 256 kernel and the rest
// to 128 x 128 tiles.  A tile count just past a multiple of the CU count
// leaves most CUs idle in the last round of 256 x 256 tiles; running only
// whole rounds of 256-row tiles there and the remaining rows as 128 x 128
// tiles ends sooner.  Both kernels add an element's K tiles in the same order;
// their MFMA shapes differ (16x16x32 and 32x32x16), and on gfx950 they give
// the same bits for every element (tested on random data against GEMMs run
// on each 256-row block alone), so the split changes no results.
inline int64_t gemm_big_rows(int64_t M, int N, int cus) {
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

// The 256 x 256 plan of rows [row0, row0 + M): one or two parts; *rounds
// gets its estimated time.
inline int gemm_plan_square(int64_t row0, int64_t M, int N, int K, GemmPart* parts, size_t ordered_bytes,
                            bool vec_stores, const GemmPlanOpts& o, double* rounds) {
  const int cus = o.cus;
  const int64_t tiles_big = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles_big < cus) {
    // the rows after another part's whole rounds stream all of W through few
    // tiles: 128 x 64 tiles (the same MFMA shape) put twice as many CUs on it
    const int64_t small = ((M + 127) / 128) * ((N + 127) / 128);
    const bool narrow = row0 > 0 && small * 2 <= cus;
    *rounds = narrow ? kNarrowRoundCost : kSmallTileCost * (double)((small + cus - 1) / cus);
    parts[0] = GemmPart{row0, M, narrow ? kGemm128x64 : kGemm128x128, false};
    return 1;
  }
  const int big = K >= o.deep_w_k ? kGemmBig3 : kGemmBig2;
  const int64_t p =
      o.persist && vec_stores ? ordered_wgs(M, N, K, (int)std::min<int64_t>(tiles_big, cus), ordered_bytes) : 0;
  if (p > 0) {
    // whole rounds, then the extra tiles' K steps shared by p workgroups
    *rounds = (double)(tiles_big / cus) + (double)(tiles_big % cus) / p + kLaunchCost;
    parts[0] = GemmPart{row0, M, big, true};  // the launch splits its partial last round itself
    return 1;
  }
  const int64_t m_big = gemm_big_rows(M, N, cus);
  parts[0] = GemmPart{row0, m_big, big, false};
  const int64_t tn = (N + 255) / 256;
  *rounds = (double)((((m_big + 255) / 256) * tn + cus - 1) / cus);
  if (m_big == M) return 1;
  // Few remaining rows stream all of W through few tiles: 128 x 64 tiles
  // (the same MFMA shape) put twice as many CUs on it.
  const int64_t rest = M - m_big;
  const int64_t small = ((rest + 127) / 128) * ((N + 127) / 128);
  const bool narrow = small * 2 <= cus;
  *rounds += narrow ? kNarrowRoundCost : kSmallTileCost * (double)((small + cus - 1) / cus);
  parts[1] = GemmPart{row0 + m_big, rest, narrow ? kGemm128x64 : kGemm128x128, false};
  return 2;
}

// The parts of an M x N x K problem (M >= 1, K % 64 == 0), at most
// kGemmMaxParts, in row order.  vec_stores: N and C's pitch are multiples of
// 8 and C and the residual 16-byte aligned (the in-order split needs it);
// ordered_bytes: its scratch (0: none).  The 256 x 256 plan, or 256 x 384
// tiles where N % 384 == 0 and the estimate says they end sooner: on every
// row (the last round partial, or split into in-order pieces), or on the rows
// that fill whole rounds of them with the rest on the 256 x 256 plan.
inline int gemm_plan_parts(int64_t M, int N, int K, GemmPart* parts, size_t ordered_bytes, bool vec_stores,
                           const GemmPlanOpts& o) {
  if (M <= 0) return 0;
  const int cus = o.cus;
  double t_square = 0.0;
  const int n_square = gemm_plan_square(0, M, N, K, parts, ordered_bytes, vec_stores, o, &t_square);
  if (!(o.wide && o.persist && N % 384 == 0 && K >= 2 * kPlanBK)) return n_square;
  const double wide_cost =
      K >= o.deep_w_k ? kWideRoundCostLongK : K >= kWideMinGainK ? kWideRoundCost : kWideRoundCostShortK;
  const int64_t tn = N / 384, mt = (M + 255) / 256, tiles_w = mt * tn;
  // the rows that fill whole rounds: M tiles in groups of `step`
  const int64_t step = cus / std::gcd<int64_t>(cus, tn);
  const int64_t m_tiles = mt / step * step;
  const int64_t rows_w = std::min<int64_t>(M, m_tiles * 256);
  GemmPart rest[kGemmMaxParts - 1];
  double t_rest = 0.0;
  const int n_rest = rows_w < M && rows_w > 0
                         ? gemm_plan_square(rows_w, M - rows_w, N, K, rest, ordered_bytes, vec_stores, o, &t_rest)
                         : 0;
  const bool rest_square = n_rest > 0 && (rest[0].cfg == kGemmBig2 || rest[0].cfg == kGemmBig3);
  const double t_split = rows_w > 0 ? (double)(m_tiles * tn / cus) * wide_cost +
                                          t_rest * (rest_square ? kWideRestSquareCost : 1.0) +
                                          (n_rest > 0 ? kLaunchCost : 0.0)
                                    : 1e30;
  const double t_all = tiles_w >= cus ? (double)((tiles_w + cus - 1) / cus) * wide_cost : 1e30;
  const int64_t p_w =
      vec_stores && tiles_w >= cus && tiles_w % cus != 0 ? ordered_wgs(M, N, K, cus, ordered_bytes, 384) : 0;
  const double t_ord =
      p_w > 0 ? ((double)(tiles_w / cus) + (double)(tiles_w % cus) / p_w) * wide_cost + kLaunchCost : 1e30;
  if (p_w > 0 && t_ord < t_all && t_ord <= t_split && t_ord < t_square) {
    parts[0] = GemmPart{0, M, kGemmWide, true};
    return 1;
  }
  if (t_all <= t_split && t_all < t_square) {
    parts[0] = GemmPart{0, M, kGemmWide, false};
    return 1;
  }
  if (t_split < t_square) {
    parts[0] = GemmPart{0, rows_w, kGemmWide, false};
    for (int i = 0; i < n_rest; ++i) parts[1 + i] = rest[i];
    return 1 + n_rest;
  }
  return n_square;
}

}  // namespace ee
