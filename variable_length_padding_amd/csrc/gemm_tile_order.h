// Which output tile a GEMM workgroup computes (gemm_f16.hip), in a plain
// header so that the host can test the mapping without a GPU.
#pragma once

#if defined(__HIPCC__)
#define EE_HOST_DEVICE __host__ __device__
#else
#define EE_HOST_DEVICE
#endif

namespace ee {

// Tiles are numbered `tile` = 0 .. n_tiles-1 in launch order (a persistent
// launch of a multiple of 8 workgroups walks tile = blockIdx.x + k*gridDim.x).
// The hardware deals consecutive workgroup ids round-robin to the 8 XCDs, so
// tile % 8 is the XCD that computes the tile, tile / 8 its place in that XCD's
// sequence, and each XCD's L2 is private.
//
// With tiles_n a multiple of 8, XCD x = 2p + h takes half h of the N tiles and
// the p-th quarter of the M tiles (tiles_m / 4 of them), walked in groups of 4
// M-tiles (M fastest inside a group, then N); the tiles_m % 4 M-tiles left over
// are shared out by N, a quarter of the half's N tiles to each XCD.  So:
//   * each round of 32 tiles on an XCD is a 4 x 8 block of tiles, the split of
//     32 tiles that reads the fewest operand panels through the XCD's L2;
//   * the two XCDs of a pair work on the same M-tiles at the same time and
//     share their A panels, so the 8 XCDs hold 4 groups of A panels;
//   * the four XCDs of a half walk the same N-tiles at the same time, so each
//     W panel is read from HBM about once per 4 XCDs, through the Infinity
//     Cache.
// The last point is what splitting each half's tiles into four contiguous
// quarters of one group-major order lost when tiles_m is not a multiple of 16:
// the XCDs then entered the N range at different points, each streamed W on
// its own, and FC1 (N = 49152, K = 12288) ran 9-12% slower per round.
// Otherwise, with n_tiles a multiple of 8, each XCD takes a contiguous range of
// the group-major order; else the group-major order itself.
EE_HOST_DEVICE inline void gemm_tile_origin(int tile, int n_tiles, int tiles_m, int tiles_n, int bm, int bn, int& m0,
                                            int& n0) {
  constexpr int GM = 4;  // M-tiles per group
  if ((tiles_n & 7) == 0) {
    const int x = tile & 7, h = x & 1, p = x >> 1, k = tile >> 3;
    const int n_cols = tiles_n >> 1, mq = tiles_m >> 2;
    const int main_tiles = mq * n_cols;
    int m, n;
    if (k < main_tiles) {
      const int per_group = GM * n_cols;
      const int group = k / per_group;
      const int first_m = group * GM;
      const int gm = mq - first_m < GM ? mq - first_m : GM;
      const int ig = k - group * per_group;
      m = p * mq + first_m + ig % gm;
      n = ig / gm;
    } else {  // the tiles_m % 4 leftover M-tiles, N-tiles [p*q, (p+1)*q) of the half
      const int r = tiles_m & 3, q = n_cols >> 2, i = k - main_tiles;
      m = 4 * mq + i % r;
      n = p * q + i / r;
    }
    m0 = m * bm;
    n0 = (h * n_cols + n) * bn;
    return;
  }
  int lin = tile;
  if ((n_tiles & 7) == 0) lin = (tile & 7) * (n_tiles >> 3) + (tile >> 3);
  const int per_group = GM * tiles_n;
  const int group = lin / per_group;
  const int first_m = group * GM;
  const int gm = tiles_m - first_m < GM ? tiles_m - first_m : GM;
  const int ig = lin - group * per_group;
  m0 = (first_m + ig % gm) * bm;
  n0 = (ig / gm) * bn;
}

}  // namespace ee
