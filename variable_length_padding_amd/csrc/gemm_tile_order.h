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
// tile % 8 is the XCD that computes the tile, and each XCD's L2 is private.
//
// With tiles_n a multiple of 8, XCD x = 2p + h takes half h of the N tiles and
// the p-th quarter of that half's tiles, walked in groups of 4 M-tiles (M
// fastest inside a group).  Each round of 32 tiles on an XCD is then 4 M-tiles
// by 8 N-tiles -- the split of 32 tiles that reads the fewest operand panels
// through the XCD's L2 -- and the two XCDs of a pair share their A panels.  At
// any time the 8 XCDs hold 4 groups of A panels, not 8: at 8192 rows and
// K = 12288 that is 100 MB of A beside the W panels streaming through the
// 256 MB Infinity Cache, instead of 200 MB (2-3% faster on the FC1 and QKV
// shapes there; the same tiles at 4096 rows).  Otherwise, with n_tiles a
// multiple of 8, each XCD takes a contiguous range of the group-major order;
// else the group-major order itself.
EE_HOST_DEVICE inline void gemm_tile_origin(int tile, int n_tiles, int tiles_m, int tiles_n, int bm, int bn, int& m0,
                                            int& n0) {
  constexpr int GM = 4;  // M-tiles per group
  int lin = tile, m_tiles = tiles_m, n_cols = tiles_n, n_base = 0;
  if ((tiles_n & 7) == 0) {
    const int x = tile & 7, h = x & 1, p = x >> 1;
    n_cols = tiles_n >> 1;
    n_base = h * n_cols;
    lin = p * ((tiles_m * n_cols) >> 2) + (tile >> 3);
  } else if ((n_tiles & 7) == 0) {
    lin = (tile & 7) * (n_tiles >> 3) + (tile >> 3);
  }
  const int per_group = GM * n_cols;
  const int group = lin / per_group;
  const int first_m = group * GM;
  const int gm = m_tiles - first_m < GM ? m_tiles - first_m : GM;
  const int ig = lin - group * per_group;
  m0 = (first_m + ig % gm) * bm;
  n0 = (n_base + ig / gm) * bn;
}

}  // namespace ee
