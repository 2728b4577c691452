// The work of one workgroup of a persistent GEMM launch whose partial last
// round runs as in-order stream-K pieces (gemm_f16.hip), in a plain header so
// that the host can check the decomposition without a GPU.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define EE_HOST_DEVICE __host__ __device__
#else
#define EE_HOST_DEVICE
#endif

namespace ee {

// A launch of G workgroups over n_tiles tiles of KT K tiles each.  Without a
// split (extra == 0) workgroup b computes tiles b, b + G, ... whole.  With one,
// it computes the `rounds` whole tiles b + r * G, r < rounds, and the `extra`
// tiles left (rounds * G ..) are cut into `wgs` equal contiguous ranges of
// their (tile, K tile) steps, range b for workgroup b < wgs.  A range holds at
// most two pieces: A, its start, which continues a tile when it does not start
// at K tile 0, and B, the start of the next tile when the range crosses a tile
// boundary.  A range ends at a tile's end or inside a tile; in the second case
// its last piece leaves its sums for workgroup b + 1, whose piece A continues
// the tile.
struct OrderedWork {
  int n_whole, nA, nB, posA;  // whole tiles; pieces A and B (0 or 1); A's place in the order
  int a_tile, a_k0, a_k1;     // piece A: tile, K tiles [a_k0, a_k1)
  int b_k1;                   // piece B: tile a_tile + 1, K tiles [0, b_k1)
};

struct OrderedItem {
  int tile, k0, k1;
  int pred;      // >= 0: continues the sums left by that workgroup (b - 1)
  bool partial;  // leaves its sums for workgroup b + 1 (k1 < KT)
};

EE_HOST_DEVICE inline OrderedWork ordered_work(int b, int G, int n_tiles, int KT, int rounds, int extra, int wgs) {
  OrderedWork w{};
  if (extra <= 0) {
    w.n_whole = b < n_tiles ? (n_tiles - b + G - 1) / G : 0;
    return w;
  }
  w.n_whole = rounds;
  if (b >= wgs) return w;
  // X < 2^31 / wgs: at most 256 workgroups and extra * KT below 2^23
  const int X = extra * KT;
  const int lo = (int)((int64_t)X * b / wgs), hi = (int)((int64_t)X * (b + 1) / wgs);
  if (hi <= lo) return w;
  const int ea = lo / KT;
  const int end_a = hi < (ea + 1) * KT ? hi : (ea + 1) * KT;
  w.nA = 1;
  w.a_tile = rounds * G + ea;
  w.a_k0 = lo - ea * KT;
  w.a_k1 = end_a - ea * KT;
  w.nB = hi > end_a;
  w.b_k1 = hi - end_a;
  // A runs after about as many whole tiles as its first K tile is far into
  // the tile (its predecessor, which starts earlier in the tile, has an
  // earlier or the same slot); B, a tile's start, runs first
  const int slot = w.a_k0 == 0 ? 0 : (int)(((int64_t)w.a_k0 * rounds + KT - 1) / KT);
  w.posA = (slot < rounds ? slot : rounds) + w.nB;
  return w;
}

EE_HOST_DEVICE inline int ordered_items(const OrderedWork& w) { return w.n_whole + w.nA + w.nB; }

// Item c (0 <= c < ordered_items(w)) of workgroup b, in the order it runs them.
EE_HOST_DEVICE inline OrderedItem ordered_item(const OrderedWork& w, int b, int G, int KT, int c) {
  if (w.nB && c == 0) return OrderedItem{w.a_tile + 1, 0, w.b_k1, -1, w.b_k1 < KT};
  if (w.nA && c == w.posA) return OrderedItem{w.a_tile, w.a_k0, w.a_k1, w.a_k0 > 0 ? b - 1 : -1, w.a_k1 < KT};
  const int r = c - w.nB - (w.nA && c > w.posA ? 1 : 0);
  return OrderedItem{b + r * G, 0, KT, -1, false};
}

// Workgroups that take a range of the extra tiles, or 0 for no split: at
// most one per partial-sum slot (`slots`), pieces of at least `min_piece` K
// tiles, and at least 1/rounds of a tile each (so the two pieces of a tile
// that meet at a range boundary do not share a slot in the order above).
//
// And a count that divides 8 * extra, so that the ranges of the workgroups of
// one XCD (b, b + 8, ...: consecutive workgroups go to the 8 XCDs in turn) lie
// at the same place in their tiles.  Those workgroups then run pieces of the
// same length at the same points, and stay in step on the blocks of whole
// tiles they share through the XCD's L2; measured on a request-stream QKV
// GEMM (176 extra tiles, for which no such count exists), the split was 3.6%
// slower than the plain last round, while 64 extra tiles on 256 workgroups
// gained 2.8%.
//
// A piece costs about what a tile's prologue and epilogue cost, plus storing
// or loading its sums, so the split is taken only where it saves at least
// half a round: each workgroup gets at most half a tile of extra steps (192
// extra tiles on 256 workgroups, three quarters of a tile each, ran 1.5%
// slower than the plain last round on the FC1 GEMM; 112 on 224, half a tile,
// ran 2-7% faster on the QKV, out and FC2 GEMMs).
inline int ordered_split_wgs(int64_t n_tiles, int G, int KT, int slots, int min_piece) {
  if (G < 2 || KT < 1) return 0;
  const int64_t rounds = n_tiles / G, extra = n_tiles - rounds * G;
  if (rounds < 1 || extra < 1 || extra * KT >= (int64_t(1) << 23)) return 0;
  int64_t cap = G;
  if (extra * rounds < cap) cap = extra * rounds;
  if (extra * KT / min_piece < cap) cap = extra * KT / min_piece;
  if (slots < cap) cap = slots;
  for (int64_t p = cap; p >= 2 * extra; --p)
    if ((8 * extra) % p == 0) return (int)p;
  return 0;
}

}  // namespace ee
