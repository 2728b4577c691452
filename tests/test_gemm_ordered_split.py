"""The in-order stream-K decomposition of a persistent GEMM launch's partial
last round (csrc/gemm_ordered_split.h), compiled with g++ and checked on the
host: every (tile, K tile) step is computed exactly once; the pieces of each
extra tile start at K tile 0 and meet end to end, each continuing piece names
as its predecessor the workgroup that leaves it the sums, and only the last
piece stores the tile; a workgroup leaves at most one partial tile, in a slot
below the split's workgroup count; the workgroups of one XCD (b % 8) run the
same items in the same order, apart from which tiles; and an event simulation
of the workgroups running their items in order, a piece waiting for its
predecessor, ends with every item done (no wait cycle), within a few per cent
of the ideal balance."""
import heapq
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_padding_amd", "csrc")

# (tiles_m, tiles_n, KT) of 256 x 256 tiles on 256 workgroups: the layer's
# GEMMs at the request stream's row counts, the tensor-parallel shard, the
# shapes of the GPU tests, and small or odd ones
CASES = [(31, 192, 192), (33, 192, 192), (29, 192, 192), (31, 144, 192), (35, 144, 192), (29, 48, 192),
         (33, 48, 768), (29, 48, 769), (17, 36, 192), (17, 48, 48), (17, 48, 768), (31, 192, 16), (17, 36, 16),
         (33, 48, 32), (17, 16, 8), (3, 100, 4), (2, 129, 64), (9, 57, 7), (40, 13, 1000), (16, 48, 192)]
# partial-sum slots: a forward's workspace (256) and an extend step's (255)
SLOT_COUNTS, MIN_PIECE, G = (256, 255), 32, 256

SRC = r'''
#include "gemm_ordered_split.h"
#include <cstdio>
int main() {
  int tm, tn, KT, G, slots, minp;
  while (std::scanf("%d %d %d %d %d %d", &tm, &tn, &KT, &G, &slots, &minp) == 6) {
    const int n_tiles = tm * tn;
    const int wgs = ee::ordered_split_wgs(n_tiles, G, KT, slots, minp);
    const int rounds = n_tiles / G, extra = wgs ? n_tiles - rounds * G : 0;
    std::printf("case %d %d %d\n", wgs, rounds, extra);
    for (int b = 0; b < G; ++b) {
      const ee::OrderedWork w = ee::ordered_work(b, G, n_tiles, KT, rounds, extra, wgs);
      const int n = ee::ordered_items(w);
      std::printf("wg %d %d\n", b, n);
      for (int c = 0; c < n; ++c) {
        const ee::OrderedItem it = ee::ordered_item(w, b, G, KT, c);
        std::printf("%d %d %d %d %d\n", it.tile, it.k0, it.k1, it.pred, (int)it.partial);
      }
    }
  }
  return 0;
}
'''


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    d = tmp_path_factory.mktemp("ordered")
    (d / "o.cpp").write_text(SRC)
    exe = d / "o"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(d / "o.cpp"), "-o", str(exe)], check=True)
    runs = [(case, slots) for slots in SLOT_COUNTS for case in CASES]
    inp = "".join(f"{tm} {tn} {kt} {G} {slots} {MIN_PIECE}\n" for (tm, tn, kt), slots in runs)
    toks = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    out, i = {}, 0
    for case in runs:
        _, wgs, rounds, extra = toks[i].split()
        i += 1
        wgs_items = []
        for _ in range(G):
            _, b, n = toks[i].split()
            i += 1
            items = [tuple(map(int, toks[i + c].split())) for c in range(int(n))]
            i += int(n)
            wgs_items.append(items)
        out[case] = (int(wgs), int(rounds), int(extra), wgs_items)
    return out


def test_every_step_once_and_chains(plans):
    split_cases = 0
    for ((tm, tn, kt), slots), (wgs, rounds, extra, items) in plans.items():
        n_tiles = tm * tn
        cover = {}
        partials = {}
        for b, its in enumerate(items):
            assert sum(p for *_, p in its) <= 1, (tm, tn, kt, b)
            for (tile, k0, k1, pred, partial) in its:
                assert 0 <= tile < n_tiles and 0 <= k0 < k1 <= kt, (tm, tn, kt, b)
                assert partial == (k1 < kt) and (pred >= 0) == (k0 > 0)
                if partial:
                    assert b < wgs <= slots
                    partials[b] = (tile, k1)
                cover.setdefault(tile, []).append((k0, k1, b, pred))
        assert sorted(cover) == list(range(n_tiles)), (tm, tn, kt)
        for tile, pcs in cover.items():
            pcs.sort()
            assert pcs[0][0] == 0 and pcs[-1][1] == kt, (tm, tn, kt, tile)
            for prev, nxt in zip(pcs, pcs[1:]):
                assert prev[1] == nxt[0], (tm, tn, kt, tile)        # end to end, no overlap
                assert nxt[3] == prev[2], (tm, tn, kt, tile)       # names the workgroup before it
                assert partials[prev[2]] == (tile, nxt[0])         # which left these sums
        if extra:
            split_cases += 1
            assert wgs >= 2 * extra and rounds >= 1 and (8 * extra) % wgs == 0
            # in step within an XCD: the same (k0, k1, partial, waits) sequence on every participant
            for x in range(8):
                shapes = {tuple((k0, k1, pred >= 0, p) for (_, k0, k1, pred, p) in items[b])
                          for b in range(x, wgs, 8)}
                assert len(shapes) == 1, (tm, tn, kt, x)
        else:
            assert all(len(c) == 1 for c in cover.values())        # no split: whole tiles
    assert split_cases >= 16


def _simulate(items, kt):
    """Each workgroup runs its items in order; a waiting piece starts once its
    predecessor's piece is done.  Returns the makespan in K-tile steps, or
    None when some workgroup can never proceed."""
    t = [0.0] * len(items)
    pos = [0] * len(items)
    done = {}                                     # (tile, k1) -> finish time of the piece ending there
    progress = True
    while progress:
        progress = False
        for b, its in enumerate(items):
            while pos[b] < len(its):
                tile, k0, k1, pred, _ = its[pos[b]]
                start = t[b]
                if pred >= 0:
                    if (tile, k0) not in done:
                        break
                    start = max(start, done[(tile, k0)])
                t[b] = start + (k1 - k0)
                done[(tile, k1)] = t[b]
                pos[b] += 1
                progress = True
    if any(pos[b] < len(its) for b, its in enumerate(items)):
        return None
    return max(t)


def test_no_wait_cycle_and_balance(plans):
    for ((tm, tn, kt), slots), (wgs, rounds, extra, items) in plans.items():
        span = _simulate(items, kt)
        assert span is not None, (tm, tn, kt)
        whole = rounds + (1 if (tm * tn) % G else 0)          # tiles of the slowest workgroup, unsplit
        ideal = (tm * tn) * kt / G
        if extra:
            # at most one tile's worth of waiting or imbalance beyond the ideal, and never worse than unsplit
            assert span <= ideal + kt * max(1.0, 1.0 / rounds) + 1, (tm, tn, kt, span, ideal)
            assert span <= whole * kt, (tm, tn, kt, span, whole * kt)
