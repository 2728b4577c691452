"""The GEMM's tile order (csrc/gemm_tile_order.h), compiled with g++ and
checked on the host: every tile of every tested shape is computed exactly
once; in a persistent launch of 256 workgroups (32 per XCD, tile % 8 = the
XCD) each full round of an XCD is a block of 4 M-tiles by 8 N-tiles, and the
two XCDs of a pair work on the same M-tiles at the same time."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_padding_amd", "csrc")

# (tiles_m, tiles_n): the layer's GEMMs at 4096 and 8192 rows, ragged row
# counts of the request stream, small and odd shapes (other branches)
SHAPES = [(16, 192), (32, 192), (16, 144), (32, 144), (16, 48), (32, 48), (26, 192), (31, 144), (35, 48),
          (1, 8), (3, 16), (7, 24), (5, 6), (9, 3), (4, 2), (13, 5), (2, 12)]


@pytest.fixture(scope="module")
def tile_map(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    d = tmp_path_factory.mktemp("tiles")
    src = d / "tiles.cpp"
    src.write_text('#include "gemm_tile_order.h"\n#include <cstdio>\nint main() {\n  int tm, tn;\n'
                   '  while (std::scanf("%d %d", &tm, &tn) == 2)\n'
                   '    for (int t = 0; t < tm * tn; ++t) {\n      int m0, n0;\n'
                   '      ee::gemm_tile_origin(t, tm * tn, tm, tn, 1, 1, m0, n0);\n'
                   '      std::printf("%d %d\\n", m0, n0);\n    }\n  return 0;\n}\n')
    exe = d / "tiles"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], input="".join(f"{m} {n}\n" for m, n in SHAPES), capture_output=True,
                         text=True, check=True).stdout.split()
    vals = list(map(int, out))
    res, i = {}, 0
    for m, n in SHAPES:
        res[(m, n)] = [(vals[i + 2 * t], vals[i + 2 * t + 1]) for t in range(m * n)]
        i += 2 * m * n
    return res


def test_every_tile_once(tile_map):
    for (tm, tn), tiles in tile_map.items():
        assert sorted(tiles) == [(m, n) for m in range(tm) for n in range(tn)], (tm, tn)


def test_persistent_rounds_are_4x8_blocks_shared_by_xcd_pairs(tile_map):
    for (tm, tn), tiles in tile_map.items():
        if tn % 8 or tm % 4:
            continue
        n = tm * tn
        for k in range(n // 256):                       # full rounds of a 256-workgroup launch
            by_xcd = {x: [tiles[k * 256 + c] for c in range(x, 256, 8)] for x in range(8)}
            for x, ts in by_xcd.items():
                ms, ns = {m for m, _ in ts}, {c for _, c in ts}
                if len(ms) == 4:                        # inside one group: a 4 x 8 block
                    assert len(ns) == 8, (tm, tn, k, x)
                if x % 2 == 0:                          # the pair shares its M-tiles, N halves differ
                    assert ms == {m for m, _ in by_xcd[x + 1]}, (tm, tn, k, x)
                    assert max(ns) < tn // 2 <= min(c for _, c in by_xcd[x + 1]), (tm, tn, k, x)
