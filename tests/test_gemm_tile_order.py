"""The GEMM's tile order (csrc/gemm_tile_order.h), compiled with g++ and
checked on the host: every tile of every tested shape is computed exactly
once; in a persistent launch of 256 workgroups (32 per XCD, tile % 8 = the
XCD) every XCD gets the same number of tiles, the two XCDs of a pair work on
the same M-tiles at the same time, the four XCDs of an N half work on the same
N-tiles at the same time (outside the leftover M-tiles), and a round inside a
group of 4 M-tiles is a block of 4 M-tiles by 8 N-tiles."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_padding_amd", "csrc")

# (tiles_m, tiles_n): the layer's GEMMs at 4096 and 8192 rows, ragged row
# counts of the request stream, small and odd shapes (other branches)
SHAPES = [(16, 192), (32, 192), (16, 144), (32, 144), (16, 48), (32, 48), (26, 192), (31, 144), (35, 48),
          (28, 192), (29, 192), (33, 192), (36, 192), (30, 144), (27, 48), (17, 36),
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


def _rounds(tm, tn, tiles):
    """Full rounds of a 256-workgroup persistent launch: {xcd: its 32 tiles}."""
    n = tm * tn
    for k in range(n // 256):
        yield k, {x: [tiles[k * 256 + c] for c in range(x, 256, 8)] for x in range(8)}


def test_every_xcd_gets_the_same_tiles_count(tile_map):
    for (tm, tn), tiles in tile_map.items():
        if (tm * tn) % 8:
            continue
        counts = [len(tiles[x::8]) for x in range(8)]
        assert len(set(counts)) == 1, (tm, tn, counts)


def test_persistent_rounds_share_panels_across_xcds(tile_map):
    for (tm, tn), tiles in tile_map.items():
        if tn % 8:
            continue
        mq, half = tm // 4, tn // 2
        for k, by_xcd in _rounds(tm, tn, tiles):
            for x in range(0, 8, 2):                    # a pair: the same M-tiles, the two N halves
                assert {m for m, _ in by_xcd[x]} == {m for m, _ in by_xcd[x + 1]}, (tm, tn, k, x)
                assert max(c for _, c in by_xcd[x]) < half <= min(c for _, c in by_xcd[x + 1]), (tm, tn, k, x)
            if (k + 1) * 32 > mq * half:                # the round reaches the leftover M-tiles
                continue
            for h in (0, 1):                            # a half: the same N-tiles on its four XCDs
                ns = [sorted({c for _, c in by_xcd[2 * p + h]}) for p in range(4)]
                assert ns[0] == ns[1] == ns[2] == ns[3], (tm, tn, k, h)
            for x, ts in by_xcd.items():
                ms, ns = {m for m, _ in ts}, {c for _, c in ts}
                if len(ms) == 4:                        # inside a group of 4: a 4 x 8 block
                    assert len(ns) == 8, (tm, tn, k, x)


def test_whole_groups_keep_the_order_of_the_quarters(tile_map):
    """When tiles_m is a multiple of 16, the order is each half's group-major
    order cut into four contiguous quarters (the order the 4096- and 8192-row
    GEMMs were measured with)."""
    for (tm, tn), tiles in tile_map.items():
        if tn % 8 or tm % 16:
            continue
        half = tn // 2
        for t, (m, n) in enumerate(tiles):
            x, k = t % 8, t // 8
            h, p = x % 2, x // 2
            lin = p * (tm * half // 4) + k
            g, ig = divmod(lin, 4 * half)
            assert (m, n) == (4 * g + ig % 4, h * half + ig // 4), (tm, tn, t)
