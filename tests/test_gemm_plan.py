"""The plan of a large fp16 GEMM (csrc/gemm_plan.h), compiled with g++ and
checked on the host: the parts cover the rows in order with valid tile
configurations, only persistent tiles split their last round, a 256 x 384
part followed by others fills whole rounds, and the layer's shapes get the
plans their round estimates call for (the request stream's batch sizes, the
tensor-parallel shard, the 12-layer workload, small problems)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_padding_amd", "csrc")
WS = 4096 + 256 * 256 * 384 * 4   # ee_linear_ws_workspace_size(): a layer's own split scratch
BIG2, BIG3, T128, T64, WIDE = range(5)

SRC = r'''
#include "gemm_plan.h"
#include <cstdio>
int main() {
  long long M; int N, K, vec; unsigned long long bytes;
  while (std::scanf("%lld %d %d %llu %d", &M, &N, &K, &bytes, &vec) == 5) {
    ee::GemmPart parts[ee::kGemmMaxParts];
    const int n = ee::gemm_plan_parts(M, N, K, parts, bytes, vec != 0, ee::GemmPlanOpts{256, true, true, 32768});
    std::printf("%d", n);
    for (int i = 0; i < n; ++i)
      std::printf(" %lld %lld %d %d", (long long)parts[i].row0, (long long)parts[i].rows, parts[i].cfg, (int)parts[i].ordered);
    std::printf("\n");
  }
}
'''


@pytest.fixture(scope="module")
def plan(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    d = tmp_path_factory.mktemp("plan")
    (d / "p.cpp").write_text(SRC)
    exe = d / "p"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(d / "p.cpp"), "-o", str(exe)], check=True)

    def run(problems):
        inp = "".join(f"{M} {N} {K} {b} {v}\n" for M, N, K, b, v in problems)
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
        res = []
        for ln in out[:len(problems)]:
            f = [int(x) for x in ln.split()]
            res.append([tuple(f[1 + 4 * i:5 + 4 * i]) for i in range(f[0])])
        return res
    return run


# the layer's GEMMs at GPT-3 width: (N, K)
SHAPES = {"qkv": (36864, 12288), "out": (12288, 12288), "fc1": (49152, 12288), "fc2": (12288, 49152)}
# FIFO batch sizes of the request stream (T = 7034 ... 9036), the shard, the 12-layer batch, small and odd ones
ROWS = [7034, 7317, 7889, 8125, 8192, 8436, 8731, 9036, 4096, 4205, 4300, 300, 1, 2048, 16000]


def test_parts_cover_the_rows(plan):
    problems = [(M, N, K, b, v) for M in ROWS for N, K in list(SHAPES.values()) + [(9216, 12288), (4096, 512)]
                for b, v in ((WS, 1), (0, 0), (64 << 20, 1))]
    for (M, N, K, b, v), parts in zip(problems, plan(problems)):
        assert 1 <= len(parts) <= 3
        row = 0
        for i, (r0, rows, cfg, ordered) in enumerate(parts):
            assert r0 == row and rows > 0 and cfg in range(5), (M, N, K, parts)
            assert not ordered or (cfg in (BIG2, BIG3, WIDE) and b > 0 and v), (M, N, K, parts)
            if cfg == WIDE:
                assert N % 384 == 0 and i == 0
                if len(parts) > 1:   # whole rounds of 256 x 384 tiles
                    assert rows % 256 == 0 and (rows // 256) * (N // 384) % 256 == 0, (M, N, K, parts)
            row += rows
        assert row == M


def test_the_layers_plans(plan):
    cases = {
        # whole rounds of 256 x 384 tiles: one plain launch
        (8125, *SHAPES["fc1"], WS, 1): [(0, 8125, WIDE, 0)],
        (4096, *SHAPES["fc1"], WS, 1): [(0, 4096, WIDE, 0)],
        # 15.5 rounds: the last split among all 256 workgroups
        (7889, *SHAPES["fc1"], WS, 1): [(0, 7889, WIDE, 1)],
        # without scratch: the whole rounds, then 209 rows on 128 x 128 tiles
        (7889, *SHAPES["fc1"], 0, 0): [(0, 7680, WIDE, 0), (7680, 209, T128, 0)],
        # FC2 (K = 49152): 4 rounds and 32 extra tiles on 128 workgroups
        (8436, *SHAPES["fc2"], WS, 1): [(0, 8436, WIDE, 1)],
        # the shard: split into 256 x 384 pieces, 32 extra tiles would go to
        # 64 workgroups (2.5 wide tiles each, 3.6 rounds); two whole wide rounds
        # and 109 rows on 128 x 64 tiles take 3.43; 256 x 256 tiles split 48
        # over 128 (3.42)
        (4205, 12288, 12288, WS, 1): [(0, 4205, BIG2, 1)],
        # its out projection (K = 3072: no gain from wide tiles; pieces too
        # short to split): whole 256 x 256 rounds and 109 rows on 128 x 64 tiles
        (4205, 12288, 3072, WS, 1): [(0, 4096, BIG2, 0), (4096, 109, T64, 0)],
        # QKV: 24 wide N tiles never fill whole rounds of 17 M tiles
        (4205, 9216, 12288, WS, 1): [(0, 4205, BIG2, 1)],
        # out projection at 7317 rows: 256 x 256 tiles split 112 extra tiles
        # over 224 workgroups (5.5) against 4 rounds of 256 x 384 (5.7)
        (7317, *SHAPES["out"], WS, 1): [(0, 7317, BIG2, 1)],
        # the shapes the GPU tests run on 256 x 384 tiles (ee_linear: no scratch)
        (8192, 49152, 8192, 0, 0): [(0, 8192, WIDE, 0)],
        (4096, 36864, 8192, 0, 0): [(0, 4096, WIDE, 0)],
        (7889, 49152, 4096, 0, 0): [(0, 7680, WIDE, 0), (7680, 209, T128, 0)],
        (7889, 49152, 1024, 0, 0): [(0, 7680, WIDE, 0), (7680, 209, T128, 0)],
        (4205, 12288, 12288, 0, 0): [(0, 4096, WIDE, 0), (4096, 109, T64, 0)],
        (7889, 36864, 1024, 0, 0): [(0, 7889, BIG2, 0)],
        # whole wide rounds, then the 256 x 256 plan for the remaining rows
        (2700, 36864, 12288, 0, 0): [(0, 2048, WIDE, 0), (2048, 652, BIG2, 0)],
        # the request stream's QKV at 31 M-tiles: wide tiles on every row, the
        # last round 62% full (a 256 x 256 launch for the last 1745 rows after
        # 9 wide rounds measured 3.4% slower)
        (7889, 36864, 12288, WS, 1): [(0, 7889, WIDE, 0)],
        (4205, 12288, 49152, 0, 0): [(0, 4096, WIDE, 0), (4096, 109, T64, 0)],
        (8457, 12288, 49152, 0, 0): [(0, 8192, WIDE, 0), (8192, 265, T128, 0)],
        # ... and with a workspace, as in-order pieces of one launch
        (7889, 49152, 4096, WS, 1): [(0, 7889, WIDE, 1)],
        (8436, 36864, 4096, WS, 1): [(0, 8436, WIDE, 1)],
        # the in-order split tests' 256 x 256 shapes
        (7889, 49408, 4096, WS, 1): [(0, 7889, BIG2, 1)],
        (4205, 12288, 4096, WS, 1): [(0, 4205, BIG2, 1)],
        (8436, 12544, 4096, WS, 1): [(0, 8436, BIG2, 1)],
        (4205, 12544, 49152, WS, 1): [(0, 4205, BIG3, 1)],
        (8192, 16384, 4096, WS, 1): [(0, 8192, BIG2, 0)],
        (8500, 16384, 4096, WS, 1): [(0, 8500, BIG2, 1)],
        # small problems: 128 x 128 tiles
        (300, 768, 768, WS, 1): [(0, 300, T128, 0)],
        (1, 4096, 512, 0, 0): [(0, 1, T128, 0)],
    }
    keys = list(cases)
    for k, parts in zip(keys, plan(keys)):
        assert parts == cases[k], (k, parts)
