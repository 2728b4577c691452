"""The 32-bit addressing guard of the head_dim 64/128 attention kernel,
checked on the host against a model of the byte offsets the kernel forms (no
GPU): for every sequence length the guard admits, each key/value load offset
of every key tile, and the buffer descriptor's range, fit a signed 32-bit int.
The guard comes from the library's own header, compiled here with g++."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_padding_amd", "csrc")
KEY_TILE = 32


def _max_offset(L, ld, hd):
    """Largest byte offset the kernel forms for a sequence of L rows at row
    stride ld (halves): tile row k0 + r (k0 the last multiple of the key tile
    below L, r < the key tile), plus the last 16-byte chunk of the head slice."""
    k0 = (L - 1) // KEY_TILE * KEY_TILE
    chunks = hd // 8
    return max((k0 + KEY_TILE - 1) * ld * 2 + (chunks - 1) * 16, L * ld * 2)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_guard_admits_only_lengths_whose_offsets_fit(tmp_path):
    cases = []
    for ld in (3 * 12288, 3 * 96 * 64, 3 * 4096, 128):     # GPT-3 width, GPT-2-like, smaller
        edge = (1 << 31) // (2 * ld)
        cases += [(L, ld) for L in range(max(1, edge - 80), edge + 8)]
    src = tmp_path / "guard.cpp"
    src.write_text('#include "attention_limits.h"\n#include <cstdio>\nint main() {\n  long long L, ld;\n'
                   '  while (std::scanf("%lld %lld", &L, &ld) == 2) std::printf("%d\\n", (int)ee::attn_tr_offsets_fit(L, ld));\n'
                   '  return 0;\n}\n')
    exe = tmp_path / "guard"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], input="".join(f"{L} {ld}\n" for L, ld in cases), capture_output=True,
                         text=True, check=True).stdout.split()
    admitted = {c: o == "1" for c, o in zip(cases, out)}
    assert len(admitted) == len(cases)
    for (L, ld), ok in admitted.items():
        if ok:   # every shorter sequence too (the kernel serves lengths up to max_len)
            for hd in (64, 128):
                assert _max_offset(L, ld, hd) < 1 << 31, (L, ld, hd)
    # the lengths just below the old limit (max_len * row bytes < 2^31) whose
    # last key tile reaches past 2^31 are no longer admitted at GPT-3 width
    ld = 3 * 12288
    assert not admitted[(29126, ld)] and _max_offset(29126, ld, 128) >= 1 << 31
    assert admitted[(29095, ld)] and not admitted[(29096, ld)]
