"""Pins for the oracle's offsets and remove/rebuild (CPU only).

Offsets and indices have exactly one correct answer: they are pinned to
hand-worked examples, to a brute-force count that does not use a prefix sum,
and to numpy's boolean-mask selection."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_packed_index(lens, P):
    """Packed index of (b, p) = number of valid positions strictly before it in
    row-major order (a direct count, no running sum)."""
    B = len(lens)
    valid = [[p < lens[b] for p in range(P)] for b in range(B)]
    out = {}
    for b in range(B):
        for p in range(P):
            if valid[b][p]:
                out[(b, p)] = sum(1 for b2 in range(B) for p2 in range(P)
                                  if valid[b2][p2] and (b2, p2) < (b, p))
    return out


def test_worked_examples():
    with open(os.path.join(GOLDEN, "offsets_worked_example.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        cu, src, p2p, T = oracle.offsets_from_lengths(case["lens"], case["pad_len"])
        assert cu.tolist() == case["cu"]
        assert T == case["total"]
        assert src.tolist() == case["token_src"]
        assert p2p.tolist() == case["pad2pack"]
        mask = np.array([[p < n for p in range(case["pad_len"])] for n in case["lens"]], dtype=np.uint8)
        cu2, src2, p2p2, T2 = oracle.offsets_from_mask(mask)
        assert cu2.tolist() == case["cu"] and src2.tolist() == case["token_src"]
        assert p2p2.tolist() == case["pad2pack"] and T2 == case["total"]


@pytest.mark.parametrize("B,P", [(1, 1), (1, 4), (2, 3), (3, 4), (3, 2)])
def test_brute_force_all_length_vectors(B, P):
    for lens in itertools.product(range(P + 1), repeat=B):
        cu, src, p2p, T = oracle.offsets_from_lengths(lens, P)
        assert T == sum(lens) == cu[-1]
        brute = _brute_packed_index(lens, P)
        assert len(brute) == T
        for b in range(B):
            assert cu[b] == sum(lens[:b])
            for p in range(P):
                r = b * P + p
                if p < lens[b]:
                    assert p2p[r] == brute[(b, p)]
                    assert src[brute[(b, p)]] == r
                else:
                    assert p2p[r] == -1
        mask = np.array([[p < n for p in range(P)] for n in lens], dtype=np.uint8).reshape(B, P)
        assert int(mask.sum()) == T
        cu2, src2, p2p2, T2 = oracle.offsets_from_mask(mask)
        assert T2 == T and np.array_equal(cu2, cu) and np.array_equal(src2, src) and np.array_equal(p2p2, p2p)


def test_mask_scan_general_mask():
    """A non-right-padded mask still packs valid positions in row-major order."""
    rng = np.random.default_rng(3)
    mask = (rng.random((5, 7)) < 0.5).astype(np.uint8)
    cu, src, p2p, T = oracle.offsets_from_mask(mask)
    flat = mask.reshape(-1)
    assert np.array_equal(src, np.nonzero(flat)[0])
    assert T == int(flat.sum())
    for b in range(5):
        assert cu[b] == int(mask[:b].sum())


def test_bad_lengths_rejected():
    with pytest.raises(ValueError):
        oracle.offsets_from_lengths([3, 5], 4)
    with pytest.raises(ValueError):
        oracle.offsets_from_lengths([-1], 4)


def test_remove_rebuild_round_trip_and_numpy_selection():
    rng = np.random.default_rng(11)
    B, P, H = 6, 9, 5
    lens = [0, 9, 1, 4, 9, 2]
    x = rng.standard_normal((B, P, H)).astype(np.float32)
    mask = np.array([[p < n for p in range(P)] for n in lens])
    packed = oracle.remove_padding(x, lens)
    assert np.array_equal(packed, x[mask])                      # numpy boolean selection
    y = oracle.rebuild_padding(packed, lens, P)
    assert np.array_equal(y[mask], x[mask])                     # identity on valid rows
    assert np.all(y[~mask] == 0) and not np.any(np.signbit(y[~mask]))   # +0.0 on pads
    assert np.array_equal(oracle.remove_padding(y, lens), packed)
    z = rng.standard_normal((sum(lens), H))
    assert np.array_equal(oracle.remove_padding(oracle.rebuild_padding(z, lens, P), lens), z)


def test_nan_pads_never_reach_output():
    B, P, H = 3, 5, 4
    lens = [2, 5, 0]
    x = np.full((B, P, H), np.nan, dtype=np.float32)
    for b, n in enumerate(lens):
        x[b, :n] = 1.0 + b
    y = oracle.rebuild_padding(oracle.remove_padding(x, lens), lens, P)
    assert not np.isnan(y).any()
