"""Pins for the oracle's row operations and attention (CPU only).

Each pin ties the oracle to something other than itself: a textbook value, a
closed form, an invariant, or torch's own library routine in float64."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


# ---------------- LayerNorm ----------------
def test_layernorm_matches_torch_fp64():
    x = RNG.standard_normal((7, 96)) * 3 + 0.5
    g = 1 + 0.1 * RNG.standard_normal(96)
    b = 0.1 * RNG.standard_normal(96)
    ref = F.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, b, 1e-5), ref, rtol=1e-12, atol=1e-12)


def test_layernorm_constant_row_gives_beta():
    x = np.full((3, 16), 2.75)
    g = RNG.standard_normal(16)
    b = RNG.standard_normal(16)
    assert np.array_equal(oracle.layer_norm(x, g, b, 1e-5), np.broadcast_to(b, (3, 16)))


def test_layernorm_moments_with_unit_affine():
    x = RNG.standard_normal((4, 256)) * 0.02          # small variance: eps matters
    y = oracle.layer_norm(x, np.ones(256), np.zeros(256), 1e-5)
    var = x.var(axis=1)                                # biased
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-10)


# ---------------- GeLU ----------------
def test_gelu_textbook_values():
    with open(os.path.join(GOLDEN, "gelu_values.json")) as f:
        g = json.load(f)
    for form in ("erf", "tanh"):
        for u, v in g[form]:
            assert abs(float(oracle.gelu(np.array([u]), form)[0]) - v) < 1e-15


def test_gelu_matches_torch_and_symmetry():
    u = np.linspace(-8, 8, 1001)
    tu = torch.from_numpy(u)
    np.testing.assert_allclose(oracle.gelu(u, "tanh"), F.gelu(tu, approximate="tanh").numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu(u, "erf"), F.gelu(tu).numpy(), rtol=1e-13, atol=1e-15)
    for form in ("tanh", "erf"):
        np.testing.assert_allclose(oracle.gelu(u, form) - oracle.gelu(-u, form), u, atol=1e-13)
    assert oracle.gelu(np.zeros(1), "tanh")[0] == 0.0
    # the two forms differ by less than 5e-4 everywhere
    assert np.max(np.abs(oracle.gelu(u, "tanh") - oracle.gelu(u, "erf"))) < 5e-4


# ---------------- linear ----------------
def test_linear_matches_torch_and_layout():
    x = RNG.standard_normal((5, 12))
    w = RNG.standard_normal((7, 12))   # [out, in]
    b = RNG.standard_normal(7)
    ref = F.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(oracle.linear(x, w, b), ref, rtol=1e-12, atol=1e-12)
    # output j is the dot product of x with row j of W
    assert abs(oracle.linear(x, w, b)[2, 3] - (x[2] @ w[3] + b[3])) < 1e-12


# ---------------- attention ----------------
def _qkv(T, nh, hd):
    return RNG.standard_normal((T, 3 * nh * hd))


def test_attention_worked_example():
    with open(os.path.join(GOLDEN, "attention_worked_example.json")) as f:
        g = json.load(f)
    qkv = np.concatenate([np.array(g["q"]), np.array(g["k"]), np.array(g["v"])], axis=1)
    o = oracle.causal_attention_packed(qkv, [0, 2], 1, g["head_dim"])
    np.testing.assert_allclose(o, np.array(g["o"]), rtol=0, atol=1e-14)


def test_attention_first_query_is_v0_exactly():
    nh, hd = 3, 8
    lens = [5, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qkv = _qkv(int(cu[-1]), nh, hd)
    o = oracle.causal_attention_packed(qkv, cu, nh, hd)
    Hp = nh * hd
    for b in range(3):
        assert np.array_equal(o[cu[b]], qkv[cu[b], 2 * Hp:3 * Hp])


def test_attention_zero_queries_give_prefix_mean():
    nh, hd, L = 2, 4, 9
    qkv = _qkv(L, nh, hd)
    Hp = nh * hd
    qkv[:, :Hp] = 0
    o = oracle.causal_attention_packed(qkv, [0, L], nh, hd)
    v = qkv[:, 2 * Hp:]
    for i in range(L):
        np.testing.assert_allclose(o[i], v[:i + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("nh,hd", [(2, 16), (3, 64), (1, 128)])
def test_attention_matches_torch_sdpa_fp64(nh, hd):
    lens = [1, 6, 13]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qkv = _qkv(int(cu[-1]), nh, hd)
    o = oracle.causal_attention_packed(qkv, cu, nh, hd)
    Hp = nh * hd
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        t = torch.from_numpy(qkv[s0:s1])
        q = t[:, :Hp].reshape(-1, nh, hd).transpose(0, 1)
        k = t[:, Hp:2 * Hp].reshape(-1, nh, hd).transpose(0, 1)
        v = t[:, 2 * Hp:].reshape(-1, nh, hd).transpose(0, 1)
        ref = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(-1, Hp).numpy()
        np.testing.assert_allclose(o[s0:s1], ref, rtol=1e-11, atol=1e-12)


def test_attention_query_matches_torch_sdpa_fp64():
    """The single-query form against torch's causal SDPA (fp64), row by row; rows
    after the query change nothing (causality); out-of-range queries raise."""
    nh, hd, L = 3, 32, 40
    qkv = _qkv(L, nh, hd)
    Hp = nh * hd
    t = torch.from_numpy(qkv)
    q = t[:, :Hp].reshape(-1, nh, hd).transpose(0, 1)
    k = t[:, Hp:2 * Hp].reshape(-1, nh, hd).transpose(0, 1)
    v = t[:, 2 * Hp:].reshape(-1, nh, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(-1, Hp).numpy()
    for i in range(L):
        o = oracle.causal_attention_query(qkv, i, nh, hd)
        np.testing.assert_allclose(o, ref[i], rtol=1e-11, atol=1e-12)
        assert np.array_equal(o, oracle.causal_attention_query(qkv[:i + 1], i, nh, hd))
    with pytest.raises(ValueError):
        oracle.causal_attention_query(qkv, L, nh, hd)


def test_attention_batch_permutation_permutes_outputs():
    nh, hd = 2, 8
    lens = [3, 5, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qkv = _qkv(int(cu[-1]), nh, hd)
    o = oracle.causal_attention_packed(qkv, cu, nh, hd)
    perm = [2, 0, 1]
    blocks = [qkv[cu[b]:cu[b + 1]] for b in perm]
    lens_p = [lens[b] for b in perm]
    cu_p = np.concatenate([[0], np.cumsum(lens_p)])
    o_p = oracle.causal_attention_packed(np.concatenate(blocks), cu_p, nh, hd)
    for i, b in enumerate(perm):
        assert np.array_equal(o_p[cu_p[i]:cu_p[i + 1]], o[cu[b]:cu[b + 1]])


def test_attention_padded_equals_packed_on_valid_rows():
    nh, hd, P = 2, 8, 7
    lens = [4, 7, 0, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qkv_pad = RNG.standard_normal((len(lens), P, 3 * nh * hd))
    packed = np.concatenate([qkv_pad[b, :n] for b, n in enumerate(lens)])
    o = oracle.causal_attention_packed(packed, cu, nh, hd)
    for b, n in enumerate(lens):
        op = oracle.causal_attention_padded(qkv_pad[b], n, nh, hd)
        assert np.array_equal(op[:n], o[cu[b]:cu[b + 1]])
        if n == 0:
            assert np.all(op == 0)      # empty key set -> zero output
