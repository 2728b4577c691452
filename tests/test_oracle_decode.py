"""Pins for the incremental-decoding oracle (CPU only): extending a sequence
step by step through a cache gives the causal forward of the whole sequence at
the new positions, however the tokens are split into steps; the cached keys
and values are the K/V projections of each layer's input; one query over the
cache matches torch's scaled_dot_product_attention."""
import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _setup(n_layers=2, seed=3):
    w = dataclasses.replace(workloads.get("tiny-fp32"), batch=3, pad_len=12)
    ps = [oracle.to_f64_params(workloads.layer_params(w, seed, l, variant="affine")) for l in range(n_layers)]
    return w, ps


@pytest.mark.parametrize("splits", [[12], [1] * 12, [5, 1, 1, 3, 2], [7, 5]])
def test_incremental_equals_full_causal_forward(splits):
    w, ps = _setup()
    x = workloads.activations(w, 8, 1, 12, [12]).double().numpy()[0]
    cu = [0, 12]
    full = x
    for p in ps:
        full = oracle.layer_forward_packed(full, cu, p, w.n_heads, w.head_dim)
    cache = oracle.SequenceCache(len(ps), w.n_heads, w.head_dim)
    got, r = [], 0
    for n in splits:
        got.append(oracle.extend_sequence(cache, x[r:r + n], ps, w.n_heads, w.head_dim))
        r += n
    np.testing.assert_allclose(np.concatenate(got), full, rtol=1e-11, atol=1e-12)
    assert cache.length == 12


def test_cache_holds_the_kv_projections_of_each_layer_input():
    w, ps = _setup()
    x = workloads.activations(w, 9, 1, 12, [12]).double().numpy()[0]
    cache = oracle.SequenceCache(len(ps), w.n_heads, w.head_dim)
    oracle.extend_sequence(cache, x[:4], ps, w.n_heads, w.head_dim)
    oracle.extend_sequence(cache, x[4:], ps, w.n_heads, w.head_dim)
    Hp = w.n_heads * w.head_dim
    inp = x
    for l, p in enumerate(ps):
        keep = {}
        out = oracle.layer_forward_packed(inp, [0, 12], p, w.n_heads, w.head_dim, keep=keep)
        a = oracle.layer_norm(inp, p["ln1_g"], p["ln1_b"], 1e-5)
        qkv = oracle.linear(a, p["w_qkv"], p["b_qkv"])
        k = qkv[:, Hp:2 * Hp].reshape(12, w.n_heads, w.head_dim).transpose(1, 0, 2)
        v = qkv[:, 2 * Hp:].reshape(12, w.n_heads, w.head_dim).transpose(1, 0, 2)
        np.testing.assert_allclose(cache.k[l], k, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(cache.v[l], v, rtol=1e-11, atol=1e-12)
        inp = out


def test_first_layer_cache_prefill_equals_extend():
    """Filling a one-layer cache without the outputs leaves the cache that
    extend_sequence leaves (bitwise for the same rows in one call, to rounding
    in chunks), and the next step's output is the same."""
    w, ps = _setup(n_layers=1)
    x = workloads.activations(w, 10, 1, 12, [12]).double().numpy()[0]
    ref = oracle.SequenceCache(1, w.n_heads, w.head_dim)
    oracle.extend_sequence(ref, x[:11], ps, w.n_heads, w.head_dim)
    one = oracle.SequenceCache(1, w.n_heads, w.head_dim)
    oracle.prefill_first_layer_cache(one, x[:11], ps[0], w.n_heads, w.head_dim)
    assert np.array_equal(one.k[0], ref.k[0]) and np.array_equal(one.v[0], ref.v[0])
    chunks = oracle.SequenceCache(1, w.n_heads, w.head_dim)
    oracle.prefill_first_layer_cache(chunks, x[:6], ps[0], w.n_heads, w.head_dim)
    oracle.prefill_first_layer_cache(chunks, x[6:11], ps[0], w.n_heads, w.head_dim)
    np.testing.assert_allclose(chunks.k[0], ref.k[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(chunks.v[0], ref.v[0], rtol=1e-12, atol=1e-13)
    y_ref = oracle.extend_sequence(ref, x[11:], ps, w.n_heads, w.head_dim)
    y_one = oracle.extend_sequence(one, x[11:], ps, w.n_heads, w.head_dim)
    assert np.array_equal(y_one, y_ref)
    with pytest.raises(ValueError):
        oracle.prefill_first_layer_cache(oracle.SequenceCache(2, w.n_heads, w.head_dim), x, ps[0], w.n_heads,
                                         w.head_dim)


def test_one_decode_query_matches_torch_sdpa():
    w, ps = _setup(n_layers=1)
    x = workloads.activations(w, 10, 1, 12, [12]).double().numpy()[0]
    cache = oracle.SequenceCache(1, w.n_heads, w.head_dim)
    oracle.extend_sequence(cache, x[:11], ps, w.n_heads, w.head_dim)
    # the attention output of the 12th token: rebuild it from the oracle's pieces and torch
    p = ps[0]
    Hp = w.n_heads * w.head_dim
    a = oracle.layer_norm(x[11:], p["ln1_g"], p["ln1_b"], 1e-5)
    qkv = oracle.linear(a, p["w_qkv"], p["b_qkv"])
    q = torch.from_numpy(qkv[:, :Hp].reshape(1, w.n_heads, w.head_dim).transpose(1, 0, 2))  # [nh, 1, hd]
    K = torch.cat([torch.from_numpy(cache.k[0]),
                   torch.from_numpy(qkv[:, Hp:2 * Hp].reshape(1, w.n_heads, w.head_dim).transpose(1, 0, 2))], dim=1)
    V = torch.cat([torch.from_numpy(cache.v[0]),
                   torch.from_numpy(qkv[:, 2 * Hp:].reshape(1, w.n_heads, w.head_dim).transpose(1, 0, 2))], dim=1)
    o_ref = F.scaled_dot_product_attention(q, K, V).transpose(0, 1).reshape(1, Hp).numpy()
    hres = x[11:] + oracle.linear(o_ref, p["w_out"], p["b_out"])
    c = oracle.layer_norm(hres, p["ln2_g"], p["ln2_b"], 1e-5)
    ref = hres + oracle.linear(oracle.gelu(oracle.linear(c, p["w_fc1"], p["b_fc1"])), p["w_fc2"], p["b_fc2"])
    got = oracle.extend_sequence(cache, x[11:], ps, w.n_heads, w.head_dim)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_batch_extend_keeps_sequences_apart():
    w, ps = _setup()
    xs = [workloads.activations(w, 20 + b, 1, 12, [12]).double().numpy()[0] for b in range(3)]
    caches = [oracle.SequenceCache(len(ps), w.n_heads, w.head_dim) for _ in range(3)]
    steps = [[3, 0, 5], [1, 2, 0], [0, 1, 1]]   # new tokens per sequence per step (0 = idle)
    pos = [0, 0, 0]
    for new_len in steps:
        rows = np.concatenate([xs[b][pos[b]:pos[b] + n] for b, n in enumerate(new_len)])
        out = oracle.extend_batch(caches, rows, new_len, ps, w.n_heads, w.head_dim)
        r = 0
        for b, n in enumerate(new_len):
            if n:
                alone = oracle.SequenceCache(len(ps), w.n_heads, w.head_dim)
                full = oracle.extend_sequence(alone, xs[b][:pos[b] + n], ps, w.n_heads, w.head_dim)
                np.testing.assert_allclose(out[r:r + n], full[pos[b]:], rtol=1e-11, atol=1e-12)
            r += n
            pos[b] += n
