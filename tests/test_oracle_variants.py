"""Pins for the oracle's page-literal RCE form (transposing rebuild/remove
around padded attention) and the post-LN encoder block (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

RNG = np.random.default_rng(77)


def _mask(lens, P):
    return np.array([[p < n for p in range(P)] for n in lens])


def test_transposing_rebuild_matches_reshape_formulation():
    nh, hd, P = 3, 4, 6
    lens = [6, 0, 2, 5]
    T = sum(lens)
    packed = RNG.standard_normal((T, 3 * nh * hd))
    got = oracle.transpose_padding_rebuild_heads(packed, lens, P, nh, hd)
    # independent formulation: scatter rows by boolean mask, then reshape/transpose
    pad = np.zeros((len(lens), P, 3 * nh * hd))
    pad[_mask(lens, P)] = packed
    ref = pad.reshape(len(lens), P, 3, nh, hd).transpose(2, 0, 3, 1, 4)
    assert np.array_equal(got, ref)
    assert np.all(got[:, 1] == 0) and np.all(got[:, 2, :, 2:] == 0)


def test_transposing_remove_matches_reshape_formulation_and_round_trip():
    B, nh, P, hd = 4, 2, 5, 3
    lens = [5, 1, 0, 3]
    x = RNG.standard_normal((B, nh, P, hd))
    got = oracle.transpose_padding_remove_heads(x, lens)
    ref = x.transpose(0, 2, 1, 3).reshape(B, P, nh * hd)[_mask(lens, P)]
    assert np.array_equal(got, ref)
    back = oracle.transpose_padding_rebuild_heads(got, lens, P, nh, hd)[0]
    m = _mask(lens, P)
    for b in range(B):
        assert np.array_equal(back[b][:, m[b]], x[b][:, m[b]])


@pytest.mark.parametrize("causal", [True, False])
def test_padded_attention_matches_torch_sdpa_with_masks(causal):
    B, nh, P, hd = 3, 2, 7, 8
    lens = [7, 3, 1]
    q, k, v = (RNG.standard_normal((B, nh, P, hd)) for _ in range(3))
    o = oracle.attention_padded_heads(q, k, v, lens, causal)
    for b, n in enumerate(lens):
        allowed = np.zeros((P, P), dtype=bool)
        allowed[:, :n] = True
        if causal:
            allowed &= np.tril(np.ones((P, P), dtype=bool))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[b]), torch.from_numpy(k[b]), torch.from_numpy(v[b]),
                                             attn_mask=torch.from_numpy(allowed)).numpy()
        np.testing.assert_allclose(o[b, :, :n], ref[:, :n], rtol=1e-11, atol=1e-12)
        assert np.all(o[b, :, n:] == 0)


def test_page_literal_attention_equals_varlen_bit_exact():
    nh, hd, P = 2, 8, 9
    lens = [9, 4, 1, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qkv = RNG.standard_normal((int(cu[-1]), 3 * nh * hd))
    a = oracle.attention_via_padded_heads(qkv, cu, P, nh, hd, causal=True)
    assert np.array_equal(a, oracle.causal_attention_packed(qkv, cu, nh, hd))
    b = oracle.attention_via_padded_heads(qkv, cu, P, nh, hd, causal=False)
    assert np.array_equal(b, oracle.attention_packed_bidirectional(qkv, cu, nh, hd))


def test_bidirectional_attention_matches_torch_sdpa():
    nh, hd = 3, 16
    lens = [5, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    qkv = RNG.standard_normal((int(cu[-1]), 3 * nh * hd))
    o = oracle.attention_packed_bidirectional(qkv, cu, nh, hd)
    Hp = nh * hd
    for b in range(len(lens)):
        t = torch.from_numpy(qkv[cu[b]:cu[b + 1]])
        q, k, v = (t[:, i * Hp:(i + 1) * Hp].reshape(-1, nh, hd).transpose(0, 1) for i in range(3))
        ref = F.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(-1, Hp).numpy()
        np.testing.assert_allclose(o[cu[b]:cu[b + 1]], ref, rtol=1e-11, atol=1e-12)
    # the last query sees the same keys as the first: bidirectional, not causal
    assert not np.allclose(o[cu[2]], qkv[cu[2], 2 * Hp:])


def test_add_bias_residual_layernorm_matches_torch():
    u, r = RNG.standard_normal((6, 40)), RNG.standard_normal((6, 40))
    b, g, be = RNG.standard_normal(40), 1 + 0.1 * RNG.standard_normal(40), RNG.standard_normal(40)
    ref = F.layer_norm(torch.from_numpy(u + b + r), (40,), torch.from_numpy(g), torch.from_numpy(be), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.add_bias_residual_layernorm(u, b, r, g, be, 1e-5), ref, rtol=1e-12, atol=1e-12)


def _torch_encoder(x_seq, p, nh, hd, eps=1e-5):
    """BERT-style post-LN block from torch routines (fp64), one unpadded sequence."""
    t = {k: torch.from_numpy(v) for k, v in p.items()}
    x = torch.from_numpy(x_seq)
    H, Hp = x.shape[1], nh * hd
    qkv = F.linear(x, t["w_qkv"], t["b_qkv"])
    q, k, v = (qkv[:, i * Hp:(i + 1) * Hp].reshape(-1, nh, hd).transpose(0, 1) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(-1, Hp)
    h = F.layer_norm(x + F.linear(o, t["w_out"], t["b_out"]), (H,), t["ln1_g"], t["ln1_b"], eps)
    g = F.gelu(F.linear(h, t["w_fc1"], t["b_fc1"]))
    return F.layer_norm(h + F.linear(g, t["w_fc2"], t["b_fc2"]), (H,), t["ln2_g"], t["ln2_b"], eps).numpy()


def test_encoder_matches_torch_composition_and_packed_equals_padded():
    import dataclasses
    w = dataclasses.replace(workloads.get("tiny-fp32"), batch=3, pad_len=8)
    lens = [8, 3, 1]
    x = workloads.activations(w, 4, 3, 8, lens).double().numpy()
    p = oracle.to_f64_params(workloads.layer_params(w, 4, 0, variant="affine"))
    y = oracle.encoder_layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(y[b, :n], _torch_encoder(x[b, :n], p, w.n_heads, w.head_dim), rtol=1e-10, atol=1e-11)
        assert np.all(y[b, n:] == 0)
    cu, _, _, _ = oracle.offsets_from_lengths(lens, 8)
    xp = oracle.remove_padding(x, lens)
    yp = oracle.encoder_layer_forward_packed(xp, cu, p, w.n_heads, w.head_dim)
    np.testing.assert_allclose(oracle.rebuild_padding(yp, lens, 8), y, rtol=1e-12, atol=1e-13)
    yl = oracle.encoder_layer_forward_packed(xp, cu, p, w.n_heads, w.head_dim, attention="padded", pad_len=8)
    assert np.array_equal(yl, yp)


def test_encoder_zero_weights_closed_form():
    import dataclasses
    w = dataclasses.replace(workloads.get("tiny-fp32"), batch=2, pad_len=4)
    lens = [4, 2]
    x = workloads.activations(w, 6, 2, 4, lens).double().numpy()
    p = oracle.to_f64_params(workloads.layer_params(w, 6, 0, variant="zero-weights"))
    y = oracle.encoder_layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    for b, n in enumerate(lens):
        xb = torch.from_numpy(x[b, :n])
        h = F.layer_norm(xb + torch.from_numpy(p["b_out"]), (w.hidden,), torch.from_numpy(p["ln1_g"]),
                         torch.from_numpy(p["ln1_b"]), eps=1e-5)
        ref = F.layer_norm(h + torch.from_numpy(p["b_fc2"]), (w.hidden,), torch.from_numpy(p["ln2_g"]),
                           torch.from_numpy(p["ln2_b"]), eps=1e-5).numpy()
        np.testing.assert_allclose(y[b, :n], ref, rtol=1e-12, atol=1e-12)


def test_decoder_page_literal_equals_varlen():
    import dataclasses
    w = dataclasses.replace(workloads.get("tiny-fp32"), batch=3, pad_len=10)
    lens = [10, 4, 7]
    x = workloads.activations(w, 2, 3, 10, lens).double().numpy()
    p = workloads.layer_params(w, 2, 0, variant="affine")
    cu, _, _, _ = oracle.offsets_from_lengths(lens, 10)
    xp = oracle.remove_padding(x, lens)
    a = oracle.layer_forward_packed(xp, cu, p, w.n_heads, w.head_dim)
    b = oracle.layer_forward_packed(xp, cu, p, w.n_heads, w.head_dim, attention="padded", pad_len=10)
    assert np.array_equal(a, b)
