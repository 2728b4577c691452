"""Pins for the oracle's whole-layer forward (CPU only).

The layer is pinned by (a) special cases with closed forms (zero weights),
(b) the RCE invariants (valid rows do not depend on pads; each sequence alone,
unpadded, gives its rows of the padded batch; packed == padded on valid rows),
and (c) a float64 composition of torch library routines (layer_norm, linear,
scaled_dot_product_attention with is_causal, gelu).  A mutation test plants
plausible mistakes in the oracle and checks that these pins catch each one."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.layer as OL
import workloads


def _small(name="tiny-fp32", **kw):
    import dataclasses
    return dataclasses.replace(workloads.get(name), **kw)


def _params64(w, seed=5, layer=0, variant="affine"):
    return oracle.to_f64_params(workloads.layer_params(w, seed, layer, variant=variant))


def _torch_layer(x_seq, p, nh, hd, eps=1e-5, gelu="tanh"):
    """One unpadded sequence [L, H] through a pre-LN block built from torch routines (fp64)."""
    t = {k: torch.from_numpy(v) for k, v in p.items()}
    x = torch.from_numpy(x_seq)
    H = x.shape[1]
    Hp = nh * hd
    a = F.layer_norm(x, (H,), t["ln1_g"], t["ln1_b"], eps)
    qkv = F.linear(a, t["w_qkv"], t["b_qkv"])
    q, k, v = (qkv[:, i * Hp:(i + 1) * Hp].reshape(-1, nh, hd).transpose(0, 1) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(-1, Hp)
    h = x + F.linear(o, t["w_out"], t["b_out"])
    c = F.layer_norm(h, (H,), t["ln2_g"], t["ln2_b"], eps)
    g = F.gelu(F.linear(c, t["w_fc1"], t["b_fc1"]), approximate="tanh" if gelu == "tanh" else "none")
    return (h + F.linear(g, t["w_fc2"], t["b_fc2"])).numpy()


def _inputs(w, seed=5, lens=None, pad_fill="random"):
    if lens is None:
        lens = workloads.lengths(w, seed)
    x = workloads.activations(w, seed, w.batch, w.pad_len, lens, pad_fill=pad_fill).double().numpy()
    return x, lens


@pytest.mark.parametrize("gelu", ["tanh", "erf"])
def test_layer_matches_torch_composition(gelu):
    w = _small(batch=3, pad_len=9)
    x, lens = _inputs(w, lens=[9, 1, 5])
    p = _params64(w)
    y = oracle.layer_forward_padded(x, lens, p, w.n_heads, w.head_dim, gelu_form=gelu)
    for b, n in enumerate(lens):
        ref = _torch_layer(x[b, :n], p, w.n_heads, w.head_dim, gelu=gelu)
        np.testing.assert_allclose(y[b, :n], ref, rtol=1e-10, atol=1e-12)
        assert np.all(y[b, n:] == 0) and not np.any(np.signbit(y[b, n:]))


def test_layer_gpt2_shape_matches_torch_composition():
    w = _small("gpt2-small", batch=2, pad_len=12, hidden=128, n_heads=2, ffn=256)
    x, lens = _inputs(w, lens=[12, 7])
    p = _params64(w)
    y = oracle.layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(y[b, :n], _torch_layer(x[b, :n], p, w.n_heads, w.head_dim), rtol=1e-10, atol=1e-11)


def test_zero_weights_and_biases_is_identity_bit_exact():
    w = _small(batch=3, pad_len=6)
    x, lens = _inputs(w, lens=[6, 2, 3])
    p = _params64(w, variant="zero-weights")
    for k in ("b_qkv", "b_out", "b_fc1", "b_fc2"):
        p[k] = np.zeros_like(p[k])
    y = oracle.layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    for b, n in enumerate(lens):
        assert np.array_equal(y[b, :n], x[b, :n])


def test_zero_weights_with_biases_adds_output_biases():
    w = _small(batch=2, pad_len=5)
    x, lens = _inputs(w, lens=[5, 3])
    p = _params64(w, variant="zero-weights")
    y = oracle.layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(y[b, :n], x[b, :n] + p["b_out"] + p["b_fc2"], rtol=0, atol=1e-15)


def test_valid_rows_independent_of_pads_bit_exact():
    w = _small(batch=4, pad_len=8)
    lens = [8, 3, 1, 5]
    x_r, _ = _inputs(w, lens=lens, pad_fill="random")
    x_n, _ = _inputs(w, lens=lens, pad_fill="nan")
    p = _params64(w)
    y_r = oracle.layer_forward_padded(x_r, lens, p, w.n_heads, w.head_dim)
    y_n = oracle.layer_forward_padded(x_n, lens, p, w.n_heads, w.head_dim)
    assert not np.isnan(y_n).any()
    assert np.array_equal(y_r, y_n)


def test_each_sequence_alone_equals_its_rows_in_batch():
    w = _small(batch=4, pad_len=10)
    lens = [10, 4, 1, 7]
    x, _ = _inputs(w, lens=lens)
    p = _params64(w)
    y = oracle.layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    for b, n in enumerate(lens):
        alone = oracle.layer_forward_padded(x[b:b + 1, :n], [n], p, w.n_heads, w.head_dim)
        np.testing.assert_allclose(alone[0], y[b, :n], rtol=1e-13, atol=1e-14)


def test_packed_forward_equals_padded_forward():
    w = _small(batch=5, pad_len=11)
    lens = [11, 0, 6, 1, 9]
    x, _ = _inputs(w, lens=lens)
    p = _params64(w)
    y_pad = oracle.layer_forward_padded(x, lens, p, w.n_heads, w.head_dim)
    cu, _, _, T = oracle.offsets_from_lengths(lens, w.pad_len)
    keep = {}
    y_pk = oracle.layer_forward_packed(oracle.remove_padding(x, lens), cu, p, w.n_heads, w.head_dim, keep=keep)
    assert y_pk.shape == (T, w.hidden) and set(keep) == {"a", "qkv", "o", "h", "c", "u", "g", "y"}
    np.testing.assert_allclose(oracle.rebuild_padding(y_pk, lens, w.pad_len), y_pad, rtol=1e-13, atol=1e-14)


def test_stack_packed_equals_padded():
    w = _small(batch=3, pad_len=6)
    lens = [6, 2, 4]
    x, _ = _inputs(w, lens=lens)
    ps = [_params64(w, layer=l) for l in range(3)]
    a = oracle.stack_forward_padded(x, lens, ps, w.n_heads, w.head_dim)
    b = oracle.stack_forward_packed(x, lens, ps, w.n_heads, w.head_dim)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    assert np.all(a[1, 2:] == 0)


# ---------------------------------------------------------------------------
# Mutation test: plausible mistakes planted in the oracle (on the CPU) must be
# caught by the pins above.
# ---------------------------------------------------------------------------
def _mut_attention_no_scale(q, K, V, scale):
    return _ORIG_ATTEND(q, K, V, 1.0)


def _mut_attention_noncausal(qkv, cu, nh, hd):
    return _ORIG_PACKED(qkv, cu, nh, hd)  # replaced below per mutant


_ORIG_ATTEND = OL._attend_one_query
_ORIG_PACKED = OL.causal_attention_packed
_ORIG_PADDED = OL.causal_attention_padded
_ORIG_LN = OL.layer_norm
_ORIG_LINEAR = OL.linear
_ORIG_GELU = OL.gelu
_ORIG_BLOCK = OL._block


def _padded_peek_future(qkv, length, nh, hd):
    qkv = np.asarray(qkv, np.float64)
    P = qkv.shape[0]
    Hp = nh * hd
    o = np.zeros((P, Hp))
    for n in range(nh):
        c = slice(n * hd, (n + 1) * hd)
        for p in range(P):
            jmax = min(p + 2, int(length))   # one key too many
            o[p, c] = _ORIG_ATTEND(qkv[p, c], qkv[:jmax, Hp:2 * Hp][:, c], qkv[:jmax, 2 * Hp:][:, c], 1 / math.sqrt(hd))
    return o


def _block_no_residual(x, attn_fn, p, eps, gelu_form, keep=None):
    a = OL.layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    h = x + OL.linear(attn_fn(OL.linear(a, p["w_qkv"], p["b_qkv"])), p["w_out"], p["b_out"])
    c = OL.layer_norm(h, p["ln2_g"], p["ln2_b"], eps)
    return OL.linear(OL.gelu(OL.linear(c, p["w_fc1"], p["b_fc1"]), gelu_form), p["w_fc2"], p["b_fc2"])  # drops "h +"


MUTANTS = {
    "attention without 1/sqrt(hd)": ("_attend_one_query", _mut_attention_no_scale),
    "attention sees one future key": ("causal_attention_padded", _padded_peek_future),
    "LayerNorm with unbiased variance": ("layer_norm", lambda x, g, b, e: (np.asarray(x) - np.asarray(x).mean(-1, keepdims=True)) / np.sqrt(np.asarray(x).var(-1, ddof=1, keepdims=True) + e) * g + b),
    "LayerNorm eps outside sqrt": ("layer_norm", lambda x, g, b, e: (np.asarray(x) - np.asarray(x).mean(-1, keepdims=True)) / (np.sqrt(np.asarray(x).var(-1, keepdims=True)) + e) * g + b),
    "linear drops bias": ("linear", lambda x, w, b: np.asarray(x, np.float64) @ np.asarray(w, np.float64).T),
    "gelu sign flip": ("gelu", lambda u, form="tanh": 0.5 * np.asarray(u) * (1 - np.tanh(math.sqrt(2 / math.pi) * (np.asarray(u) + 0.044715 * np.asarray(u) ** 3)))),
    "second residual dropped": ("_block", _block_no_residual),
}


def _run_pins():
    """Runs the layer pins; returns the names of those that fail."""
    failed = []
    for fn in (test_layer_matches_torch_composition, test_zero_weights_with_biases_adds_output_biases,
               test_zero_weights_and_biases_is_identity_bit_exact, test_layer_gpt2_shape_matches_torch_composition):
        try:
            if fn is test_layer_matches_torch_composition:
                fn("tanh")
            else:
                fn()
        except AssertionError:
            failed.append(fn.__name__)
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(OL, attr, fn)
    assert _run_pins(), f"no pin caught the planted mistake: {mutant}"


def test_unmutated_oracle_passes_the_pin_set():
    assert _run_pins() == []
