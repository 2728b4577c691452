"""Plain float64 CPU implementation of the padding-removed GPT layer forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: loops
follow the definitions one sequence / head / query at a time, and the only
library primitives used are numpy's matrix product, exp, tanh and sqrt
(scipy's erf for the erf-form GeLU).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

_F64 = np.float64


# ---------------------------------------------------------------------------
# Offsets.  Energon-AI announcement article, "Runtime": the remove/rebuild ops
# need, for every valid token, its place in the packed buffer.  The packed
# order is sequence-major, valid tokens first (right padding).
# ---------------------------------------------------------------------------
def offsets_from_lengths(lens: Sequence[int], pad_len: int):
    """Per-sequence offsets from host lengths.

    Returns (cu [B+1], token_src [T], pad2pack [B*P], T):
      cu[0] = 0, cu[b+1] = cu[b] + len[b]             (exclusive prefix sum)
      token_src[t] = b*P + (t - cu[b])  for t in [cu[b], cu[b+1])
      pad2pack[b*P + p] = cu[b] + p if p < len[b] else -1
    """
    lens = [int(n) for n in lens]
    B, P = len(lens), int(pad_len)
    for n in lens:
        if n < 0 or n > P:
            raise ValueError(f"length {n} outside [0, {P}]")
    cu = np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        cu[b + 1] = cu[b] + lens[b]
    T = int(cu[B])
    token_src = np.empty(T, dtype=np.int64)
    pad2pack = np.full(B * P, -1, dtype=np.int64)
    for b in range(B):
        for p in range(lens[b]):
            t = int(cu[b]) + p
            token_src[t] = b * P + p
            pad2pack[b * P + p] = t
    return cu, token_src, pad2pack, T


def offsets_from_mask(mask: np.ndarray):
    """The attention mask [B, P] (nonzero = valid token) prefix-summed.

    The flattened exclusive prefix sum of the mask gives each valid position its
    packed index; cu[b] counts the valid tokens of rows before b.
    """
    mask = np.asarray(mask) != 0
    B, P = mask.shape
    flat = mask.reshape(-1)
    excl = np.zeros(B * P + 1, dtype=np.int64)
    running = 0
    for r in range(B * P):
        excl[r] = running
        running += int(flat[r])
    excl[B * P] = running
    T = running
    pad2pack = np.full(B * P, -1, dtype=np.int64)
    token_src = np.empty(T, dtype=np.int64)
    for r in range(B * P):
        if flat[r]:
            pad2pack[r] = excl[r]
            token_src[excl[r]] = r
    cu = np.array([excl[b * P] for b in range(B)] + [T], dtype=np.int64)
    return cu, token_src, pad2pack, T


# ---------------------------------------------------------------------------
# transpose_padding_remove / transpose_padding_rebuild (announcement article,
# "Runtime"), read as a pure gather/scatter between the padded
# [B, P, H] layout and the packed [T, H] layout.
# ---------------------------------------------------------------------------
def remove_padding(x_padded: np.ndarray, lens: Sequence[int]) -> np.ndarray:
    """packed[t] = x[token_src[t]]: the valid rows, sequence by sequence."""
    B, P, H = x_padded.shape
    rows = []
    for b in range(B):
        for p in range(int(lens[b])):
            rows.append(x_padded[b, p])
    if not rows:
        return np.zeros((0, H), dtype=x_padded.dtype)
    return np.stack(rows, axis=0)


def rebuild_padding(packed: np.ndarray, lens: Sequence[int], pad_len: int) -> np.ndarray:
    """Y[b, p] = packed[cu[b] + p] for p < len[b], and +0.0 on every pad."""
    B = len(lens)
    H = packed.shape[1]
    out = np.zeros((B, pad_len, H), dtype=packed.dtype)
    t = 0
    for b in range(B):
        for p in range(int(lens[b])):
            out[b, p] = packed[t]
            t += 1
    assert t == packed.shape[0]
    return out


# ---------------------------------------------------------------------------
# Row operations of the layer.
# ---------------------------------------------------------------------------
def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """Per row: (x - mean) / sqrt(var + eps) * gamma + beta, biased variance.
    LayerNorm appears in the announcement article's "Ease of use" listing
    (add bias + input + LayerNorm); the pre-LN placement is a reading of the pages (GPT-2/3 blocks)."""
    x = np.asarray(x, dtype=_F64)
    H = x.shape[-1]
    mu = x.sum(axis=-1, keepdims=True) / H
    d = x - mu
    var = (d * d).sum(axis=-1, keepdims=True) / H
    return d / np.sqrt(var + eps) * np.asarray(gamma, _F64) + np.asarray(beta, _F64)


def gelu(u: np.ndarray, form: str = "tanh") -> np.ndarray:
    """GELU of the "add bias + activation (GELU)" step in the announcement
    article's "Ease of use" listing.  tanh form:
    0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))); erf form: 0.5 u (1 + erf(u/sqrt 2))."""
    u = np.asarray(u, dtype=_F64)
    if form == "tanh":
        return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u * u * u)))
    if form == "erf":
        from scipy.special import erf
        return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))
    raise ValueError(form)


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x @ W^T + b with W in [out, in] layout (the pages' Linear1D layers are
    PyTorch-like, announcement article "Ease of use")."""
    return np.asarray(x, _F64) @ np.asarray(w, _F64).T + np.asarray(b, _F64)


def _attend_one_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax over the given keys of (q . k_j) * scale, times V.  K, V hold
    exactly the allowed keys; an empty key set gives zeros."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=_F64)
    s = (K @ q) * scale
    m = s.max()
    e = np.exp(s - m)
    return (e @ V) / e.sum()


def _split_qkv(qkv: np.ndarray, n_heads: int, head_dim: int):
    Hp = n_heads * head_dim
    return qkv[:, :Hp], qkv[:, Hp:2 * Hp], qkv[:, 2 * Hp:3 * Hp]


def causal_attention_packed(qkv: np.ndarray, cu: Sequence[int], n_heads: int, head_dim: int) -> np.ndarray:
    """Causal attention run per sequence over the packed offsets: query i of
    sequence b attends to keys cu[b] .. cu[b]+i.  qkv: [T, 3H'] -> o: [T, H']."""
    qkv = np.asarray(qkv, _F64)
    q, k, v = _split_qkv(qkv, n_heads, head_dim)
    T = qkv.shape[0]
    o = np.zeros((T, n_heads * head_dim), dtype=_F64)
    scale = 1.0 / math.sqrt(head_dim)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for n in range(n_heads):
            c = slice(n * head_dim, (n + 1) * head_dim)
            for i in range(s1 - s0):
                o[s0 + i, c] = _attend_one_query(q[s0 + i, c], k[s0:s0 + i + 1, c], v[s0:s0 + i + 1, c], scale)
    return o


def causal_attention_query(qkv_seq: np.ndarray, i: int, n_heads: int, head_dim: int) -> np.ndarray:
    """Output row [H'] of query i of one sequence, given that sequence's packed
    rows qkv_seq [n, 3H'] (n > i): every head attends to keys 0 .. i, the
    keys causal_attention_packed gives query i.  For checking single rows of
    sequences too long to run whole."""
    qkv_seq = np.asarray(qkv_seq, _F64)
    if not 0 <= i < qkv_seq.shape[0]:
        raise ValueError(f"query {i} outside the sequence's {qkv_seq.shape[0]} rows")
    q, k, v = _split_qkv(qkv_seq, n_heads, head_dim)
    scale = 1.0 / math.sqrt(head_dim)
    o = np.zeros(n_heads * head_dim, dtype=_F64)
    for n in range(n_heads):
        c = slice(n * head_dim, (n + 1) * head_dim)
        o[c] = _attend_one_query(q[i, c], k[:i + 1, c], v[:i + 1, c], scale)
    return o


def causal_attention_padded(qkv: np.ndarray, length: int, n_heads: int, head_dim: int) -> np.ndarray:
    """Attention of one padded sequence qkv [P, 3H'] with `length` valid tokens:
    position p attends to the keys J(p) = {j : j <= p and j < length}."""
    qkv = np.asarray(qkv, _F64)
    q, k, v = _split_qkv(qkv, n_heads, head_dim)
    P = qkv.shape[0]
    o = np.zeros((P, n_heads * head_dim), dtype=_F64)
    scale = 1.0 / math.sqrt(head_dim)
    for n in range(n_heads):
        c = slice(n * head_dim, (n + 1) * head_dim)
        for p in range(P):
            jmax = min(p + 1, int(length))
            o[p, c] = _attend_one_query(q[p, c], k[:jmax, c], v[:jmax, c], scale)
    return o


def to_f64_params(params: Dict) -> Dict[str, np.ndarray]:
    """Host float64 copies of a parameter dict (torch tensors or arrays)."""
    out = {}
    for k_, t in params.items():
        if hasattr(t, "detach"):
            t = t.detach().to("cpu").double().numpy()
        out[k_] = np.asarray(t, dtype=_F64)
    return out


def _block(x: np.ndarray, attn_fn, p: Dict[str, np.ndarray], eps: float, gelu_form: str, keep: Dict = None):
    """One pre-LN GPT decoder block on rows x, with the attention given by attn_fn(qkv)."""
    a = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    qkv = linear(a, p["w_qkv"], p["b_qkv"])
    o = attn_fn(qkv)
    h = x + linear(o, p["w_out"], p["b_out"])
    c = layer_norm(h, p["ln2_g"], p["ln2_b"], eps)
    u = linear(c, p["w_fc1"], p["b_fc1"])
    g = gelu(u, gelu_form)
    y = h + linear(g, p["w_fc2"], p["b_fc2"])
    if keep is not None:
        keep.update(a=a, qkv=qkv, o=o, h=h, c=c, u=u, g=g, y=y)
    return y


def layer_forward_packed(x_packed: np.ndarray, cu: Sequence[int], params: Dict, n_heads: int, head_dim: int,
                         eps: float = 1e-5, gelu_form: str = "tanh", keep: Dict = None, attention: str = "varlen",
                         pad_len: int = 0) -> np.ndarray:
    """The RCE form: every row operation on the T packed valid rows; attention
    per sequence over cu ("varlen"), or, in the page-literal form ("padded"),
    through the transposing rebuild, padded attention and transposing remove.
    `keep` (a dict) receives every intermediate."""
    p = to_f64_params(params)
    x = np.asarray(x_packed, _F64)
    if attention == "varlen":
        attn = lambda qkv: causal_attention_packed(qkv, cu, n_heads, head_dim)  # noqa: E731
    else:
        attn = lambda qkv: attention_via_padded_heads(qkv, cu, pad_len, n_heads, head_dim, causal=True)  # noqa: E731
    return _block(x, attn, p, eps, gelu_form, keep)


def layer_forward_padded(x_padded: np.ndarray, lens: Sequence[int], params: Dict, n_heads: int, head_dim: int,
                         eps: float = 1e-5, gelu_form: str = "tanh") -> np.ndarray:
    """The definition: the layer over every padded row of every sequence (pads
    included, as a padded implementation computes them), then pads of the output
    set to +0.0.  Valid rows never read pad rows: attention keys stop at len."""
    p = to_f64_params(params)
    x = np.asarray(x_padded, _F64)
    B, P, H = x.shape
    out = np.zeros((B, P, H), dtype=_F64)
    for b in range(B):
        n = int(lens[b])
        y = _block(x[b], lambda qkv: causal_attention_padded(qkv, n, n_heads, head_dim), p, eps, gelu_form)
        out[b, :n] = y[:n]
    return out


def stack_forward_padded(x_padded, lens, params_list: List[Dict], n_heads: int, head_dim: int,
                         eps: float = 1e-5, gelu_form: str = "tanh") -> np.ndarray:
    """Layers applied in turn to the padded batch; each output (zero pads) is the next input."""
    y = np.asarray(x_padded, _F64)
    for params in params_list:
        y = layer_forward_padded(y, lens, params, n_heads, head_dim, eps, gelu_form)
    return y


def stack_forward_packed(x_padded, lens, params_list: List[Dict], n_heads: int, head_dim: int,
                         eps: float = 1e-5, gelu_form: str = "tanh") -> np.ndarray:
    """remove -> layers on the packed rows -> rebuild."""
    x_padded = np.asarray(x_padded, _F64)
    cu, _, _, _ = offsets_from_lengths(lens, x_padded.shape[1])
    y = remove_padding(x_padded, lens)
    for params in params_list:
        y = layer_forward_packed(y, cu, params, n_heads, head_dim, eps, gelu_form)
    return rebuild_padding(y, lens, x_padded.shape[1])


# ---------------------------------------------------------------------------
# The page-literal form of RCE (announcement article, "Runtime": the
# remove/rebuild ops serve the MLP layers of encoders and decoders), read as:
# attention stays padded.  A transposing rebuild scatters the packed q|k|v rows
# into head-major padded tensors [B, nh, P, hd] (pads zero), attention runs on
# the padded tensors with a key mask, and a transposing remove gathers the
# valid rows back into the packed [T, nh*hd] layout.
# ---------------------------------------------------------------------------
def transpose_padding_rebuild_heads(packed: np.ndarray, lens: Sequence[int], pad_len: int, n_heads: int,
                                    head_dim: int) -> np.ndarray:
    """packed [T, n*nh*hd] (n blocks of nh*hd columns, each head-major) ->
    [n, B, nh, P, hd]: out[m, b, h, p, d] = packed[cu[b]+p, m*nh*hd + h*hd + d]
    for p < len[b], else 0."""
    packed = np.asarray(packed)
    Hp = n_heads * head_dim
    n = packed.shape[1] // Hp
    B = len(lens)
    out = np.zeros((n, B, n_heads, pad_len, head_dim), dtype=packed.dtype)
    t = 0
    for b in range(B):
        for p in range(int(lens[b])):
            for m in range(n):
                for h in range(n_heads):
                    out[m, b, h, p] = packed[t, m * Hp + h * head_dim:m * Hp + (h + 1) * head_dim]
            t += 1
    return out


def transpose_padding_remove_heads(x: np.ndarray, lens: Sequence[int]) -> np.ndarray:
    """[B, nh, P, hd] -> packed [T, nh*hd]: row cu[b]+p holds x[b, h, p, :] for
    every head h, in head order."""
    x = np.asarray(x)
    B, nh, P, hd = x.shape
    rows = []
    for b in range(B):
        for p in range(int(lens[b])):
            rows.append(np.concatenate([x[b, h, p] for h in range(nh)]))
    if not rows:
        return np.zeros((0, nh * hd), dtype=x.dtype)
    return np.stack(rows)


def attention_padded_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, lens: Sequence[int],
                           causal: bool) -> np.ndarray:
    """Attention on padded head-major tensors [B, nh, P, hd]: valid query p of
    sequence b attends to the keys j < len[b] (and j <= p when causal); pad
    query positions give 0."""
    q, k, v = (np.asarray(a, _F64) for a in (q, k, v))
    B, nh, P, hd = q.shape
    o = np.zeros((B, nh, P, hd), dtype=_F64)
    scale = 1.0 / math.sqrt(hd)
    for b in range(B):
        n = int(lens[b])
        for h in range(nh):
            for p in range(n):
                jmax = p + 1 if causal else n
                o[b, h, p] = _attend_one_query(q[b, h, p], k[b, h, :jmax], v[b, h, :jmax], scale)
    return o


def add_bias_residual_layernorm(u: np.ndarray, bias: np.ndarray, residual: np.ndarray, gamma: np.ndarray,
                                beta: np.ndarray, eps: float) -> np.ndarray:
    """LN(u + bias + residual): the add bias + input + LayerNorm step of the
    announcement article's "Ease of use" listing (post-LN blocks)."""
    return layer_norm(np.asarray(u, _F64) + np.asarray(bias, _F64) + np.asarray(residual, _F64), gamma, beta, eps)


def attention_packed_bidirectional(qkv: np.ndarray, cu: Sequence[int], n_heads: int, head_dim: int) -> np.ndarray:
    """Encoder attention per sequence over the packed offsets: every query of
    sequence b attends to all of that sequence's keys (key-padding mask only)."""
    qkv = np.asarray(qkv, _F64)
    q, k, v = _split_qkv(qkv, n_heads, head_dim)
    o = np.zeros((qkv.shape[0], n_heads * head_dim), dtype=_F64)
    scale = 1.0 / math.sqrt(head_dim)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for n in range(n_heads):
            c = slice(n * head_dim, (n + 1) * head_dim)
            for i in range(s1 - s0):
                o[s0 + i, c] = _attend_one_query(q[s0 + i, c], k[s0:s1, c], v[s0:s1, c], scale)
    return o


def attention_via_padded_heads(qkv: np.ndarray, cu: Sequence[int], pad_len: int, n_heads: int, head_dim: int,
                               causal: bool) -> np.ndarray:
    """The page-literal attention on packed qkv: transposing rebuild, padded
    attention, transposing remove."""
    lens = [int(cu[b + 1]) - int(cu[b]) for b in range(len(cu) - 1)]
    heads = transpose_padding_rebuild_heads(np.asarray(qkv, _F64), lens, pad_len, n_heads, head_dim)
    o = attention_padded_heads(heads[0], heads[1], heads[2], lens, causal)
    return transpose_padding_remove_heads(o, lens)


def encoder_layer_forward_packed(x_packed: np.ndarray, cu: Sequence[int], params: Dict, n_heads: int,
                                 head_dim: int, eps: float = 1e-5, gelu_form: str = "erf",
                                 attention: str = "varlen", pad_len: int = 0, keep: Dict = None) -> np.ndarray:
    """Post-LN encoder block (BERT-style; the EnergonAI README lists BERT among
    its models) on the packed rows, with the chain of the "Ease of use" listing:
      h = LN1(x + Out(Attn(QKV(x))))          (add bias + input + LayerNorm)
      y = LN2(h + FC2(gelu(FC1(h))))          (GEMM, add bias + GELU, GEMM, add bias + input + LayerNorm)
    Attention is bidirectional within each sequence.  The parameter names are
    the decoder's: ln1_* is the attention-output LayerNorm, ln2_* the FFN one."""
    p = to_f64_params(params)
    x = np.asarray(x_packed, _F64)
    qkv = linear(x, p["w_qkv"], p["b_qkv"])
    if attention == "varlen":
        o = attention_packed_bidirectional(qkv, cu, n_heads, head_dim)
    else:
        o = attention_via_padded_heads(qkv, cu, pad_len, n_heads, head_dim, causal=False)
    a = o @ p["w_out"].T
    h = add_bias_residual_layernorm(a, p["b_out"], x, p["ln1_g"], p["ln1_b"], eps)
    g = gelu(linear(h, p["w_fc1"], p["b_fc1"]), gelu_form)
    u = g @ p["w_fc2"].T
    y = add_bias_residual_layernorm(u, p["b_fc2"], h, p["ln2_g"], p["ln2_b"], eps)
    if keep is not None:
        keep.update(qkv=qkv, o=o, h=h, g=g, y=y)
    return y


def encoder_layer_forward_padded(x_padded: np.ndarray, lens: Sequence[int], params: Dict, n_heads: int,
                                 head_dim: int, eps: float = 1e-5, gelu_form: str = "erf") -> np.ndarray:
    """The encoder definition on the padded batch: every padded row goes
    through the block, keys masked to the valid ones, pads of the output +0.0."""
    p = to_f64_params(params)
    x = np.asarray(x_padded, _F64)
    B, P, H = x.shape
    out = np.zeros((B, P, H), dtype=_F64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        xb = x[b]
        qkv = linear(xb, p["w_qkv"], p["b_qkv"])
        q, k, v = _split_qkv(qkv, n_heads, head_dim)
        o = np.zeros((P, n_heads * head_dim))
        for hh in range(n_heads):
            c = slice(hh * head_dim, (hh + 1) * head_dim)
            for i in range(P):
                o[i, c] = _attend_one_query(q[i, c], k[:n, c], v[:n, c], 1.0 / math.sqrt(head_dim))
        h = add_bias_residual_layernorm(o @ p["w_out"].T, p["b_out"], xb, p["ln1_g"], p["ln1_b"], eps)
        g = gelu(linear(h, p["w_fc1"], p["b_fc1"]), gelu_form)
        y = add_bias_residual_layernorm(g @ p["w_fc2"].T, p["b_fc2"], h, p["ln2_g"], p["ln2_b"], eps)
        out[b, :n] = y[:n]
    return out
