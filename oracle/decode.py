"""Oracle of incremental decoding with a KV cache (test infrastructure only;
see the package docstring).

Generation (the README's "Latency" section, a GPT-3 text-generation service;
the EET page's decoder-layer figures): each new token of a sequence attends,
in every layer, to all earlier tokens of its sequence.  An implementation
keeps each layer's keys and values of the earlier tokens (the cache) and
computes only the new tokens.  The result must be the causal forward of the
whole sequence, read at the new positions; the pins check exactly that.

Written step by step with an explicit cache, one query at a time, in float64,
from the oracle's LayerNorm, linear and GeLU.  Cache layout per layer and
sequence: k, v [n_heads, positions, head_dim].
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np

from .layer import gelu, layer_norm, linear, to_f64_params

_F64 = np.float64


class SequenceCache:
    """Keys and values of the tokens seen so far, per layer."""

    def __init__(self, n_layers: int, n_heads: int, head_dim: int):
        self.k = [np.zeros((n_heads, 0, head_dim), _F64) for _ in range(n_layers)]
        self.v = [np.zeros((n_heads, 0, head_dim), _F64) for _ in range(n_layers)]

    @property
    def length(self) -> int:
        return self.k[0].shape[1]


def _heads(rows: np.ndarray, n_heads: int, head_dim: int) -> np.ndarray:
    """[n, n_heads*head_dim] -> [n_heads, n, head_dim]"""
    return rows.reshape(rows.shape[0], n_heads, head_dim).transpose(1, 0, 2)


def extend_sequence(cache: SequenceCache, x_new: np.ndarray, params_list: List[Dict], n_heads: int, head_dim: int,
                    eps: float = 1e-5, gelu_form: str = "tanh") -> np.ndarray:
    """Runs the pre-LN decoder stack on the new tokens x_new [n, hidden] of one
    sequence, appending each layer's new keys and values to `cache`; returns
    the stack output of the new tokens [n, hidden]."""
    x = np.asarray(x_new, _F64)
    n = x.shape[0]
    Hp = n_heads * head_dim
    scale = 1.0 / math.sqrt(head_dim)
    start = cache.length
    for l, params in enumerate(params_list):
        p = to_f64_params(params)
        a = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
        qkv = linear(a, p["w_qkv"], p["b_qkv"])
        q = _heads(qkv[:, :Hp], n_heads, head_dim)
        cache.k[l] = np.concatenate([cache.k[l], _heads(qkv[:, Hp:2 * Hp], n_heads, head_dim)], axis=1)
        cache.v[l] = np.concatenate([cache.v[l], _heads(qkv[:, 2 * Hp:], n_heads, head_dim)], axis=1)
        o = np.zeros((n, Hp), _F64)
        for i in range(n):
            pos = start + i                      # keys 0..pos: the earlier tokens and this one
            for h in range(n_heads):
                s = cache.k[l][h, :pos + 1] @ q[h, i] * scale
                e = np.exp(s - s.max())
                o[i, h * head_dim:(h + 1) * head_dim] = (e / e.sum()) @ cache.v[l][h, :pos + 1]
        hres = x + linear(o, p["w_out"], p["b_out"])
        c = layer_norm(hres, p["ln2_g"], p["ln2_b"], eps)
        x = hres + linear(gelu(linear(c, p["w_fc1"], p["b_fc1"]), gelu_form), p["w_fc2"], p["b_fc2"])
    return x


def prefill_first_layer_cache(cache: SequenceCache, x_new: np.ndarray, params: Dict, n_heads: int, head_dim: int,
                              eps: float = 1e-5) -> None:
    """Appends the first layer's keys and values of the new tokens x_new
    [n, hidden] to a one-layer cache, without computing the tokens' outputs.
    The first layer's keys and values depend on its inputs only (LayerNorm,
    then the QKV projection), so this is the cache extend_sequence leaves,
    for prompts too long to run the oracle's attention over every token."""
    if len(cache.k) != 1:
        raise ValueError("only a one-layer cache can be filled without the layer outputs")
    p = to_f64_params(params)
    Hp = n_heads * head_dim
    qkv = linear(layer_norm(np.asarray(x_new, _F64), p["ln1_g"], p["ln1_b"], eps), p["w_qkv"], p["b_qkv"])
    cache.k[0] = np.concatenate([cache.k[0], _heads(qkv[:, Hp:2 * Hp], n_heads, head_dim)], axis=1)
    cache.v[0] = np.concatenate([cache.v[0], _heads(qkv[:, 2 * Hp:], n_heads, head_dim)], axis=1)


def extend_batch(caches: List[SequenceCache], x_packed: np.ndarray, new_len: Sequence[int], params_list: List[Dict],
                 n_heads: int, head_dim: int, eps: float = 1e-5, gelu_form: str = "tanh") -> np.ndarray:
    """One extend step of a batch: x_packed [sum new_len, hidden], sequence by
    sequence; returns the outputs in the same packing."""
    out = np.zeros(np.asarray(x_packed).shape, _F64)
    r = 0
    for b, n in enumerate(new_len):
        if n:
            out[r:r + n] = extend_sequence(caches[b], np.asarray(x_packed)[r:r + n], params_list, n_heads, head_dim,
                                           eps, gelu_form)
        r += n
    return out
