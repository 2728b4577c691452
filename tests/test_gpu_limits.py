"""The ABI's size limits, on the GPU, against the oracle.

- The layer at the largest batch (EE_MAX_BATCH = 512 sequences, the lengths
  travel as a by-value kernel argument): fp32 and fp16, ragged lengths
  including empty sequences, pads +0.0.
- One extend step at the largest batch (EE_MAX_EXTEND_BATCH = 256 sequences):
  a prefill of ragged prompts, then a decode step with a token for every
  sequence, checked step by step.
- Extend steps over long contexts after a GPU prefill: past 32768 positions
  (GPT-2-small width, 79 key chunks merged by the second kernel; a decode
  step, then a mixed step of several new tokens) and 2000 positions at GPT-3
  width (96 heads of 128).
- Causal attention at GPT-3 width (96 heads of 128) over a sequence whose
  QKV rows span more than 2^31 bytes, then one that starts past that point:
  sampled queries and heads against the oracle's single-query form.
Bars: fp16 <= 2e-2, fp32 <= 1e-4 normwise (attention: fp16 <= 3e-3); pads
exactly +0.0."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, normwise_rel, say, to_host64, valid_mask
from test_gpu_decode import Decoder, _token_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,P,tol", [("tiny-fp32", 16, 1e-4), ("gpt2-small", 8, 2e-2)])
def test_layer_at_max_batch(name, P, tol):
    assert ee.MAX_BATCH == 512
    w = dataclasses.replace(workloads.get(name), batch=ee.MAX_BATCH, pad_len=P)
    g = torch.Generator().manual_seed(512)
    lens = torch.randint(0, P + 1, (w.batch,), generator=g).tolist()   # zeros included
    lens[0], lens[-1] = 0, P
    x = workloads.activations(w, 9, w.batch, P, lens)
    p = workloads.layer_params(w, 9, 0, variant="affine")
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    layer = ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, {k: v.to(DEV) for k, v in p.items()}, dtype=dt)
    ws = torch.empty(layer.workspace_size(w.batch, P, sum(lens)), dtype=torch.uint8, device=DEV)
    xd = x.to(DEV)
    y = torch.full_like(xd, 9.0)
    layer.forward(xd, lens, y, ws)
    torch.cuda.synchronize()
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim)
    got = to_host64(y)
    m = valid_mask(lens, P)
    err = normwise_rel(got[m], ref[m])
    say(f"{name} layer at B={w.batch}, T={sum(lens)}: rel {err:.3e}")
    assert np.all(got[~m] == 0) and not np.any(np.signbit(got[~m]))
    assert err <= tol


@pytest.mark.parametrize("name,tol", [("tiny-fp32", 1e-4), ("gpt2-small", 2e-2)])
def test_extend_at_max_batch(name, tol):
    assert ee.MAX_EXTEND_BATCH == 256
    w = workloads.get(name)
    B = ee.MAX_EXTEND_BATCH
    g = torch.Generator().manual_seed(256)
    prompts = torch.randint(1, 9, (B,), generator=g).tolist()
    # a prefill, a decode step, then 0-3 new tokens per sequence: with 256
    # sequences that last step fills the GPU on the MFMA kernel
    third = [b % 4 for b in range(B)]
    dec = Decoder(w, 88, 1, prompts, max_new=4)
    rows_all = [_token_rows(w, 700 + b, prompts[b] + 4) for b in range(B)]
    pos = [0] * B
    for k, new_len in enumerate([prompts, [1] * B, third]):
        rows = torch.cat([rows_all[b][pos[b]:pos[b] + n] for b, n in enumerate(new_len)])
        pos = [p + n for p, n in zip(pos, new_len)]
        got, ref = dec.step(rows, new_len)
        err = normwise_rel(got, ref)
        say(f"{name} extend at B={B}, step {k} (T={sum(new_len)}): rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= tol


def test_attention_rows_past_2gib():
    """A 29200-token sequence at 96 heads of 128: its QKV rows span 2.15 GB, so
    byte offsets within the sequence pass 2^31.  The second sequence starts
    2.15 GB into the buffer.  Sampled queries of three heads against the
    oracle (heads are independent, so the oracle gets those heads only)."""
    nh, hd = 96, 128
    Hp = nh * hd
    lens = [29200, 100]
    assert lens[0] * 3 * Hp * 2 >= 2 ** 31
    T = sum(lens)
    cu_h = np.array([0, lens[0], T], dtype=np.int32)
    g = torch.Generator(device=DEV).manual_seed(2031)
    qkv = torch.randn(T, 3 * Hp, device=DEV, generator=g, dtype=torch.float16)
    o = torch.full((T, Hp), 7.0, dtype=torch.float16, device=DEV)
    say(f"attention past 2 GiB: lens {lens}, qkv {qkv.numel() * 2 / 1e9:.2f} GB")
    ee.ee_attention_varlen(qkv, torch.tensor(cu_h, device=DEV), len(lens), max(lens), nh, hd, o)
    torch.cuda.synchronize()
    heads = [0, 47, 95]
    head_cols = np.concatenate([np.arange(h * hd, (h + 1) * hd) for h in heads])
    cols = torch.tensor(np.concatenate([m * Hp + head_cols for m in range(3)]), device=DEV)
    got, ref = [], []
    for b, queries in ((0, [0, 1, 127, 128, 12345, 29199]), (1, [0, 57, 99])):
        s0, s1 = int(cu_h[b]), int(cu_h[b + 1])
        sub = qkv[s0:s1].index_select(1, cols).double().cpu().numpy()  # q | k | v of the three heads
        for i in queries:
            ref.append(oracle.causal_attention_query(sub[:i + 1], i, len(heads), hd))
            got.append(o[s0 + i].double().cpu().numpy()[head_cols])
    err = normwise_rel(np.stack(got), np.stack(ref))
    say(f"attention past 2 GiB: {len(got)} sampled rows x {len(heads)} heads, rel {err:.2e}")
    assert err <= 3e-3


@pytest.mark.parametrize("name,prompts,steps", [
    # past 32768 positions: 79 key chunks, a mixed step, then 200 and 17 new
    # tokens on the MFMA kernel over the 40k cached keys
    ("gpt2-small", [40000, 5], [[1, 1], [3, 2], [200, 17]]),
    # GPT-3 width (96 heads of 128): 4 key chunks, then 130, 20 and 0 new
    # tokens on the MFMA kernel
    ("gpt3-12l", [2000, 1, 700], [[1, 1, 1], [130, 20, 0]]),
])
def test_decode_long_context(name, prompts, steps):
    """One layer: long prompts prefilled on the GPU, then extend steps over the
    long cache.  The cache attention splits the keys into chunks whose softmax
    states a second kernel merges; steps with 16 or more new tokens in a
    sequence run on the MFMA kernel instead.  The oracle's cache of a long prompt is its
    first layer's keys and values (no attention over the prompt is needed for
    them); every step's outputs and both caches are checked against it."""
    w = workloads.get(name)
    dec = Decoder(w, 77, 1, prompts, max_new=sum(s[0] for s in steps) + 3)
    B = len(prompts)
    extra = [sum(s[b] for s in steps) for b in range(B)]
    rows = [_token_rows(w, 900 + b, prompts[b] + extra[b]) for b in range(B)]
    x = torch.cat([rows[b][:prompts[b]] for b in range(B)]).to(DEV)
    y = torch.empty_like(x)
    ws = torch.empty(ee.ee_extend_workspace_size(dec.layers[0], B, x.shape[0]), dtype=torch.uint8, device=DEV)
    say(f"{name} long context: prefill {prompts}")
    ee.ee_stack_extend(dec.layers, x, prompts, [0] * B, dec.slot_base, dec.cache, dec.capacity, y, ws)
    torch.cuda.synchronize()
    for b in range(B):
        oracle.prefill_first_layer_cache(dec.ocaches[b], rows[b][:prompts[b]].double().numpy(), dec.params[0],
                                         w.n_heads, w.head_dim)
    dec.ctx = list(prompts)
    pos = list(prompts)
    for new in steps:
        toks = torch.cat([rows[b][pos[b]:pos[b] + new[b]] for b in range(B)])
        got, ref = dec.step(toks, new)
        err = normwise_rel(got, ref)
        say(f"{name}: step of {new} new tokens after {pos} positions: rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= 2e-2
        pos = [p + n for p, n in zip(pos, new)]
    assert dec.ctx == pos and max(pos) > (32768 if name == "gpt2-small" else 2000)
    cv = dec.cache_view()
    for b in range(B):
        n, s0 = dec.ctx[b], dec.slot_base[b]
        k = cv[0, 0, :, s0:s0 + n].double().cpu().numpy()
        v = cv[0, 1, :, s0:s0 + n].double().cpu().numpy()
        assert normwise_rel(k, dec.ocaches[b].k[0]) <= 2e-3 and normwise_rel(v, dec.ocaches[b].v[0]) <= 2e-3
    assert ee.ee_extend_max_positions() == 2 ** 31 - 1
