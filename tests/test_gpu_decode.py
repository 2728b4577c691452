"""Incremental decoding through the C ABI (ee_stack_extend) against the
oracle: a prefill, decode steps and a mixed step (several new tokens for some
sequences, none for others), step by step; the KV cache contents; the prefill
against the padded-batch forward; a decode step against the full forward.
Bars: fp16 <= 2e-2, fp32 <= 1e-4 (layer outputs); cache fp16 <= 2e-3,
fp32 <= 1e-5; slots no sequence owns keep their bytes."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, normwise_rel, say, to_host64

pytestmark = pytest.mark.gpu


class Decoder:
    def __init__(self, w, seed, n_layers, prompts, max_new, residual=ee.RESIDUAL_AUTO):
        self.w = w
        dt = ee.F16 if w.dtype == "f16" else ee.F32
        self.params = [workloads.layer_params(w, seed, l, variant="affine") for l in range(n_layers)]
        self.layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, {k: v.to(DEV) for k, v in p.items()},
                                dtype=dt, residual=residual) for p in self.params]
        caps = [n + max_new for n in prompts]
        self.slot_base = list(np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(int))
        self.capacity = int(sum(caps)) + 7                      # a few slots nobody owns
        nbytes = ee.ee_kv_cache_bytes(self.layers[0], n_layers, self.capacity)
        self.cache = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN sentinel
        self.ctx = [0] * len(prompts)
        self.ocaches = [oracle.SequenceCache(n_layers, w.n_heads, w.head_dim) for _ in prompts]
        self.p64 = [oracle.to_f64_params(p) for p in self.params]

    def step(self, rows, new_len):
        w = self.w
        T = sum(new_len)
        x = rows.to(DEV)
        y = torch.full_like(x, 7.0)
        ws = torch.empty(ee.ee_extend_workspace_size(self.layers[0], len(new_len), T), dtype=torch.uint8,
                         device=DEV)
        ee.ee_stack_extend(self.layers, x, new_len, self.ctx, self.slot_base, self.cache, self.capacity, y, ws)
        torch.cuda.synchronize()
        ref = oracle.extend_batch(self.ocaches, rows.double().numpy(), new_len, self.p64, w.n_heads, w.head_dim)
        self.ctx = [c + n for c, n in zip(self.ctx, new_len)]
        return to_host64(y), ref

    def cache_view(self):
        w = self.w
        tdt = torch.float16 if w.dtype == "f16" else torch.float32
        L = len(self.layers)
        return self.cache.view(tdt).view(L, 2, w.n_heads, self.capacity, w.head_dim)


def _token_rows(w, seed, n_tokens):
    g = torch.Generator().manual_seed(seed)
    return (w.x_std * torch.randn(n_tokens, w.hidden, generator=g)).to(w.torch_dtype)


@pytest.mark.parametrize("name,tol,ctol", [("gpt2-small", 2e-2, 2e-3), ("tiny-fp32", 1e-4, 1e-5)])
def test_prefill_decode_and_mixed_steps(name, tol, ctol):
    w = workloads.get(name)
    prompts = [1, 37, 128, 64, 5] if w.pad_len >= 128 else [1, 9, 16, 4, 2]
    dec = Decoder(w, 41, 2, prompts, max_new=8)
    rows_all = [_token_rows(w, 100 + b, prompts[b] + 8) for b in range(len(prompts))]
    pos = [0] * len(prompts)
    plan = [prompts, [1] * 5, [1] * 5, [1] * 5, [0, 3, 1, 0, 2]]
    for k, new_len in enumerate(plan):
        rows = torch.cat([rows_all[b][pos[b]:pos[b] + n] for b, n in enumerate(new_len)])
        got, ref = dec.step(rows, new_len)
        err = normwise_rel(got, ref)
        say(f"{name} step {k} new={new_len}: rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= tol
        pos = [p + n for p, n in zip(pos, new_len)]
    cv = dec.cache_view()
    for b in range(len(prompts)):
        n, s0 = dec.ctx[b], dec.slot_base[b]
        for l in range(2):
            k = cv[l, 0, :, s0:s0 + n].double().cpu().numpy()
            v = cv[l, 1, :, s0:s0 + n].double().cpu().numpy()
            assert normwise_rel(k, dec.ocaches[b].k[l]) <= ctol and normwise_rel(v, dec.ocaches[b].v[l]) <= ctol
    # slots past each sequence's used range and the unowned tail are untouched
    used = torch.zeros(dec.capacity, dtype=torch.bool)
    for b in range(len(prompts)):
        used[dec.slot_base[b]:dec.slot_base[b] + dec.ctx[b]] = True
    tail = cv[:, :, :, ~used.to(DEV)]
    assert torch.all(tail.view(torch.uint8) == 0xFF)


def test_chunked_extend_steps():
    """Extend steps with many new tokens per sequence after cached ones (a
    chunked prefill): from 16 new tokens in some sequence on, the attention
    runs on the MFMA kernel over the cached keys.  Steps of up to 200 new
    tokens (two 128-query tiles), a sequence with no cache yet beside cached
    ones, an empty one, and one new token beside 16 and 20; then a decode
    step on the cache-attention kernel.  Each step against the oracle, and the
    cache after them."""
    w = workloads.get("gpt2-small")
    prompts = [40, 130, 0, 129, 17]
    plan = [prompts, [17, 200, 33, 130, 0], [1, 16, 0, 3, 20], [1] * 5]
    extra = [sum(st[b] for st in plan[1:]) for b in range(len(prompts))]
    dec = Decoder(w, 44, 2, prompts, max_new=max(extra))
    rows_all = [_token_rows(w, 500 + b, prompts[b] + extra[b]) for b in range(len(prompts))]
    pos = [0] * len(prompts)
    for k, new_len in enumerate(plan):
        rows = torch.cat([rows_all[b][pos[b]:pos[b] + n] for b, n in enumerate(new_len)])
        got, ref = dec.step(rows, new_len)
        err = normwise_rel(got, ref)
        say(f"chunked step {k} new={new_len} after {pos}: rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= 2e-2
        pos = [p + n for p, n in zip(pos, new_len)]
    cv = dec.cache_view()
    for b in range(len(prompts)):
        n, s0 = dec.ctx[b], dec.slot_base[b]
        for l in range(2):
            k = cv[l, 0, :, s0:s0 + n].double().cpu().numpy()
            v = cv[l, 1, :, s0:s0 + n].double().cpu().numpy()
            assert normwise_rel(k, dec.ocaches[b].k[l]) <= 2e-3 and normwise_rel(v, dec.ocaches[b].v[l]) <= 2e-3


@pytest.mark.parametrize("residual", [ee.RESIDUAL_EPILOGUE, ee.RESIDUAL_PASS])
def test_prefill_equals_padded_forward_bit_exact(residual):
    w = workloads.get("gpt2-small")
    prompts = [17, 128, 1, 90]
    dec = Decoder(w, 42, 2, prompts, max_new=0, residual=residual)
    rows = [_token_rows(w, 200 + b, n) for b, n in enumerate(prompts)]
    x = torch.cat(rows).to(DEV)
    y = torch.empty_like(x)
    ws = torch.empty(ee.ee_extend_workspace_size(dec.layers[0], 4, x.shape[0]), dtype=torch.uint8, device=DEV)
    ee.ee_stack_extend(dec.layers, x, prompts, [0] * 4, dec.slot_base, dec.cache, dec.capacity, y, ws)
    xp = workloads.pad_batch(rows, 128).to(DEV)
    yp = torch.empty_like(xp)
    ws2 = torch.empty(dec.layers[0].workspace_size(4, 128), dtype=torch.uint8, device=DEV)
    ee.ee_stack_forward(dec.layers, xp, prompts, yp, ws2)
    torch.cuda.synchronize()
    packed = torch.cat([yp[b, :n] for b, n in enumerate(prompts)])
    assert torch.equal(y, packed)


def test_decode_step_matches_full_forward():
    w = workloads.get("gpt2-small")
    prompts = [33, 100, 7]
    dec = Decoder(w, 43, 2, prompts, max_new=1)
    rows = [_token_rows(w, 300 + b, n + 1) for b, n in enumerate(prompts)]
    x = torch.cat([r[:-1] for r in rows]).to(DEV)
    y = torch.empty_like(x)
    ws = torch.empty(ee.ee_extend_workspace_size(dec.layers[0], 3, x.shape[0]), dtype=torch.uint8, device=DEV)
    ee.ee_stack_extend(dec.layers, x, prompts, [0] * 3, dec.slot_base, dec.cache, dec.capacity, y, ws)
    xd = torch.cat([r[-1:] for r in rows]).to(DEV)
    yd = torch.empty_like(xd)
    ee.ee_stack_extend(dec.layers, xd, [1] * 3, prompts, dec.slot_base, dec.cache, dec.capacity, yd, ws)
    lens = [n + 1 for n in prompts]
    xp = workloads.pad_batch(rows).to(DEV)
    yp = torch.empty_like(xp)
    ws2 = torch.empty(dec.layers[0].workspace_size(3, xp.shape[1]), dtype=torch.uint8, device=DEV)
    ee.ee_stack_forward(dec.layers, xp, lens, yp, ws2)
    torch.cuda.synchronize()
    last = torch.stack([yp[b, n - 1] for b, n in enumerate(lens)])
    err = normwise_rel(to_host64(yd), to_host64(last))
    say(f"decode step vs full forward: rel {err:.3e}")
    assert err <= 1e-2
