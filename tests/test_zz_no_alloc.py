"""ee_stack_extend_noalloc (the extend step for callers that cannot allocate)
against ee_stack_extend with a caller workspace, through the C ABI: two
calls in a row on each, the second with fewer new tokens, and the outputs and
KV caches compared bit for bit (the same kernels run on the same inputs; only
where the workspace lives differs).  At GPT-2-small width, and at GPT-3 width
where the decode step's GEMMs keep their stream-K partial sums in the static
buffer.  A step too large for the buffer is rejected before any device work."""
import numpy as np
import pytest
import torch

import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def _pair(w, n_layers, prompts, steps, seed):
    params = [ee.pitched_weights(workloads.layer_params(w, seed, l, device=DEV, variant="affine"))
              for l in range(n_layers)]
    layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=ee.F16) for p in params]
    extra = sum(max(s[b] for s in steps) for b in range(len(prompts))) * len(steps)
    caps = [n + len(steps) * max(s[b] for s in steps) for b, n in enumerate(prompts)]
    base = [int(v) for v in np.concatenate([[0], np.cumsum(caps)[:-1]])]
    cap = int(sum(caps)) + extra
    nbytes = ee.ee_kv_cache_bytes(layers[0], n_layers, cap)
    cache_ws = torch.full((nbytes,), 0x3C, dtype=torch.uint8, device=DEV)
    cache_na = cache_ws.clone()
    g = torch.Generator(device=DEV).manual_seed(seed)
    ctx = [0] * len(prompts)
    for i, new in enumerate([prompts] + steps):
        T = sum(new)
        x = torch.randn(T, w.hidden, generator=g, device=DEV).half()
        y_ws = torch.full_like(x, 7.0)
        y_na = torch.full_like(x, 5.0)
        ws = torch.empty(ee.ee_extend_workspace_size(layers[0], len(new), T), dtype=torch.uint8, device=DEV)
        ee.ee_stack_extend(layers, x, new, ctx, base, cache_ws, cap, y_ws, ws)
        ee.ee_stack_extend_noalloc(layers, x, new, ctx, base, cache_na, cap, y_na)
        torch.cuda.synchronize()
        same_y = torch.equal(y_ws, y_na)
        same_cache = torch.equal(cache_ws, cache_na)
        say(f"{w.name} call {i}: {T} new tokens over {len(new)} sequences: output identical {same_y}, "
            f"cache identical {same_cache}, finite {bool(torch.isfinite(y_na).all())}")
        assert same_y and same_cache and torch.isfinite(y_na).all()
        ctx = [c + n for c, n in zip(ctx, new)]
        del ws


def test_noalloc_matches_workspace_gpt2_small():
    w = workloads.get("gpt2-small")
    prompts = [5, 17, 1, 64, 33, 2, 9, 40]
    # second call smaller than the first: a decode step of one token for some sequences
    _pair(w, 2, prompts, [[1, 0, 1, 1, 0, 1, 0, 1]], seed=71)


def test_noalloc_matches_workspace_gpt3_width():
    w = workloads.get("gpt3-12l")
    prompts = [3, 11, 7, 1, 20, 5, 9, 2]
    _pair(w, 2, prompts, [[1] * 8], seed=72)


def test_noalloc_rejects_a_step_above_the_buffer():
    w = workloads.get("gpt3-12l")
    params = ee.pitched_weights(workloads.layer_params(w, 1234, 0, device=DEV))
    layer = ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, params, dtype=ee.F16)
    T = 1000
    assert ee.ee_extend_workspace_size(layer, 1, T) > ee.NOALLOC_SCRATCH_BYTES
    cache = torch.zeros(ee.ee_kv_cache_bytes(layer, 1, T), dtype=torch.uint8, device=DEV)
    x = torch.zeros(T, w.hidden, dtype=torch.float16, device=DEV)
    y = torch.full_like(x, 3.0)
    with pytest.raises(ee.EEError) as e:
        ee.ee_stack_extend_noalloc([layer], x, [T], [0], [0], cache, T, y)
    torch.cuda.synchronize()
    assert e.value.status == 3 and "no-allocation" in str(e.value)
    assert bool((y == 3.0).all())            # nothing ran
