"""Parity at the full GPT-3-width sizes, in the launch configuration the bench
times (ee_stack_forward over the whole batch), on sampled outputs the CPU
oracle computes one sequence at a time (sequences are independent, so a
sampled sequence's rows are exact rows of the batch), plus properties that
hold at any size.  These tests hold up to ~45 GB of weights in HBM; the
48-layer request stream has a module of its own (test_gpu_stream.py)."""
import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, normwise_rel, say, to_host64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SEED = 1234  # the bench's default seed


def _setup(w, seed, lens, layers, device_batch=None):
    B = len(lens)
    P = w.pad_len if device_batch is None else device_batch
    x = workloads.activations(w, seed, B, P, lens, device=DEV)
    params = [ee.pitched_weights(workloads.layer_params(w, seed, l, device=DEV)) for l in range(layers)]
    hs = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=ee.F16) for p in params]
    return x, params, hs


def _stack(hs, x, lens):
    B, P, _ = x.shape
    ws = torch.empty(hs[0].workspace_size(B, P, sum(lens)), dtype=torch.uint8, device=DEV)
    y = torch.full_like(x, 7.0)
    ee.ee_stack_forward(hs, x, lens, y, ws)
    torch.cuda.synchronize()
    return y


def _pads_zero(y, lens):
    for b, n in enumerate(lens):
        pad = y[b, n:]
        assert torch.all(pad == 0) and not torch.any(torch.signbit(pad)), f"pads of sequence {b}"


def _oracle_rows(w, x, params, lens, picks):
    """The oracle's output rows of the picked sequences through every layer."""
    rows = np.concatenate([x[b, :lens[b]].double().cpu().numpy() for b in picks])
    cu = np.concatenate([[0], np.cumsum([lens[b] for b in picks])])
    for l, p in enumerate(params):
        rows = oracle.layer_forward_packed(rows, cu, p, w.n_heads, w.head_dim)
        say(f"  oracle layer {l + 1}/{len(params)} done")
    return rows, cu


@pytest.mark.timeout(900)
def test_gpt3_12l_stack_sampled_sequences():
    torch.cuda.empty_cache()
    w = workloads.get("gpt3-12l")
    lens = workloads.lengths(w, SEED)
    x, params, hs = _setup(w, SEED, lens, w.layers)
    y = _stack(hs, x, lens)
    _pads_zero(y, lens)
    assert torch.isfinite(y).all()
    picks = [0, len(lens) - 1]
    ref, cu = _oracle_rows(w, x, params, lens, picks)
    for i, b in enumerate(picks):
        err = normwise_rel(to_host64(y[b, :lens[b]]), ref[cu[i]:cu[i + 1]])
        say(f"gpt3-12l sequence {b} (len {lens[b]}) through 12 layers: rel {err:.3e}")
        assert err <= 2e-2


@pytest.mark.timeout(600)
def test_gpt3_tp4_shard_sampled_sequences():
    torch.cuda.empty_cache()
    w = workloads.get("gpt3-tp4-shard")
    lens = workloads.lengths(w, SEED)
    x, params, hs = _setup(w, SEED, lens, 1)
    y = _stack(hs, x, lens)
    _pads_zero(y, lens)
    order = sorted(range(len(lens)), key=lambda b: lens[b])
    picks = sorted({0, len(lens) - 1, order[0], order[-1]})
    ref, cu = _oracle_rows(w, x, params, lens, picks)
    for i, b in enumerate(picks):
        err = normwise_rel(to_host64(y[b, :lens[b]]), ref[cu[i]:cu[i + 1]])
        say(f"gpt3-tp4-shard sequence {b} (len {lens[b]}): rel {err:.3e}")
        assert err <= 2e-2


def test_gpt3_width_decode_sampled():
    """Incremental decoding at GPT-3 width (two layers, 96 heads of 128): a
    prefill of 8 prompts (lengths 1..200), then two decode steps through
    ee_stack_extend; the split-K GEMMs and the cache attention at their real
    shapes.  Sequences 0, 3 and 7 are checked step by step against the oracle's
    incremental forward (fp16 bar 2e-2); every output row is finite."""
    w = workloads.get("gpt3-12l")
    prompts = [1, 57, 128, 200, 3, 96, 33, 150]
    B, L = len(prompts), 2
    params = [ee.pitched_weights(workloads.layer_params(w, SEED, l, device=DEV)) for l in range(L)]
    hs = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=ee.F16) for p in params]
    base = list(np.concatenate([[0], np.cumsum([n + 2 for n in prompts])[:-1]]).astype(int))
    cap = sum(n + 2 for n in prompts)
    cache = torch.empty(ee.ee_kv_cache_bytes(hs[0], L, cap), dtype=torch.uint8, device=DEV)
    ws = torch.empty(ee.ee_extend_workspace_size(hs[0], B, sum(prompts)), dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(99)
    rows = [(torch.randn(n + 2, w.hidden, generator=g, device=DEV)).half() for n in prompts]
    p64 = [oracle.to_f64_params({k: v.cpu() for k, v in p.items()}) for p in params]
    picks = (0, 3, 7)
    ocache = {b: oracle.SequenceCache(L, w.n_heads, w.head_dim) for b in picks}
    ctx = [0] * B
    for step, new in enumerate([prompts, [1] * B, [1] * B]):
        x = torch.cat([rows[b][ctx[b]:ctx[b] + n] for b, n in enumerate(new)])
        y = torch.empty_like(x)
        ee.ee_stack_extend(hs, x, new, ctx, base, cache, cap, y, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        r = 0
        for b, n in enumerate(new):
            if b in picks:
                ref = oracle.extend_sequence(ocache[b], rows[b][ctx[b]:ctx[b] + n].double().cpu().numpy(), p64,
                                             w.n_heads, w.head_dim)
                err = normwise_rel(to_host64(y[r:r + n]), ref)
                say(f"gpt3 width decode step {step} sequence {b} ({n} new after {ctx[b]}): rel {err:.3e}")
                assert err <= 2e-2
            r += n
        ctx = [c + n for c, n in zip(ctx, new)]


@pytest.mark.parametrize("B", [72, 128])
def test_gpt3_width_decode_wide_batch(B):
    """Decode steps of more than 32 sequences at GPT-3 width (two layers): the
    stream-K GEMMs with their 128-row A tile (72 rows ragged, and 128 full)
    inside ee_stack_extend.  A prefill of short prompts (lengths 1..12), then
    two decode steps; sequences 0, B/2 and B-1 are checked step by step against
    the oracle's incremental forward (fp16 bar 2e-2); every output row is
    finite."""
    w = workloads.get("gpt3-12l")
    g = torch.Generator().manual_seed(B)
    prompts = torch.randint(1, 13, (B,), generator=g).tolist()
    L = 2
    params = [ee.pitched_weights(workloads.layer_params(w, SEED, l, device=DEV)) for l in range(L)]
    hs = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=ee.F16) for p in params]
    base = list(np.concatenate([[0], np.cumsum([n + 2 for n in prompts])[:-1]]).astype(int))
    cap = sum(n + 2 for n in prompts)
    cache = torch.empty(ee.ee_kv_cache_bytes(hs[0], L, cap), dtype=torch.uint8, device=DEV)
    ws = torch.empty(ee.ee_extend_workspace_size(hs[0], B, sum(prompts)), dtype=torch.uint8, device=DEV)
    gd = torch.Generator(device=DEV).manual_seed(100 + B)
    rows = [(torch.randn(n + 2, w.hidden, generator=gd, device=DEV)).half() for n in prompts]
    p64 = [oracle.to_f64_params({k: v.cpu() for k, v in p.items()}) for p in params]
    picks = (0, B // 2, B - 1)
    ocache = {b: oracle.SequenceCache(L, w.n_heads, w.head_dim) for b in picks}
    ctx = [0] * B
    for step, new in enumerate([prompts, [1] * B, [1] * B]):
        x = torch.cat([rows[b][ctx[b]:ctx[b] + n] for b, n in enumerate(new)])
        y = torch.empty_like(x)
        ee.ee_stack_extend(hs, x, new, ctx, base, cache, cap, y, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        r = 0
        for b, n in enumerate(new):
            if b in picks:
                ref = oracle.extend_sequence(ocache[b], rows[b][ctx[b]:ctx[b] + n].double().cpu().numpy(), p64,
                                             w.n_heads, w.head_dim)
                err = normwise_rel(to_host64(y[r:r + n]), ref)
                say(f"gpt3 width decode B={B} step {step} sequence {b} ({n} new after {ctx[b]}): rel {err:.3e}")
                assert err <= 2e-2
            r += n
        ctx = [c + n for c, n in zip(ctx, new)]
