"""The variable-length request stream through the 48-layer GPT-3-width stack
(174 GB of weights), in the launch configuration the bench times: FIFO batches
of 64 requests, each padded to its own longest request (Energon-AI
announcement article, "Performance tests"; EnergonAI README, "Latency" with 48
layers and "Batching"), one ee_stack_forward call per batch.

Parity against the CPU oracle on sampled sequences (sequences are
independent, so a sampled sequence's rows are exact rows of the batch):
  * the shortest and longest sequence of the first and the last FIFO batch
    through all 48 layers, end to end (no teacher forcing);
  * the same sequences teacher-forced at layers 0, 24 and 47: the oracle runs
    that one layer on the GPU's own input to it.
The first batch (T = 8125) runs every GEMM as one launch; the last (T = 8457)
runs each GEMM as whole rounds of 256 x 256 tiles plus the remaining rows on
smaller tiles.

Properties that hold at any size: pads +0.0, finite outputs, a stack split
into two calls equals the whole stack bit for bit, each sampled sequence run
alone equals its rows of the batch bit for bit, and a batch of the dynamic
plan gives every request the rows it got in its FIFO batch, bit for bit (the
announcement article, "Serving": batches are re-packed by the scheduler, and a
request's result must not depend on its batch).
"""
import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, normwise_rel, say, to_host64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SEED = 1234  # the bench's default seed
TEACHER = (0, 24, 47)


@pytest.fixture(scope="module")
def stack48():
    torch.cuda.empty_cache()
    w = workloads.get("gpt3-48l-stream")
    lens = [n for g in workloads.request_stream(w, SEED) for n in g]
    params = []
    for l in range(w.layers):
        params.append(ee.pitched_weights(workloads.layer_params(w, SEED, l, device=DEV)))
    hs = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=ee.F16) for p in params]
    reqs = workloads.request_activations(w, SEED, lens, device=DEV)
    fifo = ee.batches_of(ee.ee_plan_fifo(lens, w.batch))
    torch.cuda.synchronize()
    say(f"gpt3-48l-stream: {len(lens)} requests, {len(fifo)} FIFO batches, weights resident")
    yield w, lens, params, hs, reqs, fifo
    del hs, params, reqs
    torch.cuda.empty_cache()


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


def _rows(t, b, n):
    return to_host64(t[b, :n])


@pytest.mark.timeout(1200)
def test_stream_batches_against_oracle(stack48):
    """First and last FIFO batch; shortest and longest sequence of each against
    the float64 oracle: end to end through 48 layers, and teacher-forced at
    layers 0, 24 and 47 (normwise relative error <= 2e-2, the fp16 bar)."""
    w, lens, params, hs, reqs, fifo = stack48
    L = w.layers
    picks = []          # (batch index, sequence index in it, length)
    gpu_in, gpu_out, gpu_y, x_rows = {}, {}, {}, {}
    for gi in (0, len(fifo) - 1):
        bl = [lens[i] for i in fifo[gi]]
        x = workloads.pad_batch([reqs[i] for i in fifo[gi]])
        say(f"batch {gi}: T={sum(bl)}, P={x.shape[1]}")
        y = _stack(hs, x, bl)
        _pads_zero(y, bl)
        assert torch.isfinite(y).all()
        order = sorted(range(len(bl)), key=lambda b: bl[b])
        sel = (order[0], order[-1])
        # the GPU's input to each teacher-forced layer, and that layer's output
        inputs = {0: x}
        for l in TEACHER[1:]:
            inputs[l] = _stack(hs[:l], x, bl)
        outs = {l: _stack(hs[l:l + 1], inputs[l], bl) for l in TEACHER}
        # the stack split in two (47 layers, then the last) is the whole stack, bit for bit
        assert torch.equal(outs[L - 1], y), "stack of 47 + 1 layers differs from the 48-layer stack"
        for b in sel:
            n = bl[b]
            picks.append((gi, b, n))
            x_rows[(gi, b)] = _rows(x, b, n)
            gpu_y[(gi, b)] = _rows(y, b, n)
            for l in TEACHER:
                gpu_in[(gi, b, l)] = _rows(inputs[l], b, n)
                gpu_out[(gi, b, l)] = _rows(outs[l], b, n)
        del inputs, outs, y, x
        torch.cuda.synchronize()
    # the oracle, one layer at a time over every picked sequence (end to end),
    # plus the teacher-forced layers on the GPU's inputs
    cu = np.concatenate([[0], np.cumsum([n for _, _, n in picks])])
    rows = np.concatenate([x_rows[(gi, b)] for gi, b, _ in picks])
    for l in range(L):
        p64 = oracle.to_f64_params({k: v.detach().cpu() for k, v in params[l].items()})
        rows = oracle.layer_forward_packed(rows, cu, p64, w.n_heads, w.head_dim)
        if l in TEACHER:
            tin = np.concatenate([gpu_in[(gi, b, l)] for gi, b, _ in picks])
            ref = oracle.layer_forward_packed(tin, cu, p64, w.n_heads, w.head_dim)
            for i, (gi, b, n) in enumerate(picks):
                err = normwise_rel(gpu_out[(gi, b, l)], ref[cu[i]:cu[i + 1]])
                say(f"  layer {l} teacher-forced, batch {gi} sequence {b} (len {n}): rel {err:.3e}")
                assert err <= 2e-2
        if l % 8 == 7:
            say(f"  oracle layer {l + 1}/{L} done")
        del p64
    for i, (gi, b, n) in enumerate(picks):
        err = normwise_rel(gpu_y[(gi, b)], rows[cu[i]:cu[i + 1]])
        say(f"batch {gi} sequence {b} (len {n}) through {L} layers, end to end: rel {err:.3e}")
        assert err <= 2e-2


@pytest.mark.timeout(900)
def test_stream_sequence_alone_equals_batch(stack48):
    """The shortest and longest sequence of the first and last FIFO batch, run
    alone and unpadded through the 48 layers, reproduce their rows of the batch
    bit for bit (a GEMM row depends only on its own A row, in the same K order
    whatever M and the tile; attention and LayerNorm are per sequence / row)."""
    w, lens, params, hs, reqs, fifo = stack48
    for gi in (0, len(fifo) - 1):
        bl = [lens[i] for i in fifo[gi]]
        x = workloads.pad_batch([reqs[i] for i in fifo[gi]])
        y = _stack(hs, x, bl)
        order = sorted(range(len(bl)), key=lambda b: bl[b])
        for b in (order[0], order[-1]):
            n = bl[b]
            y1 = _stack(hs, x[b:b + 1, :n].contiguous(), [n])
            same = torch.equal(y1[0], y[b, :n])
            say(f"batch {gi} (T={sum(bl)}) sequence {b} (len {n}) alone == in batch: {same}")
            assert same


@pytest.mark.timeout(900)
def test_dynamic_plan_batch_equals_fifo_rows(stack48):
    """Every FIFO batch through the 48 layers, then the two largest batches
    of a dynamic plan (requests drawn from many FIFO batches, sorted by
    length): each request's output rows equal its rows of its FIFO batch bit
    for bit, and the dynamic batches' pads are +0.0."""
    w, lens, params, hs, reqs, fifo = stack48
    fifo_rows = {}
    for gi, b_idx in enumerate(fifo):
        bl = [lens[i] for i in b_idx]
        y = _stack(hs, workloads.pad_batch([reqs[i] for i in b_idx]), bl)
        for k, i in enumerate(b_idx):
            fifo_rows[i] = y[k, :lens[i]].clone()
        del y
    # a cost model with a per-batch and a per-token term (the planner itself
    # is checked against the oracle's planner on the CPU)
    cost = ee.BatchCost(0.05, 3e-5, 0.0, 0.0, 1, 0)
    plan = ee.batches_of(ee.ee_plan_dynamic(lens, w.batch, cost)[0])
    big = sorted(range(len(plan)), key=lambda j: sum(lens[i] for i in plan[j]))[-2:]
    for j in big:
        b_idx = plan[j]
        bl = [lens[i] for i in b_idx]
        srcs = {fifo_of for fifo_of, f in enumerate(fifo) for i in b_idx if i in f}
        y = _stack(hs, workloads.pad_batch([reqs[i] for i in b_idx]), bl)
        _pads_zero(y, bl)
        same = all(torch.equal(y[k, :lens[i]], fifo_rows[i]) for k, i in enumerate(b_idx))
        say(f"dynamic batch {j}: {len(b_idx)} requests (T={sum(bl)}, P={max(bl)}) from FIFO batches "
            f"{sorted(srcs)}: rows == FIFO rows: {same}")
        assert same
