"""The ABI's size limits, on the GPU, against the oracle.

- The layer at the largest batch (EE_MAX_BATCH = 512 sequences, the lengths
  travel as a by-value kernel argument): fp32 and fp16, ragged lengths
  including empty sequences, pads +0.0.
- One extend step at the largest batch (EE_MAX_EXTEND_BATCH = 256 sequences):
  a prefill of ragged prompts, then a decode step with a token for every
  sequence, checked step by step.
Bars: fp16 <= 2e-2, fp32 <= 1e-4 normwise; pads exactly +0.0."""
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
    dec = Decoder(w, 88, 1, prompts, max_new=1)
    rows_all = [_token_rows(w, 700 + b, prompts[b] + 1) for b in range(B)]
    for k, new_len in enumerate([prompts, [1] * B]):
        start = [0] * B if k == 0 else prompts
        rows = torch.cat([rows_all[b][start[b]:start[b] + n] for b, n in enumerate(new_len)])
        got, ref = dec.step(rows, new_len)
        err = normwise_rel(got, ref)
        say(f"{name} extend at B={B}, step {k} (T={sum(new_len)}): rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= tol
