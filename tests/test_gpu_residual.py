"""Where the pre-LN block adds its residuals (ee_residual), through the C ABI:
the GEMM epilogue or a separate pass (sum rounded to storage, then LayerNorm
of it in the same pass after the out projection; a plain add after FC2).

- Both modes against the oracle for one layer and a stack, fp16 and fp32,
  fused and unfused GeLU, rows narrow enough for the one-wave-per-row pass
  (H = 64, 768) and wide enough for the workgroup-per-row pass (H = 5120).
- AUTO is EPILOGUE at any row count: bit-identical to it, and different from
  PASS (whose sum is rounded twice).
- Incremental decoding with the pass forced: prefill and decode steps (the
  split-K GEMMs then store acc + bias and the pass adds) against the oracle.
Bars: fp16 <= 2e-2, fp32 <= 1e-4 normwise over valid rows; pads +0.0."""
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

MODES = [ee.RESIDUAL_EPILOGUE, ee.RESIDUAL_PASS]


def _stack(w, plist, lens, x, residual, fuse_gelu=True):
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, {k: v.to(DEV) for k, v in p.items()}, dtype=dt,
                       fuse_gelu=fuse_gelu, residual=residual) for p in plist]
    B, P, _ = x.shape
    ws = torch.empty(layers[0].workspace_size(B, P, sum(lens)), dtype=torch.uint8, device=DEV)
    xd = x.to(DEV)
    y = torch.full_like(xd, 9.0)
    ee.ee_stack_forward(layers, xd, lens, y, ws)
    torch.cuda.synchronize()
    return y


def _check(w, lens, y, plist, x, tol, label):
    ref = x.double().numpy()
    for p in plist:
        ref = oracle.layer_forward_padded(ref, lens, p, w.n_heads, w.head_dim)
    got = to_host64(y)
    m = valid_mask(lens, w.pad_len)
    err = normwise_rel(got[m], ref[m])
    say(f"{label}: T={sum(lens)} rel {err:.3e}")
    assert np.all(got[~m] == 0) and not np.any(np.signbit(got[~m]))
    assert err <= tol


def _wide():
    return dataclasses.replace(workloads.get("gpt2-small"), name="wide5120", batch=3, pad_len=48, hidden=5120,
                               n_heads=40, head_dim=128, ffn=1024)


@pytest.mark.parametrize("residual", MODES)
@pytest.mark.parametrize("name,fuse,n_layers,tol", [
    ("gpt2-small", True, 1, 2e-2), ("gpt2-small", False, 1, 2e-2), ("gpt2-small", True, 3, 2e-2),
    ("tiny-fp32", True, 2, 1e-4), ("wide5120", True, 1, 2e-2),
])
def test_residual_modes_match_oracle(residual, name, fuse, n_layers, tol):
    w = _wide() if name == "wide5120" else workloads.get(name)
    lens = workloads.lengths(w, 31)
    x = workloads.activations(w, 31, w.batch, w.pad_len, lens)
    plist = [workloads.layer_params(w, 31, l, variant="affine") for l in range(n_layers)]
    y = _stack(w, plist, lens, x, residual, fuse_gelu=fuse)
    _check(w, lens, y, plist, x, tol, f"{name} residual={residual} fuse={fuse} layers={n_layers}")


@pytest.mark.parametrize("batch", [16, 7])
def test_auto_is_the_epilogue(batch):
    w = dataclasses.replace(workloads.get("gpt2-small"), batch=batch)
    lens = [w.pad_len] * batch
    x = workloads.activations(w, 5, w.batch, w.pad_len, lens)
    plist = [workloads.layer_params(w, 5, 0, variant="affine")]
    y_auto = _stack(w, plist, lens, x, ee.RESIDUAL_AUTO)
    y_epi = _stack(w, plist, lens, x, ee.RESIDUAL_EPILOGUE)
    y_pass = _stack(w, plist, lens, x, ee.RESIDUAL_PASS)
    assert torch.equal(y_auto, y_epi)
    assert not torch.equal(y_auto, y_pass)      # the two roundings differ somewhere at this size
    _check(w, lens, y_auto, plist, x, 2e-2, f"gpt2-small AUTO at {batch * w.pad_len} rows")


@pytest.mark.parametrize("name,tol", [("gpt2-small", 2e-2), ("tiny-fp32", 1e-4)])
def test_extend_with_residual_pass(name, tol):
    w = workloads.get(name)
    prompts = [1, 37, 100, 5] if w.pad_len >= 128 else [1, 9, 16, 4]
    dec = Decoder(w, 61, 2, prompts, max_new=4, residual=ee.RESIDUAL_PASS)
    rows_all = [_token_rows(w, 500 + b, prompts[b] + 4) for b in range(len(prompts))]
    pos = [0] * len(prompts)
    for k, new_len in enumerate([prompts, [1] * 4, [1] * 4, [2, 0, 1, 0]]):
        rows = torch.cat([rows_all[b][pos[b]:pos[b] + n] for b, n in enumerate(new_len)])
        got, ref = dec.step(rows, new_len)
        err = normwise_rel(got, ref)
        say(f"{name} extend (residual pass) step {k} new={new_len}: rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= tol
        pos = [q + n for q, n in zip(pos, new_len)]
