"""Row pitches through the C ABI.

- ee_linear_strided on small-integer operands: bit-exact (every partial sum
  is an integer below 2^24), and the columns past N of C keep their bytes.
- A layer whose weight matrices sit at a padded pitch computes the same bits
  as with dense weights (the kernels and their summation order are the same).
- A layer whose FC1 output rows are 32 KiB (ffn 16384 in fp16, 8192 in fp32),
  which the library stores at a padded pitch in its workspace, against the
  oracle: forward with fused and unfused GeLU, and incremental decoding, whose
  split-K GEMMs read and write those rows.
Bars: as the layer tests, fp16 <= 2e-2, fp32 <= 1e-4."""
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
GEN = torch.Generator().manual_seed(5150)


def _small_ints(shape, lo=-2, hi=2):
    return torch.randint(lo, hi + 1, shape, generator=GEN).to(torch.float16)


def _strided(t, extra, fill=7.0):
    """t on the device inside a wider buffer (row pitch cols + extra whose
    extra columns hold `fill`), as a view of its first cols columns."""
    rows, cols = t.shape
    buf = torch.full((rows, cols + extra), fill, dtype=t.dtype, device=DEV)
    buf[:, :cols] = t.to(DEV)
    return buf[:, :cols]


@pytest.mark.parametrize("M,N,K,pa,pw,pc", [
    (37, 96, 128, 8, 64, 8), (300, 256, 192, 64, 8, 0), (4112, 768, 3072, 64, 64, 64),
    (4096, 4104, 128, 8, 8, 8), (4096, 4099, 64, 8, 8, 5), (100, 70, 130, 6, 2, 3),
])
@pytest.mark.parametrize("epi", [ee.EPI_BIAS, ee.EPI_BIAS_RESIDUAL])
def test_gemm_strided_integer_exact(M, N, K, pa, pw, pc, epi):
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias = _small_ints((N,))
    R = _small_ints((M, N), -8, 8)
    cbuf = torch.full((M, N + pc), 3.0, dtype=torch.float16, device=DEV)
    C = cbuf[:, :N]
    Rd = _strided(R, pc) if epi == ee.EPI_BIAS_RESIDUAL else None
    ee.ee_linear(_strided(A, pa), _strided(W, pw), bias.to(DEV), Rd, epi, C)
    torch.cuda.synchronize()
    exact = A.double().numpy() @ W.double().numpy().T + bias.double().numpy()
    if epi == ee.EPI_BIAS_RESIDUAL:
        exact = exact + R.double().numpy()
    assert np.abs(exact).max() < 2 ** 24
    ref16 = exact.astype(np.float16)
    got = cbuf.cpu().numpy()
    assert np.array_equal(got[:, :N].view(np.uint16), ref16.view(np.uint16)), \
        f"{np.count_nonzero(got[:, :N] != ref16)} of {ref16.size} differ"
    assert np.all(got[:, N:] == 3.0)


@pytest.mark.parametrize("epi", [ee.EPI_BIAS_RESIDUAL, ee.EPI_BIAS_GELU])
def test_gemm_f32_strided_parity(epi):
    M, N, K = 100, 70, 130
    A = torch.randn(M, K, generator=GEN)
    W = 0.1 * torch.randn(N, K, generator=GEN)
    bias = torch.randn(N, generator=GEN)
    R = torch.randn(M, N, generator=GEN)
    cbuf = torch.full((M, N + 4), 3.0, device=DEV)
    ee.ee_linear(_strided(A, 4), _strided(W, 8), bias.to(DEV),
                 _strided(R, 4) if epi == ee.EPI_BIAS_RESIDUAL else None, epi, cbuf[:, :N])
    torch.cuda.synchronize()
    ref = oracle.linear(A.double().numpy(), W.double().numpy(), bias.double().numpy())
    ref = ref + R.double().numpy() if epi == ee.EPI_BIAS_RESIDUAL else oracle.gelu(ref)
    assert normwise_rel(to_host64(cbuf[:, :N]), ref) <= 1e-5
    assert torch.all(cbuf[:, N:] == 3.0)


def _stack(w, plist, lens, x, fuse_gelu=True, block=ee.BLOCK_GPT_PRELN, extra=0):
    """ee_stack_forward over layers built from plist; weight matrices stored at
    row pitch cols + extra when extra > 0."""
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    layers = []
    for p in plist:
        d = {k: v.to(DEV) for k, v in p.items()}
        if extra:
            for k in ("w_qkv", "w_out", "w_fc1", "w_fc2"):
                d[k] = _strided(p[k], extra)
        layers.append(ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, d, dtype=dt, fuse_gelu=fuse_gelu,
                               block=block))
    B, P, _ = x.shape
    ws = torch.empty(layers[0].workspace_size(B, P, sum(lens)), dtype=torch.uint8, device=DEV)
    xd = x.to(DEV)
    y = torch.full_like(xd, 9.0)
    ee.ee_stack_forward(layers, xd, lens, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name,extra", [("gpt2-small", 8), ("gpt2-small", 64), ("tiny-fp32", 4)])
@pytest.mark.parametrize("block", [ee.BLOCK_GPT_PRELN, ee.BLOCK_BERT_POSTLN])
def test_layer_pitched_weights_same_bits(name, extra, block):
    w = workloads.get(name)
    lens = workloads.lengths(w, 21)
    x = workloads.activations(w, 21, w.batch, w.pad_len, lens)
    ps = [workloads.layer_params(w, 21, l, variant="affine") for l in range(2)]
    y_dense = _stack(w, ps, lens, x, block=block)
    y_pitch = _stack(w, ps, lens, x, block=block, extra=extra)
    assert torch.equal(y_dense, y_pitch)


def _wide_ffn(dtype):
    """FC1 output rows of exactly 32 KiB: the workspace stores them padded."""
    if dtype == "f16":
        w = dataclasses.replace(workloads.get("gpt2-small"), name="ffn16k", batch=4, pad_len=64, hidden=1024,
                                n_heads=16, head_dim=64, ffn=16384)
    else:
        w = dataclasses.replace(workloads.get("tiny-fp32"), name="ffn8k-fp32", ffn=8192)
    assert ee.ee_preferred_row_pitch(w.ffn, ee.F16 if dtype == "f16" else ee.F32) > w.ffn
    return w


@pytest.mark.parametrize("dtype,fuse,tol", [("f16", True, 2e-2), ("f16", False, 2e-2), ("f32", True, 1e-4)])
def test_layer_with_32k_ffn_rows(dtype, fuse, tol):
    w = _wide_ffn(dtype)
    lens = workloads.lengths(w, 8)
    x = workloads.activations(w, 8, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 8, 0, variant="affine")
    y = _stack(w, [p], lens, x, fuse_gelu=fuse)
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim)
    got = to_host64(y)
    m = valid_mask(lens, w.pad_len)
    err = normwise_rel(got[m], ref[m])
    say(f"{w.name} fuse={fuse}: T={sum(lens)} rel {err:.3e}")
    assert np.all(got[~m] == 0) and err <= tol
    if dtype == "f16":     # weight rows padded by 64 elements: the same bits
        assert torch.equal(y, _stack(w, [p], lens, x, fuse_gelu=fuse, extra=64))


def test_extend_with_32k_ffn_rows():
    """The prefill (M = 24 rows) and decode steps (M = 2 or 3) split K four ways
    in FC1 (K = 1024) and FC2 (K = 16384): FC1's reduce writes the padded rows
    and FC2's partial GEMM reads them."""
    w = _wide_ffn("f16")
    prompts = [5, 17, 2]
    dec = Decoder(w, 77, 2, prompts, max_new=3)
    rows_all = [_token_rows(w, 300 + b, prompts[b] + 3) for b in range(len(prompts))]
    pos = [0] * len(prompts)
    for k, new_len in enumerate([prompts, [1, 1, 1], [1, 1, 1], [1, 0, 1]]):
        rows = torch.cat([rows_all[b][pos[b]:pos[b] + n] for b, n in enumerate(new_len)])
        got, ref = dec.step(rows, new_len)
        err = normwise_rel(got, ref)
        say(f"ffn16k extend step {k} new={new_len}: rel {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= 2e-2
        pos = [q + n for q, n in zip(pos, new_len)]
