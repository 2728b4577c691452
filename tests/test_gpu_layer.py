"""Whole-layer and stack parity of the HIP path against the CPU oracle's padded
forward (the definition), through the C ABI, on seeded workloads.

Bars: fp16 storage / fp32 accumulation: normwise max relative error <= 2e-2
over valid rows; fp32: <= 1e-4; pads exactly +0.0; valid rows bit-identical
whatever the pads hold (NaN included)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, Guarded, normwise_rel, say, to_host64, valid_mask

pytestmark = pytest.mark.gpu


def _run_layer(w, lens, x, params, fuse_gelu=True, gelu=ee.GELU_TANH, layers_params=None,
               residual=ee.RESIDUAL_AUTO):
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    plist = layers_params or [params]
    dev_params = [{k: v.to(DEV) for k, v in p.items()} for p in plist]
    layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, dp, dtype=dt, gelu=gelu, fuse_gelu=fuse_gelu,
                       residual=residual) for dp in dev_params]
    B, P, _ = x.shape
    gws = Guarded((layers[0].workspace_size(B, P, sum(lens)),), torch.uint8)
    xd = x.to(DEV)
    gy = Guarded(xd.shape, xd.dtype, fill=9.0)
    y = gy.t
    if len(layers) == 1:
        layers[0].forward(xd, lens, y, gws.t)
    else:
        ee.ee_stack_forward(layers, xd, lens, y, gws.t)
    torch.cuda.synchronize()
    gy.check("y")
    gws.check("the workspace")
    return y


def _check(w, lens, y, ref, tol, label):
    got = to_host64(y)
    m = valid_mask(lens, got.shape[1])
    err = normwise_rel(got[m], ref[m]) if m.any() else 0.0
    pads = got[~m]
    say(f"{label}: T={sum(lens)} rel {err:.3e}")
    assert np.all(pads == 0) and not np.any(np.signbit(pads)), "pads must be +0.0"
    assert err <= tol, f"{label}: rel {err}"
    return err


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("variant", ["init", "affine"])
def test_tiny_fp32_layer(seed, variant):
    w = workloads.get("tiny-fp32")
    lens = workloads.lengths(w, seed)
    x = workloads.activations(w, seed, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, seed, 0, variant=variant)
    y = _run_layer(w, lens, x, p)
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim)
    _check(w, lens, y, ref, 1e-4, f"tiny-fp32 seed={seed} {variant}")


@pytest.mark.parametrize("seed,variant,fuse,gelu", [
    (1234, "init", True, ee.GELU_TANH), (1234, "affine", True, ee.GELU_TANH),
    (7, "affine", False, ee.GELU_TANH), (8, "affine", True, ee.GELU_ERF),
])
def test_gpt2_small_layer(seed, variant, fuse, gelu):
    w = workloads.get("gpt2-small")
    lens = workloads.lengths(w, seed)
    x = workloads.activations(w, seed, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, seed, 0, variant=variant)
    y = _run_layer(w, lens, x, p, fuse_gelu=fuse, gelu=gelu)
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim,
                                      gelu_form="tanh" if gelu == ee.GELU_TANH else "erf")
    _check(w, lens, y, ref, 2e-2, f"gpt2-small seed={seed} {variant} fuse={fuse} gelu={gelu}")


@pytest.mark.parametrize("lens", [[0] * 8, [128] * 8, [1] * 8, [0, 128, 0, 1, 0, 77, 0, 0], [100]])
def test_gpt2_small_edge_lengths(lens):
    w = dataclasses.replace(workloads.get("gpt2-small"), batch=len(lens))
    x = workloads.activations(w, 3, len(lens), w.pad_len, lens)
    p = workloads.layer_params(w, 3, 0, variant="affine")
    y = _run_layer(w, lens, x, p)
    if sum(lens) == 0:
        assert torch.all(y == 0) and not torch.any(torch.signbit(y))
        return
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim)
    _check(w, lens, y, ref, 2e-2, f"gpt2-small lens={lens[:4]}...")


def test_gpt2_small_long_sequences():
    """A padding length of 1024: one full sequence, ragged ones (several query
    tiles of 128 and key tiles past them), an empty one and a single token."""
    lens = [1024, 300, 0, 1, 777]
    w = dataclasses.replace(workloads.get("gpt2-small"), batch=len(lens), pad_len=1024)
    x = workloads.activations(w, 5, len(lens), w.pad_len, lens)
    p = workloads.layer_params(w, 5, 0, variant="affine")
    y = _run_layer(w, lens, x, p)
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim)
    _check(w, lens, y, ref, 2e-2, f"gpt2-small P=1024 lens={lens}")


def test_nan_pads_do_not_reach_valid_rows():
    w = workloads.get("gpt2-small")
    lens = workloads.lengths(w, 11)
    p = workloads.layer_params(w, 11, 0, variant="affine")
    x_r = workloads.activations(w, 11, w.batch, w.pad_len, lens)
    x_n = workloads.activations(w, 11, w.batch, w.pad_len, lens, pad_fill="nan")
    y_r = _run_layer(w, lens, x_r, p)
    y_n = _run_layer(w, lens, x_n, p)
    assert not torch.isnan(y_n).any()
    assert torch.equal(y_r, y_n)


@pytest.mark.parametrize("residual", [ee.RESIDUAL_EPILOGUE, ee.RESIDUAL_PASS])
def test_each_sequence_alone_matches_batch(residual):
    """Sequences are independent: running one alone, unpadded, gives its rows of
    the batch bit for bit (every GEMM output element accumulates its K tiles in
    the same order whatever M and the tile shape are; attention is per
    sequence, LayerNorm and the residual pass per row), in either residual
    mode."""
    w = workloads.get("gpt2-small")
    lens = workloads.lengths(w, 21)
    x = workloads.activations(w, 21, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 21, 0, variant="affine")
    y = to_host64(_run_layer(w, lens, x, p, residual=residual))
    for b in (0, 5):
        n = lens[b]
        w1 = dataclasses.replace(w, batch=1, pad_len=n)
        y1 = to_host64(_run_layer(w1, [n], x[b:b + 1, :n].contiguous(), p, residual=residual))
        assert np.array_equal(y1[0], y[b, :n])


def test_stack_matches_oracle():
    w = dataclasses.replace(workloads.get("gpt2-small"), batch=6, layers=3)
    lens = [128, 1, 77, 0, 100, 64]
    x = workloads.activations(w, 5, w.batch, w.pad_len, lens)
    ps = [workloads.layer_params(w, 5, l, variant="affine") for l in range(3)]
    y = _run_layer(w, lens, x, None, layers_params=ps)
    ref = oracle.stack_forward_packed(x.double().numpy(), lens, ps, w.n_heads, w.head_dim)
    _check(w, lens, y, ref, 2e-2, "gpt2-small 3-layer stack")


def test_tiny_fp32_stack_matches_padded_definition():
    w = workloads.get("tiny-fp32")
    lens = workloads.lengths(w, 9)
    x = workloads.activations(w, 9, w.batch, w.pad_len, lens)
    ps = [workloads.layer_params(w, 9, l, variant="affine") for l in range(4)]
    y = _run_layer(w, lens, x, None, layers_params=ps)
    ref = oracle.stack_forward_padded(x.double().numpy(), lens, ps, w.n_heads, w.head_dim)
    _check(w, lens, y, ref, 1e-4, "tiny-fp32 4-layer stack")


def test_profile_records_every_launch_site():
    w = workloads.get("gpt2-small")
    lens = workloads.lengths(w, 1)
    x = workloads.activations(w, 1, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 1, 0)
    ee.ee_profile_enable(True)
    try:
        _run_layer(w, lens, x, p)
        stats = ee.ee_profile_collect()
    finally:
        ee.ee_profile_enable(False)
    for site in ("offsets", "remove", "ln1", "gemm_qkv", "attention", "gemm_out", "ln2", "gemm_fc1", "gemm_fc2",
                 "rebuild"):
        assert stats[site]["launches"] == 1 and stats[site]["total_ms"] > 0
    # GEMM sites carry their algorithmic flops and the kernel they ran (few
    # 256 x 256 tiles at this size: the 128 x 128 tile kernel)
    T = sum(lens)
    for site, (K, N, epi) in {"gemm_qkv": (768, 3 * 768, 1), "gemm_out": (768, 768, 2), "gemm_fc1": (768, 3072, 3),
                              "gemm_fc2": (3072, 768, 2)}.items():
        assert stats[site]["flops"] == 2.0 * T * K * N
        assert stats[site]["kernel"] == f"gemm_f16_mfma_kernel<32, 128, 128, 2, 2, {epi}, 2, false>"
    assert stats["attention"]["flops"] == 0 and not any(s.endswith("_rest") for s in stats)


def test_profile_filter_times_one_site():
    """With ee_profile_filter("gemm_fc1") only that site is timed; with the
    filter cleared every site is again; the outputs are the same bits."""
    w = workloads.get("gpt2-small")
    lens = workloads.lengths(w, 2)
    x = workloads.activations(w, 2, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 2, 0)
    ee.ee_profile_enable(True)
    try:
        ee.ee_profile_filter("gemm_fc1")
        y1 = _run_layer(w, lens, x, p)
        only = ee.ee_profile_collect()
        ee.ee_profile_filter(None)
        y2 = _run_layer(w, lens, x, p)
        every = ee.ee_profile_collect()
    finally:
        ee.ee_profile_filter(None)
        ee.ee_profile_enable(False)
    assert set(only) == {"gemm_fc1"} and only["gemm_fc1"]["launches"] == 1 and only["gemm_fc1"]["total_ms"] > 0
    assert {"gemm_fc1", "attention", "rebuild"} <= set(every)
    assert torch.equal(y1, y2)


def test_debug_sync_mode_gives_the_same_bits():
    """With ee_debug_sync on, every launch is followed by a stream
    synchronisation; the layer's outputs are the same bits as without it."""
    w = workloads.get("gpt2-small")
    lens = workloads.lengths(w, 3)
    x = workloads.activations(w, 3, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 3, 0, variant="affine")
    y0 = _run_layer(w, lens, x, p)
    ee.ee_debug_sync(True)
    try:
        y1 = _run_layer(w, lens, x, p, layers_params=[p, p])
        y2 = _run_layer(w, lens, x, p)
    finally:
        ee.ee_debug_sync(False)
    assert torch.equal(y0, y2) and torch.isfinite(y1).all()
