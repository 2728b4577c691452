"""The page-literal RCE form (transposing rebuild/remove around padded
attention) and the post-LN BERT-style encoder block on the GPU, against the
oracle, through the C ABI.

Bars: transposing rebuild/remove bit-exact; attention fp16 <= 3e-3, fp32 <=
1e-5; fused add-bias-residual-LayerNorm fp16 <= 2e-3, fp32 <= 1e-5; layers
fp16 <= 2e-2, fp32 <= 1e-4; the decoder's page-literal form bit-identical to
the varlen form."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
import workloads
from gpu_helpers import DEV, normwise_rel, say, to_host64, valid_mask

pytestmark = pytest.mark.gpu
GEN = torch.Generator().manual_seed(424242)


def _cu(lens):
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=DEV)


@pytest.mark.parametrize("dtype,nh,hd,n_mats", [(torch.float16, 3, 64, 3), (torch.float16, 2, 128, 1),
                                                 (torch.float32, 4, 16, 3), (torch.float16, 1, 16, 2)])
@pytest.mark.parametrize("lens,P", [([5, 0, 16, 1], 16), ([128] * 3, 256), ([7], 7)])
def test_transposing_rebuild_and_remove_bit_exact(dtype, nh, hd, n_mats, lens, P):
    B, T = len(lens), sum(lens)
    packed = torch.randn(max(T, 1), n_mats * nh * hd, generator=GEN).to(dtype)
    ws = torch.empty(ee.ee_padding_workspace_size(B, P), dtype=torch.uint8, device=DEV)
    heads = torch.full((n_mats, B, nh, P, hd), 9.0, dtype=dtype, device=DEV)
    ee.ee_transpose_padding_rebuild_heads(packed.to(DEV), lens, heads, ws)
    torch.cuda.synchronize()
    ref = oracle.transpose_padding_rebuild_heads(packed.numpy()[:T], lens, P, nh, hd)
    got = heads.cpu().numpy()
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))      # pads +0.0 bit for bit
    back = torch.full((max(T, 1), nh * hd), 3.0, dtype=dtype, device=DEV)
    ee.ee_transpose_padding_remove_heads(heads[0].contiguous(), lens, back, ws)
    torch.cuda.synchronize()
    ref_back = oracle.transpose_padding_remove_heads(got[0], lens)
    if T:
        assert np.array_equal(back.cpu().numpy()[:T].view(np.uint8), ref_back.view(np.uint8))
        assert np.array_equal(back.cpu().numpy()[:T], packed.numpy()[:T, :nh * hd])


ATT_LENS = [1, 31, 33, 128, 129, 200, 5]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype,hd,nh,tol", [(torch.float16, 128, 2, 3e-3), (torch.float16, 64, 3, 3e-3),
                                             (torch.float32, 16, 2, 1e-5)])
def test_padded_attention(causal, dtype, hd, nh, tol):
    lens, P = ATT_LENS, 256
    B = len(lens)
    q, k, v = (torch.randn(B, nh, P, hd, generator=GEN).to(dtype) for _ in range(3))
    o = torch.zeros(B, nh, P, hd, dtype=dtype, device=DEV)
    ee.ee_attention_padded(q.to(DEV), k.to(DEV), v.to(DEV), _cu(lens), o, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.attention_padded_heads(q.double().numpy(), k.double().numpy(), v.double().numpy(), lens, causal)
    got = to_host64(o)
    err = max(normwise_rel(got[b, :, :n], ref[b, :, :n]) for b, n in enumerate(lens))
    say(f"padded attention causal={causal} {dtype} hd={hd}: rel {err:.2e}")
    assert err <= tol


@pytest.mark.parametrize("dtype,hd,nh,tol", [(torch.float16, 128, 2, 3e-3), (torch.float16, 64, 3, 3e-3),
                                             (torch.float32, 64, 2, 1e-5)])
def test_bidirectional_varlen_attention(dtype, hd, nh, tol):
    lens = ATT_LENS
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu_h[-1])
    qkv = torch.randn(T, 3 * nh * hd, generator=GEN).to(dtype)
    o = torch.empty(T, nh * hd, dtype=dtype, device=DEV)
    ee.ee_attention_varlen(qkv.to(DEV), _cu(lens), len(lens), max(lens), nh, hd, o, causal=False)
    torch.cuda.synchronize()
    ref = oracle.attention_packed_bidirectional(qkv.double().numpy(), cu_h, nh, hd)
    err = normwise_rel(to_host64(o), ref)
    say(f"bidirectional varlen attention {dtype} hd={hd}: rel {err:.2e}")
    assert err <= tol


@pytest.mark.parametrize("dtype,H,tol", [(torch.float16, 768, 2e-3), (torch.float16, 12288, 2e-3),
                                         (torch.float32, 64, 1e-5)])
def test_add_bias_residual_layernorm(dtype, H, tol):
    rows = 37
    u, r = (torch.randn(rows, H, generator=GEN).to(dtype) for _ in range(2))
    b, g, be = (0.5 * torch.randn(H, generator=GEN)).to(dtype), (1 + 0.1 * torch.randn(H, generator=GEN)).to(dtype), \
        (0.1 * torch.randn(H, generator=GEN)).to(dtype)
    y = torch.empty(rows, H, dtype=dtype, device=DEV)
    ee.ee_add_bias_residual_layernorm(u.to(DEV), b.to(DEV), r.to(DEV), g.to(DEV), be.to(DEV), 1e-5, y)
    torch.cuda.synchronize()
    ref = oracle.add_bias_residual_layernorm(u.double().numpy(), b.double().numpy(), r.double().numpy(),
                                             g.double().numpy(), be.double().numpy(), 1e-5)
    assert normwise_rel(to_host64(y), ref) <= tol


def _run(w, lens, x, plist, block, attention, gelu=ee.GELU_TANH, residual=ee.RESIDUAL_AUTO):
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, {k: v.to(DEV) for k, v in p.items()}, dtype=dt,
                       gelu=gelu, block=block, attention=attention, residual=residual) for p in plist]
    B, P, _ = x.shape
    ws = torch.empty(layers[0].workspace_size(B, P, sum(lens)), dtype=torch.uint8, device=DEV)
    xd = x.to(DEV)
    y = torch.full_like(xd, 9.0)
    ee.ee_stack_forward(layers, xd, lens, y, ws)
    torch.cuda.synchronize()
    return y


def _check(y, ref, lens, tol, label):
    got = to_host64(y)
    m = valid_mask(lens, got.shape[1])
    err = normwise_rel(got[m], ref[m])
    say(f"{label}: rel {err:.3e}")
    assert np.all(got[~m] == 0) and not np.any(np.signbit(got[~m]))
    assert err <= tol


@pytest.mark.parametrize("name,tol", [("gpt2-small", 2e-2), ("tiny-fp32", 1e-4)])
def test_decoder_page_literal_equals_varlen(name, tol):
    w = workloads.get(name)
    lens = workloads.lengths(w, 31)
    x = workloads.activations(w, 31, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 31, 0, variant="affine")
    y_v = _run(w, lens, x, [p], ee.BLOCK_GPT_PRELN, ee.ATTN_VARLEN)
    y_p = _run(w, lens, x, [p], ee.BLOCK_GPT_PRELN, ee.ATTN_PADDED)
    assert torch.equal(y_v, y_p)
    ref = oracle.layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim)
    _check(y_p, ref, lens, tol, f"{name} decoder, page-literal attention")


@pytest.mark.parametrize("name,attention,tol", [
    ("gpt2-small", ee.ATTN_VARLEN, 2e-2), ("gpt2-small", ee.ATTN_PADDED, 2e-2),
    ("tiny-fp32", ee.ATTN_VARLEN, 1e-4), ("tiny-fp32", ee.ATTN_PADDED, 1e-4),
])
def test_encoder_layer(name, attention, tol):
    w = workloads.get(name)          # gpt2-small shapes = BERT-base shapes (768, 12 heads, 3072)
    lens = workloads.lengths(w, 12)
    x = workloads.activations(w, 12, w.batch, w.pad_len, lens)
    p = workloads.layer_params(w, 12, 0, variant="affine")
    y = _run(w, lens, x, [p], ee.BLOCK_BERT_POSTLN, attention, gelu=ee.GELU_ERF)
    ref = oracle.encoder_layer_forward_padded(x.double().numpy(), lens, p, w.n_heads, w.head_dim, gelu_form="erf")
    _check(y, ref, lens, tol, f"{name} encoder attention={attention}")


def test_encoder_stack_and_nan_pads():
    w = dataclasses.replace(workloads.get("gpt2-small"), batch=5)
    lens = [128, 3, 0, 77, 1]
    ps = [workloads.layer_params(w, 13, l, variant="affine") for l in range(3)]
    x = workloads.activations(w, 13, w.batch, w.pad_len, lens)
    y = _run(w, lens, x, ps, ee.BLOCK_BERT_POSTLN, ee.ATTN_VARLEN, gelu=ee.GELU_ERF)
    ref = x.double().numpy()
    for p in ps:
        ref = oracle.encoder_layer_forward_padded(ref, lens, p, w.n_heads, w.head_dim, gelu_form="erf")
    _check(y, ref, lens, 2e-2, "gpt2-small 3-layer encoder stack")
    x_n = workloads.activations(w, 13, w.batch, w.pad_len, lens, pad_fill="nan")
    y_n = _run(w, lens, x_n, ps, ee.BLOCK_BERT_POSTLN, ee.ATTN_PADDED, gelu=ee.GELU_ERF)
    assert not torch.isnan(y_n).any()
    y_vp = _run(w, lens, x, ps, ee.BLOCK_BERT_POSTLN, ee.ATTN_PADDED, gelu=ee.GELU_ERF)
    assert torch.equal(y_n, y_vp)


@pytest.mark.parametrize("name", ["gpt2-small", "tiny-fp32"])
@pytest.mark.parametrize("residual", [ee.RESIDUAL_EPILOGUE, ee.RESIDUAL_PASS])
def test_padding_kept_gives_the_same_valid_rows(name, residual):
    """The result the method preserves: with right padding and the causal mask,
    running all B*P rows through the layers (padding kept) leaves the valid
    rows exactly as the packed run computes them; only the work differs (in
    either residual mode)."""
    w = workloads.get(name)
    lens = workloads.lengths(w, 77)
    x = workloads.activations(w, 77, w.batch, w.pad_len, lens, pad_fill="random")
    ps = [workloads.layer_params(w, 77, l, variant="affine") for l in range(2)]
    y_rce = _run(w, lens, x, ps, ee.BLOCK_GPT_PRELN, ee.ATTN_VARLEN, residual=residual)
    y_full = _run(w, [w.pad_len] * w.batch, x, ps, ee.BLOCK_GPT_PRELN, ee.ATTN_VARLEN, residual=residual)
    m = torch.from_numpy(valid_mask(lens, w.pad_len)).to(DEV)
    diff = (y_rce[m].float() - y_full[m].float()).abs().max().item()
    say(f"{name}: padding kept vs removed, max |diff| on valid rows {diff:.3e}")
    assert torch.equal(y_rce[m], y_full[m])
