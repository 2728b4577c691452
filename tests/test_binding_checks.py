"""The Python binding checks every tensor argument before it calls the
library: a lengths list that does not match the batch, a shape or dtype that
does not match the layer or the other operands, a non-contiguous tensor, or a
tensor off the GPU raises ValueError / TypeError, and nothing is launched.
These run on the CPU: the checks come before the device check, which comes
before any call into libee (CPU tensors never reach it)."""
import pytest
import torch

import variable_length_padding_amd as ee

H, NH, HD, F = 64, 4, 16, 256


def _layer(dtype=ee.F16):
    t = torch.float16 if dtype == ee.F16 else torch.float32
    shapes = {"ln1_g": (H,), "ln1_b": (H,), "w_qkv": (3 * H, H), "b_qkv": (3 * H,), "w_out": (H, H), "b_out": (H,),
              "ln2_g": (H,), "ln2_b": (H,), "w_fc1": (F, H), "b_fc1": (F,), "w_fc2": (H, F), "b_fc2": (H,)}
    return ee.Layer(H, NH, HD, F, {k: torch.zeros(v, dtype=t) for k, v in shapes.items()}, dtype=dtype)


def _io(B=3, P=8, dtype=torch.float16):
    return torch.zeros(B, P, H, dtype=dtype), torch.zeros(B, P, H, dtype=dtype), torch.zeros(4096, dtype=torch.uint8)


def test_layer_forward_checks():
    L = _layer()
    x, y, ws = _io()
    with pytest.raises(ValueError, match="3 entries for a batch of 3|entries for a batch"):
        L.forward(x, [1, 2], y, ws)                       # lengths shorter than the batch
    with pytest.raises(ValueError, match="entries for a batch"):
        L.forward(x, [1, 2, 3, 4], y, ws)
    with pytest.raises(ValueError, match="y has shape"):
        L.forward(x, [1, 2, 3], torch.zeros(3, 7, H, dtype=torch.float16), ws)
    with pytest.raises(ValueError, match="x has shape"):
        L.forward(torch.zeros(3, 8, 2 * H, dtype=torch.float16), [1, 2, 3], y, ws)
    with pytest.raises(TypeError, match="x has dtype"):
        L.forward(x.float(), [1, 2, 3], y, ws)            # fp32 input to an fp16 layer
    with pytest.raises(TypeError, match="y has dtype"):
        L.forward(x, [1, 2, 3], y.float(), ws)
    with pytest.raises(ValueError, match="contiguous"):
        L.forward(x.transpose(0, 1).contiguous().transpose(0, 1), [1, 2, 3], y, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        L.forward(x, [1, 2, 3], y, ws)                    # every check passes but the device one
    L32 = _layer(ee.F32)
    with pytest.raises(TypeError, match="dtype"):
        L32.forward(x, [1, 2, 3], y, ws)                  # fp16 tensors to an fp32 layer


def test_stack_forward_checks():
    L = _layer()
    x, y, ws = _io()
    with pytest.raises(ValueError, match="at least one layer"):
        ee.ee_stack_forward([], x, [1, 2, 3], y, ws)
    with pytest.raises(ValueError, match="entries for a batch"):
        ee.ee_stack_forward([L, L], x, [1], y, ws)
    with pytest.raises(ValueError, match="y has shape"):
        ee.ee_stack_forward([L, L], x, [1, 2, 3], y[:2], ws)
    with pytest.raises(TypeError, match="dtype"):
        ee.ee_stack_forward([L, L], x.float(), [1, 2, 3], y.float(), ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        ee.ee_stack_forward([L, L], x, [1, 2, 3], y, ws)


def test_remove_rebuild_checks():
    x, _, ws = _io()
    packed = torch.zeros(6, H, dtype=torch.float16)
    for fn in (ee.ee_remove_padding, lambda p, l, k, w: ee.ee_rebuild_padding(k, l, p, w)):
        with pytest.raises(ValueError, match="entries for a batch"):
            fn(x, [1, 2], packed, ws)
        with pytest.raises(ValueError, match="need sum\\(lens\\) = 7"):
            fn(x, [1, 2, 4], packed, ws)                  # packed has 6 rows for T = 7
        with pytest.raises(ValueError, match="packed has shape"):
            fn(x, [1, 2, 3], torch.zeros(6, H + 8, dtype=torch.float16), ws)
        with pytest.raises(TypeError, match="packed has dtype"):
            fn(x, [1, 2, 3], packed.float(), ws)
        with pytest.raises(ValueError, match="GPU tensor"):
            fn(x, [1, 2, 3], packed, ws)
    with pytest.raises(TypeError, match="unsupported dtype"):
        ee.ee_remove_padding(x.to(torch.bfloat16), [1, 2, 3], packed, ws)


def test_row_op_and_linear_checks():
    x = torch.zeros(5, H, dtype=torch.float16)
    g = torch.ones(H, dtype=torch.float16)
    with pytest.raises(ValueError, match="y has shape"):
        ee.ee_layernorm(x, g, g, 1e-5, torch.zeros(4, H, dtype=torch.float16))
    with pytest.raises(TypeError, match="gamma has dtype"):
        ee.ee_layernorm(x, g.float(), g, 1e-5, torch.zeros_like(x))
    A, W = torch.zeros(5, H, dtype=torch.float16), torch.zeros(32, H, dtype=torch.float16)
    Cm, b = torch.zeros(5, 32, dtype=torch.float16), torch.zeros(32, dtype=torch.float16)
    with pytest.raises(ValueError, match="W has shape"):
        ee.ee_linear(A, torch.zeros(32, H + 8, dtype=torch.float16), b, None, ee.EPI_BIAS, Cm)
    with pytest.raises(ValueError, match="C_out has shape"):
        ee.ee_linear(A, W, b, None, ee.EPI_BIAS, torch.zeros(5, 31, dtype=torch.float16))
    with pytest.raises(ValueError, match="residual is required"):
        ee.ee_linear(A, W, b, None, ee.EPI_BIAS_RESIDUAL, Cm)
    with pytest.raises(ValueError, match="bias is required"):
        ee.ee_linear(A, W, None, None, ee.EPI_BIAS, Cm)
    with pytest.raises(TypeError, match="W has dtype"):
        ee.ee_linear(A, W.float(), b, None, ee.EPI_BIAS, Cm)
    with pytest.raises(ValueError, match="GPU tensor"):
        ee.ee_linear(A, W, b, None, ee.EPI_BIAS, Cm)
    with pytest.raises(ValueError, match="g has shape"):
        ee.ee_bias_gelu(Cm, b, torch.zeros(5, 30, dtype=torch.float16))


def test_attention_and_offsets_checks():
    qkv = torch.zeros(10, 3 * H, dtype=torch.float16)
    o = torch.zeros(10, H, dtype=torch.float16)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="o has shape"):
        ee.ee_attention_varlen(qkv, cu, 2, 6, NH, HD, o[:9])
    with pytest.raises(TypeError, match="cu has dtype"):
        ee.ee_attention_varlen(qkv, cu.long(), 2, 6, NH, HD, o)
    with pytest.raises(ValueError, match="cu has shape"):
        ee.ee_attention_varlen(qkv, cu, 3, 6, NH, HD, o)
    with pytest.raises(ValueError, match="GPU tensor"):
        ee.ee_attention_varlen(qkv, cu, 2, 6, NH, HD, o)
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)   # noqa: E731
    with pytest.raises(ValueError, match="token_src has shape"):
        ee.ee_compute_offsets([1, 2], 4, i32(3), i32(7), i32(8))
    with pytest.raises(ValueError, match="GPU tensor"):
        ee.ee_compute_offsets([1, 2], 4, i32(3), i32(8), i32(8))


def test_extend_checks():
    L = _layer()
    x = torch.zeros(3, H, dtype=torch.float16)
    ws = torch.zeros(16, dtype=torch.uint8)
    cache = torch.zeros(ee.ee_kv_cache_bytes(L, 2, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="one entry per sequence"):
        ee.ee_stack_extend([L, L], x, [1, 2], [0], [0, 4], cache, 8, x.clone(), ws)
    with pytest.raises(ValueError, match="x has shape"):
        ee.ee_stack_extend([L, L], x, [1, 1], [0, 0], [0, 4], cache, 8, x.clone(), ws)   # 2 new tokens, 3 rows
    with pytest.raises(ValueError, match="cache of"):
        ee.ee_stack_extend([L, L], x, [1, 2], [0, 0], [0, 4], cache[:100], 8, x.clone(), ws)
    with pytest.raises(TypeError, match="y has dtype"):
        ee.ee_stack_extend([L, L], x, [1, 2], [0, 0], [0, 4], cache, 8, x.float(), ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        ee.ee_stack_extend([L, L], x, [1, 2], [0, 0], [0, 4], cache, 8, x.clone(), ws)
