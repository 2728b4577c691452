"""The C ABI without a GPU: libee loads, exports every function include/ee.h
declares, and rejects bad arguments on the host before any device work.
(Only calls that fail validation are made here; nothing reaches a kernel.)"""
import ctypes as C
import os
import re

import pytest

import variable_length_padding_amd as ee

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "ee.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^EE_API\s+[\w\s\*]+?\b(ee_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = ee.lib()
    declared = _declared()
    assert len(declared) >= 19
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in ee.h but not exported"
    assert sorted(ee.EXPORTED_SYMBOLS) == declared


def test_status_strings_and_version():
    lib = ee.lib()
    assert lib.ee_status_string(0) == b"EE_OK"
    assert lib.ee_status_string(3) == b"EE_ERR_WORKSPACE"
    assert b"gfx950" in lib.ee_version()


def _desc(**kw):
    d = dict(hidden=64, n_heads=4, head_dim=16, ffn=256, ln_eps=1e-5, dtype=ee.F32, gelu=ee.GELU_TANH, fuse_gelu=1,
             block=ee.BLOCK_GPT_PRELN, attention=ee.ATTN_VARLEN, residual=ee.RESIDUAL_AUTO)
    d.update(kw)
    return ee.LayerDesc(*[d[k] for k, _ in ee.LayerDesc._fields_])


def _weights(base=1 << 20):
    return ee.LayerWeights(*[base + 4096 * i for i in range(12)])   # aligned, never dereferenced


def _create(desc, weights):
    h = C.c_void_p()
    st = ee.lib().ee_layer_create(C.byref(desc), C.byref(weights), C.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=24), 2), (dict(head_dim=256), 2), (dict(hidden=0), 1), (dict(ln_eps=0.0), 1),
    (dict(dtype=7), 1), (dict(gelu=5), 1), (dict(fuse_gelu=2), 1), (dict(hidden=66), 2),
    (dict(hidden=65536 * 4, ffn=256), 2), (dict(block=2), 1), (dict(attention=3), 1), (dict(residual=3), 1),
    (dict(residual=-1), 1),
])
def test_layer_create_rejects_bad_descriptors(kw, status):
    st, h = _create(_desc(**kw), _weights())
    assert st == status and not h.value
    assert len(ee.lib().ee_last_error()) > 0


def test_layer_create_rejects_null_and_misaligned_weights():
    w = _weights()
    w.b_fc2 = None
    assert _create(_desc(), w)[0] == 1
    w = _weights()
    w.w_qkv = (1 << 20) + 2
    assert _create(_desc(), w)[0] == 1


def test_forward_validation_happens_before_device_work():
    lib = ee.lib()
    st, h = _create(_desc(), _weights())
    assert st == 0 and h.value
    try:
        n = C.c_size_t(0)
        assert lib.ee_layer_workspace_size(h, 4, 16, -1, C.byref(n)) == 0 and n.value > 0
        n_small = C.c_size_t(0)
        assert lib.ee_layer_workspace_size(h, 4, 16, 10, C.byref(n_small)) == 0 and n_small.value < n.value
        lens = (C.c_int32 * 4)(16, 3, 0, 7)
        x, y, ws = 1 << 30, 1 << 31, 1 << 32
        # workspace too small -> EE_ERR_WORKSPACE
        assert lib.ee_layer_forward(h, x, lens, 4, 16, y, ws, 100, None) == 3
        # a length beyond pad_len -> EE_ERR_INVALID_ARG
        bad = (C.c_int32 * 4)(17, 3, 0, 7)
        assert lib.ee_layer_forward(h, x, bad, 4, 16, y, ws, n.value, None) == 1
        neg = (C.c_int32 * 4)(-1, 3, 0, 7)
        assert lib.ee_layer_forward(h, x, neg, 4, 16, y, ws, n.value, None) == 1
        # overlapping x / y
        assert lib.ee_layer_forward(h, x, lens, 4, 16, x + 64, ws, n.value, None) == 1
        # workspace overlapping the output
        assert lib.ee_layer_forward(h, x, lens, 4, 16, y, y + 256, n.value, None) == 1
        # misaligned input
        assert lib.ee_layer_forward(h, x + 4, lens, 4, 16, y, ws, n.value, None) == 1
        # batch above EE_MAX_BATCH
        big = (C.c_int32 * 513)(*([1] * 513))
        assert lib.ee_layer_forward(h, x, big, 513, 16, y, ws, n.value, None) == 1
        # stack with mismatched descriptors
        st2, h2 = _create(_desc(ffn=512), _weights())
        assert st2 == 0
        arr = (C.c_void_p * 2)(h.value, h2.value)
        assert lib.ee_stack_forward(arr, 2, x, lens, 4, 16, y, ws, n.value, None) == 1
        lib.ee_layer_destroy(h2)
    finally:
        lib.ee_layer_destroy(h)


def test_op_entry_points_validate():
    lib = ee.lib()
    lens = (C.c_int32 * 2)(3, 5)
    n = C.c_size_t(0)
    assert lib.ee_padding_workspace_size(2, 4, C.byref(n)) == 0 and n.value >= 4 * (3 + 16)
    # hidden*sizeof not a multiple of 16 bytes
    assert lib.ee_remove_padding(1 << 30, lens, 2, 8, 6, ee.F16, 1 << 31, 1 << 32, n.value, None) == 2
    # lengths beyond pad_len
    assert lib.ee_rebuild_padding(1 << 30, lens, 2, 4, 64, ee.F16, 1 << 31, 1 << 32, n.value, None) == 1
    # linear: unknown epilogue, missing bias, overlapping output
    assert lib.ee_linear(1 << 30, 1 << 31, 1 << 32, None, 8, 64, 64, ee.F16, 9, 0, 1 << 33, None) == 1
    assert lib.ee_linear(1 << 30, 1 << 31, None, None, 8, 64, 64, ee.F16, ee.EPI_BIAS, 0, 1 << 33, None) == 1
    assert lib.ee_linear(1 << 30, 1 << 31, 1 << 32, None, 8, 64, 64, ee.F16, ee.EPI_BIAS, 0, (1 << 30) + 16,
                         None) == 1
    assert lib.ee_linear(1 << 30, 1 << 31, 1 << 32, None, 8, 64, 64, ee.F16, ee.EPI_BIAS_RESIDUAL, 0, 1 << 33,
                         None) == 1
    # M = 0 is a valid no-op
    assert lib.ee_linear(None, 1 << 31, None, None, 0, 64, 64, ee.F16, ee.EPI_NONE, 0, None, None) == 0
    # linear with a workspace: its size, then a small, a NULL and an overlapping workspace
    need = lib.ee_linear_ws_workspace_size()
    assert need == 4096 + 256 * 256 * 384 * 4
    a, w, c, ws = 1 << 30, 1 << 31, 1 << 33, 1 << 34
    assert lib.ee_linear_ws(a, 64, w, 64, None, None, 8, 64, 64, ee.F16, ee.EPI_NONE, 0, c, 64, ws, need - 1,
                            None) == 3
    assert lib.ee_linear_ws(a, 64, w, 64, None, None, 8, 64, 64, ee.F16, ee.EPI_NONE, 0, c, 64, None, need,
                            None) == 1
    assert lib.ee_linear_ws(a, 64, w, 64, None, None, 8, 64, 64, ee.F16, ee.EPI_NONE, 0, c, 64, c - 4096, need,
                            None) == 1
    # attention: unsupported head_dim
    assert lib.ee_attention_varlen(1 << 30, 1 << 31, 2, 8, 4, 48, 10, 1, ee.F16, 1 << 32, None) == 2
    assert lib.ee_attention_padded(1 << 30, 1 << 31, 1 << 32, 1 << 33, 2, 8, 4, 24, 1, ee.F16, 1 << 34, None) == 2
    assert lib.ee_attention_padded(1 << 30, 1 << 31, 1 << 32, (1 << 30) + 64, 2, 8, 4, 16, 1, ee.F16, 1 << 30,
                                   None) == 1                               # o overlaps q
    n = C.c_size_t(0)
    assert lib.ee_padding_workspace_size(2, 8, C.byref(n)) == 0
    # head rows must be 16-byte multiples; lengths within pad_len
    assert lib.ee_transpose_padding_rebuild_heads(1 << 30, lens, 2, 8, 3, 4, 4, ee.F16, 1 << 31, 1 << 32, n.value,
                                                  None) == 2
    assert lib.ee_transpose_padding_remove_heads(1 << 30, (C.c_int32 * 2)(3, 9), 2, 8, 4, 16, ee.F16, 1 << 31,
                                                 1 << 32, n.value, None) == 1
    assert lib.ee_add_bias_residual_layernorm(1 << 30, 1 << 31, 1 << 32, 1 << 33, 1 << 34, 4, 64, 1e-5, ee.F16,
                                              1 << 30, None) == 1           # y aliases u
    # layernorm: hidden too large / eps <= 0
    assert lib.ee_layernorm(1 << 30, 1 << 31, 1 << 32, 4, 1 << 20, 1e-5, ee.F16, 1 << 33, None) == 2
    assert lib.ee_layernorm(1 << 30, 1 << 31, 1 << 32, 4, 64, -1.0, ee.F16, 1 << 33, None) == 1
    # offsets: bad lengths, null outputs
    total = C.c_int32(0)
    assert lib.ee_compute_offsets((C.c_int32 * 2)(1, 9), 2, 8, 1 << 30, 1 << 31, 1 << 32, C.byref(total), None) == 1
    assert lib.ee_compute_offsets(lens, 2, 8, None, 1 << 31, 1 << 32, C.byref(total), None) == 1
    assert lib.ee_bias_gelu(1 << 30, None, 4, 64, ee.F16, 0, 1 << 31, None) == 1


def test_extend_validation_happens_before_device_work():
    lib = ee.lib()
    st, h = _create(_desc(), _weights())
    assert st == 0
    try:
        arr = (C.c_void_p * 1)(h.value)

        def I(*v):
            return (C.c_int32 * len(v))(*v)
        n = C.c_size_t(0)
        assert lib.ee_extend_workspace_size(h, 2, 8, C.byref(n)) == 0 and n.value > 0
        cb = C.c_size_t(0)
        assert lib.ee_kv_cache_bytes(h, 3, 10, C.byref(cb)) == 0
        assert cb.value == 3 * 2 * 4 * 10 * 16 * 4          # layers x (k|v) x heads x slots x head_dim x fp32
        assert lib.ee_extend_max_positions() >= 4096
        x, y, ws, cache = 1 << 30, 1 << 31, 1 << 32, 1 << 33
        # a sequence's slots past the capacity (base 4 + ctx 5 + new 1 > 8)
        assert lib.ee_stack_extend(arr, 1, x, I(3, 1), I(0, 5), I(0, 4), 2, cache, 8, y, ws, n.value, None) == 1
        # overlapping slot ranges ([0, 3) and [2, 3))
        assert lib.ee_stack_extend(arr, 1, x, I(3, 1), I(0, 0), I(0, 2), 2, cache, 64, y, ws, n.value, None) == 1
        # an idle sequence's cached range still counts
        assert lib.ee_stack_extend(arr, 1, x, I(1, 0), I(0, 6), I(0, 0), 2, cache, 64, y, ws, n.value, None) == 1
        # negative counts, batch above the limit, workspace too small
        assert lib.ee_stack_extend(arr, 1, x, I(-1, 1), I(0, 0), I(0, 8), 2, cache, 64, y, ws, n.value, None) == 1
        big = (C.c_int32 * 257)(*([0] * 257))
        assert lib.ee_stack_extend(arr, 1, x, big, big, big, 257, cache, 64, y, ws, n.value, None) == 1
        assert lib.ee_stack_extend(arr, 1, x, I(3, 1), I(0, 0), I(0, 8), 2, cache, 64, y, ws, 64, None) == 3
        # the cache overlapping the output
        assert lib.ee_stack_extend(arr, 1, x, I(3, 1), I(0, 0), I(0, 8), 2, y + 64, 64, y, ws, n.value, None) == 1
        # nothing new: a no-op
        assert lib.ee_stack_extend(arr, 1, x, I(0, 0), I(2, 3), I(0, 8), 2, cache, 64, y, ws, n.value, None) == 0
        # post-LN encoder layers are not causal
        st2, h2 = _create(_desc(block=ee.BLOCK_BERT_POSTLN), _weights())
        arr2 = (C.c_void_p * 1)(h2.value)
        assert lib.ee_stack_extend(arr2, 1, x, I(3, 1), I(0, 0), I(0, 8), 2, cache, 64, y, ws, n.value, None) == 1
        lib.ee_layer_destroy(h2)
    finally:
        lib.ee_layer_destroy(h)


def test_extend_noalloc_rejects_before_device_work():
    """The no-allocation extend step's own checks (sizes that do not fit its
    static buffer among them) run on the host before any HIP call."""
    lib = ee.lib()
    st, h = _create(_desc(), _weights())
    assert st == 0
    try:
        arr = (C.c_void_p * 1)(h.value)

        def I(*v):
            return (C.c_int32 * len(v))(*v)
        x, y, cache = 1 << 30, 1 << 31, 1 << 33
        assert lib.ee_stack_extend_noalloc(None, 1, x, I(1), I(0), I(0), 1, cache, 8, y, None) == 1
        assert lib.ee_stack_extend_noalloc(arr, 0, x, I(1), I(0), I(0), 1, cache, 8, y, None) == 1
        assert lib.ee_stack_extend_noalloc(arr, 1, x, I(1), I(0), I(0), 0, cache, 8, y, None) == 1
        assert lib.ee_stack_extend_noalloc(arr, 1, x, I(-1, 2), I(0, 0), I(0, 4), 2, cache, 8, y, None) == 1
        n = C.c_size_t(0)
        T = 2_000_000                      # a workspace of several GB: above the static buffer
        assert lib.ee_extend_workspace_size(h, 1, T, C.byref(n)) == 0 and n.value > ee.NOALLOC_SCRATCH_BYTES
        assert lib.ee_stack_extend_noalloc(arr, 1, x, I(T), I(0), I(0), 1, cache, T, y, None) == 3
        assert b"no-allocation" in lib.ee_last_error()
    finally:
        lib.ee_layer_destroy(h)


def test_debug_sync_toggles_without_device_work():
    lib = ee.lib()
    assert lib.ee_debug_sync(1) == 0 and lib.ee_debug_sync(0) == 0


def test_preferred_row_pitch():
    lib = ee.lib()
    # a row that is a multiple of 32 KiB gets 128 bytes more; others stay dense
    assert lib.ee_preferred_row_pitch(49152, ee.F16) == 49216
    assert lib.ee_preferred_row_pitch(16384, ee.F16) == 16448
    assert lib.ee_preferred_row_pitch(8192, ee.F32) == 8224
    assert lib.ee_preferred_row_pitch(12288, ee.F16) == 12288
    assert lib.ee_preferred_row_pitch(3072, ee.F16) == 3072
    assert lib.ee_preferred_row_pitch(24576, ee.F16) == 24576
    assert lib.ee_preferred_row_pitch(0, ee.F16) == 0
    assert lib.ee_preferred_row_pitch(64, 7) == 0


def test_linear_strided_validates_pitches():
    lib = ee.lib()
    A, W, b, C_ = 1 << 30, 1 << 31, 1 << 32, 1 << 33
    # pitches below the row lengths
    assert lib.ee_linear_strided(A, 63, W, 64, b, None, 8, 32, 64, ee.F16, ee.EPI_BIAS, 0, C_, 32, None) == 1
    assert lib.ee_linear_strided(A, 64, W, 60, b, None, 8, 32, 64, ee.F16, ee.EPI_BIAS, 0, C_, 32, None) == 1
    assert lib.ee_linear_strided(A, 64, W, 64, b, None, 8, 32, 64, ee.F16, ee.EPI_BIAS, 0, C_, 31, None) == 1
    assert lib.ee_linear_strided(A, 1 << 31, W, 64, b, None, 8, 32, 64, ee.F16, ee.EPI_BIAS, 0, C_, 32, None) == 1
    # C's pitched extent (7 rows x 1000 + 32 elements) reaches the bias
    assert lib.ee_linear_strided(A, 64, W, 64, C_ + 2 * 7000, None, 8, 32, 64, ee.F16, ee.EPI_BIAS, 0, C_, 1000,
                                 None) == 1
    # M = 0 is a valid no-op with any valid pitches
    assert lib.ee_linear_strided(None, 72, W, 72, None, None, 0, 32, 64, ee.F16, ee.EPI_NONE, 0, None, 40, None) == 0


@pytest.mark.parametrize("field,value,status", [
    ("ld_fc2", 255, 1), ("ld_fc2", 257, 1), ("ld_qkv", 63, 1), ("ld_out", 1 << 31, 1),
    ("ld_fc2", 260, 0), ("ld_fc1", 0, 0), ("ld_out", 68, 0),
])
def test_layer_create_validates_weight_pitches(field, value, status):
    w = _weights()
    setattr(w, field, value)      # fp32, H = 64, H' = 64, F = 256
    st, h = _create(_desc(), w)
    assert st == status
    if h.value:
        ee.lib().ee_layer_destroy(h)


def test_profile_filter_validates_and_resets():
    """ee_profile_filter copies a site name shorter than the stat name field,
    rejects longer ones, and NULL or "" restore timing every site (host only)."""
    lib = ee.lib()
    assert lib.ee_profile_filter(b"gemm_fc1") == 0
    assert lib.ee_profile_filter(b"x" * 31) == 0
    assert lib.ee_profile_filter(b"x" * 32) == 1
    assert lib.ee_profile_filter(b"") == 0
    assert lib.ee_profile_filter(None) == 0
