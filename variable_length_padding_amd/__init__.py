"""Python binding of libee (include/ee.h): argument marshalling only.

Every function here converts torch tensors / Python values into the C ABI's
plain pointers and sizes and calls libee; all work of the padding-removed layer
forward runs in libee's HIP kernels.  torch supplies device memory and streams.
There is no fallback: if libee.so is not built, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

__all__ = [
    "EEError", "lib", "F32", "F16", "GELU_TANH", "GELU_ERF",
    "EPI_NONE", "EPI_BIAS", "EPI_BIAS_RESIDUAL", "EPI_BIAS_GELU",
    "ee_compute_offsets", "ee_compute_offsets_mask", "ee_padding_workspace_size",
    "ee_remove_padding", "ee_rebuild_padding", "ee_layernorm", "ee_linear", "ee_linear_ws",
    "ee_linear_ws_workspace_size", "ee_bias_gelu",
    "ee_linear_splitk", "ee_linear_splitk_workspace_size", "ee_linear_streamk", "ee_linear_streamk_workspace_size",
    "ee_attention_varlen", "ee_attention_padded", "ee_transpose_padding_rebuild_heads",
    "ee_transpose_padding_remove_heads", "ee_add_bias_residual_layernorm",
    "BLOCK_GPT_PRELN", "BLOCK_BERT_POSTLN", "ATTN_VARLEN", "ATTN_PADDED",
    "Layer", "ee_stack_forward", "ee_profile_enable", "ee_profile_filter", "ee_profile_collect", "ee_debug_sync",
    "ee_kv_cache_bytes", "ee_extend_workspace_size", "ee_extend_max_positions", "ee_stack_extend",
    "ee_stack_extend_noalloc", "NOALLOC_SCRATCH_BYTES",
    "MAX_EXTEND_BATCH",
    "BatchCost", "ee_batch_cost_eval", "ee_plan_fifo", "ee_plan_dynamic", "batches_of",
    "EXPORTED_SYMBOLS", "lib_path",
]

F32, F16 = 0, 1
GELU_TANH, GELU_ERF = 0, 1
EPI_NONE, EPI_BIAS, EPI_BIAS_RESIDUAL, EPI_BIAS_GELU = 0, 1, 2, 3
BLOCK_GPT_PRELN, BLOCK_BERT_POSTLN = 0, 1
ATTN_VARLEN, ATTN_PADDED = 0, 1
RESIDUAL_AUTO, RESIDUAL_EPILOGUE, RESIDUAL_PASS = 0, 1, 2
MAX_BATCH = 512
MAX_EXTEND_BATCH = 256

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree libee.so, or the build EE_LIBRARY names (a host-sanitizer
    build of the same sources, see build.py)."""
    return os.environ.get("EE_LIBRARY") or os.path.join(_HERE, "libee.so")


class EEError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "EE_OK", 1: "EE_ERR_INVALID_ARG", 2: "EE_ERR_UNSUPPORTED", 3: "EE_ERR_WORKSPACE",
           4: "EE_ERR_OOM", 5: "EE_ERR_HIP"}


class LayerDesc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("ln_eps", C.c_float), ("dtype", C.c_int), ("gelu", C.c_int), ("fuse_gelu", C.c_int32),
                ("block", C.c_int), ("attention", C.c_int), ("residual", C.c_int)]


WEIGHT_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_out", "b_out",
                 "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")


# row pitch fields (elements; 0 = dense) of the four weight matrices, in order
PITCH_FIELDS = (("w_qkv", "ld_qkv"), ("w_out", "ld_out"), ("w_fc1", "ld_fc1"), ("w_fc2", "ld_fc2"))


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS] + [(ld, C.c_int64) for _, ld in PITCH_FIELDS]


class KernelStat(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int64), ("total_ms", C.c_double), ("flops", C.c_double),
                ("kernel", C.c_char * 96)]


class BatchCost(C.Structure):
    """Per-batch cost model of the batch planners (seconds).  A token table is
    kept alive by the structure (`_table`)."""
    _fields_ = [("t_batch", C.c_double), ("t_token", C.c_double), ("t_row", C.c_double), ("t_pair", C.c_double),
                ("token_quantum", C.c_int32), ("padded_compute", C.c_int32),
                ("token_table", C.POINTER(C.c_double)), ("token_table_len", C.c_int32)]

    def set_table(self, seconds: Sequence[float]):
        self._table = (C.c_double * max(1, len(seconds)))(*[float(v) for v in seconds])
        self.token_table = self._table
        self.token_table_len = len(seconds)
        return self


_VP, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_PI32 = C.POINTER(C.c_int32)

# name -> (restype, argtypes); the list of exported functions of include/ee.h
_SIGS = {
    "ee_status_string": (C.c_char_p, [C.c_int]),
    "ee_last_error": (C.c_char_p, []),
    "ee_version": (C.c_char_p, []),
    "ee_layer_create": (C.c_int, [C.POINTER(LayerDesc), C.POINTER(LayerWeights), C.POINTER(_VP)]),
    "ee_layer_destroy": (C.c_int, [_VP]),
    "ee_layer_workspace_size": (C.c_int, [_VP, _I32, _I32, _I64, C.POINTER(_SZ)]),
    "ee_layer_forward": (C.c_int, [_VP, _VP, _PI32, _I32, _I32, _VP, _VP, _SZ, _VP]),
    "ee_stack_forward": (C.c_int, [C.POINTER(_VP), _I32, _VP, _PI32, _I32, _I32, _VP, _VP, _SZ, _VP]),
    "ee_compute_offsets": (C.c_int, [_PI32, _I32, _I32, _VP, _VP, _VP, _PI32, _VP]),
    "ee_compute_offsets_mask": (C.c_int, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
    "ee_padding_workspace_size": (C.c_int, [_I32, _I32, C.POINTER(_SZ)]),
    "ee_remove_padding": (C.c_int, [_VP, _PI32, _I32, _I32, _I32, C.c_int, _VP, _VP, _SZ, _VP]),
    "ee_rebuild_padding": (C.c_int, [_VP, _PI32, _I32, _I32, _I32, C.c_int, _VP, _VP, _SZ, _VP]),
    "ee_layernorm": (C.c_int, [_VP, _VP, _VP, _I64, _I32, C.c_float, C.c_int, _VP, _VP]),
    "ee_linear": (C.c_int, [_VP, _VP, _VP, _VP, _I64, _I32, _I32, C.c_int, C.c_int, C.c_int, _VP, _VP]),
    "ee_linear_strided": (C.c_int, [_VP, _I64, _VP, _I64, _VP, _VP, _I64, _I32, _I32, C.c_int, C.c_int, C.c_int, _VP,
                                    _I64, _VP]),
    "ee_linear_ws_workspace_size": (_SZ, []),
    "ee_linear_ws": (C.c_int, [_VP, _I64, _VP, _I64, _VP, _VP, _I64, _I32, _I32, C.c_int, C.c_int, C.c_int, _VP,
                               _I64, _VP, _SZ, _VP]),
    "ee_preferred_row_pitch": (_I64, [_I64, C.c_int]),
    "ee_bias_gelu": (C.c_int, [_VP, _VP, _I64, _I32, C.c_int, C.c_int, _VP, _VP]),
    "ee_linear_splitk_workspace_size": (C.c_int, [_I64, _I32, _I32, C.POINTER(_SZ)]),
    "ee_linear_splitk": (C.c_int, [_VP, _VP, _VP, _VP, _I64, _I32, _I32, C.c_int, C.c_int, C.c_int, _I32, _VP, _VP,
                                   _SZ, _VP]),
    "ee_linear_streamk_workspace_size": (C.c_int, [_I64, _I32, _I32, C.POINTER(_SZ)]),
    "ee_linear_streamk": (C.c_int, [_VP, _VP, _VP, _VP, _I64, _I32, _I32, C.c_int, C.c_int, C.c_int, _VP, _VP, _SZ,
                                    _VP]),
    "ee_attention_varlen": (C.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _I64, _I32, C.c_int, _VP, _VP]),
    "ee_attention_padded": (C.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32, _I32, C.c_int, _VP, _VP]),
    "ee_transpose_padding_rebuild_heads": (C.c_int, [_VP, _PI32, _I32, _I32, _I32, _I32, _I32, C.c_int, _VP, _VP,
                                                     _SZ, _VP]),
    "ee_transpose_padding_remove_heads": (C.c_int, [_VP, _PI32, _I32, _I32, _I32, _I32, C.c_int, _VP, _VP, _SZ,
                                                    _VP]),
    "ee_add_bias_residual_layernorm": (C.c_int, [_VP, _VP, _VP, _VP, _VP, _I64, _I32, C.c_float, C.c_int, _VP,
                                                 _VP]),
    "ee_profile_enable": (C.c_int, [_I32]),
    "ee_debug_sync": (C.c_int, [_I32]),
    "ee_profile_filter": (C.c_int, [C.c_char_p]),
    "ee_profile_collect": (C.c_int, [C.POINTER(KernelStat), _I32, _PI32]),
    "ee_kv_cache_bytes": (C.c_int, [_VP, _I32, _I64, C.POINTER(_SZ)]),
    "ee_extend_workspace_size": (C.c_int, [_VP, _I32, _I64, C.POINTER(_SZ)]),
    "ee_extend_max_positions": (C.c_int32, []),
    "ee_stack_extend": (C.c_int, [C.POINTER(_VP), _I32, _VP, _PI32, _PI32, _PI32, _I32, _VP, _I64, _VP, _VP, _SZ,
                                  _VP]),
    "ee_stack_extend_noalloc": (C.c_int, [C.POINTER(_VP), _I32, _VP, _PI32, _PI32, _PI32, _I32, _VP, _I64, _VP,
                                          _VP]),
    "ee_batch_cost_eval": (C.c_int, [_PI32, _I32, C.POINTER(BatchCost), C.POINTER(C.c_double)]),
    "ee_plan_fifo": (C.c_int, [_PI32, _I32, _I32, _PI32, _PI32]),
    "ee_plan_dynamic": (C.c_int, [_PI32, C.POINTER(C.c_double), _I32, _I32, _I64, C.POINTER(BatchCost), _PI32,
                                  _PI32, C.POINTER(C.c_double)]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


def lib():
    """The loaded libee (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m variable_length_padding_amd.build`")
        L = C.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, func: str):
    if status != 0:
        raise EEError(status, func, lib().ee_last_error().decode())


# ---------------------------------------------------------------- helpers
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _row_pitch(t, dense: bool = False) -> int:
    """Row pitch (elements) of a 2-D tensor with unit column stride; 0 for a
    contiguous tensor unless `dense` asks for its row length."""
    if t is None:
        return 0
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("need a 2-D tensor with unit column stride")
    if t.is_contiguous():
        return t.shape[1] if dense else 0
    return t.stride(0)


def _lens(lens: Sequence[int]):
    arr = (C.c_int32 * max(1, len(lens)))(*[int(n) for n in lens])
    return arr


# ---------------------------------------------------------------- argument checks
# Run before any library call: the library validates sizes and pointers, but
# only the binding sees a tensor's shape, dtype, layout and device, and a
# lengths list shorter than the batch would make the library read past it.
def _torch_dtype(code: int):
    import torch
    return torch.float16 if code == F16 else torch.float32


def _shape_ok(t, shape) -> bool:
    return t.dim() == len(shape) and all(s is None or int(a) == int(s) for a, s in zip(t.shape, shape))


def _need(t, name: str, shape=None, dtype=None, contiguous: bool = True):
    """A tensor argument: its shape (None entries free), dtype and layout."""
    if t is None:
        raise ValueError(f"{name} is required")
    if shape is not None and not _shape_ok(t, shape):
        want = "[" + ", ".join("*" if s is None else str(int(s)) for s in shape) + "]"
        raise ValueError(f"{name} has shape {list(t.shape)}, need {want}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, need {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_lens(lens: Sequence[int], batch: int, name: str = "lens"):
    if len(lens) != batch:
        raise ValueError(f"{name} has {len(lens)} entries for a batch of {batch}")


def _need_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (device {t.device})")


def _need_workspace(ws, name: str = "workspace"):
    _need(ws, name)
    _need_gpu(**{name: ws})


# ---------------------------------------------------------------- offsets
def ee_compute_offsets(lens: Sequence[int], pad_len: int, cu, token_src, pad2pack, stream=None) -> int:
    """Host lengths -> device cu [B+1], token_src [B*P], pad2pack [B*P] (int32); returns T."""
    import torch
    B = len(lens)
    _need(cu, "cu", (B + 1,), torch.int32)
    _need(token_src, "token_src", (B * pad_len,), torch.int32)
    _need(pad2pack, "pad2pack", (B * pad_len,), torch.int32)
    _need_gpu(cu=cu, token_src=token_src, pad2pack=pad2pack)
    total = C.c_int32(0)
    _check(lib().ee_compute_offsets(_lens(lens), len(lens), pad_len, _ptr(cu), _ptr(token_src), _ptr(pad2pack),
                                    C.byref(total), _stream(stream)), "ee_compute_offsets")
    return total.value


def ee_compute_offsets_mask(mask, cu, token_src, pad2pack, total, stream=None):
    """Device uint8 mask [B, P] -> cu, token_src, pad2pack, total (device int32)."""
    import torch
    if mask is None or mask.dim() != 2:
        raise ValueError("mask must be [batch, pad_len]")
    B, P = mask.shape
    _need(mask, "mask", (B, P), torch.uint8)
    _need(cu, "cu", (B + 1,), torch.int32)
    _need(token_src, "token_src", (B * P,), torch.int32)
    _need(pad2pack, "pad2pack", (B * P,), torch.int32)
    _need(total, "total", (1,), torch.int32)
    _need_gpu(mask=mask, cu=cu, token_src=token_src, pad2pack=pad2pack, total=total)
    _check(lib().ee_compute_offsets_mask(_ptr(mask), B, P, _ptr(cu), _ptr(token_src), _ptr(pad2pack), _ptr(total),
                                         _stream(stream)), "ee_compute_offsets_mask")


def ee_padding_workspace_size(batch: int, pad_len: int) -> int:
    n = C.c_size_t(0)
    _check(lib().ee_padding_workspace_size(batch, pad_len, C.byref(n)), "ee_padding_workspace_size")
    return n.value


def _padding_args(padded, lens, packed, workspace, packed_name):
    if padded is None or padded.dim() != 3:
        raise ValueError("the padded tensor must be [batch, pad_len, hidden]")
    B, P, H = padded.shape
    _need_lens(lens, B)
    _dtype_code(padded)
    _need(padded, "padded", (B, P, H))
    T = sum(int(n) for n in lens)
    _need(packed, packed_name, (None, H), padded.dtype)
    if packed.shape[0] < T:
        raise ValueError(f"{packed_name} has {packed.shape[0]} rows, need sum(lens) = {T}")
    _need_gpu(padded=padded, **{packed_name: packed})
    _need_workspace(workspace)
    return B, P, H


def ee_remove_padding(padded, lens: Sequence[int], packed, workspace, stream=None):
    B, P, H = _padding_args(padded, lens, packed, workspace, "packed")
    _check(lib().ee_remove_padding(_ptr(padded), _lens(lens), B, P, H, _dtype_code(padded), _ptr(packed),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "ee_remove_padding")


def ee_rebuild_padding(packed, lens: Sequence[int], padded, workspace, stream=None):
    B, P, H = _padding_args(padded, lens, packed, workspace, "packed")
    _check(lib().ee_rebuild_padding(_ptr(packed), _lens(lens), B, P, H, _dtype_code(padded), _ptr(padded),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "ee_rebuild_padding")


# ---------------------------------------------------------------- row ops
def ee_layernorm(x, gamma, beta, eps: float, y, stream=None):
    if x is None or x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    rows, H = x.shape
    _dtype_code(x)
    _need(x, "x", (rows, H))
    _need(y, "y", (rows, H), x.dtype)
    _need(gamma, "gamma", (H,), x.dtype)
    _need(beta, "beta", (H,), x.dtype)
    _need_gpu(x=x, y=y, gamma=gamma, beta=beta)
    _check(lib().ee_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), rows, H, eps, _dtype_code(x), _ptr(y),
                              _stream(stream)), "ee_layernorm")


def _linear_args(A, W, bias, residual, epi, C_out, strided):
    if A is None or A.dim() != 2 or W is None or W.dim() != 2:
        raise ValueError("A must be [M, K] and W [N, K]")
    M, K = A.shape
    N = W.shape[0]
    _dtype_code(A)
    _need(A, "A", (M, K), contiguous=not strided)
    _need(W, "W", (N, K), A.dtype, contiguous=not strided)
    _need(C_out, "C_out", (M, N), A.dtype, contiguous=not strided)
    if epi != EPI_NONE or bias is not None:
        _need(bias, "bias", (N,), A.dtype)
    if epi == EPI_BIAS_RESIDUAL or residual is not None:
        _need(residual, "residual", (M, N), A.dtype, contiguous=not strided)
    _need_gpu(A=A, W=W, bias=bias, residual=residual, C_out=C_out)
    return M, N, K


def ee_linear(A, W, bias, residual, epi: int, C_out, gelu: int = GELU_TANH, stream=None):
    """C_out = epilogue(A . W^T); 2-D tensors whose rows may be strided
    (unit column stride): their row strides are passed as the pitches."""
    M, N, K = _linear_args(A, W, bias, residual, epi, C_out, strided=True)
    if all(t is None or t.is_contiguous() for t in (A, W, residual, C_out)):
        _check(lib().ee_linear(_ptr(A), _ptr(W), _ptr(bias), _ptr(residual), M, N, K, _dtype_code(A), epi, gelu,
                               _ptr(C_out), _stream(stream)), "ee_linear")
        return
    ldc = _row_pitch(C_out, dense=True)
    if residual is not None and _row_pitch(residual, dense=True) != ldc:
        raise ValueError("residual and C_out must share a row pitch")
    _check(lib().ee_linear_strided(_ptr(A), _row_pitch(A, dense=True), _ptr(W), _row_pitch(W, dense=True), _ptr(bias),
                                   _ptr(residual), M, N, K, _dtype_code(A), epi, gelu, _ptr(C_out), ldc,
                                   _stream(stream)), "ee_linear_strided")


def ee_linear_ws_workspace_size() -> int:
    """Bytes of workspace ee_linear_ws needs."""
    return int(lib().ee_linear_ws_workspace_size())


def ee_linear_ws(A, W, bias, residual, epi: int, C_out, workspace, gelu: int = GELU_TANH, stream=None):
    """ee_linear with a workspace: a large fp16 problem runs its partial last
    round of tiles as in-order stream-K pieces (the same bits as ee_linear)."""
    M, N, K = _linear_args(A, W, bias, residual, epi, C_out, strided=True)
    _need_workspace(workspace)
    _need_gpu(workspace=workspace)
    ldc = _row_pitch(C_out, dense=True)
    if residual is not None and _row_pitch(residual, dense=True) != ldc:
        raise ValueError("residual and C_out must share a row pitch")
    _check(lib().ee_linear_ws(_ptr(A), _row_pitch(A, dense=True), _ptr(W), _row_pitch(W, dense=True), _ptr(bias),
                              _ptr(residual), M, N, K, _dtype_code(A), epi, gelu, _ptr(C_out), ldc, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream)), "ee_linear_ws")


def ee_preferred_row_pitch(cols: int, dtype: int = F16) -> int:
    """Row pitch (elements) the library suggests for a matrix of `cols` columns."""
    return int(lib().ee_preferred_row_pitch(cols, dtype))


def pitched(t):
    """A copy of the 2-D tensor t stored at ee_preferred_row_pitch (a view of
    the first t.shape[1] columns of a wider tensor), or t itself when the
    dense pitch is already the preferred one."""
    import torch
    rows, cols = t.shape
    ld = ee_preferred_row_pitch(cols, _dtype_code(t))
    if ld == cols and t.is_contiguous():
        return t
    buf = torch.zeros(rows, ld, dtype=t.dtype, device=t.device)
    buf[:, :cols] = t
    return buf[:, :cols]


def pitched_weights(params: Dict) -> Dict:
    """A layer's parameter dict with the four weight matrices stored at
    ee_preferred_row_pitch (see `pitched`); the other tensors as given."""
    return {k: pitched(v) if k in ("w_qkv", "w_out", "w_fc1", "w_fc2") else v for k, v in params.items()}


def ee_linear_splitk_workspace_size(M: int, N: int, splits: int) -> int:
    n = C.c_size_t(0)
    _check(lib().ee_linear_splitk_workspace_size(M, N, splits, C.byref(n)), "ee_linear_splitk_workspace_size")
    return n.value


def ee_linear_splitk(A, W, bias, residual, epi: int, C_out, splits: int, workspace, gelu: int = GELU_TANH,
                     stream=None):
    M, N, K = _linear_args(A, W, bias, residual, epi, C_out, strided=False)
    _need_workspace(workspace)
    _check(lib().ee_linear_splitk(_ptr(A), _ptr(W), _ptr(bias), _ptr(residual), M, N, K, _dtype_code(A), epi, gelu,
                                  splits, _ptr(C_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)), "ee_linear_splitk")


def ee_linear_streamk_workspace_size(M: int, N: int, K: int) -> int:
    n = C.c_size_t(0)
    _check(lib().ee_linear_streamk_workspace_size(M, N, K, C.byref(n)), "ee_linear_streamk_workspace_size")
    return n.value


def ee_linear_streamk(A, W, bias, residual, epi: int, C_out, workspace, gelu: int = GELU_TANH, stream=None):
    M, N, K = _linear_args(A, W, bias, residual, epi, C_out, strided=False)
    _need_workspace(workspace)
    _check(lib().ee_linear_streamk(_ptr(A), _ptr(W), _ptr(bias), _ptr(residual), M, N, K, _dtype_code(A), epi, gelu,
                                   _ptr(C_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "ee_linear_streamk")


def ee_bias_gelu(u, bias, g, gelu: int = GELU_TANH, stream=None):
    if u is None or u.dim() != 2:
        raise ValueError("u must be [rows, cols]")
    rows, cols = u.shape
    _dtype_code(u)
    _need(u, "u", (rows, cols))
    _need(bias, "bias", (cols,), u.dtype)
    _need(g, "g", (rows, cols), u.dtype)
    _need_gpu(u=u, bias=bias, g=g)
    _check(lib().ee_bias_gelu(_ptr(u), _ptr(bias), rows, cols, _dtype_code(u), gelu, _ptr(g), _stream(stream)),
           "ee_bias_gelu")


def ee_attention_varlen(qkv, cu, batch: int, max_len: int, n_heads: int, head_dim: int, o, causal: bool = True,
                        stream=None):
    import torch
    Hp = n_heads * head_dim
    if qkv is None or qkv.dim() != 2:
        raise ValueError("qkv must be [T, 3 * n_heads * head_dim]")
    _dtype_code(qkv)
    _need(qkv, "qkv", (None, 3 * Hp))
    _need(o, "o", (qkv.shape[0], Hp), qkv.dtype)
    _need(cu, "cu", (batch + 1,), torch.int32)
    _need_gpu(qkv=qkv, o=o, cu=cu)
    _check(lib().ee_attention_varlen(_ptr(qkv), _ptr(cu), batch, max_len, n_heads, head_dim, qkv.shape[0],
                                     1 if causal else 0, _dtype_code(qkv), _ptr(o), _stream(stream)),
           "ee_attention_varlen")


def ee_attention_padded(q, k, v, cu, o, causal: bool = True, stream=None):
    """q, k, v, o: [B, nh, P, hd] head-major padded; cu [B+1] device int32."""
    import torch
    if q is None or q.dim() != 4:
        raise ValueError("q must be [batch, n_heads, pad_len, head_dim]")
    B, nh, P, hd = q.shape
    _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, (B, nh, P, hd), q.dtype)
    _need(cu, "cu", (B + 1,), torch.int32)
    _need_gpu(q=q, k=k, v=v, o=o, cu=cu)
    _check(lib().ee_attention_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), B, P, nh, hd, 1 if causal else 0,
                                     _dtype_code(q), _ptr(o), _stream(stream)), "ee_attention_padded")


def ee_transpose_padding_rebuild_heads(packed, lens: Sequence[int], heads, workspace, stream=None):
    """packed [T, n*nh*hd] -> heads [n, B, nh, P, hd] (pads zero)."""
    if heads is None or heads.dim() != 5:
        raise ValueError("heads must be [n_mats, batch, n_heads, pad_len, head_dim]")
    n, B, nh, P, hd = heads.shape
    _need_lens(lens, B)
    _dtype_code(heads)
    _need(heads, "heads", (n, B, nh, P, hd))
    _need(packed, "packed", (None, n * nh * hd), heads.dtype)
    if packed.shape[0] < sum(int(x) for x in lens):
        raise ValueError(f"packed has {packed.shape[0]} rows, need sum(lens) = {sum(int(x) for x in lens)}")
    _need_gpu(packed=packed, heads=heads)
    _need_workspace(workspace)
    _check(lib().ee_transpose_padding_rebuild_heads(_ptr(packed), _lens(lens), B, P, n, nh, hd, _dtype_code(heads),
                                                    _ptr(heads), _ptr(workspace),
                                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "ee_transpose_padding_rebuild_heads")


def ee_transpose_padding_remove_heads(heads, lens: Sequence[int], packed, workspace, stream=None):
    """heads [B, nh, P, hd] -> packed [T, nh*hd]."""
    if heads is None or heads.dim() != 4:
        raise ValueError("heads must be [batch, n_heads, pad_len, head_dim]")
    B, nh, P, hd = heads.shape
    _need_lens(lens, B)
    _dtype_code(heads)
    _need(heads, "heads", (B, nh, P, hd))
    _need(packed, "packed", (None, nh * hd), heads.dtype)
    if packed.shape[0] < sum(int(x) for x in lens):
        raise ValueError(f"packed has {packed.shape[0]} rows, need sum(lens) = {sum(int(x) for x in lens)}")
    _need_gpu(packed=packed, heads=heads)
    _need_workspace(workspace)
    _check(lib().ee_transpose_padding_remove_heads(_ptr(heads), _lens(lens), B, P, nh, hd, _dtype_code(heads),
                                                   _ptr(packed), _ptr(workspace),
                                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "ee_transpose_padding_remove_heads")


def ee_add_bias_residual_layernorm(u, bias, residual, gamma, beta, eps: float, y, stream=None):
    if u is None or u.dim() != 2:
        raise ValueError("u must be [rows, hidden]")
    rows, H = u.shape
    _dtype_code(u)
    _need(u, "u", (rows, H))
    for name, t, shp in (("residual", residual, (rows, H)), ("y", y, (rows, H)), ("bias", bias, (H,)),
                         ("gamma", gamma, (H,)), ("beta", beta, (H,))):
        _need(t, name, shp, u.dtype)
    _need_gpu(u=u, bias=bias, residual=residual, gamma=gamma, beta=beta, y=y)
    _check(lib().ee_add_bias_residual_layernorm(_ptr(u), _ptr(bias), _ptr(residual), _ptr(gamma), _ptr(beta), rows, H,
                                                eps, _dtype_code(u), _ptr(y), _stream(stream)),
           "ee_add_bias_residual_layernorm")


# ---------------------------------------------------------------- layer
class Layer:
    """A layer handle: borrows the weight tensors (kept alive by this object)."""

    def __init__(self, hidden: int, n_heads: int, head_dim: int, ffn: int, weights: Dict, dtype: int = F16,
                 ln_eps: float = 1e-5, gelu: int = GELU_TANH, fuse_gelu: bool = True, block: int = BLOCK_GPT_PRELN,
                 attention: int = ATTN_VARLEN, residual: int = RESIDUAL_AUTO):
        self.desc = LayerDesc(hidden, n_heads, head_dim, ffn, ln_eps, dtype, gelu, 1 if fuse_gelu else 0, block,
                              attention, residual)
        self._weights = {k: weights[k] for k in WEIGHT_FIELDS}
        w = LayerWeights(*[_ptr(self._weights[k]) for k in WEIGHT_FIELDS],
                         *[_row_pitch(self._weights[k]) for k, _ in PITCH_FIELDS])
        h = C.c_void_p()
        _check(lib().ee_layer_create(C.byref(self.desc), C.byref(w), C.byref(h)), "ee_layer_create")
        self.handle = h

    def workspace_size(self, batch: int, pad_len: int, max_tokens: int = -1) -> int:
        n = C.c_size_t(0)
        _check(lib().ee_layer_workspace_size(self.handle, batch, pad_len, max_tokens, C.byref(n)),
               "ee_layer_workspace_size")
        return n.value

    def check_io(self, x, lens: Sequence[int], y, workspace):
        """The checks of forward()'s arguments (also used by ee_stack_forward)."""
        if x is None or x.dim() != 3:
            raise ValueError("x must be [batch, pad_len, hidden]")
        B, P, H = x.shape
        _need_lens(lens, B)
        dt = _torch_dtype(self.desc.dtype)
        _need(x, "x", (B, P, self.desc.hidden), dt)
        _need(y, "y", (B, P, self.desc.hidden), dt)
        _need_gpu(x=x, y=y)
        _need_workspace(workspace)
        return B, P

    def forward(self, x, lens: Sequence[int], y, workspace, stream=None):
        B, P = self.check_io(x, lens, y, workspace)
        _check(lib().ee_layer_forward(self.handle, _ptr(x), _lens(lens), B, P, _ptr(y), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
               "ee_layer_forward")

    def close(self):
        if self.handle:
            lib().ee_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ee_kv_cache_bytes(layer: Layer, n_layers: int, capacity: int) -> int:
    """Bytes of a KV cache of `capacity` slots per layer for n_layers layers."""
    n = C.c_size_t(0)
    _check(lib().ee_kv_cache_bytes(layer.handle, n_layers, capacity, C.byref(n)), "ee_kv_cache_bytes")
    return n.value


def ee_extend_workspace_size(layer: Layer, batch: int, max_new_tokens: int) -> int:
    n = C.c_size_t(0)
    _check(lib().ee_extend_workspace_size(layer.handle, batch, max_new_tokens, C.byref(n)),
           "ee_extend_workspace_size")
    return n.value


def ee_extend_max_positions() -> int:
    return int(lib().ee_extend_max_positions())


def ee_stack_extend(layers: List[Layer], x, new_len: Sequence[int], ctx_len: Sequence[int],
                    slot_base: Sequence[int], cache, capacity: int, y, workspace, stream=None):
    """One extend step: x/y device [sum(new_len), hidden]; cache device buffer of
    ee_kv_cache_bytes(layers[0], len(layers), capacity) bytes."""
    B = len(new_len)
    if len(ctx_len) != B or len(slot_base) != B:
        raise ValueError("new_len, ctx_len and slot_base must have one entry per sequence")
    if not layers:
        raise ValueError("need at least one layer")
    T = sum(int(n) for n in new_len)
    dt = _torch_dtype(layers[0].desc.dtype)
    H = layers[0].desc.hidden
    _need(x, "x", (T, H), dt)
    _need(y, "y", (T, H), dt)
    _need(cache, "cache")
    need = ee_kv_cache_bytes(layers[0], len(layers), capacity)
    if cache.numel() * cache.element_size() < need:
        raise ValueError(f"cache of {cache.numel() * cache.element_size()} bytes, need {need}")
    _need_gpu(x=x, y=y, cache=cache)
    _need_workspace(workspace)
    arr = (C.c_void_p * len(layers))(*[l.handle.value for l in layers])
    _check(lib().ee_stack_extend(arr, len(layers), _ptr(x), _lens(new_len), _lens(ctx_len), _lens(slot_base), B,
                                 _ptr(cache), int(capacity), _ptr(y), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)), "ee_stack_extend")


NOALLOC_SCRATCH_BYTES = 128 << 20


def ee_stack_extend_noalloc(layers: List[Layer], x, new_len: Sequence[int], ctx_len: Sequence[int],
                            slot_base: Sequence[int], cache, capacity: int, y, stream=None):
    """ee_stack_extend without a workspace argument: the library's static
    scratch buffer (NOALLOC_SCRATCH_BYTES per GPU) serves as the workspace."""
    B = len(new_len)
    if len(ctx_len) != B or len(slot_base) != B:
        raise ValueError("new_len, ctx_len and slot_base must have one entry per sequence")
    if not layers:
        raise ValueError("need at least one layer")
    T = sum(int(n) for n in new_len)
    dt = _torch_dtype(layers[0].desc.dtype)
    H = layers[0].desc.hidden
    _need(x, "x", (T, H), dt)
    _need(y, "y", (T, H), dt)
    _need(cache, "cache")
    need = ee_kv_cache_bytes(layers[0], len(layers), capacity)
    if cache.numel() * cache.element_size() < need:
        raise ValueError(f"cache of {cache.numel() * cache.element_size()} bytes, need {need}")
    _need_gpu(x=x, y=y, cache=cache)
    arr = (C.c_void_p * len(layers))(*[l.handle.value for l in layers])
    _check(lib().ee_stack_extend_noalloc(arr, len(layers), _ptr(x), _lens(new_len), _lens(ctx_len), _lens(slot_base),
                                         B, _ptr(cache), int(capacity), _ptr(y), _stream(stream)),
           "ee_stack_extend_noalloc")


def ee_stack_forward(layers: List[Layer], x, lens: Sequence[int], y, workspace, stream=None):
    if not layers:
        raise ValueError("need at least one layer")
    B, P = layers[0].check_io(x, lens, y, workspace)
    arr = (C.c_void_p * len(layers))(*[l.handle.value for l in layers])
    _check(lib().ee_stack_forward(arr, len(layers), _ptr(x), _lens(lens), B, P, _ptr(y), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)), "ee_stack_forward")


# ---------------------------------------------------------------- timing
def ee_profile_enable(on: bool = True):
    _check(lib().ee_profile_enable(1 if on else 0), "ee_profile_enable")


def ee_debug_sync(on: bool = True):
    """Synchronise the stream after every launch (a launch that fails is then
    reported by the call that made it, with its launch site)."""
    _check(lib().ee_debug_sync(1 if on else 0), "ee_debug_sync")


def ee_profile_filter(site: Optional[str] = None):
    """Time only launch site `site` (None: every site)."""
    _check(lib().ee_profile_filter(None if site is None else site.encode()), "ee_profile_filter")


def ee_profile_collect() -> Dict[str, Dict[str, float]]:
    """Per launch site: launches, total_ms, flops, the kernel label ("several
    kernels" if its launches ran more than one) and by_kernel, the same
    totals for each kernel label."""
    cap = 128
    arr = (KernelStat * cap)()
    n = C.c_int32(0)
    _check(lib().ee_profile_collect(arr, cap, C.byref(n)), "ee_profile_collect")
    out: Dict[str, Dict] = {}
    for i in range(n.value):
        name, kern = arr[i].name.decode(), arr[i].kernel.decode()
        row = {"launches": int(arr[i].launches), "total_ms": float(arr[i].total_ms), "flops": float(arr[i].flops)}
        site = out.setdefault(name, {"launches": 0, "total_ms": 0.0, "flops": 0.0, "kernel": kern, "by_kernel": {}})
        for k in ("launches", "total_ms", "flops"):
            site[k] += row[k]
        if site["kernel"] != kern:
            site["kernel"] = "several kernels"
        site["by_kernel"][kern] = row
    return out


# ---------------------------------------------------------------- batch planning (host only)
def _cost(t_batch=0.0, t_token=0.0, t_row=0.0, t_pair=0.0, token_quantum=1, padded_compute=False) -> BatchCost:
    return BatchCost(float(t_batch), float(t_token), float(t_row), float(t_pair), int(token_quantum),
                     1 if padded_compute else 0)


def ee_batch_cost_eval(lens: Sequence[int], cost: BatchCost) -> float:
    out = C.c_double(0.0)
    _check(lib().ee_batch_cost_eval(_lens(lens), len(lens), C.byref(cost), C.byref(out)), "ee_batch_cost_eval")
    return out.value


def ee_plan_fifo(lens: Sequence[int], max_batch: int) -> List[int]:
    """Batch index of each request (arrival order), FIFO groups of max_batch."""
    n = len(lens)
    out = (C.c_int32 * max(1, n))()
    nb = C.c_int32(0)
    _check(lib().ee_plan_fifo(_lens(lens), n, max_batch, out, C.byref(nb)), "ee_plan_fifo")
    return list(out)[:n]


def ee_plan_dynamic(lens: Sequence[int], max_batch: int, cost: BatchCost, max_tokens: int = 0,
                    wait: Optional[Sequence[float]] = None):
    """(batch index of each request in run order, summed cost) of the dynamic plan."""
    n = len(lens)
    out = (C.c_int32 * max(1, n))()
    nb = C.c_int32(0)
    total = C.c_double(0.0)
    w = None if wait is None else (C.c_double * max(1, n))(*[float(x) for x in wait])
    _check(lib().ee_plan_dynamic(_lens(lens), w, n, max_batch, int(max_tokens), C.byref(cost), out, C.byref(nb),
                                 C.byref(total)), "ee_plan_dynamic")
    return list(out)[:n], total.value


def batches_of(plan: Sequence[int]) -> List[List[int]]:
    """Request indices of each batch, in run order, from a batch-index plan."""
    nb = (max(plan) + 1) if plan else 0
    groups: List[List[int]] = [[] for _ in range(nb)]
    for i, b in enumerate(plan):
        groups[b].append(i)
    return groups
