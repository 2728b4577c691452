"""Seeded synthetic workloads for the padding-removed GPT layer forward.

This module only draws inputs: per-sequence lengths, padded activations and
layer parameters.  It holds none of the method's arithmetic, and both the HIP
path and the CPU oracle consume what it produces.

Workload shapes follow the pages:
  * EnergonAI README, "Scaling Ability": GPT-3, 12 layers, FP16, batch 32,
    sequence length set to half the padding length.
  * Energon-AI news article, "Performance" (tensor-parallel runtime and dynamic
    batching): GPT-3 at TP=4 with 48 layers; request lengths drawn at random
    up to 256 and each batch padded to its longest request.
  * Energon-AI news article, "Ease of use" config: ``half = True`` (fp16
    storage).

Random numbers come from torch's counter-based Philox generators, keyed by a
(seed, stream) pair hashed with splitmix64.  Streams: 0 = lengths,
1 = activations, 2 + 16*layer + tensor_id = parameters.  Small workloads are
drawn on the CPU; the GPT-3-width ones are drawn on the device (the oracle then
receives host copies of the same tensors).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch

__all__ = [
    "Workload", "WORKLOADS", "get", "lengths", "request_stream", "activations",
    "layer_params", "PARAM_NAMES", "stream_generator",
]

# Parameter tensors of one pre-LN decoder layer, in nn.Linear [out, in] layout.
PARAM_NAMES = (
    "ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_out", "b_out",
    "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2",
)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "f16": storage type of activations and weights
    batch: int
    pad_len: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    layers: int
    lens: str             # "uniform" -> U[1, pad_len]; "half" -> every len = pad_len // 2
    x_std: float
    w_std: float = 0.02
    requests: int = 0     # >0: a request stream grouped FIFO into batches of `batch`
    description: str = ""

    @property
    def inner(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.float16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def gemm_flops_per_token(self) -> int:
        """2 * (3*H*H' + H'*H + 2*H*F): the four dense contractions of one layer."""
        H, Hp, F = self.hidden, self.inner, self.ffn
        return 2 * (3 * H * Hp + Hp * H + 2 * H * F)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny-fp32", "f32", batch=4, pad_len=16, hidden=64, n_heads=4, head_dim=16,
             ffn=256, layers=1, lens="uniform", x_std=0.02,
             description="tiny pre-LN causal layer in fp32"),
    Workload("gpt2-small", "f16", batch=8, pad_len=128, hidden=768, n_heads=12, head_dim=64,
             ffn=3072, layers=1, lens="uniform", x_std=1.0,
             description="GPT-2-small-shaped layer, fp16 storage, fp32 accumulation"),
    Workload("gpt3-12l", "f16", batch=32, pad_len=256, hidden=12288, n_heads=96, head_dim=128,
             ffn=49152, layers=12, lens="half", x_std=1.0,
             description="GPT-3-width 12-layer stack, batch 32, every length = pad_len/2"),
    Workload("gpt3-tp4-shard", "f16", batch=32, pad_len=256, hidden=12288, n_heads=24,
             head_dim=128, ffn=12288, layers=1, lens="uniform", x_std=1.0,
             description="one GPU's 1/4 tensor-parallel share of a GPT-3 layer, un-reduced"),
    Workload("gpt3-48l-stream", "f16", batch=64, pad_len=256, hidden=12288, n_heads=96,
             head_dim=128, ffn=49152, layers=48, lens="uniform", x_std=1.0, requests=1024,
             description="1024 requests, FIFO batches of 64 padded to their own max, 48 layers"),
]}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return (x ^ (x >> 31)) & 0x7FFFFFFFFFFFFFFF


def stream_generator(seed: int, stream: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_splitmix64((int(seed) << 24) ^ int(stream)))
    return g


def lengths(w: Workload, seed: int) -> List[int]:
    """Per-sequence lengths of one batch (stream 0)."""
    if w.lens == "half":
        return [w.pad_len // 2] * w.batch
    g = stream_generator(seed, 0)
    return torch.randint(1, w.pad_len + 1, (w.batch,), generator=g).tolist()


def request_stream(w: Workload, seed: int) -> List[List[int]]:
    """Lengths of `w.requests` requests in arrival order, grouped FIFO into
    consecutive batches of `w.batch` (stream 0)."""
    g = stream_generator(seed, 0)
    lens = torch.randint(1, w.pad_len + 1, (w.requests,), generator=g).tolist()
    return [lens[i:i + w.batch] for i in range(0, len(lens), w.batch)]


REQUEST_STREAM_BASE = 1 << 20


def request_activations(w: Workload, seed: int, lens: List[int], device="cpu") -> List[torch.Tensor]:
    """Activations of each request of a stream, [len_i, hidden] ~ N(0, x_std^2)
    in the workload dtype, request i from stream REQUEST_STREAM_BASE + i, so a
    request carries the same values whichever batch it lands in."""
    out = []
    for i, n in enumerate(lens):
        g = stream_generator(seed, REQUEST_STREAM_BASE + i, device)
        x = torch.randn((n, w.hidden), generator=g, device=device, dtype=torch.float32)
        out.append(x.mul_(w.x_std).to(w.torch_dtype))
    return out


def pad_batch(rows: List[torch.Tensor], pad_len: Optional[int] = None) -> torch.Tensor:
    """Right-pads per-request [len_i, hidden] rows into [B, P, hidden] (pads zero)."""
    P = pad_len if pad_len is not None else max(r.shape[0] for r in rows)
    x = torch.zeros((len(rows), P, rows[0].shape[1]), dtype=rows[0].dtype, device=rows[0].device)
    for b, r in enumerate(rows):
        x[b, :r.shape[0]] = r
    return x


def activations(w: Workload, seed: int, batch: int, pad_len: int, lens: Optional[List[int]] = None,
                device="cpu", pad_fill: str = "random", stream: int = 1) -> torch.Tensor:
    """Padded activations [batch, pad_len, hidden] ~ N(0, x_std^2), stored in the
    workload dtype (fp16 by round-to-nearest-even from fp32).  Pads hold the same
    stream's values, or NaN when ``pad_fill == "nan"``."""
    g = stream_generator(seed, stream, device)
    x = torch.randn((batch, pad_len, w.hidden), generator=g, device=device, dtype=torch.float32)
    x.mul_(w.x_std)
    x = x.to(w.torch_dtype)
    if pad_fill == "nan":
        assert lens is not None
        for b, n in enumerate(lens):
            x[b, n:] = float("nan")
    elif pad_fill == "zero":
        assert lens is not None
        for b, n in enumerate(lens):
            x[b, n:] = 0
    return x


def layer_params(w: Workload, seed: int, layer: int, device="cpu", variant: str = "init") -> Dict[str, torch.Tensor]:
    """Parameters of one layer, drawn from streams 2 + 16*layer + tensor_id.

    variant "init": weights ~ N(0, w_std^2), biases 0, LayerNorm gamma 1, beta 0
    (GPT-2 initialisation).  variant "affine": additionally biases ~ N(0, 0.02^2),
    gamma = 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2), so the affine and bias paths carry
    signal.  variant "zero-weights": every matrix 0, biases as in "affine".
    """
    H, Hp, F = w.hidden, w.inner, w.ffn
    shapes = {
        "ln1_g": (H,), "ln1_b": (H,), "w_qkv": (3 * Hp, H), "b_qkv": (3 * Hp,),
        "w_out": (H, Hp), "b_out": (H,), "ln2_g": (H,), "ln2_b": (H,),
        "w_fc1": (F, H), "b_fc1": (F,), "w_fc2": (H, F), "b_fc2": (H,),
    }
    out = {}
    for tid, name in enumerate(PARAM_NAMES):
        shp = shapes[name]
        g = stream_generator(seed, 2 + 16 * layer + tid, device)
        if name.startswith("w_"):
            if variant == "zero-weights":
                t = torch.zeros(shp, device=device, dtype=torch.float32)
            else:
                t = torch.randn(shp, generator=g, device=device, dtype=torch.float32).mul_(w.w_std)
        elif name.endswith("_g"):
            t = torch.ones(shp, device=device, dtype=torch.float32)
            if variant in ("affine", "zero-weights"):
                t += torch.randn(shp, generator=g, device=device, dtype=torch.float32).mul_(0.1)
        else:  # biases and LayerNorm beta
            t = torch.zeros(shp, device=device, dtype=torch.float32)
            if variant in ("affine", "zero-weights"):
                std = 0.1 if name.startswith("ln") else 0.02
                t += torch.randn(shp, generator=g, device=device, dtype=torch.float32).mul_(std)
        out[name] = t.to(w.torch_dtype)
    return out
