"""Shared helpers for the GPU parity tests (no oracle arithmetic here)."""
import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def valid_mask(lens, P):
    m = np.zeros((len(lens), P), dtype=bool)
    for b, n in enumerate(lens):
        m[b, :n] = True
    return m


def normwise_rel(got, ref):
    """max |got - ref| / max |ref| (the layer-output error measure)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def to_host64(t):
    return t.detach().to("cpu").double().numpy()


def say(msg):
    print(msg, flush=True)
