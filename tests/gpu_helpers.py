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


GUARD_BYTES = 4096
SENTINEL = 0xA5


class Guarded:
    """A device output buffer with sentinel bands of GUARD_BYTES before and
    after it, in one allocation: `.t` is the buffer (shape, dtype; 4096-byte
    aligned), `check()` asserts that no kernel wrote into either band."""

    def __init__(self, shape, dtype, fill=None):
        shape = tuple(int(s) for s in shape)
        n = 1
        for s in shape:
            n *= s
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((2 * GUARD_BYTES + self.nbytes,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what="buffer"):
        lo = self.raw[:GUARD_BYTES]
        hi = self.raw[GUARD_BYTES + self.nbytes:]
        assert bool((lo == SENTINEL).all()), f"a write landed before {what}"
        assert bool((hi == SENTINEL).all()), f"a write landed past the end of {what}"
