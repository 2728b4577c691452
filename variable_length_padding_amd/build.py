"""Builds libee.so in-tree for gfx950 with hipcc.

    python -m variable_length_padding_amd.build      (or __graft_entry__.build())

Every source under csrc/ is compiled to an object file under _build/ (in
parallel), then linked into variable_length_padding_amd/libee.so.  Always
rebuilds: the call is the "does it build" check.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libee.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "batching.cpp", "offsets.hip", "padding.hip", "layernorm.hip", "bias_gelu.hip",
           "gemm_f16.hip", "gemm_streamk.hip", "gemm_valu.hip", "attention.hip", "decode.hip"]

# -packed-fp32-ops: keep the compiler from forming v_pk_*_f32 instructions.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libee)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # resolve every symbol now: an undefined one (e.g. a kernel stub the host
    # pass did not emit) fails the build here rather than at first use
    import ctypes
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    except OSError as e:
        raise RuntimeError(f"linked library does not load: {e}") from None
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
