"""Builds libee.so in-tree for gfx950 with hipcc.

    python -m variable_length_padding_amd.build      (or __graft_entry__.build())

Every source under csrc/ is compiled to an object file under _build/ (in
parallel), then linked into variable_length_padding_amd/libee.so.  Always
rebuilds: the call is the "does it build" check.

    python -m variable_length_padding_amd.build --sanitize address --out DIR
    python -m variable_length_padding_amd.build --sanitize undefined --out DIR

A host-only sanitizer build (CPU checking of the host code: argument
validation, workspace planning, the batch planners and the launch helpers;
the GPU code is built as usual, uninstrumented) into DIR/libee.so, linked
against clang's shared sanitizer runtime.  The binding loads it when
EE_LIBRARY is set to its path; Python itself is not instrumented, so the
runtime is preloaded:

    EE_LIBRARY=DIR/libee.so LD_PRELOAD=<runtime> ASAN_OPTIONS=detect_leaks=0 \
        python -m pytest tests -m "not gpu"

where <runtime> is what sanitizer_runtime(kind) returns.
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
           "gemm_f16.hip", "gemm_streamk.hip", "gemm_valu.hip", "attention.hip", "decode.hip", "noalloc.hip"]

# -packed-fp32-ops: keep the compiler from forming v_pk_*_f32 instructions.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libee)")


# Host-only instrumentation: each -fsanitize= goes to the host compilation only.
SANITIZE_FLAGS = {
    "address": "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer -shared-libasan".split(),
    "undefined": "-Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined".split(),
}
SANITIZE_RUNTIME = {"address": "libclang_rt.asan-x86_64.so", "undefined": "libclang_rt.ubsan_standalone-x86_64.so"}


def sanitizer_runtime(kind: str) -> str:
    """Path of clang's shared runtime for a sanitizer build (to preload)."""
    r = subprocess.run([_hipcc(), f"-print-file-name={SANITIZE_RUNTIME[kind]}"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"clang runtime {SANITIZE_RUNTIME[kind]} not found")
    return path


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, sanitize: str = "", out_dir: str = "") -> str:
    extra = SANITIZE_FLAGS[sanitize] if sanitize else []
    if sanitize and not out_dir:
        raise ValueError("a sanitizer build needs an output directory (it never replaces the in-tree libee.so)")
    build_dir = os.path.join(out_dir, "obj") if sanitize else BUILD
    lib = os.path.join(out_dir, "libee.so") if sanitize else LIB
    os.makedirs(build_dir, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    # a sanitizer build's runtime symbols resolve from the preloaded runtime
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # resolve every symbol now: an undefined one (e.g. a kernel stub the host
    # pass did not emit) fails the build here rather than at first use
    if not sanitize:   # (a sanitizer build loads only with its runtime preloaded)
        import ctypes
        try:
            ctypes.CDLL(tmp, mode=os.RTLD_NOW)
        except OSError as e:
            raise RuntimeError(f"linked library does not load: {e}") from None
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", flush=True)
        if sanitize:
            print(f"runtime to preload: {sanitizer_runtime(sanitize)}", flush=True)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--sanitize", choices=sorted(SANITIZE_FLAGS), default="")
    ap.add_argument("--out", default="")
    a = ap.parse_args()
    build(sanitize=a.sanitize, out_dir=a.out)
    sys.exit(0)
