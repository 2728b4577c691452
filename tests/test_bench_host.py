"""Host-side pieces of bench.py (no GPU): the kernel labels the library
reports map to symbols its code object holds, the defaults name the 48-layer
request stream, and a multi-GPU request is refused."""
import os
import shutil
import subprocess

import pytest

import bench
import variable_length_padding_amd as ee

# every kernel configuration gemm_f16_kernel_label can name: <MF, BM, BN, WGM, WGN> and W depth
CONFIGS = [("16, 256, 256, 2, 2", 2), ("16, 256, 256, 2, 2", 3), ("32, 128, 128, 2, 2", 2), ("32, 128, 64, 2, 2", 2),
           ("16, 256, 384, 2, 2", 2)]


@pytest.mark.skipif(shutil.which("nm") is None, reason="needs nm")
def test_kernel_labels_map_to_library_symbols():
    out = subprocess.run(["nm", ee.lib_path()], capture_output=True, text=True, check=True).stdout
    names = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for cfg, depth in CONFIGS:
        for epi in range(4):
            for ordered in ("false", "true") if cfg.startswith("16, 256") else ("false",):
                label = f"gemm_f16_mfma_kernel<{cfg}, {epi}, {depth}, {ordered}>"
                assert bench.kernel_symbol(label) in names, label
    assert bench.kernel_symbol("gemm_streamk_kernel + streamk_reduce_kernel") is None


def test_defaults_and_single_gpu_only():
    a = bench._parse([])
    assert a.workload == "gpt3-48l-stream" and a.gpus == 1
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2


def test_site_bytes():
    import workloads
    w = workloads.get("gpt3-12l")
    H, F = w.hidden, w.ffn
    # FC1 reads A [T, H] and W [F, H] and writes [T, F]; FC2 also reads the residual [T, H]
    assert bench._site_bytes(w, 4096, 32, 256, "gemm_fc1") == (4096 * H + F * H + 4096 * F) * 2
    assert bench._site_bytes(w, 96, 32, 256, "gemm_fc2_rest") == (96 * F + H * F + 2 * 96 * H) * 2
    assert bench._site_bytes(w, 4096, 32, 256, "rebuild") == (4096 + 32 * 256) * H * 2


def test_traffic_reads_the_summary_per_kernel(tmp_path, monkeypatch):
    """The roofline's traffic comes from the counter summary's entry for its
    kernel (or its top-level kernel), and only for the current GEMM code."""
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    summary = {"kernel": "plain", "hbm_bytes_per_launch": 1.0, "gemm_code_sha256": bench.gemm_code_sha256(),
               "kernels": {"plain": {"hbm_bytes_per_launch": 1.0}, "split": {"hbm_bytes_per_launch": 2.0}}}
    with open(bench.pmc_summary_path("w"), "w") as f:
        json.dump(summary, f)
    assert bench._traffic("w", "plain") == 1.0 and bench._traffic("w", "split") == 2.0
    assert bench._traffic("w", "other") is None and bench._traffic("x", "plain") is None
    summary["gemm_code_sha256"] = "0" * 64
    with open(bench.pmc_summary_path("w"), "w") as f:
        json.dump(summary, f)
    assert bench._traffic("w", "split") is None
