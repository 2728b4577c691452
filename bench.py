#!/usr/bin/env python3
"""Throughput of the padding-removed GPT layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

Default workload: the variable-length request stream through a 48-layer
GPT-3-width stack (gpt3-48l-stream: 1024 requests with lengths U[1,256],
grouped FIFO into 16 batches of 64, each padded to its own longest request;
174 GB of weights resident in HBM).  A step is one pass of the whole hot path
over one FIFO batch: offsets, remove, 48 packed layers (LayerNorm, QKV GEMM,
varlen causal attention, out GEMM, LayerNorm, FC1 GEMM + GeLU, FC2 GEMM),
rebuild -- one ee_stack_forward call.  Steps cycle through the 16 batches;
W untimed steps, then K timed ones.  Inputs and weights are resident in HBM
before the timed region.  Prints one JSON line.

Metric: valid tokens/s per layer = sum over the timed steps of T_batch * L /
their summed time ("value").  When the timed steps cover all 16 batches,
"stream" gives the rate of the first pass over them, and "batching" runs the
dynamic plan over the same requests (planned on a table of batch times
measured in the run) beside FIFO; else both are null.

roofline: the FC1 GEMM kernel (bias + GeLU epilogue, the largest single
contraction; the GEMMs together take ~97% of a step): the algorithmic flops
of its launches (2 * rows * H * F each) over their hipEvent-measured
durations on the launch stream, recorded by libee in the timed steps (the only
launch site with events there).  Its rows are the ones the 256 x 256 kernel
runs; when a batch's row count leaves a partial last round of tiles, the
remaining rows run as a second launch (site gemm_fc1_rest).  "kernels" comes
from as many further steps (at most 16) with every launch timed.
traffic: HBM bytes per launch of that kernel from the committed rocprofv3
counter summary (profiles/), when it was taken on this workload and on the
current GEMM code; else null.
cpu_baseline: the CPU oracle (numpy float64, as it stands) on a bounded sample
of the first batch through layer 0, packed (the method) and padded (the
definition); stated as valid tokens/s per layer.

    python bench.py --workload gpt3-12l     (one batch, 12 layers; also gpt2-small, gpt3-tp4-shard, tiny-fp32)
    python bench.py --decode-steps 32       (incremental decoding)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "valid tokens/s per GPT layer fwd (packed) + % HBM/MFMA roofline, 1 GPU"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROOFLINE_SITE = "gemm_fc1"
PROFILES = os.path.join(ROOT, "profiles")
# the GEMM kernel's source and the headers that shape its loads, tile order and epilogue arithmetic
GEMM_SOURCES = [os.path.join(ROOT, "variable_length_padding_amd", "csrc", f)
                for f in ("gemm_f16.hip", "gemm_tile_order.h", "lds_dma.h", "device_common.h")]
DEFAULT_WORKLOAD = "gpt3-48l-stream"


def _parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=0,
                    help="sequences of the first batch the CPU oracle runs (default: 8 for the request stream, "
                         "24 for single-batch workloads)")
    ap.add_argument("--no-dynamic", action="store_true",
                    help="request stream: skip the dynamic-batching comparison (cost table and dynamic pass)")
    ap.add_argument("--no-fuse-gelu", action="store_true", help="unfused bias+GeLU (ablation)")
    ap.add_argument("--attention", choices=("varlen", "padded"), default="varlen",
                    help="padded: transposing rebuild -> fixed-shape masked attention -> transposing remove "
                         "(the pages' form of padding removal, as an ablation)")
    ap.add_argument("--block", choices=("gpt", "bert"), default="gpt",
                    help="bert: post-LN encoder block (bidirectional attention, erf GeLU), as an ablation")
    ap.add_argument("--no-pack", action="store_true",
                    help="padding kept: every one of the B*P rows runs through the layers (the redundant "
                         "computation the method removes); value still counts valid tokens only")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="incremental decoding: prefill the batch's prompts, then time this many decode steps "
                         "(one new token per sequence each) through ee_stack_extend")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="incremental decoding: number of sequences (default: the workload's batch)")
    ap.add_argument("--max-batch", type=int, default=0,
                    help="request-stream workload: batch size cap of both planners (default: the workload's)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (scale reference for HBM byte counters)")
    ap.add_argument("--residual", choices=("auto", "epilogue", "pass"), default="auto",
                    help="where the pre-LN block adds its residuals: in the out/FC2 GEMM epilogues or in a "
                         "separate pass (auto: the library's default, the epilogues)")
    ap.add_argument("--dense-weights", action="store_true",
                    help="weight matrices stored dense instead of at ee_preferred_row_pitch (ablation)")
    return ap.parse_args(argv)


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _stored(args, params):
    """A layer's parameters as the bench hands them to libee: weight rows at
    the library's preferred pitch (dense with --dense-weights)."""
    import variable_length_padding_amd as ee
    return params if args.dense_weights else ee.pitched_weights(params)


GEMM_SHAPES = {"gemm_qkv": ("hidden", "3inner"), "gemm_out": ("inner", "hidden"), "gemm_fc1": ("hidden", "ffn"),
               "gemm_fc2": ("ffn", "hidden")}


def _gemm_kn(w, site):
    """(K, N) of a GEMM launch site (or of its "_rest" part)."""
    dims = {"hidden": w.hidden, "inner": w.inner, "3inner": 3 * w.inner, "ffn": w.ffn}
    k, n = GEMM_SHAPES[site.replace("_rest", "")]
    return dims[k], dims[n]


def _site_bytes(w, rows, B, P, site, res_in_gemm=True):
    """Algorithmic HBM bytes of one launch at a site that processes `rows`
    packed rows (B sequences padded to P for the padding ops); res_in_gemm:
    the out and FC2 GEMMs read the residual in their epilogue."""
    s = w.elem_bytes
    H, Hp, F = w.hidden, w.inner, w.ffn
    base = site.replace("_rest", "")
    if base in GEMM_SHAPES:
        K, N = _gemm_kn(w, site)
        res = rows * N * s if res_in_gemm and base in ("gemm_out", "gemm_fc2") else 0
        return float((rows * K + N * K + rows * N) * s + res)
    table = {
        "ln1": 2.0 * rows * H * s, "ln2": 2.0 * rows * H * s, "remove": 2.0 * rows * H * s,
        "rebuild": float((rows + B * P) * H * s), "attention": 4.0 * rows * Hp * s,
        # q|k|v valid rows read, [3, B, nh, P, hd] written (pads as zeros)
        "rebuild_heads": float(3 * (rows + B * P) * Hp * s), "remove_heads": 2.0 * rows * Hp * s,
        "add_ln1": 3.0 * rows * H * s, "add_ln2": 3.0 * rows * H * s,   # u and residual read, y written
        "res_ln2": 4.0 * rows * H * s,                                   # u, residual read; sum, LN(sum) written
        "res_add": 3.0 * rows * H * s, "bias_gelu": 2.0 * rows * F * s,
    }
    return table.get(base, 0.0)


def _attention_flops(w, lens, causal=True):
    # QK^T and PV: 2 * 2 * hd * nh flops per (query, key) pair; len(len+1)/2
    # pairs per sequence under the causal mask, len^2 without it
    if causal:
        return sum(2.0 * w.inner * n * (n + 1) for n in lens)
    return sum(4.0 * w.inner * n * n for n in lens)


def kernel_symbol(label):
    """The symbol rocprofv3 reports for a gemm_f16_mfma_kernel<...> label (the
    library's template label, arguments in declaration order): the Itanium
    mangling of ee::(anonymous namespace)::gemm_f16_mfma_kernel<ints...> with
    the kernel's parameter list."""
    if not label.startswith("gemm_f16_mfma_kernel<") or "+" in label:
        return None
    args = [v.strip() for v in label[label.index("<") + 1:label.rindex(">")].split(",")]
    mangled = "".join(f"Lb{int(v == 'true')}E" if v in ("true", "false") else f"Li{int(v)}E" for v in args)
    return ("_ZN2ee12_GLOBAL__N_120gemm_f16_mfma_kernelI" + mangled +
            "EEvPKDF16_iS3_iS3_S3_PDF16_iiiiiiiPfNS0_12OrderedSplitE")


def gemm_code_sha256(paths=GEMM_SOURCES):
    """sha256 of the GEMM sources' code, in order: // comments, trailing
    spaces and blank lines removed (the files hold no // inside string
    literals), so an edit of the comments keeps counters taken on the same
    code valid."""
    lines = []
    for path in paths:
        with open(path) as f:
            lines += [ln.split("//", 1)[0].rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def pmc_summary_path(workload):
    return os.path.join(PROFILES, f"gemm_fc1_{workload}_pmc.json")


def _traffic(workload, symbol):
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary, if it was taken on this workload and the current GEMM code and
    covers this kernel (its "kernel", or an entry of its "kernels")."""
    try:
        with open(pmc_summary_path(workload)) as f:
            s = json.load(f)
        if s.get("gemm_code_sha256") != gemm_code_sha256():
            return None
        if symbol in s.get("kernels", {}):
            return s["kernels"][symbol]["hbm_bytes_per_launch"]
        return s["hbm_bytes_per_launch"] if s.get("kernel") == symbol else None
    except (OSError, KeyError, ValueError, TypeError):
        return None


def _kernel_table(w, stats, steps, ms_total, rows_of_site, B, P, attn_flops, res_in_gemm):
    """Per-site figures: launches per step, average ms, share of the step,
    TFLOP/s and MFMA fraction (GEMMs: the library's algorithmic flops; attention:
    attn_flops, summed over all its launches), GB/s and HBM fraction
    (algorithmic bytes of a launch over rows_of_site(site) rows)."""
    kernels = {}
    for site, st in stats.items():
        n = st["launches"]
        avg_ms = st["total_ms"] / n
        base = site.replace("_rest", "")
        if base in GEMM_SHAPES:
            fl = st["flops"] / n
            K, N = _gemm_kn(w, site)
            rows = fl / (2.0 * K * N)
        else:
            fl = attn_flops / n if site == "attention" else 0.0
            rows = rows_of_site(site)
        by = _site_bytes(w, rows, B, P, site, res_in_gemm)
        k = {"launches_per_step": round(n / steps, 3), "avg_ms": round(avg_ms, 5),
             "share": round(st["total_ms"] / ms_total, 4)}
        if st.get("kernel"):
            k["kernel"] = st["kernel"]
        if len(st.get("by_kernel", {})) > 1:   # e.g. a GEMM with and without the in-order split
            k["kernels"] = {lb: {"launches": v["launches"],
                                 "tflops": round(v["flops"] / v["total_ms"] / 1e9, 1) if v["flops"] else None,
                                 "flops_per_launch": v["flops"] / v["launches"]}
                            for lb, v in st["by_kernel"].items()}
        if fl:
            k["tflops"] = round(fl / (avg_ms * 1e-3) / 1e12, 1)
            k["mfma_frac"] = round(k["tflops"] / PEAK_F16_TFLOPS, 4)
        if by:
            k["gbs"] = round(by / (avg_ms * 1e-3) / 1e9, 1)
            k["hbm_frac"] = round(k["gbs"] / PEAK_HBM_GBS, 4)
        kernels[site] = k
    return kernels


def _roofline(workload, st):
    """The roofline object for the FC1 site's timed launches: the kernel that
    ran most of them (a batch whose last round of tiles is partial runs the
    in-order split form of the same kernel), with the whole site's rate
    beside it."""
    by = st.get("by_kernel") or {st["kernel"]: st}
    # the kernel with the most launches; on a tie the plain form
    label, k = max(by.items(), key=lambda kv: (kv[1]["launches"], kv[0].endswith("false>")))
    ms = k["total_ms"] / k["launches"]
    flops = k["flops"] / k["launches"]
    achieved = flops / (ms * 1e-3) / 1e12
    sym = kernel_symbol(label)
    out = {"bound": "mfma", "kernel": label, "symbol": sym, "achieved": round(achieved, 1),
           "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
           "traffic": _traffic(workload, sym) if sym else None, "avg_launch_ms": round(ms, 4),
           "flops_per_launch": flops, "launches": k["launches"]}
    if len(by) > 1:
        out["site"] = {"launches": st["launches"], "achieved": round(st["flops"] / st["total_ms"] / 1e9, 1),
                       "kernels": {lb: v["launches"] for lb, v in by.items()}}
    return out


def host_info():
    """CPU model, NUMA nodes and the cores this process may run on."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nodes = len([d for d in os.listdir("/sys/devices/system/node") if d.startswith("node") and d[4:].isdigit()])
    except OSError:
        nodes = None
    return {"cpu_model": model, "numa_nodes": nodes, "host_cores": len(os.sched_getaffinity(0))}


def _cpu_baseline(w, seqs, params_dev, layers_total, tokens_total, label):
    """Times the oracle as it stands (numpy float64) on the sampled sequences
    `seqs` (a list of [len_i, H] host tensors, one batch's first ones) through
    one layer, in its packed form (the method: the valid rows only) and its
    padded form (the definition: every row of the sequences padded to the
    longest of them, pads computed, then zeroed).  Valid tokens/s per layer."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    params64 = oracle.to_f64_params({k: v.detach().cpu() for k, v in params_dev.items()})   # untimed
    lens = [int(r.shape[0]) for r in seqs]
    xs = np.concatenate([r.double().numpy() for r in seqs], axis=0)
    cu = np.concatenate([[0], np.cumsum(lens)])
    P = max(lens)
    xp = np.zeros((len(lens), P, w.hidden))
    for b, r in enumerate(seqs):
        xp[b, :lens[b]] = r.double().numpy()
    t0 = time.perf_counter()
    oracle.layer_forward_packed(xs, cu, params64, w.n_heads, w.head_dim)
    dt_packed = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.layer_forward_padded(xp, lens, params64, w.n_heads, w.head_dim)
    dt_padded = time.perf_counter() - t0
    ntok = int(cu[-1])
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    rate = ntok / dt_packed
    out = {"value": round(rate, 2), "unit": "valid tokens/s per layer", "cores": threads, "kind": "oracle",
           "sample": f"{len(lens)} sequences ({ntok} valid tokens, padded to {P}) of {label} through layer 0; "
                     f"float64 numpy oracle; packed {dt_packed:.1f} s, padded {dt_padded:.1f} s",
           "padded_value": round(ntok / dt_padded, 2),
           "packed_seconds": round(dt_packed, 2), "padded_seconds": round(dt_padded, 2),
           "threads_used": threads}
    out.update(host_info())
    if tokens_total:
        hours = tokens_total * layers_total / rate / 3600.0
        out["extrapolated"] = (f"the whole workload ({tokens_total} valid tokens x {layers_total} layers) at this rate: "
                               f"{hours:.1f} h packed, {hours * rate / out['padded_value']:.1f} h padded")
    return out


def _copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}), flush=True)


def _timed_steps(ee, stream, step_fns, site_filter):
    """Runs the step callables in turn with per-launch events on one site
    (site_filter, or every site when None); returns (ms of each step, stats)."""
    import torch
    ee.ee_profile_filter(site_filter)
    ee.ee_profile_enable(True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(step_fns) + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i, fn in enumerate(step_fns):
        fn()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ee.ee_profile_enable(False)
    ee.ee_profile_filter(None)
    stats = ee.ee_profile_collect()
    return [marks[i].elapsed_time(marks[i + 1]) for i in range(len(step_fns))], stats


def _pct(sorted_ms, q):
    return sorted_ms[min(len(sorted_ms) - 1, int(round(q * (len(sorted_ms) - 1))))]


def _stream_bench(args):
    """The request stream: FIFO batches (the workload's definition) as the
    timed steps, then the whole stream once, then (unless --no-dynamic) the
    dynamic plan over the same requests."""
    import torch

    import variable_length_padding_amd as ee
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    lens = [n for g in workloads.request_stream(w, args.seed) for n in g]
    n_req, L, P_max = len(lens), w.layers, w.pad_len
    cap = args.max_batch or w.batch
    T_all = sum(lens)
    stream = torch.cuda.current_stream()
    _log(f"request stream {w.name}: {n_req} requests, T={T_all}, {L} layers, batch cap {cap}, "
         f"padding {'kept' if args.no_pack else 'removed'}")
    t0 = time.perf_counter()
    params = []
    for l in range(L):
        params.append(_stored(args, workloads.layer_params(w, args.seed, l, device=dev)))
        if l % 12 == 11:
            torch.cuda.synchronize()
            _log(f"weights: {l + 1}/{L} layers")
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=dt) for p in params]
    reqs = workloads.request_activations(w, args.seed, lens, device=dev)
    ws = torch.empty(layers[0].workspace_size(cap, P_max, cap * P_max), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    _log(f"{sum(t.numel() * t.element_size() for p in params for t in p.values()) / 1e9:.1f} GB of weights "
         f"resident, workspace {ws.numel() / 1e6:.0f} MB ({time.perf_counter() - t0:.1f} s)")

    def run(x, batch_lens, y):
        B, P, _ = x.shape
        ee.ee_stack_forward(layers, x, [P] * B if args.no_pack else batch_lens, y, ws, stream)

    def make_batches(plan):
        xs = [workloads.pad_batch([reqs[i] for i in b]) for b in plan]
        return xs, [torch.empty_like(x) for x in xs], [[lens[i] for i in b] for b in plan]

    fifo = ee.batches_of(ee.ee_plan_fifo(lens, cap))
    xs, ys, bls = make_batches(fifo)
    nb = len(fifo)
    Tb = [sum(bl) for bl in bls]
    rows_b = [x.shape[0] * x.shape[1] for x in xs]

    def step(i):
        j = i % nb
        return lambda: run(xs[j], bls[j], ys[j])

    for i in range(args.warmup):
        step(i)()
    torch.cuda.synchronize()
    _log(f"warmup done ({args.warmup} steps)")
    K = args.steps
    first = args.warmup            # timed steps continue the cycle where the warm-up left it
    order = [(first + i) % nb for i in range(K)]
    t_host = time.perf_counter()
    ms, st_fc1 = _timed_steps(ee, stream, [step(first + i) for i in range(K)], ROOFLINE_SITE)
    t_host = time.perf_counter() - t_host
    tok_timed = sum(Tb[j] for j in order)
    sec = sum(ms) / 1e3
    value = tok_timed * L / sec
    srt = sorted(ms)
    _log(f"timed {K} steps (batches {order[0]}..): {sum(ms) / K:.2f} ms/step, {value:.0f} valid tokens/s per layer "
         f"(host clock {t_host / K * 1e3:.2f} ms/step)")
    # per-kernel figures: up to one pass of the batches with every launch site timed
    K2 = min(K, nb)
    ms2, stats = _timed_steps(ee, stream, [step(first + i) for i in range(K2)], None)
    order2 = [(first + i) % nb for i in range(K2)]
    lens2 = [n for j in order2 for n in bls[j]]
    T2 = sum(Tb[j] for j in order2)

    def rows_of_site(site):
        if site in ("remove", "rebuild", "offsets"):
            return T2 / K2
        return (sum(rows_b[j] for j in order2) if args.no_pack else T2) / K2
    kernels = _kernel_table(w, stats, K2, sum(ms2), rows_of_site, cap, sum(xs[j].shape[1] for j in order2) / K2,
                            _attention_flops(w, lens2) * L, True)
    # the whole stream once (FIFO): the first nb timed steps, when they cover it
    stream_ms = sum(ms[:nb]) if K >= nb else None
    if stream_ms is not None:
        stream_rate = T_all * L / (stream_ms / 1e3)
        _log(f"whole stream, FIFO: {nb} batches, {stream_ms / 1e3:.2f} s, {stream_rate:.0f} valid tokens/s per layer")

    batching = None
    if not args.no_dynamic and stream_ms is not None:
        batching = _dynamic_vs_fifo(args, w, ee, torch, dev, stream, run, make_batches, lens, cap, P_max, T_all, L,
                                    stream_ms / 1e3, sum(rows_b))
    roofline = _roofline(w.name, st_fc1[ROOFLINE_SITE])
    cpu = None
    if not args.no_cpu_baseline and not args.no_pack:
        nseq = args.cpu_sample_seqs or 8
        _log(f"timing the CPU oracle on {nseq} sequences of FIFO batch 0")
        cpu = _cpu_baseline(w, [reqs[i].cpu() for i in fifo[0][:nseq]], params[0], L, T_all,
                            f"FIFO batch 0 of the {w.name} stream")
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "valid tokens/s per layer", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(sum(ms) / K, 3),
        "ms_per_step_p10_p50_p90": [round(_pct(srt, q), 3) for q in (0.1, 0.5, 0.9)],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "f32",
        "data": "synthetic (seeded request lengths U[1,%d], N(0,1) activations, N(0,0.02) random-init weights)" % P_max,
        "config": {"workload": w.name, "requests": n_req, "valid_tokens": T_all, "layers": L, "max_batch": cap,
                   "batches": nb, "hidden": w.hidden, "n_heads": w.n_heads, "head_dim": w.head_dim, "ffn": w.ffn,
                   "batching": "fifo", "step": "one FIFO batch through all layers, cycling the batches",
                   "timed_valid_tokens": tok_timed, "padding_removed": not args.no_pack,
                   "weight_rows": "dense" if args.dense_weights else "preferred pitch"},
        "stream": None if stream_ms is None else {
            "batches": nb, "seconds": round(stream_ms / 1e3, 3), "value": round(stream_rate, 1),
            "padded_rows": sum(rows_b), "padded_ratio": round(sum(rows_b) / T_all, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "batching": batching,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def _dynamic_vs_fifo(args, w, ee, torch, dev, stream, run, make_batches, lens, cap, P_max, T_all, L, fifo_s,
                     fifo_rows):
    """The dynamic plan (ee_plan_dynamic on a table of whole-stack batch times
    measured here) run once over the stream, beside the FIFO pass."""
    # cost model "by machine performance" (TurboTransformers' scheduler works
    # from a table of measured batch times): the whole stack timed on batches
    # of `cap` equal-length requests, tokens = (k + 1) * 8 * cap, no padding
    # (random activations: the chip draws more power, and clocks lower, on random data than on zeros)
    import workloads
    x_cal = workloads.activations(w, args.seed + 9, cap, P_max, device=dev)

    def timed(bl, P=None):
        P = P or max(bl)
        x = x_cal[:len(bl), :P].contiguous()
        y = torch.empty_like(x)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(x, bl, y)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3
    quantum = 8 * cap
    timed([8] * cap)                                   # warm-up
    table = [timed([8 * (k + 1)] * cap) for k in range(P_max // 8)]
    _log(f"cost table: {len(table)} batch sizes timed, {table[0]:.3f} s at {quantum} tokens .. "
         f"{table[-1]:.3f} s at {quantum * len(table)}")
    t_row = 0.0
    if not args.no_pack:
        # with the padding removed, a padded row costs only its share of the
        # rebuild (written as zeros); time that on its own: one-token sequences
        x = torch.zeros((cap, P_max, w.hidden), dtype=w.torch_dtype, device=dev)
        packed = torch.zeros((cap, w.hidden), dtype=w.torch_dtype, device=dev)
        pws = torch.empty(ee.ee_padding_workspace_size(cap, P_max), dtype=torch.uint8, device=dev)
        ee.ee_rebuild_padding(packed, [1] * cap, x, pws, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            ee.ee_rebuild_padding(packed, [1] * cap, x, pws, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t_row = e0.elapsed_time(e1) / 1e3 / 10 / (cap * P_max)
        del x, packed, pws
    cost = ee.BatchCost(0.0, 0.0, t_row, 0.0, quantum, 1 if args.no_pack else 0).set_table(table)
    g = torch.Generator().manual_seed(args.seed + 7)
    checks = []
    for B, P in ((cap, P_max), (max(1, cap // 2), P_max // 2)):
        bl = torch.randint(1, P + 1, (B,), generator=g).tolist()
        checks.append((B, sum(bl), timed(bl), ee.ee_batch_cost_eval(bl, cost)))
    _log("cost model check: " + ", ".join(f"B={B} T={T}: measured {t:.3f} s, model {m:.3f} s"
                                           for B, T, t, m in checks))
    del x_cal
    plan = ee.batches_of(ee.ee_plan_dynamic(lens, cap, cost)[0])
    xs, ys, bls = make_batches(plan)
    run(xs[0], bls[0], ys[0])                     # warm-up: one batch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for x, bl, y in zip(xs, bls, ys):
        run(x, bl, y)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3
    rows = sum(x.shape[0] * x.shape[1] for x in xs)
    dyn = {"batches": len(plan), "padded_rows": rows, "padded_ratio": round(rows / T_all, 4),
           "seconds": round(sec, 3), "value": round(T_all * L / sec, 1),
           "predicted_seconds": round(sum(ee.ee_batch_cost_eval(bl, cost) for bl in bls), 3)}
    fifo_plan = ee.batches_of(ee.ee_plan_fifo(lens, cap))
    fifo_bls = [[lens[i] for i in b] for b in fifo_plan]
    fifo = {"batches": len(fifo_plan), "padded_rows": fifo_rows, "padded_ratio": round(fifo_rows / T_all, 4),
            "seconds": round(fifo_s, 3), "value": round(T_all * L / fifo_s, 1),
            "predicted_seconds": round(sum(ee.ee_batch_cost_eval(bl, cost) for bl in fifo_bls), 3)}
    _log(f"dynamic: {len(plan)} batches, padded/valid rows {rows / T_all:.3f}, {sec:.2f} s, "
         f"{T_all * L / sec:.0f} valid tokens/s per layer (model {dyn['predicted_seconds']:.2f} s); "
         f"FIFO {fifo_s:.2f} s (model {fifo['predicted_seconds']:.2f} s)")
    del xs, ys
    return {"fifo": fifo, "dynamic": dyn, "dynamic_over_fifo": round(dyn["value"] / fifo["value"], 4),
            "cost_model": {"t_row": cost.t_row, "token_quantum": quantum,
                           "token_table_s": [round(v, 4) for v in table],
                           "check": [[B, T, round(t, 4), round(m, 4)] for B, T, t, m in checks]}}


def _forward_bench(args):
    """One batch of a single-batch workload through all its layers per step."""
    import torch

    import variable_length_padding_amd as ee
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    lens = workloads.lengths(w, args.seed)
    B, P, L = w.batch, w.pad_len, w.layers
    T = sum(lens)
    # rows actually run through the layers: the valid ones, or all B*P with --no-pack
    run_lens = [P] * B if args.no_pack else lens
    T_run = sum(run_lens)
    _log(f"workload {w.name}: B={B} P={P} T={T} (rows run {T_run}) H={w.hidden} nh={w.n_heads} "
         f"hd={w.head_dim} F={w.ffn} L={L} block={args.block} attention={args.attention}")

    x = workloads.activations(w, args.seed, B, P, lens, device=dev)
    params = [_stored(args, workloads.layer_params(w, args.seed, l, device=dev)) for l in range(L)]
    torch.cuda.synchronize()
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    bert = args.block == "bert"
    layers = [ee.Layer(w.hidden, w.n_heads, w.head_dim, w.ffn, p, dtype=dt, fuse_gelu=not args.no_fuse_gelu,
                       gelu=ee.GELU_ERF if bert else ee.GELU_TANH,
                       block=ee.BLOCK_BERT_POSTLN if bert else ee.BLOCK_GPT_PRELN,
                       attention=ee.ATTN_PADDED if args.attention == "padded" else ee.ATTN_VARLEN,
                       residual={"auto": ee.RESIDUAL_AUTO, "epilogue": ee.RESIDUAL_EPILOGUE,
                                 "pass": ee.RESIDUAL_PASS}[args.residual])
              for p in params]
    ws = torch.empty(layers[0].workspace_size(B, P, T_run), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    _log(f"weights {sum(t.numel() * t.element_size() for p in params for t in p.values()) / 1e9:.1f} GB resident; "
         f"workspace {ws.numel() / 1e6:.0f} MB")

    def step():
        ee.ee_stack_forward(layers, x, run_lens, y, ws, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _log(f"warmup done ({args.warmup} steps)")
    # the timed steps, with events around the roofline site's launches only
    # (every event pair leaves a stream bubble of a few us)
    t_host = time.perf_counter()
    ms, st_fc1 = _timed_steps(ee, stream, [step] * args.steps, ROOFLINE_SITE)
    t_host = time.perf_counter() - t_host
    ms_step = sum(ms) / args.steps
    srt = sorted(ms)
    # then as many steps with every launch site timed, for the per-kernel figures
    ms2, stats = _timed_steps(ee, stream, [step] * args.steps, None)
    ms_step_all = sum(ms2) / args.steps
    _log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host clock {1e3 * t_host / args.steps:.3f}; "
         f"p10 {_pct(srt, 0.1):.3f}, median {_pct(srt, 0.5):.3f}, p90 {_pct(srt, 0.9):.3f})")

    value = T * L / (ms_step / 1e3)

    def rows_of_site(site):
        return T if site in ("remove", "rebuild", "offsets") else T_run
    kernels = _kernel_table(w, stats, args.steps, sum(ms2), rows_of_site, B, P,
                            _attention_flops(w, run_lens, causal=not bert) * L * args.steps,
                            "res_ln2" not in stats)
    roofline = _roofline(w.name, st_fc1[ROOFLINE_SITE])
    if args.no_pack or bert:
        roofline["traffic"] = None

    cpu = None
    if not args.no_cpu_baseline and not (bert or args.no_pack or args.attention != "varlen"):
        nseq = args.cpu_sample_seqs or 24
        _log(f"timing the CPU oracle on {nseq} sequences")
        xh = x.cpu()
        cpu = _cpu_baseline(w, [xh[b, :lens[b]] for b in range(min(nseq, B))], params[0], L, 0,
                            f"the {w.name} batch")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "valid tokens/s per layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_p50_p90": [round(_pct(srt, q), 4) for q in (0.1, 0.5, 0.9)],
        "ms_per_step_with_kernel_events": round(ms_step_all, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16" if w.dtype == "f16" else "f32",
        "data": "synthetic (seeded lengths, N(0,1) activations, N(0,0.02) random-init weights)",
        "config": {"workload": w.name, "batch": B, "pad_len": P, "valid_tokens": T, "layers": L,
                   "hidden": w.hidden, "n_heads": w.n_heads, "head_dim": w.head_dim, "ffn": w.ffn,
                   "fuse_gelu": not args.no_fuse_gelu, "block": "bert-postln" if bert else "gpt-preln",
                   "attention": args.attention, "rows_run": T_run, "padding_removed": not args.no_pack,
                   "weight_rows": "dense" if args.dense_weights else "preferred pitch", "residual": args.residual},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def _decode_bench(args):
    """Incremental decoding: the workload's batch as prompts (prefill, untimed),
    then --decode-steps steps of one new token per sequence, timed; then as
    many steps again with per-launch events, for the per-kernel figures."""
    import torch

    import variable_length_padding_amd as ee
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    if args.decode_batch > 0:
        w = dataclasses.replace(w, batch=args.decode_batch)
    prompts = workloads.lengths(w, args.seed)
    B, L, N = len(prompts), w.layers, args.decode_steps
    s_el = w.elem_bytes
    H, Hp, F = w.hidden, w.inner, w.ffn
    params = [_stored(args, workloads.layer_params(w, args.seed, l, device=dev)) for l in range(L)]
    dt = ee.F16 if w.dtype == "f16" else ee.F32
    layers = [ee.Layer(H, w.n_heads, w.head_dim, F, p, dtype=dt) for p in params]
    slot_base, cap = [], 0
    for n in prompts:
        slot_base.append(cap)
        cap += n + 2 * N + args.warmup
    cache = torch.empty(ee.ee_kv_cache_bytes(layers[0], L, cap), dtype=torch.uint8, device=dev)
    T0 = sum(prompts)
    ws = torch.empty(ee.ee_extend_workspace_size(layers[0], B, max(T0, B)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    g = workloads.stream_generator(args.seed, workloads.REQUEST_STREAM_BASE - 1, dev)
    x0 = (w.x_std * torch.randn(T0, H, generator=g, device=dev)).to(w.torch_dtype)
    y0 = torch.empty_like(x0)
    xs = (w.x_std * torch.randn(2 * N + args.warmup, B, H, generator=g, device=dev)).to(w.torch_dtype)
    ys = torch.empty_like(xs)
    _log(f"decode {w.name}: {B} sequences, prompts T={T0}, {L} layers, {N} timed steps; cache "
         f"{cache.numel() / 1e9:.2f} GB for {cap} slots per layer")
    ee.ee_stack_extend(layers, x0, prompts, [0] * B, slot_base, cache, cap, y0, ws, stream)
    ctx = list(prompts)
    for i in range(args.warmup):
        ee.ee_stack_extend(layers, xs[i], [1] * B, ctx, slot_base, cache, cap, ys[i], ws, stream)
        ctx = [c + 1 for c in ctx]
    torch.cuda.synchronize()
    ctx_start = list(ctx)
    # timed steps; the per-launch events are left out of them (at ~40 launches
    # per step their stream bubbles cost ~5% here), and a second run of as
    # many steps records them for the per-kernel figures
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.warmup, args.warmup + N):
        ee.ee_stack_extend(layers, xs[i], [1] * B, ctx, slot_base, cache, cap, ys[i], ws, stream)
        ctx = [c + 1 for c in ctx]
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / N
    ee.ee_profile_enable(True)
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for i in range(args.warmup + N, args.warmup + 2 * N):
        ee.ee_stack_extend(layers, xs[i], [1] * B, ctx, slot_base, cache, cap, ys[i], ws, stream)
        ctx = [c + 1 for c in ctx]
    e3.record(stream)
    torch.cuda.synchronize()
    ee.ee_profile_enable(False)
    st = ee.ee_profile_collect()
    ms_step_events = e2.elapsed_time(e3) / N
    value = B * L / (ms_step / 1e3)
    # bytes a decode step must move: every layer's weights, the cached keys and
    # values it attends over, and the new tokens' rows (small)
    w_bytes = (H * 3 * Hp + Hp * H + 2 * H * F + 3 * Hp + 2 * H + F + 4 * H) * s_el
    mid_ctx = [c + N // 2 for c in ctx_start]          # context length half-way through the timed steps
    kv_bytes = sum(2 * (c + 1) * Hp * s_el for c in mid_ctx)
    step_bytes = L * (w_bytes + kv_bytes)
    kernels = {}
    for site, v in st.items():
        kernels[site] = {"launches_per_step": v["launches"] / N, "avg_ms": round(v["total_ms"] / v["launches"], 5),
                         "share": round(v["total_ms"] / (ms_step_events * N), 4)}
    fc1_ms = st["gemm_fc1"]["total_ms"] / st["gemm_fc1"]["launches"]
    fc1_bytes = (H * F + B * H + B * F) * s_el
    achieved = fc1_bytes / (fc1_ms * 1e-3) / 1e9
    _log(f"decode: {ms_step:.3f} ms per step, {value:.0f} tokens/s per layer, "
         f"{step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s of weights + cache")
    out = {
        "metric": "decode tokens/s per GPT layer (incremental, packed KV cache), 1 GPU", "value": round(value, 1),
        "unit": "decode tokens/s per layer", "n_gpus": 1, "steps": N, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if w.dtype == "f16" else "f32",
        "data": "synthetic (seeded prompts and token rows, N(0,0.02) random-init weights)",
        "config": {"weight_rows": "dense" if args.dense_weights else "preferred pitch", "workload": w.name, "mode": "decode", "sequences": B, "prompt_tokens": T0, "layers": L,
                   "hidden": H, "n_heads": w.n_heads, "head_dim": w.head_dim, "ffn": F},
        "ms_per_step_with_kernel_events": round(ms_step_events, 4),
        "roofline": {"bound": "hbm", "kernel": "gemm_fc1 at M = %d (stream-K GEMM + reduce; weights streamed once)" % B,
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(fc1_ms, 4), "bytes_per_launch": fc1_bytes,
                     "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1)},
        "cpu_baseline": None,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


def main(argv=None):
    args = _parse(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        _copy_calibration()
        return

    import torch

    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = workloads.get(args.workload)
    if args.decode_steps > 0:
        if w.requests:
            w = workloads.get("gpt3-12l")
            args.workload = w.name
        _decode_bench(args)
    elif w.requests:
        _stream_bench(args)
    else:
        _forward_bench(args)


if __name__ == "__main__":
    main()
