#!/usr/bin/env python3
"""Throughput of the padding-removed GPT layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole hot path over one batch: offsets, remove,
L packed layers (LayerNorm, QKV GEMM, varlen causal attention, out GEMM,
LayerNorm, FC1 GEMM + GeLU, FC2 GEMM), rebuild -- one ee_stack_forward call.
Inputs (lengths, padded activations, every layer's weights) are generated
and resident in HBM before the timed region.  Prints one JSON line.

Metric: valid tokens/s per layer = T * L / (seconds per step).
roofline: the FC1 GEMM kernel (gelu epilogue, the largest single contraction;
the GEMMs together take ~97% of a step), algorithmic flops 2*T*H*F per launch
over its hipEvent-measured average duration on the launch stream, timed in the
timed steps (the only launches with events there); "kernels" comes from as
many further steps with every launch timed.
cpu_baseline: the CPU oracle's packed layer forward on a bounded sample.

    python bench.py --workload gpt3-48l-stream [--no-pack] [--max-batch N]

The request stream (1024 requests, lengths U[1,256], 48 layers): FIFO batches
and dynamically planned batches (ee_plan_dynamic, on a table of batch times
measured at the start of the run) each run once over the whole stream; the
line's value is the dynamic plan's valid tokens/s per layer, and "batching"
holds both plans' times, batch counts and padded-row ratios.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "valid tokens/s per GPT layer fwd (packed) + % HBM/MFMA roofline, 1 GPU"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROOFLINE_KERNEL = "gemm_fc1"
ROOFLINE_SYMBOL = "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, EE_EPI_BIAS_GELU, 2>"
ROOFLINE_MANGLED = "_ZN2ee12_GLOBAL__N_120gemm_f16_mfma_kernelILi16ELi256ELi256ELi2ELi2ELi3ELi2EEEvPKDF16_iS3_iS3_S3_PDF16_iiiiiiiPf"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_fc1_gpt3-12l_pmc.json")
GEMM_SOURCE = os.path.join(ROOT, "variable_length_padding_amd", "csrc", "gemm_f16.hip")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gpt3-12l")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=24)
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
    return ap.parse_args()


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _stored(args, params):
    """A layer's parameters as the bench hands them to libee: weight rows at
    the library's preferred pitch (dense with --dense-weights)."""
    import variable_length_padding_amd as ee
    return params if args.dense_weights else ee.pitched_weights(params)


def _site_work(w, T, B, P, site, res_in_gemm=True):
    """(algorithmic flops, algorithmic HBM bytes) of one launch at a site, for
    T rows run through the layer (res_in_gemm: the out and FC2 GEMMs read the
    residual in their epilogue)."""
    s = w.elem_bytes
    H, Hp, F = w.hidden, w.inner, w.ffn
    gemm = {"gemm_qkv": (H, 3 * Hp), "gemm_out": (Hp, H), "gemm_fc1": (H, F), "gemm_fc2": (F, H)}
    if site in gemm:
        K, N = gemm[site]
        res = T * N * s if res_in_gemm and site in ("gemm_out", "gemm_fc2") else 0
        return 2.0 * T * K * N, float((T * K + N * K + T * N) * s + res)
    if site in ("ln1", "ln2"):
        return 0.0, 2.0 * T * H * s
    if site == "remove":
        return 0.0, 2.0 * T * H * s
    if site == "rebuild":
        return 0.0, float((T + B * P) * H * s)
    if site == "attention":
        return 0.0, 4.0 * T * Hp * s
    if site == "rebuild_heads":          # q|k|v valid rows read, [3, B, nh, P, hd] written (pads as zeros)
        return 0.0, float(3 * (T + B * P) * Hp * s)
    if site == "remove_heads":
        return 0.0, 2.0 * T * Hp * s
    if site in ("add_ln1", "add_ln2"):   # u and residual read, y written
        return 0.0, 3.0 * T * H * s
    if site == "res_ln2":                 # u and residual read, sum and LN(sum) written
        return 0.0, 4.0 * T * H * s
    if site == "res_add":                 # u and residual read, sum written
        return 0.0, 3.0 * T * H * s
    if site == "bias_gelu":
        return 0.0, 2.0 * T * F * s
    return 0.0, 0.0


def _attention_flops(w, lens, causal=True):
    # QK^T and PV: 2 * 2 * hd * nh flops per (query, key) pair; len(len+1)/2
    # pairs per sequence under the causal mask, len^2 without it
    if causal:
        return sum(2.0 * w.inner * n * (n + 1) for n in lens)
    return sum(4.0 * w.inner * n * n for n in lens)


def gemm_code_sha256(path=GEMM_SOURCE):
    """sha256 of the GEMM source's code: // comments, trailing spaces and
    blank lines removed (the file holds no // inside string literals), so an
    edit of the comments keeps counters taken on the same code valid."""
    with open(path) as f:
        lines = [ln.split("//", 1)[0].rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def _traffic(workload):
    """HBM bytes per FC1 launch from the committed counter summary, if it was
    taken on this workload and on the current GEMM code."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
        if s.get("workload") != workload or s.get("gemm_code_sha256") != gemm_code_sha256():
            return None
        return s["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def _cpu_baseline(w, lens, x_host, params_dev, nseq):
    """Times the oracle (numpy float64, as it stands) on `nseq` sequences of the
    batch through layer 0."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    params64 = oracle.to_f64_params(params_dev)          # input preparation, untimed
    pick = list(range(min(nseq, len(lens))))
    rows = [x_host[b, :lens[b]].double().numpy() for b in pick]
    xs = np.concatenate(rows, axis=0)
    cu = np.concatenate([[0], np.cumsum([lens[b] for b in pick])])
    t0 = time.perf_counter()
    oracle.layer_forward_packed(xs, cu, params64, w.n_heads, w.head_dim)
    dt = time.perf_counter() - t0
    ntok = int(cu[-1])
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": ntok / dt, "unit": "valid tokens/s per layer", "cores": threads, "kind": "oracle",
            "sample": f"{len(pick)} sequences ({ntok} valid tokens) of the {w.name} batch through layer 0, "
                      f"float64 numpy oracle, {dt:.1f} s"}


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


def _stream_bench(args):
    """The request stream: both planners (FIFO and dynamic) over all requests
    through all layers, one timed pass each, in one process."""
    import numpy as np
    import torch

    import variable_length_padding_amd as ee
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    lens = [n for g in workloads.request_stream(w, args.seed) for n in g]
    n_req, L, P_max = len(lens), w.layers, w.pad_len
    cap = args.max_batch or w.batch
    T = sum(lens)
    stream = torch.cuda.current_stream()
    _log(f"request stream {w.name}: {n_req} requests, T={T}, {L} layers, batch cap {cap}, "
         f"padding {'kept' if args.no_pack else 'removed'}")
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

    def run(x, batch_lens, y):
        B, P, _ = x.shape
        ee.ee_stack_forward(layers, x, [P] * B if args.no_pack else batch_lens, y, ws, stream)

    # cost model "by machine performance" (TurboTransformers' scheduler works
    # from a table of measured batch times): the whole stack timed on batches
    # of `cap` equal-length requests, tokens = (k + 1) * 8 * cap, no padding
    # (random activations: the chip draws more power, and clocks lower, on random data than on zeros)
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
    plans = {"fifo": ee.batches_of(ee.ee_plan_fifo(lens, cap)),
             "dynamic": ee.batches_of(ee.ee_plan_dynamic(lens, cap, cost)[0])}
    results = {}
    fc1 = {}
    for name, plan in plans.items():
        xs = [workloads.pad_batch([reqs[i] for i in b]) for b in plan]
        ys = [torch.empty_like(x) for x in xs]
        bls = [[lens[i] for i in b] for b in plan]
        run(xs[0], bls[0], ys[0])                     # warm-up: one batch
        torch.cuda.synchronize()
        ee.ee_profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for x, bl, y in zip(xs, bls, ys):
            run(x, bl, y)
        e1.record(stream)
        torch.cuda.synchronize()
        ee.ee_profile_enable(False)
        st = ee.ee_profile_collect()
        sec = e0.elapsed_time(e1) / 1e3
        rows = sum(x.shape[0] * x.shape[1] for x in xs)
        rows_run = rows if args.no_pack else T
        fc1[name] = (st["gemm_fc1"]["total_ms"], 2.0 * rows_run * w.hidden * w.ffn * L)
        results[name] = {
            "batches": len(plan), "padded_rows": rows, "padded_ratio": round(rows / T, 4), "rows_run": rows_run,
            "seconds": round(sec, 3), "value": round(T * L / sec, 1),
            "predicted_seconds": round(sum(ee.ee_batch_cost_eval(bl, cost) for bl in bls), 3)}
        _log(f"{name}: {len(plan)} batches, padded/valid rows {rows / T:.3f}, {sec:.2f} s, "
             f"{T * L / sec:.0f} valid tokens/s per layer (model {results[name]['predicted_seconds']:.2f} s)")
        del xs, ys
        torch.cuda.synchronize()

    ms, flops = fc1["dynamic"]
    achieved = flops / (ms * 1e-3) / 1e12
    d = results["dynamic"]
    out = {
        "metric": METRIC, "value": d["value"], "unit": "valid tokens/s per layer", "n_gpus": 1, "steps": 1,
        "warmup": 1, "ms_per_step": round(1e3 * d["seconds"], 1), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16" if w.dtype == "f16" else "f32",
        "data": "synthetic (seeded request lengths U[1,%d], N(0,1) activations, N(0,0.02) random-init weights)" % P_max,
        "config": {"weight_rows": "dense" if args.dense_weights else "preferred pitch", "workload": w.name, "requests": n_req, "valid_tokens": T, "layers": L, "max_batch": cap,
                   "hidden": w.hidden, "n_heads": w.n_heads, "head_dim": w.head_dim, "ffn": w.ffn,
                   "batching": "dynamic", "padding_removed": not args.no_pack},
        "roofline": {"bound": "mfma", "kernel": ROOFLINE_SYMBOL, "achieved": round(achieved, 1),
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": None, "note": "FC1 launches of the dynamic plan: summed flops over summed time"},
        "cpu_baseline": None,
        "batching": {"fifo": results["fifo"], "dynamic": d,
                     "dynamic_over_fifo": round(d["value"] / results["fifo"]["value"], 4),
                     "cost_model": {"t_row": cost.t_row, "token_quantum": quantum,
                                    "token_table_s": [round(v, 4) for v in table],
                                    "check": [[B, T, round(t, 4), round(m, 4)] for B, T, t, m in checks]}},
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


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.copy_calibration:
        _copy_calibration()
        return

    import torch

    import variable_length_padding_amd as ee
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    if w.requests:
        _stream_bench(args)
        return
    if args.decode_steps > 0:
        _decode_bench(args)
        return
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

    for _ in range(args.warmup):
        ee.ee_stack_forward(layers, x, run_lens, y, ws, stream)
    torch.cuda.synchronize()
    _log(f"warmup done ({args.warmup} steps)")

    # the timed steps, with events around the roofline kernel's launches only
    # (every event pair leaves a stream bubble of a few us)
    ee.ee_profile_filter(ROOFLINE_KERNEL)
    ee.ee_profile_enable(True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    e0, e1 = marks[0], marks[-1]
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        ee.ee_stack_forward(layers, x, run_lens, y, ws, stream)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ee.ee_profile_enable(False)
    fc1 = ee.ee_profile_collect()[ROOFLINE_KERNEL]
    ms_step = e0.elapsed_time(e1) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    # then as many steps with every launch site timed, for the per-kernel figures
    ee.ee_profile_filter(None)
    ee.ee_profile_enable(True)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(args.steps):
        ee.ee_stack_forward(layers, x, run_lens, y, ws, stream)
    b1.record(stream)
    torch.cuda.synchronize()
    ee.ee_profile_enable(False)
    stats = ee.ee_profile_collect()
    ms_step_all = b0.elapsed_time(b1) / args.steps

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    _log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host clock {1e3 * t_host / args.steps:.3f}; "
         f"p10 {pct(0.1):.3f}, median {pct(0.5):.3f}, p90 {pct(0.9):.3f})")

    value = T * L / (ms_step / 1e3)
    kernels = {}
    for site, st in stats.items():
        n = st["launches"]
        avg_ms = st["total_ms"] / n
        fl, by = _site_work(w, T_run, B, P, site, res_in_gemm="res_ln2" not in stats)
        if site == "attention":
            fl = _attention_flops(w, run_lens, causal=not bert)
        k = {"launches_per_step": n / args.steps, "avg_ms": round(avg_ms, 5),
             "share": round(st["total_ms"] / (ms_step_all * args.steps), 4)}
        if fl:
            k["tflops"] = round(fl / (avg_ms * 1e-3) / 1e12, 1)
            k["mfma_frac"] = round(k["tflops"] / PEAK_F16_TFLOPS, 4)
        if by:
            k["gbs"] = round(by / (avg_ms * 1e-3) / 1e9, 1)
            k["hbm_frac"] = round(k["gbs"] / PEAK_HBM_GBS, 4)
        kernels[site] = k

    fc1_ms = fc1["total_ms"] / fc1["launches"]
    fc1_flops = _site_work(w, T_run, B, P, ROOFLINE_KERNEL)[0]
    achieved = fc1_flops / (fc1_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": ROOFLINE_SYMBOL, "symbol": ROOFLINE_MANGLED, "achieved": round(achieved, 1),
                "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                "traffic": _traffic(w.name) if not (args.no_pack or bert) else None, "avg_launch_ms": round(fc1_ms, 4),
                "flops_per_launch": fc1_flops}

    cpu = None
    if not args.no_cpu_baseline and not (bert or args.no_pack or args.attention != "varlen"):
        _log("timing the CPU oracle on a bounded sample")
        cpu = _cpu_baseline(w, lens, x.cpu(), params[0], args.cpu_sample_seqs)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "valid tokens/s per layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
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


if __name__ == "__main__":
    main()
