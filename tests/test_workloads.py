"""The seeded generator: determinism, stream independence, and the workload
facts the pages fix (CPU only)."""
import torch

import workloads


def test_scaling_workload_facts():
    # EnergonAI README, "Scaling Ability": GPT-3, 12 layers, FP16, batch 32,
    # sequence length = half the padding length.
    w = workloads.get("gpt3-12l")
    assert (w.layers, w.batch, w.dtype, w.hidden, w.n_heads * w.head_dim) == (12, 32, "f16", 12288, 12288)
    lens = workloads.lengths(w, 1)
    assert lens == [w.pad_len // 2] * 32 and sum(lens) == 4096


def test_request_stream_facts():
    # Announcement article, dynamic-batching test: lengths random up to 256,
    # each batch padded to its longest; 48 layers at TP=4 in the latency test.
    w = workloads.get("gpt3-48l-stream")
    groups = workloads.request_stream(w, 1234)
    assert len(groups) == 16 and all(len(g) == 64 for g in groups)
    flat = [n for g in groups for n in g]
    assert min(flat) >= 1 and max(flat) <= 256 and w.layers == 48


def test_tp_shard_shapes():
    w = workloads.get("gpt3-tp4-shard")
    assert 3 * w.inner == 9216 and w.inner == 3072 and w.ffn == 12288 and w.hidden == 12288


def test_determinism_and_streams():
    w = workloads.get("gpt2-small")
    a = workloads.activations(w, 7, 2, 16)
    b = workloads.activations(w, 7, 2, 16)
    c = workloads.activations(w, 8, 2, 16)
    assert a.dtype == torch.float16 and torch.equal(a, b) and not torch.equal(a, c)
    p0 = workloads.layer_params(w, 7, 0)
    p1 = workloads.layer_params(w, 7, 1)
    assert not torch.equal(p0["w_qkv"], p1["w_qkv"])
    assert torch.equal(p0["w_qkv"], workloads.layer_params(w, 7, 0)["w_qkv"])
    assert p0["w_qkv"].shape == (3 * 768, 768) and p0["w_fc2"].shape == (768, 3072)
    assert torch.all(p0["b_qkv"] == 0) and torch.all(p0["ln1_g"] == 1)
    pa = workloads.layer_params(w, 7, 0, variant="affine")
    assert torch.any(pa["b_qkv"] != 0) and torch.any(pa["ln1_g"] != 1)
    lens = workloads.lengths(w, 7)
    assert len(lens) == 8 and all(1 <= n <= 128 for n in lens)
    assert lens == workloads.lengths(w, 7)


def test_nan_pad_fill():
    w = workloads.get("tiny-fp32")
    x = workloads.activations(w, 1, 2, 4, lens=[1, 4], pad_fill="nan")
    assert torch.isnan(x[0, 1:]).all() and not torch.isnan(x[0, :1]).any() and not torch.isnan(x[1]).any()
