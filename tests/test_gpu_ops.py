"""Per-kernel parity of the HIP path against the CPU oracle, through the C ABI.

Bars: bit-exact for offsets, indices and remove/rebuild; bit-exact for the
integer-valued GEMM test; otherwise a normwise relative error bound derived
from fp16 output rounding (2^-11 relative, plus fp32 accumulation), written
in each test."""
import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
from gpu_helpers import DEV, Guarded, normwise_rel, say, to_host64, valid_mask

pytestmark = pytest.mark.gpu

GEN = torch.Generator().manual_seed(20240607)


def _i32(n):
    return torch.empty(max(1, n), dtype=torch.int32, device=DEV)


# ------------------------------------------------------------------ offsets
LEN_CASES = [
    ([2, 0, 3], 4), ([1] * 7, 5), ([9] * 3, 9), ([0, 0, 0], 6), ([5], 5), ([0], 3),
    ([0, 128, 1, 64, 127, 128, 33, 2], 128),
]


def _rand_lens(B, P, seed, lo=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, P + 1, (B,), generator=g).tolist()


@pytest.mark.parametrize("lens,P", LEN_CASES + [(_rand_lens(512, 256, 1), 256), (_rand_lens(64, 3000, 2), 3000)])
def test_offsets_bit_exact(lens, P):
    B = len(lens)
    cu, src, p2p = _i32(B + 1), _i32(B * P), _i32(B * P)
    src.fill_(-7)
    T = ee.ee_compute_offsets(lens, P, cu, src, p2p)
    torch.cuda.synchronize()
    rcu, rsrc, rp2p, rT = oracle.offsets_from_lengths(lens, P)
    assert T == rT
    assert cu.cpu().tolist() == rcu.tolist()
    assert p2p.cpu().tolist() == rp2p.tolist()
    assert src.cpu()[:T].tolist() == rsrc.tolist()
    assert torch.all(src.cpu()[T:] == -7)   # entries past T untouched


@pytest.mark.parametrize("lens,P", LEN_CASES + [(_rand_lens(64, 256, 3), 256), (_rand_lens(40, 1000, 4), 1000)])
def test_offsets_from_mask_bit_exact(lens, P):
    B = len(lens)
    mask = torch.tensor(valid_mask(lens, P).astype(np.uint8), device=DEV)
    cu, src, p2p, tot = _i32(B + 1), _i32(B * P), _i32(B * P), _i32(1)
    ee.ee_compute_offsets_mask(mask, cu, src, p2p, tot)
    torch.cuda.synchronize()
    rcu, rsrc, rp2p, rT = oracle.offsets_from_mask(mask.cpu().numpy())
    assert int(tot.item()) == rT == sum(lens)
    assert cu.cpu().tolist() == rcu.tolist()
    assert p2p.cpu().tolist() == rp2p.tolist()
    assert src.cpu()[:rT].tolist() == rsrc.tolist()


def test_offsets_from_general_mask():
    g = torch.Generator().manual_seed(5)
    m = (torch.rand(33, 77, generator=g) < 0.4).to(torch.uint8)
    B, P = m.shape
    cu, src, p2p, tot = _i32(B + 1), _i32(B * P), _i32(B * P), _i32(1)
    ee.ee_compute_offsets_mask(m.to(DEV), cu, src, p2p, tot)
    torch.cuda.synchronize()
    rcu, rsrc, rp2p, rT = oracle.offsets_from_mask(m.numpy())
    assert int(tot.item()) == rT
    assert cu.cpu().tolist() == rcu.tolist() and p2p.cpu().tolist() == rp2p.tolist()
    assert src.cpu()[:rT].tolist() == rsrc.tolist()


# ------------------------------------------------------------------ remove / rebuild
@pytest.mark.parametrize("dtype,H", [(torch.float16, 768), (torch.float16, 12288), (torch.float32, 64),
                                     (torch.float16, 8), (torch.float32, 1028)])
@pytest.mark.parametrize("lens,P", [([3, 0, 16, 1, 9], 16), ([128] * 4, 256), ([0, 0], 4), ([7], 7)])
def test_remove_rebuild_bit_exact(dtype, H, lens, P):
    B = len(lens)
    x = torch.randn(B, P, H, generator=GEN).to(dtype)
    mask = valid_mask(lens, P)
    x[torch.from_numpy(~mask)] = float("nan")          # pads must never reach the output
    xd = x.to(DEV)
    T = sum(lens)
    gp = Guarded((max(T, 1), H), dtype, fill=3.0)
    packed = gp.t
    gws = Guarded((ee.ee_padding_workspace_size(B, P),), torch.uint8)
    ws = gws.t
    ee.ee_remove_padding(xd, lens, packed, ws)
    gy = Guarded((B, P, H), dtype, fill=5.0)
    y = gy.t
    ee.ee_rebuild_padding(packed, lens, y, ws)
    torch.cuda.synchronize()
    gp.check("packed")
    gy.check("y")
    gws.check("the workspace")
    xn = x.numpy()
    ref_packed = oracle.remove_padding(xn, lens)
    if T:
        assert np.array_equal(packed.cpu().numpy()[:T].view(np.uint8), ref_packed.view(np.uint8))
    yr = y.cpu().numpy()
    ref_y = oracle.rebuild_padding(ref_packed, lens, P)
    assert np.array_equal(yr.view(np.uint8), ref_y.view(np.uint8))      # +0.0 pads, bit for bit
    assert not np.isnan(yr).any()


# ------------------------------------------------------------------ LayerNorm
@pytest.mark.parametrize("dtype,H,rows,tol", [
    (torch.float16, 768, 37, 2e-3), (torch.float16, 12288, 19, 2e-3), (torch.float16, 64, 300, 2e-3),
    (torch.float32, 64, 33, 1e-5), (torch.float32, 12288, 7, 1e-5), (torch.float16, 4096, 5, 2e-3),
    # more rows than the grid's workgroups: each walks several rows with gamma/beta held in registers
    (torch.float16, 12288, 2000, 2e-3), (torch.float32, 4096, 3001, 1e-5), (torch.float16, 8192, 1537, 2e-3),
])
def test_layernorm_parity(dtype, H, rows, tol):
    x = (torch.randn(rows, H, generator=GEN) * 3 + 0.7).to(dtype)
    g = (1 + 0.1 * torch.randn(H, generator=GEN)).to(dtype)
    b = (0.1 * torch.randn(H, generator=GEN)).to(dtype)
    gy = Guarded((rows, H), dtype)
    y = gy.t
    ee.ee_layernorm(x.to(DEV), g.to(DEV), b.to(DEV), 1e-5, y)
    torch.cuda.synchronize()
    gy.check("y")
    ref = oracle.layer_norm(x.double().numpy(), g.double().numpy(), b.double().numpy(), 1e-5)
    err = normwise_rel(to_host64(y), ref)
    say(f"layernorm {dtype} H={H}: rel {err:.2e}")
    assert err <= tol


# ------------------------------------------------------------------ GEMM
def _small_ints(shape, lo=-2, hi=2):
    return torch.randint(lo, hi + 1, shape, generator=GEN).to(torch.float16)


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (37, 96, 128), (300, 256, 192), (516, 2304, 768),
                                   (1000, 1000, 640), (4112, 768, 3072), (2048, 4096, 12288),
                                   (4100, 4200, 320), (4096, 4096, 1024), (4096, 4096, 64), (4300, 4096, 192),
                                   (4096, 4104, 128), (4096, 4099, 64), (4096, 4096, 256), (4096, 4352, 384),
                                   (4096, 4096, 12288), (4205, 9216, 512), (4205, 12288, 512)])
@pytest.mark.parametrize("epi", [ee.EPI_NONE, ee.EPI_BIAS, ee.EPI_BIAS_RESIDUAL])
def test_gemm_integer_exact(M, N, K, epi):
    """Small-integer fp16 operands: every product and partial sum is an integer
    below 2^24, exact in fp32 in any order, so the only rounding is the final
    fp32 -> fp16 one; the result must equal the fp16 rounding (nearest-even) of
    the exact sum, bit for bit."""
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias = _small_ints((N,)) if epi != ee.EPI_NONE else None
    R = _small_ints((M, N), -8, 8) if epi == ee.EPI_BIAS_RESIDUAL else None
    gc = Guarded((M, N), torch.float16)
    C = gc.t
    ee.ee_linear(A.to(DEV), W.to(DEV), None if bias is None else bias.to(DEV), None if R is None else R.to(DEV),
                 epi, C)
    torch.cuda.synchronize()
    gc.check("C")
    exact = A.double().numpy() @ W.double().numpy().T
    if bias is not None:
        exact = exact + bias.double().numpy()
    if R is not None:
        exact = exact + R.double().numpy()
    assert np.abs(exact).max() < 2 ** 24
    ref16 = exact.astype(np.float16)
    got = C.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), ref16.view(np.uint16)), \
        f"{np.count_nonzero(got != ref16)} of {got.size} differ"


@pytest.mark.parametrize("M,N,epi,gelu", [(4205, 9216, ee.EPI_BIAS, ee.GELU_TANH),
                                          (4205, 12288, ee.EPI_BIAS_GELU, ee.GELU_TANH),
                                          (4205, 12288, ee.EPI_BIAS_RESIDUAL, ee.GELU_TANH),
                                          (4300, 4096, ee.EPI_BIAS_GELU, ee.GELU_ERF)])
def test_gemm_row_split_bit_identical(M, N, epi, gelu):
    """Tile counts just past a multiple of the CU count run whole rounds of
    256 x 256 tiles and the remaining rows on 128 x 128 tiles (128 x 64 when
    few: the 12288-wide shapes and 4300 x 4096).  On random data
    the result must equal, bit for bit, GEMMs over each 256-row block alone
    (each small enough for 128 x 128 tiles only): every element sums the same
    K tiles in the same order whichever tile computes it."""
    K = 1024
    A = torch.randn(M, K, generator=GEN).half().to(DEV)
    W = (0.05 * torch.randn(N, K, generator=GEN)).half().to(DEV)
    bias = (0.1 * torch.randn(N, generator=GEN)).half().to(DEV)
    R = torch.randn(M, N, generator=GEN).half().to(DEV) if epi == ee.EPI_BIAS_RESIDUAL else None
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ee.ee_linear(A, W, bias, R, epi, C, gelu=gelu)
    parts = torch.empty_like(C)
    for r0 in range(0, M, 256):
        r1 = min(M, r0 + 256)
        ee.ee_linear(A[r0:r1], W, bias, None if R is None else R[r0:r1], epi, parts[r0:r1], gelu=gelu)
    torch.cuda.synchronize()
    diff = (C != parts).any(dim=1).nonzero().flatten().tolist()
    say(f"row split {M}x{N} epi={epi}: {len(diff)} rows differ from the per-block GEMMs")
    assert not diff, f"rows {diff[:8]}... differ"


@pytest.mark.parametrize("M,N", [(7317, 49152), (7889, 36864), (8731, 12288), (9036, 49152), (8192, 12288)])
def test_gemm_integer_exact_request_stream_rows(M, N):
    """Row counts of the request stream's batches at the layer's GEMM widths:
    29, 31, 35 and 36 M-tiles of 256, whose tiles_m % 4 leftover M-tiles the
    tile order shares out by N, some with a row split.  C starts as NaN; on
    small-integer operands two rows of every 256-row tile (its first and last),
    over all N, must be the fp16 rounding of the exact sum, bit for bit, so a
    tile computed twice or never shows."""
    K = 128
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias = _small_ints((N,))
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    ee.ee_linear(A.to(DEV), W.to(DEV), bias.to(DEV), None, ee.EPI_BIAS, C)
    torch.cuda.synchronize()
    rows = sorted({r for t in range(0, M, 256) for r in (t, min(M, t + 256) - 1)})
    exact = A[rows].double().numpy() @ W.double().numpy().T + bias.double().numpy()
    got = C[rows].cpu().numpy()
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16)), \
        f"{np.count_nonzero(got != exact.astype(np.float16))} of {got.size} differ"


# (M, N, K, epi): 256 x 256 tile counts that leave the persistent launch's last
# round partial, with whole rounds R and extra tiles E of 256 workgroups, split
# over P of them: R 23 / E 95 / P 190 (pieces of 32 K tiles), R 2 / E 100 /
# P 200 (the TP-shard QKV), R 3 / E 48 / P 96 (the TP-shard out projection
# width, K = 4096), R 3 / E 65 / P 130 (three W stages, K = 49152), R 6 / E
# 81 / P 162 with the residual, and R 1 / E 16 (too few rounds: the row split
# instead).  N is not a multiple of 384 where 256 x 384 tiles would be planned
# instead (the plans: tests/test_gemm_plan.py).
ORDERED = [(7889, 49408, 4096, ee.EPI_BIAS_GELU), (4205, 9216, 4096, ee.EPI_BIAS),
           (4205, 12288, 4096, ee.EPI_BIAS_RESIDUAL), (8436, 12544, 4096, ee.EPI_BIAS_RESIDUAL),
           (4205, 12544, 49152, ee.EPI_BIAS_RESIDUAL), (4300, 4096, 512, ee.EPI_NONE)]


@pytest.fixture(scope="module")
def linear_ws():
    return torch.empty(ee.ee_linear_ws_workspace_size(), dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("M,N,K,epi", ORDERED)
def test_gemm_ordered_split_bit_identical(M, N, K, epi, linear_ws):
    """The partial last round as in-order stream-K pieces (ee_linear_ws) gives
    ee_linear's bits on random data, twice in a row with the workspace's
    flags from the first call in place (each launch has its own tag), and
    after the workspace is filled with random bytes."""
    gen = torch.Generator(device="cpu").manual_seed(M + N + K)
    A = torch.randn(M, K, generator=gen).half().to(DEV)
    W = (0.05 * torch.randn(N, K, generator=gen)).half().to(DEV)
    bias = (0.1 * torch.randn(N, generator=gen)).half().to(DEV) if epi != ee.EPI_NONE else None
    R = torch.randn(M, N, generator=gen).half().to(DEV) if epi == ee.EPI_BIAS_RESIDUAL else None
    ref = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    ee.ee_linear(A, W, bias, R, epi, ref)
    for rep in range(3):
        if rep == 2:
            linear_ws.copy_(torch.randint(0, 256, linear_ws.shape, dtype=torch.uint8, generator=gen).to(DEV))
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        ee.ee_linear_ws(A, W, bias, R, epi, C, linear_ws)
        torch.cuda.synchronize()
        diff = (C.view(torch.int16) != ref.view(torch.int16)).any(dim=1).nonzero().flatten().tolist()
        say(f"ordered split {M}x{N}x{K} epi={epi} call {rep}: {len(diff)} rows differ from ee_linear")
        assert not diff, f"rows {diff[:8]}... differ"


# (M, N, K, epi) whose 256 x 384 tiles leave a partial last round that
# ee_linear_ws runs as in-order stream-K pieces of the same launch: R 15 / E
# 128 / P 256 (FC1 width), R 12 / E 96 / P 256 (QKV width), R 4 / E 32 / P 128
# (FC2: K = 49152, with the residual)
WIDE_ORDERED = [(7889, 49152, 4096, ee.EPI_BIAS_GELU), (8436, 36864, 4096, ee.EPI_BIAS),
                (8436, 12288, 49152, ee.EPI_BIAS_RESIDUAL)]


@pytest.mark.parametrize("M,N,K,epi", WIDE_ORDERED)
def test_gemm_wide_ordered_split_bit_identical(M, N, K, epi, linear_ws):
    """The in-order split of a 256 x 384 launch (ee_linear_ws) gives
    ee_linear's bits on random data, three calls in a row, the third on a
    workspace filled with random bytes first."""
    gen = torch.Generator().manual_seed(M + N + K)
    A = torch.randn(M, K, generator=gen).half().to(DEV)
    W = (0.05 * torch.randn(N, K, generator=gen)).half().to(DEV)
    bias = (0.1 * torch.randn(N, generator=gen)).half().to(DEV)
    R = torch.randn(M, N, generator=gen).half().to(DEV) if epi == ee.EPI_BIAS_RESIDUAL else None
    ref = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    ee.ee_linear(A, W, bias, R, epi, ref)
    for rep in range(3):
        if rep == 2:
            linear_ws.copy_(torch.randint(0, 256, linear_ws.shape, dtype=torch.uint8, generator=gen).to(DEV))
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        ee.ee_profile_enable(True)
        try:
            ee.ee_linear_ws(A, W, bias, R, epi, C, linear_ws)
            st = ee.ee_profile_collect()
        finally:
            ee.ee_profile_enable(False)
        torch.cuda.synchronize()
        assert st["linear"]["kernel"] == f"gemm_f16_mfma_kernel<16, 256, 384, 2, 2, {epi}, 2, true>"
        assert st["linear"]["launches"] == 1 and "linear_rest" not in st
        diff = (C.view(torch.int16) != ref.view(torch.int16)).any(dim=1).nonzero().flatten().tolist()
        say(f"wide ordered split {M}x{N}x{K} epi={epi} call {rep}: {len(diff)} rows differ from ee_linear")
        assert not diff, f"rows {diff[:8]}... differ"


def test_profile_splits_a_site_by_kernel(linear_ws):
    """A GEMM site whose launches ran the plain and the in-order split form of
    the large kernel (N = 16384, 64 tile columns; 8192 rows: whole rounds;
    8500 rows: 128 extra tiles) is reported per kernel: by_kernel holds both
    labels with their launches and flops, and the site's kernel reads
    "several kernels"."""
    N, K = 16384, 4096
    W = (0.05 * torch.randn(N, K, generator=GEN)).half().to(DEV)
    bias = torch.zeros(N, dtype=torch.float16, device=DEV)
    ee.ee_profile_enable(True)
    try:
        for M in (8192, 8500):
            A = torch.randn(M, K, generator=GEN).half().to(DEV)
            C = torch.empty(M, N, dtype=torch.float16, device=DEV)
            ee.ee_linear_ws(A, W, bias, None, ee.EPI_BIAS_GELU, C, linear_ws)
        st = ee.ee_profile_collect()["linear"]
    finally:
        ee.ee_profile_enable(False)
    plain = "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 3, 2, false>"
    split = "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 3, 2, true>"
    assert st["launches"] == 2 and st["kernel"] == "several kernels"
    assert set(st["by_kernel"]) == {plain, split}
    assert st["by_kernel"][plain]["flops"] == 2.0 * 8192 * N * K
    assert st["by_kernel"][split]["flops"] == 2.0 * 8500 * N * K


@pytest.mark.parametrize("M,N,K", [(7889, 49408, 4096), (4205, 12288, 4096)])
def test_gemm_ordered_split_integer_exact(M, N, K, linear_ws):
    """Small-integer operands through ee_linear_ws: two rows of every 256-row
    tile, over all N, are the fp16 rounding of the exact sum, bit for bit."""
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias = _small_ints((N,))
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    ee.ee_linear_ws(A.to(DEV), W.to(DEV), bias.to(DEV), None, ee.EPI_BIAS, C, linear_ws)
    torch.cuda.synchronize()
    rows = sorted({r for t in range(0, M, 256) for r in (t, min(M, t + 256) - 1)})
    exact = A[rows].double().numpy() @ W.double().numpy().T + bias.double().numpy()
    got = C[rows].cpu().numpy()
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("K", [32768, 49152 + 64])
def test_gemm_integer_exact_long_k(K):
    """Long K ranges (>= 32768) take the three-W-stage ring of the 256 x 256 tile
    (W requested two K tiles ahead): bit-exact on small-integer operands, checked
    on sampled rows (rows are independent), bias + residual epilogue."""
    M, N = 4096, 4096
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias, R = _small_ints((N,)), _small_ints((M, N), -8, 8)
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ee.ee_linear(A.to(DEV), W.to(DEV), bias.to(DEV), R.to(DEV), ee.EPI_BIAS_RESIDUAL, C)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 2047, 3840, 4095]
    exact = A[rows].double().numpy() @ W.double().numpy().T + bias.double().numpy() + R[rows].double().numpy()
    assert np.abs(exact).max() < 2 ** 24
    got = C[rows].cpu().numpy()
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))


# (M, N, K, epi) planned on 256 x 384 tiles (N a multiple of 384): whole
# rounds of them (16 rounds at 8192 x 49152; 6 at 4096 x 36864), and rows
# past the whole rounds on the 256 x 256 plan's smaller tiles (7889 rows: 209
# rows on 128 x 128 tiles; 4205 rows: 109 rows on 128 x 64 tiles)
WIDE = [(8192, 49152, 8192, ee.EPI_BIAS_GELU), (7889, 49152, 4096, ee.EPI_BIAS),
        (4096, 36864, 8192, ee.EPI_BIAS_RESIDUAL), (4205, 12288, 12288, ee.EPI_NONE)]
WIDE_LABEL = "gemm_f16_mfma_kernel<16, 256, 384, 2, 2, {}, 2, false>"


@pytest.mark.parametrize("M,N,K,epi", WIDE)
def test_gemm_wide_tile_matches_square_tile(M, N, K, epi):
    """The 256 x 384 tile against the 256 x 256 one on random data: the same
    problem with 256 more W rows (N + 256 columns, which no 256 x 384 plan
    covers) gives the same bits in the first N columns, since every output
    element adds its K tiles in the same order with the same MFMA shape."""
    gen = torch.Generator().manual_seed(M + N + K + epi)
    A = torch.randn(M, K, generator=gen).half().to(DEV)
    W = (0.05 * torch.randn(N + 256, K, generator=gen)).half().to(DEV)
    bias = (0.1 * torch.randn(N + 256, generator=gen)).half().to(DEV)
    R = torch.randn(M, N + 256, generator=gen).half().to(DEV) if epi == ee.EPI_BIAS_RESIDUAL else None
    wide = Guarded((M, N), torch.float16, fill=float("nan"))
    ee.ee_profile_enable(True)
    try:
        ee.ee_linear(A, W[:N], None if epi == ee.EPI_NONE else bias[:N],
                     None if R is None else R[:, :N].contiguous(), epi, wide.t)
        st = ee.ee_profile_collect()
    finally:
        ee.ee_profile_enable(False)
    square = torch.full((M, N + 256), float("nan"), dtype=torch.float16, device=DEV)
    ee.ee_linear(A, W, None if epi == ee.EPI_NONE else bias, R, epi, square)
    torch.cuda.synchronize()
    wide.check("C")
    assert st["linear"]["kernel"] == WIDE_LABEL.format(epi)
    rows_w = st["linear"]["flops"] / (2.0 * N * K)
    say(f"wide {M}x{N}x{K} epi={epi}: {rows_w:.0f} rows on 256 x 384 tiles, rest {st.get('linear_rest', {}).get('kernel')}")
    diff = (wide.t.view(torch.int16) != square[:, :N].view(torch.int16)).any(dim=1).nonzero().flatten().tolist()
    assert not diff, f"{len(diff)} rows differ, first {diff[:8]}"


@pytest.mark.parametrize("M,N,K", [(8192, 49152, 8192), (2700, 36864, 12288)])
def test_gemm_wide_tile_integer_exact(M, N, K):
    """Small-integer operands on 256 x 384 tiles (and the rows after their
    whole rounds): two rows of every 256-row tile, over all N, are the fp16
    rounding of the exact sum, bit for bit."""
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias = _small_ints((N,))
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
    ee.ee_profile_enable(True)
    try:
        ee.ee_linear(A.to(DEV), W.to(DEV), bias.to(DEV), None, ee.EPI_BIAS, C)
        st = ee.ee_profile_collect()
    finally:
        ee.ee_profile_enable(False)
    torch.cuda.synchronize()
    assert st["linear"]["kernel"] == WIDE_LABEL.format(ee.EPI_BIAS)
    rows = sorted({r for t in range(0, M, 256) for r in (t, min(M, t + 256) - 1)})
    exact = A[rows].double().numpy() @ W.double().numpy().T + bias.double().numpy()
    got = C[rows].cpu().numpy()
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))


def test_profile_reports_wide_tiles_and_rest():
    """7889 x 49152: 30 M-tiles of 256 x 384 tiles fill 15 whole rounds (site
    "linear"); the last 209 rows run on 128 x 128 tiles (site "linear_rest")."""
    M, N, K = 7889, 49152, 1024
    A = torch.randn(M, K, generator=GEN).half().to(DEV)
    W = (0.05 * torch.randn(N, K, generator=GEN)).half().to(DEV)
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ee.ee_profile_enable(True)
    try:
        ee.ee_linear(A, W, None, None, ee.EPI_NONE, C)
        st = ee.ee_profile_collect()
    finally:
        ee.ee_profile_enable(False)
    assert st["linear"]["kernel"] == WIDE_LABEL.format(ee.EPI_NONE)
    assert st["linear"]["flops"] == 2.0 * 7680 * N * K
    assert st["linear_rest"]["kernel"] == "gemm_f16_mfma_kernel<32, 128, 128, 2, 2, 0, 2, false>"
    assert st["linear_rest"]["flops"] == 2.0 * 209 * N * K


@pytest.mark.parametrize("M,rest_kernel", [(4205, "gemm_f16_mfma_kernel<32, 128, 64, 2, 2, 2, 2, false>"),
                                           (8457, "gemm_f16_mfma_kernel<32, 128, 128, 2, 2, 2, 2, false>")])
def test_gemm_integer_exact_row_split_long_k(M, rest_kernel):
    """The FC2 shape of the layer (N = 12288, K = 49152, A and W rows at the
    preferred 49216-element pitch) at row counts past whole rounds of 256 x
    384 tiles: those rounds (timed as site "linear"), the remaining rows on
    smaller tiles (site "linear_rest").  Small-integer operands, so the result
    is the fp16 rounding of the exact sum, bit for bit, on sampled rows of
    both parts."""
    N, K = 12288, 49152
    ld = ee.ee_preferred_row_pitch(K)
    assert ld == K + 64
    A = torch.zeros(M, ld, dtype=torch.float16)
    A[:, :K] = _small_ints((M, K))
    W = torch.zeros(N, ld, dtype=torch.float16)
    W[:, :K] = _small_ints((N, K))
    bias, R = _small_ints((N,)), _small_ints((M, N), -8, 8)
    Ad, Wd = A.to(DEV)[:, :K], W.to(DEV)[:, :K]
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ee.ee_profile_enable(True)
    try:
        ee.ee_linear(Ad, Wd, bias.to(DEV), R.to(DEV), ee.EPI_BIAS_RESIDUAL, C)
        st = ee.ee_profile_collect()
    finally:
        ee.ee_profile_enable(False)
    torch.cuda.synchronize()
    m_big = M // 256 * 256 if M == 4205 else 8192
    assert st["linear"]["kernel"] == "gemm_f16_mfma_kernel<16, 256, 384, 2, 2, 2, 2, false>"
    assert st["linear_rest"]["kernel"] == rest_kernel
    assert st["linear"]["flops"] == 2.0 * m_big * N * K and st["linear_rest"]["flops"] == 2.0 * (M - m_big) * N * K
    rows = [0, 1, 255, m_big - 1, m_big, m_big + 1, (m_big + M) // 2, M - 1]
    exact = (A[rows, :K].double().numpy() @ W[:, :K].double().numpy().T + bias.double().numpy() +
             R[rows].double().numpy())
    assert np.abs(exact).max() < 2 ** 24
    got = C[rows].cpu().numpy()
    say(f"row split M={M} at K={K}: rest {M - m_big} rows on {rest_kernel}")
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("M,N,K,splits", [(1, 1024, 1024, 2), (32, 12288, 4096, 8), (100, 4104, 1024, 4),
                                          (128, 4099, 512, 2), (32, 640, 2048, 16), (77, 256, 128, 2)])
@pytest.mark.parametrize("epi", [ee.EPI_NONE, ee.EPI_BIAS, ee.EPI_BIAS_RESIDUAL])
def test_gemm_splitk_integer_exact(M, N, K, splits, epi):
    """Split-K on small-integer operands: each K range's partial sum and the
    sum of the partials are integers below 2^24, exact in fp32, so the result
    is the fp16 rounding of the exact sum, bit for bit, as unsplit."""
    A, W = _small_ints((M, K)), _small_ints((N, K))
    bias = _small_ints((N,)) if epi != ee.EPI_NONE else None
    R = _small_ints((M, N), -8, 8) if epi == ee.EPI_BIAS_RESIDUAL else None
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ws = torch.empty(ee.ee_linear_splitk_workspace_size(M, N, splits), dtype=torch.uint8, device=DEV)
    ee.ee_linear_splitk(A.to(DEV), W.to(DEV), None if bias is None else bias.to(DEV),
                        None if R is None else R.to(DEV), epi, C, splits, ws)
    torch.cuda.synchronize()
    exact = A.double().numpy() @ W.double().numpy().T
    if bias is not None:
        exact = exact + bias.double().numpy()
    if R is not None:
        exact = exact + R.double().numpy()
    assert np.abs(exact).max() < 2 ** 24
    ref16 = exact.astype(np.float16)
    got = C.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), ref16.view(np.uint16)), \
        f"{np.count_nonzero(got != ref16)} of {got.size} differ"


@pytest.mark.parametrize("gelu", [ee.GELU_TANH, ee.GELU_ERF])
def test_gemm_splitk_random_matches_unsplit(gelu):
    M, N, K = 32, 4096, 12288
    A = torch.randn(M, K, generator=GEN).to(torch.float16).to(DEV)
    W = (0.02 * torch.randn(N, K, generator=GEN)).to(torch.float16).to(DEV)
    bias = (0.1 * torch.randn(N, generator=GEN)).to(torch.float16).to(DEV)
    C1 = torch.empty(M, N, dtype=torch.float16, device=DEV)
    C8 = torch.empty_like(C1)
    ee.ee_linear(A, W, bias, None, ee.EPI_BIAS_GELU, C1, gelu=gelu)
    ws = torch.empty(ee.ee_linear_splitk_workspace_size(M, N, 8), dtype=torch.uint8, device=DEV)
    ee.ee_linear_splitk(A, W, bias, None, ee.EPI_BIAS_GELU, C8, 8, ws, gelu=gelu)
    torch.cuda.synchronize()
    u = oracle.linear(A.double().cpu().numpy(), W.double().cpu().numpy(), bias.double().cpu().numpy())
    ref = oracle.gelu(u, "tanh" if gelu == ee.GELU_TANH else "erf")
    assert normwise_rel(to_host64(C8), ref) <= 2e-3 and normwise_rel(to_host64(C1), ref) <= 2e-3


@pytest.mark.parametrize("M,N,K,epi,gelu", [
    (129, 768, 768, ee.EPI_BIAS_GELU, ee.GELU_TANH), (516, 3072, 768, ee.EPI_BIAS_GELU, ee.GELU_ERF),
    (4100, 1024, 1024, ee.EPI_BIAS_GELU, ee.GELU_TANH), (77, 2304, 768, ee.EPI_BIAS, ee.GELU_TANH),
])
def test_gemm_f16_random_parity(M, N, K, epi, gelu):
    A = torch.randn(M, K, generator=GEN).to(torch.float16)
    W = (0.02 * torch.randn(N, K, generator=GEN)).to(torch.float16)
    bias = (0.1 * torch.randn(N, generator=GEN)).to(torch.float16)
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ee.ee_linear(A.to(DEV), W.to(DEV), bias.to(DEV), None, epi, C, gelu=gelu)
    torch.cuda.synchronize()
    u = oracle.linear(A.double().numpy(), W.double().numpy(), bias.double().numpy())
    ref = oracle.gelu(u, "tanh" if gelu == ee.GELU_TANH else "erf") if epi == ee.EPI_BIAS_GELU else u
    err = normwise_rel(to_host64(C), ref)
    say(f"gemm f16 {M}x{N}x{K} epi={epi}: rel {err:.2e}")
    assert err <= 2e-3


@pytest.mark.parametrize("M,N,K", [(5, 7, 3), (64, 256, 64), (100, 70, 130)])
@pytest.mark.parametrize("epi", [ee.EPI_BIAS, ee.EPI_BIAS_RESIDUAL, ee.EPI_BIAS_GELU])
def test_gemm_f32_parity(M, N, K, epi):
    A = torch.randn(M, K, generator=GEN)
    W = 0.1 * torch.randn(N, K, generator=GEN)
    bias = torch.randn(N, generator=GEN)
    R = torch.randn(M, N, generator=GEN)
    C = torch.empty(M, N, device=DEV)
    ee.ee_linear(A.to(DEV), W.to(DEV), bias.to(DEV), R.to(DEV) if epi == ee.EPI_BIAS_RESIDUAL else None, epi, C)
    torch.cuda.synchronize()
    ref = oracle.linear(A.double().numpy(), W.double().numpy(), bias.double().numpy())
    if epi == ee.EPI_BIAS_RESIDUAL:
        ref = ref + R.double().numpy()
    if epi == ee.EPI_BIAS_GELU:
        ref = oracle.gelu(ref)
    assert normwise_rel(to_host64(C), ref) <= 1e-5


@pytest.mark.parametrize("dtype,tol", [(torch.float16, 2e-3), (torch.float32, 1e-6)])
@pytest.mark.parametrize("gelu", [ee.GELU_TANH, ee.GELU_ERF])
def test_bias_gelu_parity(dtype, tol, gelu):
    u = (2 * torch.randn(300, 3072, generator=GEN)).to(dtype)
    b = torch.randn(3072, generator=GEN).to(dtype)
    g = torch.empty_like(u, device=DEV)
    ee.ee_bias_gelu(u.to(DEV), b.to(DEV), g, gelu=gelu)
    torch.cuda.synchronize()
    ref = oracle.gelu(u.double().numpy() + b.double().numpy(), "tanh" if gelu == ee.GELU_TANH else "erf")
    assert normwise_rel(to_host64(g), ref) <= tol


# ------------------------------------------------------------------ attention
ATTN_LENS = [1, 31, 32, 33, 127, 128, 129, 200, 256, 5]


@pytest.mark.parametrize("dtype,hd,nh,tol", [
    (torch.float16, 128, 2, 3e-3), (torch.float16, 64, 3, 3e-3), (torch.float16, 32, 2, 3e-3),
    (torch.float16, 16, 4, 3e-3), (torch.float32, 16, 4, 1e-5), (torch.float32, 64, 2, 1e-5),
    (torch.float32, 128, 1, 1e-5),
])
def test_attention_varlen_parity(dtype, hd, nh, tol):
    lens = ATTN_LENS
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu_h[-1])
    qkv = torch.randn(T, 3 * nh * hd, generator=GEN).to(dtype)
    go = Guarded((T, nh * hd), dtype, fill=7.0)
    o = go.t
    cu = torch.tensor(cu_h, device=DEV)
    ee.ee_attention_varlen(qkv.to(DEV), cu, len(lens), max(lens), nh, hd, o)
    torch.cuda.synchronize()
    go.check("o")
    ref = oracle.causal_attention_packed(qkv.double().numpy(), cu_h, nh, hd)
    got = to_host64(o)
    err = normwise_rel(got, ref)
    say(f"attention {dtype} hd={hd} nh={nh}: rel {err:.2e}")
    assert err <= tol
    # query 0 of every sequence sees only key 0: o = v0 (up to the output rounding)
    Hp = nh * hd
    v = qkv.double().numpy()[:, 2 * Hp:]
    for b in range(len(lens)):
        assert np.allclose(got[cu_h[b]], v[cu_h[b]], rtol=1e-3 if dtype == torch.float16 else 1e-6, atol=1e-6)


@pytest.mark.parametrize("dtype,hd,nh,tol", [
    (torch.float16, 128, 1, 3e-3), (torch.float16, 64, 2, 3e-3), (torch.float16, 32, 2, 3e-3),
    (torch.float32, 64, 1, 1e-5),
])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_long_sequences(dtype, hd, nh, tol, causal):
    """Sequences of thousands of keys (up to 128 key tiles per query tile,
    ragged ends) against the whole oracle, causal and bidirectional."""
    lens = [2048, 1, 4095, 777]
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu_h[-1])
    qkv = torch.randn(T, 3 * nh * hd, generator=GEN).to(dtype)
    go = Guarded((T, nh * hd), dtype, fill=7.0)
    o = go.t
    ee.ee_attention_varlen(qkv.to(DEV), torch.tensor(cu_h, device=DEV), len(lens), max(lens), nh, hd, o,
                           causal=causal)
    torch.cuda.synchronize()
    go.check("o")
    if causal:
        ref = oracle.causal_attention_packed(qkv.double().numpy(), cu_h, nh, hd)
    else:
        ref = oracle.attention_packed_bidirectional(qkv.double().numpy(), cu_h, nh, hd)
    err = normwise_rel(to_host64(o), ref)
    say(f"attention long causal={causal} {dtype} hd={hd} nh={nh} lens={lens}: rel {err:.2e}")
    assert err <= tol


@pytest.mark.parametrize("hd", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_growing_and_spiking_scores(hd, causal):
    """Scores that rise along the sequence: by about 1.4 per key (log2 units)
    on one sequence and in one jump of ~115 at a late key on another, so the
    running maximum of the softmax moves by far more than its slack between
    key tiles (rescales); and by about 0.2 per key on a third, below the
    slack (kept maxima, probabilities above 1 before the final division).
    Against the oracle, causal and bidirectional."""
    nh = 2
    lens = [300, 257, 200, 40]
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, Hp = int(cu_h[-1]), nh * hd
    g = torch.Generator().manual_seed(7)
    q = 0.5 + 0.05 * torch.randn(T, Hp, generator=g)
    k = 0.05 * torch.randn(T, Hp, generator=g)
    v = torch.randn(T, Hp, generator=g)
    # sequence 0: k_j grows linearly, so q.k_j / sqrt(hd) rises ~1 per key at the end
    r0 = torch.arange(lens[0], dtype=torch.float32)
    k[:lens[0]] += (r0 / lens[0] * 2.0 * 300 / (0.5 * hd ** 0.5))[:, None] * 0.5
    # sequence 1: one key (position 220) far above the rest
    k[cu_h[1] + 220] += 80.0 / (0.5 * hd ** 0.5)
    # sequence 2: a slow rise, ~0.2 per key in log2 units (~7 per key tile:
    # below the slack, so maxima are kept and probabilities exceed 1)
    r2 = torch.arange(lens[2], dtype=torch.float32)
    k[cu_h[2]:cu_h[3]] += (0.15 * r2 / (0.5 * hd ** 0.5))[:, None]
    qkv = torch.cat([q, k, v], dim=1).half()
    o = torch.empty(T, Hp, dtype=torch.float16, device=DEV)
    ee.ee_attention_varlen(qkv.to(DEV), torch.tensor(cu_h, device=DEV), len(lens), max(lens), nh, hd, o,
                           causal=causal)
    torch.cuda.synchronize()
    qkv64 = qkv.double().numpy()
    ref = (oracle.causal_attention_packed(qkv64, cu_h, nh, hd) if causal
           else oracle.attention_packed_bidirectional(qkv64, cu_h, nh, hd))
    got = to_host64(o)
    assert np.isfinite(got).all()
    err = normwise_rel(got, ref)
    say(f"attention growing/spiking scores hd={hd} causal={causal}: rel {err:.2e}")
    assert err <= 3e-3


def test_attention_sequences_are_independent():
    """Permuting the sequences of the batch permutes the output rows exactly."""
    nh, hd = 4, 128
    lens = [100, 3, 256, 40]
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qkv = torch.randn(int(cu_h[-1]), 3 * nh * hd, generator=GEN).half()
    o = torch.empty(int(cu_h[-1]), nh * hd, dtype=torch.float16, device=DEV)
    ee.ee_attention_varlen(qkv.to(DEV), torch.tensor(cu_h, device=DEV), 4, 256, nh, hd, o)
    perm = [2, 0, 3, 1]
    lp = [lens[i] for i in perm]
    cu_p = np.concatenate([[0], np.cumsum(lp)]).astype(np.int32)
    qkv_p = torch.cat([qkv[cu_h[i]:cu_h[i + 1]] for i in perm])
    o_p = torch.empty_like(o)
    ee.ee_attention_varlen(qkv_p.to(DEV), torch.tensor(cu_p, device=DEV), 4, 256, nh, hd, o_p)
    torch.cuda.synchronize()
    for j, i in enumerate(perm):
        assert torch.equal(o_p[cu_p[j]:cu_p[j + 1]], o[cu_h[i]:cu_h[i + 1]])
