"""The stream-K GEMM for at most 128 rows of A (ee_linear_streamk), through the C ABI.

- Integer-exact: small-integer fp16 operands make every piece's partial sum
  and the sum of a tile's pieces integers below 2^24, exact in fp32 in any
  order, so the result must be the fp16 rounding of the exact sum, bit for
  bit.  Shapes: the four GEMMs of a GPT-3-width decode step at M = 32 (QKV,
  out, FC1, FC2), FC1 and FC2 at M = 128 and 64 (the 128- and 64-row A
  tiles), and ragged ones: M below a tile height (1, 5, 7, 17, 33, 100), N not
  a multiple of the 256-row tile, N % 8 != 0 (the scalar reduce), more N
  tiles than CUs (two rounds of workgroups), and pieces crossing a tile
  boundary.
- Random data with the GeLU epilogue against the oracle (fp64 linear + gelu).
- The workspace query and the errors (fp32, M > 128, a problem too small to
  give every workgroup 8 K tiles, a short workspace).
Bars: bit-exact for the integer cases; normwise 2e-3 for random data (fp16
output rounding plus fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle
import variable_length_padding_amd as ee
from gpu_helpers import DEV, normwise_rel, say, to_host64

pytestmark = pytest.mark.gpu

GEN = torch.Generator().manual_seed(20241203)


def _ints(shape, lo=-2, hi=2):
    return torch.randint(lo, hi + 1, shape, generator=GEN, dtype=torch.int8).to(torch.float16)


def _exact_check(M, N, K, epi):
    A, W = _ints((M, K)), _ints((N, K))
    bias = _ints((N,)) if epi != ee.EPI_NONE else None
    R = _ints((M, N), -8, 8) if epi == ee.EPI_BIAS_RESIDUAL else None
    C = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    ws = torch.empty(ee.ee_linear_streamk_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # NaN patterns: a partial slot the reduce reads without its piece being written shows
    ee.ee_linear_streamk(A.to(DEV), W.to(DEV), None if bias is None else bias.to(DEV),
                         None if R is None else R.to(DEV), epi, C, ws)
    torch.cuda.synchronize()
    # integer sums below 2^24 are exact in fp32 whatever the order
    exact = A.float() @ W.float().T
    if bias is not None:
        exact = exact + bias.float()
    if R is not None:
        exact = exact + R.float()
    assert exact.abs().max().item() < 2 ** 24
    ref16 = exact.to(torch.float16).numpy()
    got = C.cpu().numpy()
    bad = np.count_nonzero(got.view(np.uint16) != ref16.view(np.uint16))
    say(f"stream-K {M}x{N}x{K} epi={epi}: {bad} of {got.size} differ")
    assert bad == 0


@pytest.mark.parametrize("M,N,K,epi", [
    (32, 36864, 12288, ee.EPI_BIAS),            # QKV of a decode step
    (32, 12288, 12288, ee.EPI_BIAS_RESIDUAL),   # out projection
    (32, 49152, 12288, ee.EPI_BIAS),            # FC1 (GeLU below, on random data)
    (32, 12288, 49152, ee.EPI_BIAS_RESIDUAL),   # FC2
    (128, 49152, 12288, ee.EPI_BIAS),           # FC1, 128 sequences
    (64, 12288, 49152, ee.EPI_BIAS_RESIDUAL),   # FC2, 64 sequences
])
def test_streamk_decode_shapes_integer_exact(M, N, K, epi):
    _exact_check(M, N, K, epi)


@pytest.mark.parametrize("M,N,K", [(7, 1000, 64 * 600), (1, 777, 64 * 600), (5, 8200, 64 * 64),
                                   (32, 2056, 64 * 256), (32, 76808, 64 * 16), (17, 4096, 64 * 130),
                                   (33, 1000, 64 * 600), (100, 8200, 64 * 64), (128, 76808, 64 * 16),
                                   (64, 4104, 64 * 130)])
@pytest.mark.parametrize("epi", [ee.EPI_NONE, ee.EPI_BIAS, ee.EPI_BIAS_RESIDUAL])
def test_streamk_ragged_integer_exact(M, N, K, epi):
    _exact_check(M, N, K, epi)


@pytest.mark.parametrize("gelu", [ee.GELU_TANH, ee.GELU_ERF])
def test_streamk_gelu_random(gelu):
    M, N, K = 32, 8192, 12288
    A = torch.randn(M, K, generator=GEN).to(torch.float16)
    W = (0.02 * torch.randn(N, K, generator=GEN)).to(torch.float16)
    bias = (0.1 * torch.randn(N, generator=GEN)).to(torch.float16)
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    ws = torch.empty(ee.ee_linear_streamk_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    ee.ee_linear_streamk(A.to(DEV), W.to(DEV), bias.to(DEV), None, ee.EPI_BIAS_GELU, C, ws, gelu=gelu)
    torch.cuda.synchronize()
    u = oracle.linear(A.double().numpy(), W.double().numpy(), bias.double().numpy())
    ref = oracle.gelu(u, "tanh" if gelu == ee.GELU_TANH else "erf")
    err = normwise_rel(to_host64(C), ref)
    say(f"stream-K gelu={gelu}: rel {err:.2e}")
    assert err <= 2e-3


def test_streamk_repeated_calls_same_bits():
    """A second call on a workspace holding the first call's partials gives the
    same bits (every slot the reduce reads is rewritten)."""
    M, N, K = 32, 12288, 12288
    A = torch.randn(M, K, generator=GEN).to(torch.float16).to(DEV)
    W = (0.02 * torch.randn(N, K, generator=GEN)).to(torch.float16).to(DEV)
    bias = (0.1 * torch.randn(N, generator=GEN)).to(torch.float16).to(DEV)
    ws = torch.empty(ee.ee_linear_streamk_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    C1, C2 = (torch.empty(M, N, dtype=torch.float16, device=DEV) for _ in range(2))
    ee.ee_linear_streamk(A, W, bias, None, ee.EPI_BIAS, C1, ws)
    ee.ee_linear_streamk(A, W, bias, None, ee.EPI_BIAS, C2, ws)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)


def test_streamk_errors():
    with pytest.raises(ee.EEError, match="EE_ERR_UNSUPPORTED"):
        ee.ee_linear_streamk_workspace_size(129, 12288, 12288)       # M above 128
    with pytest.raises(ee.EEError, match="EE_ERR_UNSUPPORTED"):
        ee.ee_linear_streamk_workspace_size(32, 768, 768)            # 36 K tiles in all
    assert ee.ee_linear_streamk_workspace_size(0, 768, 768) == 0
    M, N, K = 32, 4096, 64 * 512
    need = ee.ee_linear_streamk_workspace_size(M, N, K)
    assert need > 0 and need % (M * 256 * 4) == 0
    A = torch.zeros(M, K, dtype=torch.float16, device=DEV)
    W = torch.zeros(N, K, dtype=torch.float16, device=DEV)
    C = torch.empty(M, N, dtype=torch.float16, device=DEV)
    short = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(ee.EEError, match="EE_ERR_WORKSPACE"):
        ee.ee_linear_streamk(A, W, None, None, ee.EPI_NONE, C, short)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    with pytest.raises(ee.EEError, match="EE_ERR_UNSUPPORTED"):
        ee.ee_linear_streamk(A.float(), W.float(), None, None, ee.EPI_NONE, C.float(), ws)
    with pytest.raises(ee.EEError, match="EE_ERR_INVALID_ARG"):
        ee.ee_linear_streamk(A, W, None, None, ee.EPI_NONE, A.view(-1)[:M * N].view(M, N), ws)   # C overlaps A
