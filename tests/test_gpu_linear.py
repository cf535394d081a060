"""GPU parity of the linear (spec_linear) at every weight shape of the
8B-shaped target and of the small target against the oracle's linear: the
weight-streaming kernel for M <= 8 (several 8-row blocks for fp32) and the
matrix-core kernel for bf16 with M > 8 (ragged 64-row blocks, up to the
1280 rows of a B = 256 verify pass).  bf16 weights and inputs, float32
accumulate: the tolerance is relative to sum |x||w|."""
import numpy as np
import pytest
import torch

from draft_then_verify_amd import binding as bd
from oracle.model import linear

pytestmark = pytest.mark.gpu

SHAPES_8B = [(6144, 4096), (4096, 4096), (12288, 4096), (4096, 12288), (151936, 4096)]


def _check(N, K, M, epi, seed, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda").manual_seed(seed)
    rows = 2 * N if epi == 2 else N
    W = (torch.randn((rows, K), generator=g, device="cuda") * 0.02).to(dtype)
    x = torch.randn((M, K), generator=g, device="cuda").to(dtype)
    y0 = torch.randn((M, N), generator=g, device="cuda")
    y = y0.clone() if epi == 1 else torch.empty((M, N), device="cuda")
    z = torch.empty((M, N), dtype=dtype, device="cuda") if epi == 2 else None
    bd.spec_linear(W, x, M, N, K, epilogue=epi, y=None if epi == 2 else y, z=z)
    torch.cuda.synchronize()
    # sampled output columns (all of them for the smaller matrices)
    cols = np.arange(N) if N <= 16384 else np.sort(np.random.default_rng(seed).choice(N, 4096, replace=False))
    Wc = W.float().cpu().numpy()
    xs = x.float().cpu().numpy().astype(np.float64)
    bf = dtype == torch.bfloat16
    ref = linear(xs, Wc[cols], bf)
    bound = np.abs(xs) @ np.abs(Wc[cols].astype(np.float64)).T
    if epi == 0:
        got = y.cpu().numpy()[:, cols]
    elif epi == 1:
        got = y.cpu().numpy()[:, cols] - y0.cpu().numpy()[:, cols]
    else:
        gate, up = ref, linear(xs, Wc[N + cols], bf)
        ref = gate / (1 + np.exp(-gate)) * up
        got = z.float().cpu().numpy()[:, cols]
        bound = (np.abs(ref) + 1e-3) * 2 ** -7 + 1e-4 * (bound + np.abs(xs) @ np.abs(Wc[N + cols].astype(np.float64)).T)
        assert (np.abs(got - ref) <= bound).all()
        return
    assert (np.abs(got - ref) <= 1e-4 * bound + 1e-6).all()


@pytest.mark.parametrize("N,K", SHAPES_8B)
def test_linear_8b_shapes_m5(N, K):
    _check(N, K, 5, 0, seed=N + K)


@pytest.mark.parametrize("epi", [1, 2])
def test_linear_epilogues(epi):
    _check(4096, 4096, 5, epi, seed=7 + epi)
    _check(2816, 1024, 3, epi, seed=9 + epi)


@pytest.mark.parametrize("M", [1, 2, 7, 8, 9, 13])
def test_linear_row_counts(M):
    _check(1000, 1024, M, 0, seed=M)
    _check(6144, 4096, M, 1, seed=100 + M)


@pytest.mark.parametrize("M", [16, 40, 64, 65, 320])
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_linear_matrix_cores(M, epi):
    _check(4096, 4096, M, epi, seed=200 + M + epi)


def test_linear_matrix_cores_large():
    _check(2816, 1024, 1280, 2, seed=301)   # SwiGLU, small-config MLP, B = 256 verify rows
    _check(32000, 1024, 1280, 0, seed=302)  # small-config LM head
    _check(151936, 4096, 40, 0, seed=303)   # 8B LM head, B = 8 verify rows


@pytest.mark.parametrize("N,K,M,epi", [(40000, 1024, 257, 0),   # 2 x 157 tiles of 256 x 256, 1 row in the last
                                       (13100, 1024, 1280, 1),  # 5 x 52, the last 44 columns wide
                                       (8200, 2048, 1000, 2)])  # SwiGLU: 4 x 65 tiles of 128 outputs
def test_linear_matrix_cores_wide_tiles(N, K, M, epi):
    """Launches with at least one 256 x 256 tile per CU (8-wave workgroups),
    ragged in rows and columns."""
    _check(N, K, M, epi, seed=400 + epi)


def test_linear_float32():
    _check(704, 256, 5, 0, seed=3, dtype=torch.float32)
    _check(256, 704, 4, 1, seed=4, dtype=torch.float32)


@pytest.mark.parametrize("epi,N", [(2, 12288), (0, 6144)])
def test_linear_rmsnorm_staging(epi, N):
    """The linear fed from float32 residual rows: the kernel makes its input
    bf16(RMSNorm(h) * gain) while staging it (the form the verify pass uses
    for QKV, gate/up and the LM head).  Against the oracle's RMSNorm, bf16
    rounding and linear; an input element whose float32 norm lands on the
    other side of a bf16 rounding boundary moves its term by at most one
    bf16 spacing (2^-8 |x| |w|)."""
    from oracle.model import rms_norm, silu

    K, M = 4096, 5
    g = torch.Generator(device="cuda").manual_seed(N + epi)
    rows = 2 * N if epi == 2 else N
    W = (torch.randn((rows, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    h = torch.randn((M, K), generator=g, device="cuda") * 3
    gain = 1 + 0.1 * torch.randn(K, generator=g, device="cuda")
    y = torch.empty((M, N), device="cuda")
    z = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    bd.spec_linear(W, None, M, N, K, epilogue=epi, y=y if epi == 0 else None, z=z if epi == 2 else None,
                   hn=h, gain=gain, eps=1e-6)
    torch.cuda.synchronize()
    Wc = W.float().cpu().numpy().astype(np.float64)
    x = rms_norm(h.cpu().numpy().astype(np.float64), gain.cpu().numpy().astype(np.float64), 1e-6)
    a = np.abs(x) @ np.abs(Wc).T  # sum |x||w| per output
    ref = linear(x, Wc, True)
    slack = 1e-4 * a + 2 ** -8 * a
    if epi == 0:
        assert (np.abs(y.cpu().numpy() - ref) <= slack + 1e-6).all()
    else:
        gate, up = ref[:, :N], ref[:, N:]
        zr = silu(gate) * up
        # |d silu / dg| <= 1.1
        dz = np.abs(silu(gate)) * slack[:, N:] + 1.1 * np.abs(up) * slack[:, :N]
        assert (np.abs(z.float().cpu().numpy() - zr) <= (np.abs(zr) + 1e-3) * 2 ** -7 + dz + 1e-6).all()
