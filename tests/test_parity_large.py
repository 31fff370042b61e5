"""GPU parity at large sizes: the 32-bit offset arithmetic, deep-K slicing and
long grids near the documented limits, checked on sampled outputs against
the fp64 oracle.  Inputs are hundreds of MB, so each case draws them once;
the oracle computes only the sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._parity import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def say(msg):
    print(f"[large] {msg}", flush=True)


def gen(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.rand(shape, generator=g) * 2 - 1


def test_addmm_deep_k_near_the_limit():
    """K just below 2^21 with a 5 x 37 output: 32-row tiles in many K slices."""
    import bias_addmm_im2col_amd as baim
    M, N, K = 5, 37, (1 << 21) - 12
    say(f"addmm M={M} N={N} K={K} plan {baim.gemm_plan(M, N, K)}")
    a, b, s = gen((M, K), 1), gen((K, N), 2), gen((N,), 3)
    out = baim.addmm(s.cuda(), a.cuda(), b.cuda(), beta=1.0, alpha=1.0)
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), oracle.addmm(a, b, s, False, 1.0, 1.0), K, 1.0, "deep K")


@pytest.mark.parametrize("spec", ["7", "7,s5", "7,3"])
def test_addmm_wide_mat2_with_a_128_row_tile(spec, monkeypatch):
    """N past 2^22: the 128-row B tile of mat2 [K, N] would need offsets of
    127*N floats, beyond 32 bits; forced, the launcher moves the plan to a
    64-row tile, and every sampled output (the last rows of each k-tile
    included) matches the oracle."""
    import bias_addmm_im2col_amd as baim
    monkeypatch.setenv("BAIM_TILE", spec)
    M, K, N = 3, 200, (1 << 22) + 200000
    say(f"addmm M={M} N={N} K={K} BAIM_TILE={spec}")
    a, b, s = gen((M, K), 7), gen((K, N), 8), gen((N,), 9)
    out = baim.addmm(s.cuda(), a.cuda(), b.cuda(), beta=1.0, alpha=1.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    cols = np.concatenate([[0, N - 1, N // 2, (1 << 22) + 7], rng.integers(0, N, 3000)])
    rows = rng.integers(0, M, cols.size)
    got = out.cpu().numpy()[rows, cols]
    check_close(got, oracle.addmm_at(a, b, s, False, 1.0, 1.0, rows, cols), K, 1.0, "wide mat2")


def test_linear_long_m():
    """M = 2^20 + 3 rows: a long grid of row tiles."""
    import bias_addmm_im2col_amd as baim
    M, K, N = (1 << 20) + 3, 64, 48
    say(f"linear M={M} K={K} N={N}")
    x, w, b = gen((M, K), 4), gen((N, K), 5), gen((N,), 6)
    out = baim.linear(x.cuda(), w.cuda(), b.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.concatenate([[0, M - 1, M // 2], rng.integers(0, M, 2000)])
    cols = rng.integers(0, N, rows.size)
    got = out.cpu().numpy()[rows, cols]
    check_close(got, oracle.linear_at(x, w, b, rows, cols), K, 1.0, "long M")


def _conv_points(B, OC, OH, OW, n, seed):
    g = np.random.default_rng(seed)
    P = OH * OW
    edge = [0, OW - 1, P - OW, P - 1]
    idx = [(b * OC + oc) * P + p for b in (0, B - 1) for oc in (0, OC - 1) for p in edge]
    return np.unique(np.concatenate([idx, g.integers(0, B * OC * P, n)]).astype(np.int64))


def test_conv_large_input():
    """A 537 MB NCHW input (2^27 elements) and a 268 MB output."""
    import bias_addmm_im2col_amd as baim
    B, IC, H, W, OC = 2, 32, 1448, 1448, 16
    say(f"conv2d x=[{B},{IC},{H},{W}] w=[{OC},{IC},3,3]")
    x, w, bias = gen((B, IC, H, W), 7), gen((OC, IC, 3, 3), 8), gen((OC,), 9)
    out = baim.conv2d(x.cuda(), w.cuda(), bias.cuda(), 1, 1, 1)
    torch.cuda.synchronize()
    idx = _conv_points(B, OC, H, W, 3000, 1)
    got = out.reshape(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()
    check_close(got, oracle.conv2d_at(x, w, bias, 1, 1, 1, idx), IC * 9, 1.0, "large conv")
    say("conv2d_nhwc on the same numbers read channels-last")
    xn = x.view(B, H, W, IC)
    wn = w.view(OC, 3, 3, IC)
    out = baim.conv2d_nhwc(xn.cuda(), wn.cuda(), bias.cuda(), 1, 1, 1)
    torch.cuda.synchronize()
    g = np.random.default_rng(2)
    idx = np.unique(np.concatenate([[0, out.numel() - 1], g.integers(0, out.numel(), 3000)]))
    got = out.reshape(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()
    check_close(got, oracle.conv2d_nhwc_at(xn, wn, bias, 1, 1, 1, idx), IC * 9, 1.0, "large nhwc")


def test_sdpa_with_a_half_gigabyte_mask():
    """Sq = Skv = 8192 with a [2, 8192, 8192] mask (2^27 elements)."""
    import bias_addmm_im2col_amd as baim
    BH, S, D = 2, 8192, 64
    say(f"sdpa BH={BH} S={S} D={D} with mask")
    q, k, v = gen((BH, S, D), 10), gen((BH, S, D), 11), gen((BH, S, D), 12)
    m = gen((BH, S, S), 13)
    out = baim.sdpa(q.cuda(), k.cuda(), v.cuda(), m.cuda())
    torch.cuda.synchronize()
    rows = np.array([0, S - 1, S, 2 * S - 1, 5000, 12345], dtype=np.int64)
    got = out.reshape(-1, D)[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    res = oracle.sdpa_rows(q, k, v, m, None, rows)
    assert (np.abs(got - res.ref) <= oracle.sdpa_tolerance(res)).all()
