"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against facts fixed independently of its own code:
exact rational brute force on tiny inputs, closed forms of special cases
(identity mat2, alpha = 0, K = 1, 1x1 conv, a delta kernel), two formulations
of the conv, linearity of the epilogue, hand-worked examples and the
float64 CPU routines of an outside library (torch.addmm / F.conv2d).

Definitions pinned:
  addmm  -- "[ExecuTorch][WebGPU] Add optimized addmm op", Solution paragraph:
            out = beta*self + alpha*(mat1 @ mat2), self [N] or [M,N].
  conv2d -- "et_vk conv2d: route standard (groups==1) conv through an im2col
            tiled GEMM", Solution/Implementation: M=OC, N=B*OH*OW,
            K=IC*KH*KW, ih = oh*sH - pH + kh*dH, out-of-range taps read 0,
            bias per OC, NCHW output.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from bias_addmm_im2col_amd import inputs as I

U64 = 2.0 ** -53  # unit roundoff of float64


def rand32(shape, seed, lo=-1.0, hi=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo).numpy()


def int32v(shape, seed, lo=-4, hi=4):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.float32).numpy()


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("M,K,N,self_2d,beta,alpha", [
    (1, 1, 1, False, 1.0, 1.0),
    (3, 5, 4, False, 1.0, 1.0),
    (4, 7, 3, True, 0.5, 2.0),
    (5, 2, 6, True, -1.25, 0.75),
    (2, 8, 2, False, 0.0, 3.0),
])
def test_addmm_matches_exact_rationals(M, K, N, self_2d, beta, alpha):
    """P-6: tiny addmm against exact rational arithmetic.

    fp32 values are exact rationals; the true result differs from the fp64
    oracle only by fp64 rounding: at most (K+2) roundings of size U64 times
    the magnitude sum."""
    a, b = rand32((M, K), 1), rand32((K, N), 2)
    s = rand32((M, N) if self_2d else (N,), 3)
    r = oracle.addmm(a, b, s, self_2d, beta, alpha)
    for i in range(M):
        for j in range(N):
            acc = sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(K))
            sv = Fraction(float(s[i, j] if self_2d else s[j]))
            exact = Fraction(float(np.float32(beta))) * sv + Fraction(float(np.float32(alpha))) * acc
            sabs = sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j]))) for k in range(K))
            mag = abs(alpha) * float(sabs) + abs(beta * float(sv))
            assert abs(Fraction(r.ref[i, j]) - exact) <= (K + 3) * U64 * mag + 1e-300
            assert abs(Fraction(r.sabs[i, j]) - sabs) <= K * U64 * float(sabs) + 1e-300


def _conv_brute(x, w, bias, stride, pad, dil):
    """Exact conv by definition: padded input, strided/dilated taps, Fractions."""
    B, IC, H, W = x.shape
    OC, _, KH, KW = w.shape
    sH, sW = stride
    pH, pW = pad
    dH, dW = dil
    Hp, Wp = H + 2 * pH, W + 2 * pW
    xp = [[[[Fraction(0)] * Wp for _ in range(Hp)] for _ in range(IC)] for _ in range(B)]
    for b in range(B):
        for c in range(IC):
            for h in range(H):
                for v in range(W):
                    xp[b][c][h + pH][v + pW] = Fraction(float(x[b, c, h, v]))
    OH = (Hp - dH * (KH - 1) - 1) // sH + 1
    OW = (Wp - dW * (KW - 1) - 1) // sW + 1
    out = {}
    for b in range(B):
        for o in range(OC):
            for oh in range(OH):
                for ow in range(OW):
                    acc = Fraction(0) if bias is None else Fraction(float(bias[o]))
                    for c in range(IC):
                        for kh in range(KH):
                            for kw in range(KW):
                                acc += Fraction(float(w[o, c, kh, kw])) * \
                                    xp[b][c][oh * sH + kh * dH][ow * sW + kw * dW]
                    out[b, o, oh, ow] = acc
    return out, (OH, OW)


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,has_bias", [
    (1, 1, 5, 5, 1, 3, 3, (1, 1), (0, 0), (1, 1), True),
    (2, 3, 6, 7, 2, 3, 2, (2, 1), (1, 0), (1, 2), True),
    (1, 2, 7, 7, 3, 7, 7, (4, 4), (3, 3), (1, 1), False),
    (1, 2, 6, 5, 2, 3, 3, (1, 2), (2, 2), (2, 2), True),
])
def test_conv_matches_exact_rationals(B, IC, H, W, OC, KH, KW, stride, pad, dil, has_bias):
    """P-6: tiny direct conv against an exact computation on a zero-padded input."""
    x = rand32((B, IC, H, W), 4)
    w = rand32((OC, IC, KH, KW), 5)
    bias = rand32((OC,), 6) if has_bias else None
    r = oracle.conv2d(x, w, bias, stride, pad, dil)
    exact, (OH, OW) = _conv_brute(x, w, bias, stride, pad, dil)
    assert r.ref.shape == (B, OC, OH, OW)
    K = IC * KH * KW
    for key, e in exact.items():
        mag = r.sabs[key] + (abs(float(bias[key[1]])) if has_bias else 0.0)
        assert abs(Fraction(r.ref[key]) - e) <= (K + 2) * U64 * mag + 1e-300


# ------------------------------------------------------------ closed forms

def test_identity_mat2_gives_alpha_mat1_plus_beta_self():
    """P-1: mat2 = I (K = N) -> alpha*mat1 + beta*self, exactly in fp64."""
    M, K = 37, 29
    a = rand32((M, K), 7)
    s = rand32((K,), 8)
    eye = np.eye(K, dtype=np.float32)
    r = oracle.addmm(a, eye, s, False, 0.5, 3.0)
    expect = 3.0 * a.astype(np.float64) + 0.5 * s.astype(np.float64)[None, :]
    assert np.array_equal(r.ref, expect)


@pytest.mark.parametrize("self_2d", [False, True])
def test_alpha_zero_gives_exactly_beta_self(self_2d):
    """P-2: alpha = 0 -> beta*self exactly, whatever mat1 @ mat2 is."""
    M, K, N = 9, 13, 11
    a, b = rand32((M, K), 9), rand32((K, N), 10)
    s = rand32((M, N) if self_2d else (N,), 11)
    r = oracle.addmm(a, b, s, self_2d, -1.5, 0.0)
    full = s.astype(np.float64) if self_2d else np.broadcast_to(s.astype(np.float64), (M, N))
    assert np.array_equal(r.ref, -1.5 * full)


def test_k1_is_outer_product():
    """P-3: K = 1 -> beta*self + alpha * a_i * b_j (one exact product)."""
    M, N = 17, 23
    a, b = rand32((M, 1), 12), rand32((1, N), 13)
    s = rand32((N,), 14)
    r = oracle.addmm(a, b, s, False, 1.0, 2.0)
    outer = a.astype(np.float64) * b.astype(np.float64)  # (M,1)*(1,N)
    assert np.array_equal(r.ref, s.astype(np.float64)[None, :] + 2.0 * outer)
    assert np.array_equal(r.sabs, np.abs(outer))


def test_k0_is_beta_self():
    """Empty contraction: out = beta*self, sabs = 0."""
    s = rand32((4, 5), 15)
    r = oracle.addmm(np.zeros((4, 0), np.float32), np.zeros((0, 5), np.float32), s, True, 2.0, 1.0)
    assert np.array_equal(r.ref, 2.0 * s.astype(np.float64))
    assert not r.sabs.any()


def test_beta_zero_never_reads_self():
    """beta = 0: the self term is exactly 0 even if self holds NaN/Inf."""
    a, b = rand32((6, 4), 16), rand32((4, 5), 17)
    s = np.full((5,), np.nan, np.float32)
    s[1] = np.inf
    r = oracle.addmm(a, b, s, False, 0.0, 1.0)
    assert np.isfinite(r.ref).all()
    r2 = oracle.addmm(a, b, np.zeros(5, np.float32), False, 1.0, 1.0)
    assert np.array_equal(r.ref, r2.ref)


def test_hand_worked_addmm():
    """A worked example small enough to check by hand.

    mat1 @ mat2 = [[1+3, 2+3], [4+6, 5+6]] = [[4, 5], [10, 11]];
    out = [10, 20] + 2*that = [[18, 30], [30, 42]];
    sabs = [[1+3, 2+3], [4+6, 5+6]] (all terms non-negative)."""
    a = np.array([[1, 2, 3], [4, 5, 6]], np.float32)
    b = np.array([[1, 0], [0, 1], [1, 1]], np.float32)
    s = np.array([10, 20], np.float32)
    r = oracle.addmm(a, b, s, False, 1.0, 2.0)
    assert r.ref.tolist() == [[18.0, 30.0], [30.0, 42.0]]
    assert r.sabs.tolist() == [[4.0, 5.0], [10.0, 11.0]]
    r2 = oracle.addmm(a, b, np.array([[1, 2], [3, 4]], np.float32), True, -1.0, 1.0)
    assert r2.ref.tolist() == [[3.0, 3.0], [7.0, 7.0]]


def test_hand_worked_conv():
    """Worked conv examples checkable by hand on x = [[1,2,3],[4,5,6],[7,8,9]].

    * kernel [[1,0],[0,-1]], no padding: out[i,j] = x[i,j] - x[i+1,j+1] = -4.
    * kernel [[1]] with padding 1 and stride 2: samples the zero-padded input
      at rows/cols {-1, 1, 3} -> [[0,0,0],[0,5,0],[0,0,0]], plus bias 0.5.
    * 2x2 all-ones kernel, dilation 2, padding 1: a 3x3 output whose entry
      (oh, ow) sums the input at (oh-1 or oh+1, ow-1 or ow+1) where inside.
    """
    x = np.arange(1, 10, dtype=np.float32).reshape(1, 1, 3, 3)
    k = np.array([[1, 0], [0, -1]], np.float32).reshape(1, 1, 2, 2)
    r = oracle.conv2d(x, k, None)
    assert r.ref.tolist() == [[[[-4.0, -4.0], [-4.0, -4.0]]]]
    r = oracle.conv2d(x, np.ones((1, 1, 1, 1), np.float32), np.array([0.5], np.float32), 2, 1, 1)
    assert r.ref.tolist() == [[[[0.5, 0.5, 0.5], [0.5, 5.5, 0.5], [0.5, 0.5, 0.5]]]]
    # dilation 2, pad 1: taps at (oh-1, ow-1), (oh-1, ow+1), (oh+1, ow-1), (oh+1, ow+1)
    # OH = (3 + 2 - 2 - 1)//1 + 1 = 3.
    # (0,0): only (1,1) is inside -> 5.  (0,1): (1,0)=4, (1,2)=6 -> 10.
    # (1,1): (0,0)=1,(0,2)=3,(2,0)=7,(2,2)=9 -> 20.  (2,2): (1,1) -> 5.
    r = oracle.conv2d(x, np.ones((1, 1, 2, 2), np.float32), None, 1, 1, 2)
    assert r.ref.tolist() == [[[[5.0, 10.0, 5.0], [10.0, 20.0, 10.0], [5.0, 10.0, 5.0]]]]


def test_1x1_conv_is_a_matmul_per_image():
    """P-4: a 1x1, stride-1, unpadded conv is W[OC,IC] @ x[b][IC, H*W] + bias."""
    B, IC, H, W, OC = 3, 5, 4, 6, 7
    x = rand32((B, IC, H, W), 18)
    w = rand32((OC, IC, 1, 1), 19)
    bias = rand32((OC,), 20)
    r = oracle.conv2d(x, w, bias)
    w2 = w.reshape(OC, IC).astype(np.float64)
    for b in range(B):
        mm = w2 @ x[b].reshape(IC, H * W).astype(np.float64) + bias.astype(np.float64)[:, None]
        np.testing.assert_allclose(r.ref[b].reshape(OC, H * W), mm, rtol=1e-13, atol=1e-14)
    # and the same numbers come out of the addmm oracle with mat1 = W, mat2 = x[b]
    for b in range(B):
        ra = oracle.addmm(w.reshape(OC, IC), np.ascontiguousarray(x[b].reshape(IC, H * W)),
                          np.ascontiguousarray(np.repeat(bias[:, None], H * W, 1)), True)
        assert np.array_equal(ra.ref, r.ref[b].reshape(OC, H * W))


@pytest.mark.parametrize("kh0,kw0,pad,dil", [
    (1, 1, (1, 1), (1, 1)),   # centre tap with "same" padding -> identity
    (0, 2, (1, 1), (1, 1)),
    (2, 0, (2, 1), (2, 1)),
    (1, 2, (0, 3), (1, 2)),
])
def test_delta_kernel_shifts_input(kh0, kw0, pad, dil):
    """P-5: W[oc,ic,kh0,kw0] = delta(oc,ic), stride 1 -> the input shifted by
    (kh0*dH - pH, kw0*dW - pW) with zero fill, plus bias."""
    B, C, H, W, KH, KW = 2, 3, 7, 8, 3, 3
    x = rand32((B, C, H, W), 21)
    w = np.zeros((C, C, KH, KW), np.float32)
    for c in range(C):
        w[c, c, kh0, kw0] = 1.0
    bias = rand32((C,), 22)
    r = oracle.conv2d(x, w, bias, 1, pad, dil)
    OH, OW = r.ref.shape[2:]
    dy, dx = kh0 * dil[0] - pad[0], kw0 * dil[1] - pad[1]
    expect = np.zeros((B, C, OH, OW))
    for oh in range(OH):
        for ow in range(OW):
            ih, iw = oh + dy, ow + dx
            if 0 <= ih < H and 0 <= iw < W:
                expect[:, :, oh, ow] = x[:, :, ih, iw]
    expect += bias.astype(np.float64)[None, :, None, None]
    assert np.array_equal(r.ref, expect)
    if (kh0, kw0, pad, dil) == (1, 1, (1, 1), (1, 1)):
        assert np.array_equal(r.ref, x.astype(np.float64) + bias.astype(np.float64)[None, :, None, None])


@pytest.mark.parametrize("stride,pad,dil", [((1, 1), (1, 1), (1, 1)), ((2, 3), (0, 2), (2, 1)),
                                            ((4, 4), (3, 3), (1, 1))])
def test_direct_conv_equals_explicit_im2col_gemm(stride, pad, dil):
    """P-8: the direct 7-loop conv == W[OC,K] @ im2col [K, B*OH*OW] + bias."""
    B, IC, H, W, OC, KH, KW = 2, 3, 11, 10, 4, 3, 4
    x = rand32((B, IC, H, W), 23)
    w = rand32((OC, IC, KH, KW), 24)
    bias = rand32((OC,), 25)
    r = oracle.conv2d(x, w, bias, stride, pad, dil)
    col = oracle.im2col(x, KH, KW, stride, pad, dil)
    OH, OW = r.ref.shape[2:]
    gemm = w.reshape(OC, -1).astype(np.float64) @ col + bias.astype(np.float64)[:, None]
    gemm = gemm.reshape(OC, B, OH, OW).transpose(1, 0, 2, 3)
    np.testing.assert_allclose(r.ref, gemm, rtol=1e-12, atol=1e-13)


def test_im2col_matches_sliding_windows():
    """The explicit im2col against numpy's sliding windows of the padded input."""
    B, IC, H, W, KH, KW, p = 2, 3, 6, 5, 3, 2, 1
    x = rand32((B, IC, H, W), 26)
    col = oracle.im2col(x, KH, KW, 1, p, 1)
    xp = np.pad(x.astype(np.float64), ((0, 0), (0, 0), (p, p), (p, p)))
    win = np.lib.stride_tricks.sliding_window_view(xp, (KH, KW), axis=(2, 3))  # B,IC,OH,OW,KH,KW
    expect = win.transpose(1, 4, 5, 0, 2, 3).reshape(IC * KH * KW, -1)
    assert np.array_equal(col, expect)


def test_epilogue_linearity():
    """P-10: out(alpha, beta) = alpha*out(1, 0) + beta*self."""
    M, K, N = 12, 30, 9
    a, b, s = rand32((M, K), 27), rand32((K, N), 28), rand32((M, N), 29)
    r10 = oracle.addmm(a, b, s, True, 0.0, 1.0)
    r = oracle.addmm(a, b, s, True, -0.75, 2.5)
    np.testing.assert_allclose(r.ref, 2.5 * r10.ref - 0.75 * s.astype(np.float64), rtol=1e-14, atol=1e-14)


def test_self_broadcast_equals_repeated_rows():
    """self [N] is the same as the full [M,N] self with every row equal."""
    M, K, N = 8, 10, 6
    a, b, s = rand32((M, K), 30), rand32((K, N), 31), rand32((N,), 32)
    r1 = oracle.addmm(a, b, s, False, 0.5, 1.0)
    r2 = oracle.addmm(a, b, np.ascontiguousarray(np.tile(s, (M, 1))), True, 0.5, 1.0)
    assert np.array_equal(r1.ref, r2.ref)


def test_sabs_equals_ref_for_nonnegative_terms():
    """With non-negative operands, beta = 0, alpha = 1: ref == sabs."""
    a = rand32((5, 40), 33, 0.0, 1.0)
    b = rand32((40, 7), 34, 0.0, 1.0)
    r = oracle.addmm(a, b, np.zeros(7, np.float32), False, 0.0, 1.0)
    assert np.array_equal(r.ref, r.sabs)


# ------------------------------------------------------- library cross-check

@pytest.mark.parametrize("M,K,N,self_2d,beta,alpha", [
    (64, 96, 80, False, 1.0, 1.0), (33, 127, 65, True, 0.5, 2.0), (1, 300, 3, False, -2.0, 0.25)])
def test_addmm_vs_torch_float64(M, K, N, self_2d, beta, alpha):
    """P-9: against torch.addmm in float64 on the CPU (an outside routine)."""
    a, b = rand32((M, K), 35), rand32((K, N), 36)
    s = rand32((M, N) if self_2d else (N,), 37)
    r = oracle.addmm(a, b, s, self_2d, beta, alpha)
    t = torch.addmm(torch.from_numpy(s).double(), torch.from_numpy(a).double(),
                    torch.from_numpy(b).double(), beta=beta, alpha=alpha).numpy()
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil", [
    (1, 3, 32, 32, 8, 7, 7, (4, 4), (3, 3), (1, 1)),
    (2, 8, 12, 12, 6, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 8, 12, 12, 6, 3, 3, (1, 1), (2, 2), (2, 2)),
    (2, 8, 13, 13, 6, 3, 3, (2, 2), (1, 1), (1, 1)),
    (1, 4, 9, 11, 5, 2, 3, (3, 2), (0, 2), (2, 3)),
])
def test_conv_vs_torch_float64(B, IC, H, W, OC, KH, KW, stride, pad, dil):
    """P-9: against torch.nn.functional.conv2d in float64 on the CPU."""
    x = rand32((B, IC, H, W), 38)
    w = rand32((OC, IC, KH, KW), 39)
    bias = rand32((OC,), 40)
    r = oracle.conv2d(x, w, bias, stride, pad, dil)
    t = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                 torch.from_numpy(bias).double(), stride, pad, dil).numpy()
    assert r.ref.shape == t.shape
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ sampled entry

def test_sampled_addmm_equals_full():
    M, K, N = 21, 17, 19
    a, b, s = rand32((M, K), 41), rand32((K, N), 42), rand32((M, N), 43)
    full = oracle.addmm(a, b, s, True, 0.5, -1.0)
    g = np.random.default_rng(0)
    rows, cols = g.integers(0, M, 100), g.integers(0, N, 100)
    at = oracle.addmm_at(a, b, s, True, 0.5, -1.0, rows, cols)
    assert np.array_equal(at.ref, full.ref[rows, cols])
    assert np.array_equal(at.sabs, full.sabs[rows, cols])
    assert np.array_equal(at.selfabs, full.selfabs[rows, cols])


def test_sampled_conv_equals_full():
    x = rand32((2, 3, 9, 8), 44)
    w = rand32((5, 3, 3, 3), 45)
    bias = rand32((5,), 46)
    full = oracle.conv2d(x, w, bias, (2, 1), (1, 2), (1, 2))
    idx = np.random.default_rng(1).integers(0, full.ref.size, 200)
    at = oracle.conv2d_at(x, w, bias, (2, 1), (1, 2), (1, 2), idx)
    assert np.array_equal(at.ref, full.ref.reshape(-1)[idx])
    assert np.array_equal(at.sabs, full.sabs.reshape(-1)[idx])


# --------------------------------------------------------------- workloads

def test_workload_output_sizes():
    """The stem conv's stated output is [1,128,192,192]; the 3x3 cases give
    56x56 (s1 p1, and d2 p2) and 29x29 (s2 p1 on 57x57)."""
    assert oracle.conv_out_size(768, 7, 4, 3, 1) == 192
    assert oracle.conv_out_size(56, 3, 1, 1, 1) == 56
    assert oracle.conv_out_size(56, 3, 1, 2, 2) == 56
    assert oracle.conv_out_size(57, 3, 2, 1, 1) == 29
    assert oracle.conv_out_size(2, 5, 1, 0, 1) == 0  # kernel larger than input
    for c in I.CASES.values():
        if c.kind == "conv":
            assert c.out_hw() == (oracle.conv_out_size(c.H, c.KH, c.stride[0], c.padding[0], c.dilation[0]),
                                  oracle.conv_out_size(c.W, c.KW, c.stride[1], c.padding[1], c.dilation[1]))


def test_input_generator_is_seeded_and_shaped():
    c = I.CASES["addmm_small_64x96x80"]
    a1, b1, s1 = I.addmm_inputs(c)
    a2, b2, s2 = I.addmm_inputs(c)
    assert a1.shape == (64, 96) and b1.shape == (96, 80) and s1.shape == (80,)
    assert torch.equal(a1, a2) and torch.equal(b1, b2) and torch.equal(s1, s2)
    assert a1.dtype == torch.float32 and float(a1.min()) >= -1 and float(a1.max()) < 1
    cc = I.CASES["stem_conv7x7_s4_768"]
    x, w, b = I.conv_inputs(cc)
    assert x.shape == (1, 3, 768, 768) and w.shape == (128, 3, 7, 7) and b.shape == (128,)
    assert float(x.min()) >= 0.0


def test_regression_fixture_unchanged():
    """The stored oracle outputs (tests/golden/make_golden.py) still come out."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")
    g = json.load(open(path))
    ga = g["addmm"]
    a, b, s = (rand32(sh, sd) for sh, sd in zip([(3, 5), (5, 4), (4,)], ga["seeds"]))
    r = oracle.addmm(a, b, s, False, ga["beta"], ga["alpha"])
    assert r.ref.tolist() == ga["ref"] and r.sabs.tolist() == ga["sabs"]
    gc = g["conv2d"]
    x, w, bias = (rand32(sh, sd) for sh, sd in zip([(1, 2, 5, 5), (3, 2, 3, 3), (3,)], gc["seeds"]))
    r = oracle.conv2d(x, w, bias, gc["stride"], gc["padding"], gc["dilation"])
    assert r.ref.tolist() == gc["ref"] and r.sabs.tolist() == gc["sabs"]


# ------------------------------------------------------------------ linear

def test_linear_matches_exact_rationals():
    """Tiny linear against exact rational arithmetic."""
    M, K, N = 3, 6, 4
    x, w, b = rand32((M, K), 64), rand32((N, K), 65), rand32((N,), 66)
    r = oracle.linear(x, w, b)
    for i in range(M):
        for j in range(N):
            exact = Fraction(float(b[j])) + sum(Fraction(float(x[i, k])) * Fraction(float(w[j, k]))
                                                for k in range(K))
            mag = float(r.sabs[i, j]) + abs(float(b[j]))
            assert abs(Fraction(r.ref[i, j]) - exact) <= (K + 2) * U64 * mag


def test_linear_is_addmm_with_transposed_weight():
    """linear(x, W, b) == addmm(b, x, W^T) bit for bit (same terms, same order)."""
    x, w, b = rand32((17, 29), 67), rand32((13, 29), 68), rand32((13,), 69)
    r = oracle.linear(x, w, b)
    ra = oracle.addmm(x, np.ascontiguousarray(w.T), b, False, 1.0, 1.0)
    assert np.array_equal(r.ref, ra.ref) and np.array_equal(r.sabs, ra.sabs)
    rn = oracle.linear(x, w, None)
    assert np.array_equal(rn.ref, oracle.addmm(x, np.ascontiguousarray(w.T), b, False, 0.0, 1.0).ref)


def test_linear_identity_weight_and_library():
    x = rand32((9, 12), 70)
    r = oracle.linear(x, np.eye(12, dtype=np.float32), None)
    assert np.array_equal(r.ref, x.astype(np.float64))
    w, b = rand32((7, 12), 71), rand32((7,), 72)
    t = F.linear(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                 torch.from_numpy(b).double()).numpy()
    np.testing.assert_allclose(oracle.linear(x, w, b).ref, t, rtol=1e-12, atol=1e-12)


def test_sampled_linear_equals_full():
    x, w, b = rand32((21, 17), 73), rand32((19, 17), 74), rand32((19,), 75)
    full = oracle.linear(x, w, b)
    g = np.random.default_rng(2)
    rows, cols = g.integers(0, 21, 100), g.integers(0, 19, 100)
    at = oracle.linear_at(x, w, b, rows, cols)
    assert np.array_equal(at.ref, full.ref[rows, cols])
    assert np.array_equal(at.selfabs, full.selfabs[rows, cols])


# ------------------------------------------------------------ grouped conv

def test_grouped_conv_with_one_group_is_the_conv():
    x, w, b = rand32((2, 6, 9, 8), 76), rand32((5, 6, 3, 2), 77), rand32((5,), 78)
    r1 = oracle.conv2d(x, w, b, (2, 1), (1, 0), (1, 2))
    rg = oracle.conv2d_grouped(x, w, b, (2, 1), (1, 0), (1, 2), groups=1)
    assert np.array_equal(r1.ref, rg.ref) and np.array_equal(r1.sabs, rg.sabs)


def test_grouped_conv_is_per_group_convs():
    """Closed form: group g's outputs are the ungrouped conv of its channel
    slice of the input with its slice of the weight."""
    G, B, IC, OC, H, W = 3, 2, 6, 9, 10, 7
    x, w, b = rand32((B, IC, H, W), 79), rand32((OC, IC // G, 3, 3), 80), rand32((OC,), 81)
    r = oracle.conv2d_grouped(x, w, b, 1, 1, 1, groups=G)
    icg, ocg = IC // G, OC // G
    for g in range(G):
        rg = oracle.conv2d(np.ascontiguousarray(x[:, g * icg:(g + 1) * icg]),
                           np.ascontiguousarray(w[g * ocg:(g + 1) * ocg]),
                           np.ascontiguousarray(b[g * ocg:(g + 1) * ocg]), 1, 1, 1)
        assert np.array_equal(r.ref[:, g * ocg:(g + 1) * ocg], rg.ref)


@pytest.mark.parametrize("G,IC,OC,stride,pad,dil", [(2, 4, 6, 1, 1, 1), (4, 8, 8, 2, 1, 1),
                                                    (8, 8, 16, 1, 2, 2), (3, 3, 3, (2, 1), (0, 1), 1)])
def test_grouped_conv_vs_torch_float64(G, IC, OC, stride, pad, dil):
    x, w, b = rand32((2, IC, 11, 9), 82), rand32((OC, IC // G, 3, 3), 83), rand32((OC,), 84)
    r = oracle.conv2d_grouped(x, w, b, stride, pad, dil, groups=G)
    t = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                 torch.from_numpy(b).double(), stride, pad, dil, G).numpy()
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-12)


def test_depthwise_delta_kernel_shifts_each_channel():
    """Depthwise (G = IC = OC), each channel's kernel a delta at (2, 0): the
    output is the input shifted by (2 - 1, 0 - 1) with zero fill."""
    C = 5
    x = rand32((1, C, 7, 6), 85)
    w = np.zeros((C, 1, 3, 3), np.float32)
    w[:, 0, 2, 0] = 1.0
    r = oracle.conv2d_grouped(x, w, None, 1, 1, 1, groups=C)
    expect = np.zeros((1, C, 7, 6))
    expect[:, :, 0:6, 1:6] = x[:, :, 1:7, 0:5]
    assert np.array_equal(r.ref, expect)


def test_sampled_grouped_conv_equals_full():
    x, w, b = rand32((2, 6, 9, 8), 86), rand32((9, 2, 3, 3), 87), rand32((9,), 88)
    full = oracle.conv2d_grouped(x, w, b, (2, 1), 1, (1, 2), groups=3)
    idx = np.random.default_rng(3).integers(0, full.ref.size, 150)
    at = oracle.conv2d_grouped_at(x, w, b, (2, 1), 1, (1, 2), 3, idx)
    assert np.array_equal(at.ref, full.ref.reshape(-1)[idx])


# ------------------------------------------------------------------ attention
# "[ExecuTorch][WebGPU] Add optimized SDPA op", Problem/Solution paragraphs:
# out = softmax(q @ k^T * scale + attn_mask) @ v over [B,H,S,D], softmax along
# the keys, optional additive [B,H,Sq,Skv] mask, Sq may differ from Skv,
# scale 1/sqrt(D) by default.

def _qkv(BH, Sq, Skv, D, seed, mask=False):
    q = rand32((BH, Sq, D), seed)
    k = rand32((BH, Skv, D), seed + 1)
    v = rand32((BH, Skv, D), seed + 2)
    m = rand32((BH, Sq, Skv), seed + 3, -2.0, 2.0) if mask else None
    return q, k, v, m


def test_sdpa_zero_scale_averages_the_values():
    q, k, v, _ = _qkv(3, 5, 7, 8, 10)
    r = oracle.sdpa(q, k, v, None, scale=0.0)
    want = np.broadcast_to(v.astype(np.float64).mean(axis=1, keepdims=True), r.ref.shape)
    np.testing.assert_allclose(r.ref, want, rtol=0, atol=1e-15)


def test_sdpa_one_hot_mask_selects_one_value_row():
    BH, Sq, Skv, D = 2, 6, 9, 4
    q, k, v, _ = _qkv(BH, Sq, Skv, D, 20)
    pick = np.random.default_rng(3).integers(0, Skv, size=(BH, Sq))
    mask = np.full((BH, Sq, Skv), -np.inf, np.float32)
    for b in range(BH):
        for i in range(Sq):
            mask[b, i, pick[b, i]] = 0.0
    r = oracle.sdpa(q, k, v, mask)
    for b in range(BH):
        for i in range(Sq):
            assert (r.ref[b, i] == v[b, pick[b, i]].astype(np.float64)).all()


def test_sdpa_two_keys_is_a_logistic_blend():
    # With two keys the softmax weight of key 0 is 1 / (1 + exp(s1 - s0)).
    q, k, v, m = _qkv(1, 4, 2, 6, 30, mask=True)
    scale = np.float32(0.375)
    r = oracle.sdpa(q, k, v, m, scale=scale)
    for i in range(4):
        s = [float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[0, i], k[0, j]))
                   * Fraction(float(scale)) + Fraction(float(m[0, i, j]))) for j in range(2)]
        w0 = 1.0 / (1.0 + np.exp(s[1] - s[0]))
        want = w0 * v[0, 0].astype(np.float64) + (1.0 - w0) * v[0, 1].astype(np.float64)
        np.testing.assert_allclose(r.ref[0, i], want, rtol=0, atol=1e-14)


def test_sdpa_single_key_returns_its_value():
    q, k, v, m = _qkv(2, 5, 1, 8, 40, mask=True)
    r = oracle.sdpa(q, k, v, m)
    assert (r.ref == np.broadcast_to(v.astype(np.float64), r.ref.shape)).all()


def test_sdpa_values_of_ones_give_ones():
    q, k, _, m = _qkv(2, 5, 11, 8, 50, mask=True)
    v = np.ones((2, 11, 8), np.float32)
    r = oracle.sdpa(q, k, v, m)
    np.testing.assert_allclose(r.ref, 1.0, rtol=0, atol=4e-16)


@pytest.mark.parametrize("shape,masked,scale", [
    ((2, 3, 5, 5, 8), False, None), ((1, 4, 7, 13, 16), True, None),
    ((3, 1, 9, 4, 12), True, 0.3), ((2, 2, 33, 65, 64), True, None), ((1, 1, 1, 3, 4), False, 2.0)])
def test_sdpa_vs_torch_float64(shape, masked, scale):
    B, H, Sq, Skv, D = shape
    q = rand32((B, H, Sq, D), 60)
    k = rand32((B, H, Skv, D), 61)
    v = rand32((B, H, Skv, D), 62)
    m = rand32((B, H, Sq, Skv), 63, -3, 3) if masked else None
    r = oracle.sdpa(q, k, v, m, scale)
    sc = float(np.float32(1.0 / np.sqrt(D) if scale is None else scale))
    t = F.scaled_dot_product_attention(
        torch.from_numpy(q).double(), torch.from_numpy(k).double(), torch.from_numpy(v).double(),
        attn_mask=None if m is None else torch.from_numpy(m).double(), scale=sc).numpy()
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-14)


def test_sdpa_default_scale_is_inverse_sqrt_d():
    q, k, v, _ = _qkv(2, 4, 6, 36, 70)
    a = oracle.sdpa(q, k, v).ref
    b = oracle.sdpa(q, k, v, scale=np.float32(1.0 / 6.0)).ref
    assert (a == b).all()
    assert not np.allclose(a, oracle.sdpa(q, k, v, scale=np.float32(1.0 / 36.0)).ref)


def test_sdpa_row_offset_of_the_mask_cancels():
    q, k, v, m = _qkv(2, 5, 9, 8, 80, mask=True)
    shift = rand32((2, 5, 1), 81, -4, 4)
    a = oracle.sdpa(q, k, v, m).ref
    b = oracle.sdpa(q, k, v, (m + shift).astype(np.float32)).ref
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-6)  # the shifted mask is rounded to fp32


def test_sdpa_key_permutation_invariance():
    q, k, v, m = _qkv(2, 5, 9, 8, 90, mask=True)
    perm = np.random.default_rng(5).permutation(9)
    a = oracle.sdpa(q, k, v, m).ref
    b = oracle.sdpa(q, k[:, perm].copy(), v[:, perm].copy(), m[:, :, perm].copy()).ref
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_sdpa_masked_rows():
    q, k, v, m = _qkv(1, 4, 6, 4, 100, mask=True)
    m[0, 1, :] = -np.inf                      # every key masked: no softmax
    m[0, 2, :3] = -np.inf                     # first keys masked
    m[0, 3, 3:] = -np.inf                     # last keys masked
    r = oracle.sdpa(q, k, v, m)
    assert np.isnan(r.ref[0, 1]).all() and np.isnan(r.err[0, 1]).all()
    assert np.isfinite(r.ref[0, [0, 2, 3]]).all() and np.isfinite(r.err[0, [0, 2, 3]]).all()
    r2 = oracle.sdpa(q[:, 2:3], k[:, 3:], v[:, 3:], m[:, 2:3, 3:].copy())
    np.testing.assert_allclose(r.ref[0, 2], r2.ref[0, 0], rtol=0, atol=1e-15)
    r3 = oracle.sdpa(q[:, 3:4], k[:, :3], v[:, :3], m[:, 3:4, :3].copy())
    np.testing.assert_allclose(r.ref[0, 3], r3.ref[0, 0], rtol=0, atol=1e-15)


def test_sdpa_sampled_rows_equal_full():
    q, k, v, m = _qkv(3, 7, 10, 12, 110, mask=True)
    full = oracle.sdpa(q, k, v, m, 0.5)
    rows = np.array([0, 6, 7, 13, 20])
    s = oracle.sdpa_rows(q, k, v, m, 0.5, rows)
    assert (s.ref == full.ref.reshape(-1, 12)[rows]).all()
    assert (s.err == full.err.reshape(-1, 12)[rows]).all()


def test_sdpa_error_scale_covers_an_fp32_evaluation():
    # A plain float32 evaluation (numpy, one order of summation) must sit
    # inside the acceptance bound 4e-6 * err, with room to spare.
    B, H, Sq, Skv, D = 2, 2, 48, 300, 64
    g = torch.Generator("cpu").manual_seed(120)
    q = (torch.randn(B, H, Sq, D, generator=g) * 1.5).numpy()
    k = (torch.randn(B, H, Skv, D, generator=g) * 1.5).numpy()
    v = torch.randn(B, H, Skv, D, generator=g).numpy()
    m = (torch.randn(B, H, Sq, Skv, generator=g)).numpy()
    r = oracle.sdpa(q, k, v, m)
    sc = np.float32(1.0 / 8.0)
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * sc + m
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    f32 = np.matmul(p / p.sum(axis=-1, keepdims=True), v)
    assert f32.dtype == np.float32
    bound = oracle.sdpa_tolerance(r)
    assert (np.abs(f32 - r.ref) <= 0.25 * bound).all()
    assert (r.err > 0).all()


# ------------------------------------------------------- channels-last conv
# The conv page's Constraints paragraph: NCHW keeps the GEMM's K dimension
# strided; channels-last (input [B,H,W,IC], weight [OC,KH,KW,IC], output
# [B,OH,OW,OC]) makes it contiguous.  Same convolution, other layout.

def _nchw(t):
    return np.ascontiguousarray(np.transpose(t, (0, 3, 1, 2)))


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil", [
    (2, 4, 9, 7, 5, 3, 3, 1, 1, 1), (1, 3, 12, 11, 6, 7, 7, 4, 3, 1),
    (2, 8, 10, 10, 4, 3, 2, (2, 1), (1, 0), (2, 3)), (1, 5, 6, 6, 3, 1, 1, 1, 0, 1)])
def test_nhwc_conv_is_the_nchw_conv_in_another_layout(B, IC, H, W, OC, KH, KW, stride, pad, dil):
    x = rand32((B, H, W, IC), 140)
    w = rand32((OC, KH, KW, IC), 141)
    b = rand32((OC,), 142)
    r = oracle.conv2d_nhwc(x, w, b, stride, pad, dil)
    n = oracle.conv2d(_nchw(x), _nchw(w), b, stride, pad, dil)
    np.testing.assert_allclose(r.ref, np.transpose(n.ref, (0, 2, 3, 1)), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r.sabs, np.transpose(n.sabs, (0, 2, 3, 1)), rtol=1e-13, atol=0)
    t = F.conv2d(torch.from_numpy(_nchw(x)).double(), torch.from_numpy(_nchw(w)).double(),
                 torch.from_numpy(b).double(), stride, pad, dil).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-12)


def test_nhwc_conv_1x1_is_a_matmul():
    x, w, b = rand32((2, 5, 4, 6), 143), rand32((7, 1, 1, 6), 144), rand32((7,), 145)
    r = oracle.conv2d_nhwc(x, w, b)
    want = x.reshape(-1, 6).astype(np.float64) @ w.reshape(7, 6).T.astype(np.float64) + b
    np.testing.assert_allclose(r.ref.reshape(-1, 7), want, rtol=1e-14, atol=1e-14)


def test_nhwc_conv_delta_kernel_shifts_input():
    # w[oc, kh0, kw0, ic] = delta(oc, ic): out[b, oh, ow, c] = x[b, oh*s - p + kh0*d, ..., c]
    C, KH, KW, kh0, kw0 = 4, 3, 3, 2, 0
    x = rand32((2, 8, 9, C), 146)
    w = np.zeros((C, KH, KW, C), np.float32)
    for c in range(C):
        w[c, kh0, kw0, c] = 1.0
    r = oracle.conv2d_nhwc(x, w, None, 1, 1, 2)
    xp = np.pad(x.astype(np.float64), ((0, 0), (1, 1), (1, 1), (0, 0)))
    OH, OW = r.ref.shape[1:3]
    want = xp[:, kh0 * 2: kh0 * 2 + OH, kw0 * 2: kw0 * 2 + OW, :]
    assert (r.ref == want).all()


def test_sampled_nhwc_conv_equals_full():
    x, w, b = rand32((2, 7, 6, 4), 147), rand32((5, 3, 3, 4), 148), rand32((5,), 149)
    full = oracle.conv2d_nhwc(x, w, b, 2, 1, 1)
    idx = np.array([0, 3, 17, full.ref.size - 1, full.ref.size // 2])
    s = oracle.conv2d_nhwc_at(x, w, b, 2, 1, 1, idx)
    assert (s.ref == full.ref.reshape(-1)[idx]).all() and (s.sabs == full.sabs.reshape(-1)[idx]).all()


# ----------------------------------------------------------- transposed conv
# The conv page keeps transposed convs on their own gather kernels; the
# definition taken is the adjoint of conv2d (aten's conv_transpose2d):
# weight [IC,OC,KH,KW], x[b,ic,ih,iw]*w[ic,oc,kh,kw] lands on
# out[b, oc, ih*sH - pH + kh*dH, iw*sW - pW + kw*dW].

CONVT_SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, dil, out_pad
    (2, 3, 5, 4, 4, 3, 3, 1, 0, 1, 0), (1, 4, 6, 5, 3, 4, 4, 2, 1, 1, 0),
    (2, 2, 4, 7, 5, 3, 2, (2, 3), (1, 0), (1, 2), (1, 2)), (1, 3, 3, 3, 2, 2, 2, 2, 0, 1, 1),
    (1, 5, 7, 6, 4, 5, 3, 3, 2, 2, (2, 0))]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,opad", CONVT_SHAPES)
def test_conv_transpose_vs_torch_float64(B, IC, H, W, OC, KH, KW, stride, pad, dil, opad):
    x, w, b = rand32((B, IC, H, W), 150), rand32((IC, OC, KH, KW), 151), rand32((OC,), 152)
    r = oracle.conv_transpose2d(x, w, b, stride, pad, dil, opad)
    t = F.conv_transpose2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                           torch.from_numpy(b).double(), stride, pad, opad, 1, dil).numpy()
    assert r.ref.shape == t.shape
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,opad", CONVT_SHAPES)
def test_conv_transpose_is_the_adjoint_of_conv(B, IC, H, W, OC, KH, KW, stride, pad, dil, opad):
    # <convT(x), y> = <x, conv(y)> for the same weight read as a conv weight
    # [OC', IC'] = [IC, OC] (no bias): the defining property, checked with
    # the oracle's own direct conv.
    x, w = rand32((B, IC, H, W), 153), rand32((IC, OC, KH, KW), 154)
    r = oracle.conv_transpose2d(x, w, None, stride, pad, dil, opad)
    y = rand32(r.ref.shape, 155)
    c = oracle.conv2d(y, w, None, stride, pad, dil)   # y [B,OC,OH,OW] -> [B,IC,H',W']
    h, wd = min(H, c.ref.shape[2]), min(W, c.ref.shape[3])
    # with output padding the conv of y may see fewer rows than x has; the
    # missing rows of x only reach output rows past OH, which do not exist
    lhs = float((r.ref * y.astype(np.float64)).sum())
    rhs = float((x[:, :, :h, :wd].astype(np.float64) * c.ref[:, :, :h, :wd]).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_conv_transpose_stride1_is_a_flipped_conv():
    # stride 1: convT(x, w) = conv(x, flip(w)^T, pad = d*(K-1) - p)
    x, w, b = rand32((2, 3, 6, 7), 156), rand32((3, 4, 3, 2), 157), rand32((4,), 158)
    r = oracle.conv_transpose2d(x, w, b, 1, (1, 0), (2, 1), 0)
    wf = np.ascontiguousarray(np.flip(w, (2, 3)).transpose(1, 0, 2, 3))
    c = oracle.conv2d(x, wf, b, 1, (2 * 2 - 1, 1 * 1 - 0), (2, 1))
    np.testing.assert_allclose(r.ref, c.ref, rtol=1e-13, atol=1e-13)


def test_conv_transpose_single_pixel_places_the_kernel():
    # one nonzero input pixel at (ih, iw) stamps x * w[ic, oc] at
    # (ih*s - p + kh*d, iw*s - p + kw*d)
    x = np.zeros((1, 1, 4, 5), np.float32)
    x[0, 0, 2, 3] = 2.0
    w = rand32((1, 2, 3, 3), 159)
    r = oracle.conv_transpose2d(x, w, None, 2, 1, 2, 0)
    want = np.zeros_like(r.ref)
    for oc in range(2):
        for kh in range(3):
            for kw in range(3):
                want[0, oc, 2 * 2 - 1 + 2 * kh, 3 * 2 - 1 + 2 * kw] += 2.0 * w[0, oc, kh, kw]
    assert (r.ref == want).all()


def test_conv_transpose_output_size():
    assert oracle.convt_out_size(5, 3, 1, 0, 1, 0) == 7
    assert oracle.convt_out_size(6, 4, 2, 1, 1, 0) == 12     # the usual 2x upsampling
    assert oracle.convt_out_size(4, 3, 2, 1, 2, 1) == 10     # (4-1)*2 - 2 + 4 + 1 + 1
    assert oracle.convt_out_size(3, 2, 2, 0, 1, 1) == 7


def test_sampled_conv_transpose_equals_full():
    # the sampled form gathers (divisibility test) where the full form
    # scatters: the two formulations must agree
    for shape in CONVT_SHAPES:
        B, IC, H, W, OC, KH, KW, stride, pad, dil, opad = shape
        x, w, b = rand32((B, IC, H, W), 160), rand32((IC, OC, KH, KW), 161), rand32((OC,), 162)
        full = oracle.conv_transpose2d(x, w, b, stride, pad, dil, opad)
        idx = np.arange(full.ref.size)
        s = oracle.conv_transpose2d_at(x, w, b, stride, pad, dil, opad, idx)
        np.testing.assert_allclose(s.ref, full.ref.reshape(-1), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(s.sabs, full.sabs.reshape(-1), rtol=1e-13, atol=0)


# Grouped transposed conv: weight [IC, OC/G, KH, KW]; input channel ic feeds
# only the output channels of its group ic // (IC/G) (aten's groups).
CONVT_GROUPED_SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, dil, out_pad, groups
    (2, 4, 5, 4, 6, 3, 3, 2, 1, 1, 1, 2), (1, 6, 4, 5, 3, 2, 3, (2, 1), (0, 1), 1, (1, 0), 3),
    (1, 8, 3, 3, 8, 3, 3, 1, 1, 2, 0, 8), (2, 4, 3, 4, 8, 4, 4, 2, 1, 1, 0, 4)]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,opad,groups", CONVT_GROUPED_SHAPES)
def test_grouped_conv_transpose_vs_torch_float64(B, IC, H, W, OC, KH, KW, stride, pad, dil, opad,
                                                 groups):
    x = rand32((B, IC, H, W), 163)
    w, b = rand32((IC, OC // groups, KH, KW), 164), rand32((OC,), 165)
    r = oracle.conv_transpose2d(x, w, b, stride, pad, dil, opad, groups)
    t = F.conv_transpose2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                           torch.from_numpy(b).double(), stride, pad, opad, groups, dil).numpy()
    assert r.ref.shape == t.shape
    np.testing.assert_allclose(r.ref, t, rtol=1e-12, atol=1e-12)
    idx = np.arange(r.ref.size)
    s = oracle.conv_transpose2d_at(x, w, b, stride, pad, dil, opad, idx, groups)
    np.testing.assert_allclose(s.ref, r.ref.reshape(-1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s.sabs, r.sabs.reshape(-1), rtol=1e-13, atol=0)


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,opad,groups", CONVT_GROUPED_SHAPES)
def test_grouped_conv_transpose_is_the_adjoint_of_grouped_conv(B, IC, H, W, OC, KH, KW, stride,
                                                               pad, dil, opad, groups):
    # <convT_G(x), y> = <x, conv_G(y)>: the weight [IC, OC/G, KH, KW] read as
    # a grouped conv weight [OC' = IC, IC'/G = OC/G, KH, KW].
    x, w = rand32((B, IC, H, W), 166), rand32((IC, OC // groups, KH, KW), 167)
    r = oracle.conv_transpose2d(x, w, None, stride, pad, dil, opad, groups)
    y = rand32(r.ref.shape, 168)
    c = oracle.conv2d_grouped(y, w, None, stride, pad, dil, groups)
    h, wd = min(H, c.ref.shape[2]), min(W, c.ref.shape[3])
    lhs = float((r.ref * y.astype(np.float64)).sum())
    rhs = float((x[:, :, :h, :wd].astype(np.float64) * c.ref[:, :, :h, :wd]).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_grouped_conv_transpose_block_structure():
    # a group's output channels are untouched by the other groups' inputs:
    # zeroing every input channel outside group 1 leaves groups 0 and 2 at
    # their bias, and group 1 equals the ungrouped transposed conv of its
    # own channels and weight slice
    G, icg, ocg = 3, 2, 4
    x, w, b = rand32((1, G * icg, 4, 5), 169), rand32((G * icg, ocg, 3, 3), 170), rand32((G * ocg,), 171)
    x[:, :icg] = 0.0
    x[:, 2 * icg:] = 0.0
    r = oracle.conv_transpose2d(x, w, b, 2, 1, 1, 1, G)
    for g in (0, 2):
        assert (r.ref[:, g * ocg:(g + 1) * ocg] ==
                b[g * ocg:(g + 1) * ocg].astype(np.float64)[None, :, None, None]).all()
    one = oracle.conv_transpose2d(np.ascontiguousarray(x[:, icg:2 * icg]),
                                  np.ascontiguousarray(w[icg:2 * icg]),
                                  np.ascontiguousarray(b[ocg:2 * ocg]), 2, 1, 1, 1)
    assert (r.ref[:, ocg:2 * ocg] == one.ref).all()
