"""Pins of the acceptance bound every GPU parity verdict rests on.

The bound is stated with the workload for the addmm page's
``out = beta*self + alpha*(mat1 @ mat2)`` ("[ExecuTorch][WebGPU] Add
optimized addmm op", Solution paragraph) and reused for the conv page's GEMM
("et_vk conv2d: route standard (groups==1) conv through an im2col tiled
GEMM", Implementation paragraph) with alpha = beta = 1 and self = bias[oc]:

    |out - ref| <= 4e-6 * sqrt(K) * (|alpha| * sum_k |a_ik * b_kj| + |beta * self_ij|)

The helpers that compute it (``oracle.tolerance`` and the ``selfabs`` terms
each oracle function returns) are checked here against values worked out by
hand on inputs small enough to read, with dyadic numbers so every figure is
exact; and ``check_close`` must accept an error of 0.99x the bound and reject
1.01x.  The attention bound (``oracle.sdpa_tolerance``) is pinned by hand
values of its error scale and from above: a plausible mistake in a kernel
(one key dropped) must fall outside it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests._parity import check_close

SQ3 = math.sqrt(3.0)

# mat1 [2,3], mat2 [3,2]; every product and sum below is exact in binary.
A = np.array([[1.0, -2.0, 0.5], [3.0, 0.25, -1.0]], np.float32)
B = np.array([[2.0, -1.0], [0.5, 4.0], [-3.0, 1.0]], np.float32)
# (A @ B) by hand: row 0: 2 - 1 - 1.5 = -0.5, -1 - 8 + 0.5 = -8.5
#                  row 1: 6 + 0.125 + 3 = 9.125, -3 + 1 - 1 = -3
ACC = np.array([[-0.5, -8.5], [9.125, -3.0]])
# sum_k |a_ik b_kj|: row 0: 2 + 1 + 1.5 = 4.5, 1 + 8 + 0.5 = 9.5
#                    row 1: 6 + 0.125 + 3 = 9.125, 3 + 1 + 1 = 5
SABS = np.array([[4.5, 9.5], [9.125, 5.0]])
BETA, ALPHA = 0.5, -2.0


def test_addmm_bound_by_hand_self_row():
    s = np.array([1.5, -4.0], np.float32)
    r = oracle.addmm(A, B, s, False, BETA, ALPHA)
    assert (r.ref == np.array([[1.75, 15.0], [-17.5, 4.0]])).all()
    assert (r.sabs == SABS).all()
    # |beta * self_j| broadcast over rows: 0.75, 2
    assert (r.selfabs == np.array([[0.75, 2.0], [0.75, 2.0]])).all()
    # |alpha| * sabs + |beta*self| = 9 + 0.75, 19 + 2, 18.25 + 0.75, 10 + 2
    want = 4e-6 * SQ3 * np.array([[9.75, 21.0], [19.0, 12.0]])
    np.testing.assert_allclose(oracle.tolerance(r, 3, ALPHA), want, rtol=1e-15, atol=0)


def test_addmm_bound_by_hand_full_self():
    s = np.array([[1.5, -4.0], [-0.5, 8.0]], np.float32)
    r = oracle.addmm(A, B, s, True, BETA, ALPHA)
    assert (r.ref == np.array([[1.75, 15.0], [-18.5, 10.0]])).all()
    assert (r.selfabs == np.array([[0.75, 2.0], [0.25, 4.0]])).all()
    want = 4e-6 * SQ3 * np.array([[9.75, 21.0], [18.5, 14.0]])
    np.testing.assert_allclose(oracle.tolerance(r, 3, ALPHA), want, rtol=1e-15, atol=0)


def test_addmm_bound_by_hand_sampled():
    # the sampled form carries the same terms at each (row, col)
    s = np.array([[1.5, -4.0], [-0.5, 8.0]], np.float32)
    rows, cols = np.array([1, 0, 1]), np.array([0, 1, 1])
    r = oracle.addmm_at(A, B, s, True, BETA, ALPHA, rows, cols)
    assert (r.ref == np.array([-18.5, 15.0, 10.0])).all()
    assert (r.sabs == np.array([9.125, 9.5, 5.0])).all()
    assert (r.selfabs == np.array([0.25, 2.0, 4.0])).all()
    np.testing.assert_allclose(oracle.tolerance(r, 3, ALPHA), 4e-6 * SQ3 * np.array([18.5, 21.0, 14.0]),
                               rtol=1e-15, atol=0)
    s1 = np.array([1.5, -4.0], np.float32)
    r1 = oracle.addmm_at(A, B, s1, False, BETA, ALPHA, rows, cols)
    assert (r1.selfabs == np.array([0.75, 2.0, 2.0])).all()


def test_addmm_bound_beta_zero_has_no_self_term():
    # beta = 0: the self term is 0 and self is not read (NaN there is fine)
    s = np.array([np.nan, 7.0], np.float32)
    r = oracle.addmm(A, B, s, False, 0.0, ALPHA)
    assert (r.selfabs == 0).all()
    np.testing.assert_allclose(oracle.tolerance(r, 3, ALPHA), 4e-6 * SQ3 * 2.0 * SABS, rtol=1e-15, atol=0)


def test_linear_bound_by_hand():
    # x [2,3] @ w[2,3]^T + bias: weight rows are mat2's columns (B^T)
    w = np.ascontiguousarray(B.T)
    bias = np.array([-0.25, 3.0], np.float32)
    r = oracle.linear(A, w, bias)
    assert (r.ref == ACC + np.array([-0.25, 3.0])).all()
    assert (r.sabs == SABS).all()
    assert (r.selfabs == np.array([[0.25, 3.0], [0.25, 3.0]])).all()
    want = 4e-6 * SQ3 * (SABS + np.array([0.25, 3.0]))
    np.testing.assert_allclose(oracle.tolerance(r, 3), want, rtol=1e-15, atol=0)
    rs = oracle.linear_at(A, w, bias, np.array([1, 0]), np.array([1, 0]))
    assert (rs.selfabs == np.array([3.0, 0.25])).all()


X22 = np.array([[[[1.0, 2.0], [3.0, 4.0]]]], np.float32)             # [1,1,2,2]
W22 = np.array([[[[1.0, -1.0], [0.5, 2.0]]], [[[-2.0, 0.0], [1.0, 1.0]]]], np.float32)  # [2,1,2,2]
BIAS2 = np.array([0.25, -3.0], np.float32)


def test_conv_bound_by_hand():
    # one output pixel per channel; K = 4 taps
    # oc 0: 1 - 2 + 1.5 + 8 = 8.5 (+0.25), sabs 12.5; oc 1: -2 + 0 + 3 + 4 = 5 (-3), sabs 9
    r = oracle.conv2d(X22, W22, BIAS2)
    assert (r.ref.reshape(-1) == np.array([8.75, 2.0])).all()
    assert (r.sabs.reshape(-1) == np.array([12.5, 9.0])).all()
    assert (np.asarray(r.selfabs).reshape(-1) == np.array([0.25, 3.0])).all()
    want = 4e-6 * 2.0 * np.array([12.75, 12.0])
    np.testing.assert_allclose(oracle.tolerance(r, 4).reshape(-1), want, rtol=1e-15, atol=0)
    for fn in (oracle.conv2d_grouped,):
        g = fn(X22, W22, BIAS2, 1, 0, 1, 1)
        np.testing.assert_allclose(oracle.tolerance(g, 4).reshape(-1), want, rtol=1e-15, atol=0)
    s = oracle.conv2d_at(X22, W22, BIAS2, 1, 0, 1, np.array([1, 0]))
    np.testing.assert_allclose(oracle.tolerance(s, 4), want[::-1], rtol=1e-15, atol=0)
    gs = oracle.conv2d_grouped_at(X22, W22, BIAS2, 1, 0, 1, 1, np.array([1, 0]))
    np.testing.assert_allclose(oracle.tolerance(gs, 4), want[::-1], rtol=1e-15, atol=0)


def test_conv_bound_padding_taps_add_nothing():
    # a 1x1 input under a 3x3 kernel with pad 2: output (oh, ow) of the 3x3
    # output sees only tap (2 - oh, 2 - ow); its bound is
    # 4e-6*3*(|2*w| + |bias[oc]|): the eight padding taps add nothing to sum|x*w|
    x = np.array([[[[2.0]]]], np.float32)
    taps = np.arange(1, 10, dtype=np.float32).reshape(3, 3)
    w = np.stack([taps * np.float32(-0.5), taps * np.float32(0.25)])[:, None]   # [2,1,3,3]
    b = np.array([1.0, -2.0], np.float32)
    r = oracle.conv2d(x, w, b, 1, 2, 1)
    want_sabs = np.abs(2.0 * w[:, 0, ::-1, ::-1].astype(np.float64))            # [2,3,3]
    assert (r.sabs[0] == want_sabs).all()
    want = 4e-6 * 3.0 * (want_sabs + np.abs(b.astype(np.float64))[:, None, None])
    np.testing.assert_allclose(oracle.tolerance(r, 9)[0], want, rtol=1e-15, atol=0)
    # sampled outputs: flat NCHW index oc*9 + oh*3 + ow
    idx = np.array([10, 3, 17, 0, 9])
    rs = oracle.conv2d_at(x, w, b, 1, 2, 1, idx)
    np.testing.assert_allclose(oracle.tolerance(rs, 9), want.reshape(-1)[idx], rtol=1e-15, atol=0)
    rg = oracle.conv2d_grouped_at(x, w, b, 1, 2, 1, 1, idx)
    np.testing.assert_allclose(oracle.tolerance(rg, 9), want.reshape(-1)[idx], rtol=1e-15, atol=0)
    # channels-last: the same numbers at NHWC positions
    xn, wn = x.transpose(0, 2, 3, 1).copy(), w.transpose(0, 2, 3, 1).copy()
    rn = oracle.conv2d_nhwc(xn, wn, b, 1, 2, 1)
    np.testing.assert_allclose(oracle.tolerance(rn, 9)[0], want.transpose(1, 2, 0), rtol=1e-15, atol=0)
    nidx = np.array([4 * 2 + 1, 4 * 2, 8 * 2 + 1, 0, 1])     # (pix, oc) -> pix*2 + oc
    rns = oracle.conv2d_nhwc_at(xn, wn, b, 1, 2, 1, nidx)
    np.testing.assert_allclose(oracle.tolerance(rns, 9), want.transpose(1, 2, 0).reshape(-1)[nidx],
                               rtol=1e-15, atol=0)


def test_conv_transpose_bound_by_hand():
    # one input pixel: output (kh, kw) gets x*w[kh, kw]; bias 0.5
    x = np.array([[[[-2.0]]]], np.float32)
    w = np.array([[[[1.0, -3.0], [0.25, 2.0]]]], np.float32)
    b = np.array([0.5], np.float32)
    r = oracle.conv_transpose2d(x, w, b, 1, 0, 1, 0)
    assert (r.ref[0, 0] == np.array([[-1.5, 6.5], [0.0, -3.5]])).all()
    assert (r.sabs[0, 0] == np.array([[2.0, 6.0], [0.5, 4.0]])).all()
    np.testing.assert_allclose(oracle.tolerance(r, 4)[0, 0],
                               4e-6 * 2.0 * np.array([[2.5, 6.5], [1.0, 4.5]]), rtol=1e-15, atol=0)
    s = oracle.conv_transpose2d_at(x, w, b, 1, 0, 1, 0, np.array([3, 1]))
    np.testing.assert_allclose(oracle.tolerance(s, 4), 4e-6 * 2.0 * np.array([4.5, 6.5]),
                               rtol=1e-15, atol=0)


@pytest.mark.parametrize("self_2d", [False, True])
def test_check_close_accepts_inside_and_rejects_outside(self_2d):
    s = (np.array([[1.5, -4.0], [-0.5, 8.0]], np.float32) if self_2d
         else np.array([1.5, -4.0], np.float32))
    r = oracle.addmm(A, B, s, self_2d, BETA, ALPHA)
    tol = oracle.tolerance(r, 3, ALPHA)
    sign = np.array([[1.0, -1.0], [-1.0, 1.0]])
    check_close(r.ref + 0.99 * sign * tol, r, 3, ALPHA, "inside")
    for i in range(2):
        for j in range(2):
            out = r.ref.copy()
            out[i, j] += 1.01 * sign[i, j] * tol[i, j]
            with pytest.raises(AssertionError):
                check_close(out, r, 3, ALPHA, "outside")
    # alpha enters as |alpha|: the bound with alpha = +2 is the same
    check_close(r.ref + 0.99 * tol, r, 3, 2.0, "alpha sign")
    with pytest.raises(AssertionError):
        check_close(r.ref + 0.99 * tol, r, 3, 1.0, "smaller alpha")


def test_check_close_rejects_nan():
    r = oracle.addmm(A, B, np.array([1.5, -4.0], np.float32), False, BETA, ALPHA)
    out = r.ref.copy()
    out[1, 0] = np.nan
    with pytest.raises(AssertionError):
        check_close(out, r, 3, ALPHA, "nan")


def test_bound_covers_fp32_rounding_with_room_to_spare():
    # 4e-6*sqrt(K) is about 67 fp32 rounding units times sqrt(K); the worst
    # case of a length-K fp32 dot product is K units: the bound exceeds it
    # for every K up to 4503 (sqrt(K) <= 4e-6 / u), in particular at the workload depths
    u = 2.0 ** -24
    for K in (96, 147, 768, 1024, 2304, 4096):
        assert 4e-6 * math.sqrt(K) >= K * u
    assert 4e-6 * math.sqrt(4503) >= 4503 * u and 4e-6 * math.sqrt(4504) < 4504 * u


# ------------------------------------------------------------- attention

def test_sdpa_error_scale_by_hand_single_key():
    # one key: weight 1, out = v.  err_d = 1*(|v_d| + |v_d|)*(sqrt(D)*a + 0 + sqrt(1) + 1)
    # with a = |scale|*sum_d|q_d k_d| + |mask| = 0.5*4.5 + 0.25 = 2.5: factor 7
    q = np.array([[[1.0, -1.0, 2.0, 0.5]]], np.float32)
    k = np.array([[[0.5, 1.0, -1.0, 2.0]]], np.float32)
    v = np.array([[[1.0, -2.0, 0.5, 3.0]]], np.float32)
    m = np.array([[[0.25]]], np.float32)
    r = oracle.sdpa(q, k, v, m, 0.5)
    assert (r.ref[0, 0] == v[0, 0]).all()
    assert (r.err[0, 0] == np.array([14.0, 28.0, 7.0, 42.0])).all()
    np.testing.assert_allclose(oracle.sdpa_tolerance(r)[0, 0], 4e-6 * np.array([14.0, 28.0, 7.0, 42.0]),
                               rtol=1e-15, atol=0)


def test_sdpa_error_scale_by_hand_two_keys():
    # scale 0, mask [0, -1]: logits s = (0, -1), max 0; weights e^s / (1 + e^-1);
    # a_j = |mask_j| = (0, 1); D = 4, Skv = 2:
    # err_d = w0 (|v0d| + |o_d|) (0 + 0 + sqrt2 + 1) + w1 (|v1d| + |o_d|) (2*1 + 1 + sqrt2 + 1)
    q = np.ones((1, 1, 4), np.float32)
    k = np.ones((1, 2, 4), np.float32)
    v = np.array([[[1.0, -2.0, 0.0, 4.0], [3.0, 1.0, -1.0, -4.0]]], np.float32)
    m = np.array([[[0.0, -1.0]]], np.float32)
    r = oracle.sdpa(q, k, v, m, 0.0)
    e1 = math.exp(-1.0)
    w0, w1 = 1.0 / (1.0 + e1), e1 / (1.0 + e1)
    o = w0 * v[0, 0].astype(np.float64) + w1 * v[0, 1].astype(np.float64)
    np.testing.assert_allclose(r.ref[0, 0], o, rtol=1e-14, atol=1e-15)
    want = (w0 * (np.abs(v[0, 0]) + np.abs(o)) * (math.sqrt(2.0) + 1.0) +
            w1 * (np.abs(v[0, 1]) + np.abs(o)) * (2.0 + 1.0 + math.sqrt(2.0) + 1.0))
    np.testing.assert_allclose(r.err[0, 0], want, rtol=1e-14, atol=0)


def test_sdpa_bound_rejects_a_dropped_key():
    # from above: leaving out one key of 197 (a plausible kernel mistake at a
    # ragged edge) must fall outside the bound on most outputs
    g = torch.Generator("cpu").manual_seed(172)
    q = torch.randn(2, 16, 64, generator=g).numpy()
    k = torch.randn(2, 197, 64, generator=g).numpy()
    v = torch.randn(2, 197, 64, generator=g).numpy()
    r = oracle.sdpa(q, k, v)
    scale = np.float32(1.0 / 8.0)
    for drop in (0, 196):
        keep = np.ones(197, bool)
        keep[drop] = False
        d = oracle.sdpa(q, np.ascontiguousarray(k[:, keep]), np.ascontiguousarray(v[:, keep]), None,
                        scale)
        outside = np.abs(d.ref - r.ref) > oracle.sdpa_tolerance(r)
        assert outside.mean() > 0.5, (drop, outside.mean())


def test_sdpa_bound_rejects_a_wrong_scale():
    # from above: a 1% error in the softmax scale must not pass
    g = torch.Generator("cpu").manual_seed(173)
    q = torch.randn(1, 32, 64, generator=g).numpy()
    k = torch.randn(1, 128, 64, generator=g).numpy()
    v = torch.randn(1, 128, 64, generator=g).numpy()
    r = oracle.sdpa(q, k, v, None, 0.125)
    d = oracle.sdpa(q, k, v, None, 0.125 * 1.01)
    assert (np.abs(d.ref - r.ref) > oracle.sdpa_tolerance(r)).mean() > 0.5
