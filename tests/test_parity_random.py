"""GPU: seeded random sweeps of every entry point against the fp64 oracle.

Each op runs on a few dozen shapes drawn from a fixed seed (ragged sizes,
strides, paddings, dilations, groups, masks, scales, alpha/beta), so edge
combinations that no hand-picked case names are still compared element by
element.  Same acceptance bounds as the op's own parity file.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._parity import check_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def say(msg):
    print(f"[random] {msg}", flush=True)


def gen(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.rand(shape, generator=g) * 2 - 1


def test_random_addmm_and_linear():
    import bias_addmm_im2col_amd as baim
    rng = np.random.default_rng(1000)
    for i in range(40):
        M, K, N = (int(v) for v in rng.integers(1, 400, 3))
        self_2d = bool(rng.integers(0, 2))
        beta, alpha = float(rng.choice([0.0, 1.0, -0.5, 2.0])), float(rng.choice([1.0, 0.25, -3.0]))
        say(f"{i}: addmm M={M} K={K} N={N} self_2d={self_2d} beta={beta} alpha={alpha}")
        a, b = gen((M, K), 3 * i), gen((K, N), 3 * i + 1)
        s = gen((M, N) if self_2d else (N,), 3 * i + 2)
        out = baim.addmm(dev(s), dev(a), dev(b), beta=beta, alpha=alpha)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), oracle.addmm(a, b, s, self_2d, beta, alpha), K, alpha,
                    f"random addmm {i}")
        w = gen((N, K), 3 * i + 7)
        bias = gen((N,), 3 * i + 8) if i % 2 else None
        say(f"{i}: linear M={M} K={K} N={N} bias={bias is not None}")
        out = baim.linear(dev(a), dev(w), dev(bias))
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), oracle.linear(a, w, bias), K, 1.0, f"random linear {i}")


def _conv_geometry(rng):
    while True:
        KH, KW = (int(v) for v in rng.integers(1, 6, 2))
        sH, sW = (int(v) for v in rng.integers(1, 4, 2))
        dH, dW = (int(v) for v in rng.integers(1, 3, 2))
        pH, pW = int(rng.integers(0, KH)), int(rng.integers(0, KW))
        H, W = (int(v) for v in rng.integers(1, 30, 2))
        if H + 2 * pH - dH * (KH - 1) - 1 >= 0 and W + 2 * pW - dW * (KW - 1) - 1 >= 0:
            return KH, KW, (sH, sW), (pH, pW), (dH, dW), H, W


def test_random_conv_nchw_grouped_and_nhwc():
    import bias_addmm_im2col_amd as baim
    rng = np.random.default_rng(2000)
    for i in range(40):
        KH, KW, st, pd, dl, H, W = _conv_geometry(rng)
        G = int(rng.choice([1, 1, 2, 4, 8]))
        IC = G * int(rng.integers(1, 12))
        OC = G * int(rng.integers(1, 40))
        B = int(rng.integers(1, 3))
        say(f"{i}: conv2d B={B} IC={IC} H={H} W={W} OC={OC} k=({KH},{KW}) s={st} p={pd} d={dl} G={G}")
        x, w = gen((B, IC, H, W), 5 * i), gen((OC, IC // G, KH, KW), 5 * i + 1)
        bias = gen((OC,), 5 * i + 2) if i % 3 else None
        out = baim.conv2d(dev(x), dev(w), dev(bias), st, pd, dl, G)
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(), oracle.conv2d_grouped(x, w, bias, st, pd, dl, G),
                    IC // G * KH * KW, 1.0, f"random conv {i}")
        if G == 1:
            xn = x.permute(0, 2, 3, 1).contiguous()
            wn = w.permute(0, 2, 3, 1).contiguous()
            say(f"{i}: conv2d_nhwc")
            out = baim.conv2d_nhwc(dev(xn), dev(wn), dev(bias), st, pd, dl)
            torch.cuda.synchronize()
            check_close(out.cpu().numpy(), oracle.conv2d_nhwc(xn, wn, bias, st, pd, dl),
                        IC * KH * KW, 1.0, f"random nhwc {i}")


def test_random_conv_transpose():
    import bias_addmm_im2col_amd as baim
    rng = np.random.default_rng(3000)
    for i in range(30):
        KH, KW = (int(v) for v in rng.integers(1, 6, 2))
        sH, sW = (int(v) for v in rng.integers(1, 5, 2))
        dH, dW = (int(v) for v in rng.integers(1, 3, 2))
        pH, pW = int(rng.integers(0, KH)), int(rng.integers(0, KW))
        oH, oW = int(rng.integers(0, max(sH, dH))), int(rng.integers(0, max(sW, dW)))
        H, W = (int(v) for v in rng.integers(1, 14, 2))
        if oracle.convt_out_size(H, KH, sH, pH, dH, oH) < 1 or \
                oracle.convt_out_size(W, KW, sW, pW, dW, oW) < 1:
            continue
        IC, OC, B = int(rng.integers(1, 40)), int(rng.integers(1, 70)), int(rng.integers(1, 3))
        say(f"{i}: conv_transpose2d B={B} IC={IC} H={H} W={W} OC={OC} k=({KH},{KW}) "
            f"s=({sH},{sW}) p=({pH},{pW}) d=({dH},{dW}) op=({oH},{oW})")
        x, w = gen((B, IC, H, W), 7 * i), gen((IC, OC, KH, KW), 7 * i + 1)
        bias = gen((OC,), 7 * i + 2) if i % 2 else None
        out = baim.conv_transpose2d(dev(x), dev(w), dev(bias), (sH, sW), (pH, pW), (oH, oW), 1,
                                    (dH, dW))
        torch.cuda.synchronize()
        check_close(out.cpu().numpy(),
                    oracle.conv_transpose2d(x, w, bias, (sH, sW), (pH, pW), (dH, dW), (oH, oW)),
                    IC * KH * KW, 1.0, f"random convT {i}")


def test_random_sdpa():
    import bias_addmm_im2col_amd as baim
    rng = np.random.default_rng(4000)
    for i in range(30):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
        Sq, Skv = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        D = 4 * int(rng.integers(1, 33))
        masked = bool(rng.integers(0, 2))
        scale = None if rng.integers(0, 2) else float(rng.uniform(0.05, 0.5))
        say(f"{i}: sdpa B={B} H={H} Sq={Sq} Skv={Skv} D={D} mask={masked} scale={scale}")
        q, k, v = gen((B, H, Sq, D), 9 * i), gen((B, H, Skv, D), 9 * i + 1), gen((B, H, Skv, D), 9 * i + 2)
        m = gen((B, H, Sq, Skv), 9 * i + 3) * 3 if masked else None
        out = baim.sdpa(dev(q), dev(k), dev(v), dev(m), scale)
        torch.cuda.synchronize()
        res = oracle.sdpa(q, k, v, m, scale)
        got = out.cpu().numpy().astype(np.float64)
        err = np.abs(got - res.ref)
        tol = oracle.sdpa_tolerance(res)
        assert (err <= tol).all(), f"random sdpa {i}: worst err/tol {float(np.max(err / tol)):.3g}"
