"""GPU parity of the LDS-window conv kernel (3x3 at stride 1, dilation 1 or 2,
and 3x3 at stride 2) against the fp64 oracle, through conv2d_gemm_f32.

The kernel copies the input rows a block's output pixels touch into LDS
and reads every im2col element from there; what it must get right is the
window (rows above and below the image, columns left and right of it),
output pixel runs that cross output rows and end past an image, k-tiles of
sixteen input channels with a partial last one, ragged output channels, and
the two-piece schedules; at stride 2 also rows of any width (whole
16-byte quads from a 4-byte-aligned row start plus a tail of 1 to 3
columns) and the column parity of the taps.  Every case first checks through baim_conv2d_plan
that the window kernel really is what runs.  Acceptance as in
tests/test_parity.py; integer-valued inputs must match bit for bit.
"""
import pytest
import torch

import oracle
from tests._parity import check_bitwise, check_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def say(msg):
    print(f"[window] {msg}", flush=True)


def gen(shape, seed, kind="U"):
    g = torch.Generator("cpu").manual_seed(seed)
    if kind == "U":
        return torch.rand(shape, generator=g) * 2 - 1
    return torch.randint(-4, 5, shape, generator=g).float()


def run(x, w, b, pad, dil, stride=1):
    import bias_addmm_im2col_amd as baim
    out = baim.conv2d(dev(x), dev(w), dev(b), stride, pad, dil)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def plan(x, w, pad, dil, stride=1):
    import bias_addmm_im2col_amd as baim
    return baim.conv2d_plan(tuple(x.shape), tuple(w.shape), stride, pad, dil)


SHAPES = [
    # B, IC, H, W, OC, pad, dil, bias
    (1, 16, 48, 48, 64, 1, 1, True),        # one k-tile; 2304 pixels = 18 runs of 128
    (2, 20, 33, 44, 100, 1, 1, True),       # partial last k-tile, ragged OC, runs past each image
    (1, 4, 7, 44, 64, (2, 1), 1, False),    # tall pad, short image: most window rows are padding
    (3, 36, 34, 48, 136, 0, 1, True),       # no padding: OW = 46
    (2, 20, 38, 48, 72, 2, 2, True),        # dilation 2, pad 2
    (1, 16, 40, 52, 96, (1, 0), 2, False),  # dilation 2, pads smaller than the reach: OW = 48
    (1, 12, 9, 60, 40, (1, 0), 1, True),    # widest row the window holds (W + pW + 4 = 64)
    (2, 64, 56, 56, 256, 1, 1, True),       # the mid-stage shape at reduced batch and depth
]


@pytest.mark.parametrize("spec", ["", "tile", "2", "s7", "s3"])
@pytest.mark.parametrize("B,IC,H,W,OC,pad,dil,has_bias", SHAPES)
def test_window_conv(B, IC, H, W, OC, pad, dil, has_bias, spec, monkeypatch):
    if spec:
        monkeypatch.setenv("BAIM_CONV_WIN", spec)
    x, w = gen((B, IC, H, W), 1), gen((OC, IC, 3, 3), 2)
    b = gen((OC,), 3) if has_bias else None
    p = plan(x, w, pad, dil)
    say(f"BAIM_CONV_WIN={spec!r} x=[{B},{IC},{H},{W}] OC={OC} p={pad} d={dil} plan {p}")
    assert p["kernel"] == 1
    if spec == "2" and IC > p["bk"] // 9:
        assert p["splits"] == 2
    if spec.startswith("s") and p["stream_blocks"] == 0:
        # fewer workers than tiles is required for a stream; else one tile per block
        assert p["splits"] == 1
    check_close(run(x, w, b, pad, dil), oracle.conv2d(x, w, b, 1, pad, dil), IC * 9, 1.0,
                f"window {spec}")
    xi, wi, bi = gen((B, IC, H, W), 4, "I"), gen((OC, IC, 3, 3), 5, "I"), gen((OC,), 6, "I")
    check_bitwise(run(xi, wi, bi, pad, dil), oracle.conv2d(xi, wi, bi, 1, pad, dil),
                  f"window integer {spec}")


def test_window_stream_pieces_are_reproducible(monkeypatch):
    """A stream plan cuts tiles into two pieces; the exchange combines them
    in an order-free way, so repeated launches give the same bits."""
    import bias_addmm_im2col_amd as baim
    monkeypatch.setenv("BAIM_CONV_WIN", "s13")
    x, w, b = gen((2, 40, 36, 48), 7), gen((136, 40, 3, 3), 8), gen((136,), 9)
    assert plan(x, w, 1, 1)["stream_blocks"] == 13
    outs = [baim.conv2d(dev(x), dev(w), dev(b), 1, 1, 1).cpu() for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    check_close(outs[0].numpy(), oracle.conv2d(x, w, b, 1, 1, 1), 360, 1.0, "stream s13")


def test_window_matches_the_gather_kernel_bitwise(monkeypatch):
    """On integer inputs the window kernel and the general implicit-im2col
    kernel (BAIM_CONV_WIN=off) both give the exact result."""
    x, w, b = gen((2, 24, 32, 48), 10, "I"), gen((96, 24, 3, 3), 11, "I"), gen((96,), 12, "I")
    win = run(x, w, b, 1, 1)
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    import bias_addmm_im2col_amd as baim
    assert baim.conv2d_plan(tuple(x.shape), tuple(w.shape), 1, 1, 1)["kernel"] == 0
    gat = run(x, w, b, 1, 1)
    assert (win == gat).all()
    check_bitwise(win, oracle.conv2d(x, w, b, 1, 1, 1), "window vs gather")


def test_window_nonfinite_input_stays_local():
    """An Inf in the input reaches exactly the outputs whose taps read it
    (the padding columns and rows are zeros, not neighbouring data)."""
    import numpy as np
    x, w, b = gen((1, 8, 34, 48), 13), gen((64, 8, 3, 3), 14), gen((64,), 15)
    x[0, 3, 0, 47] = float("inf")   # last column of the first row
    x[0, 5, 33, 0] = float("-inf")  # first column of the last row
    out = run(x, w, b, 1, 1)
    ref = oracle.conv2d(x, w, b, 1, 1, 1)
    bad = ~np.isfinite(ref.ref)
    assert (~np.isfinite(out) == bad).all()
    finite = np.isfinite(ref.ref)
    assert (np.abs(out[finite] - ref.ref[finite]) <= oracle.tolerance(ref, 72)[finite]).all()


S2_SHAPES = [
    # B, IC, H, W, OC, pad, bias
    (1, 16, 57, 57, 64, 1, True),        # one k-tile; W % 4 = 1; 841 pixels = 13 runs of 64 + 9
    (2, 20, 45, 46, 70, 1, True),        # W % 4 = 2, partial last k-tile, ragged OC, two images
    (1, 32, 48, 59, 64, 1, False),       # W % 4 = 3 and the widest row held (W + pW + 4 = 64)
    (3, 16, 40, 44, 64, 0, True),        # whole quads only, no padding, OW = 21 (runs touch 4 rows)
    (1, 8, 43, 42, 136, (0, 1), True),   # fewer channels than a k-tile, unequal pads, 3 OC blocks
    (2, 64, 57, 57, 256, 1, True),       # the stride-2 mid-stage shape at reduced batch and depth
]


@pytest.mark.parametrize("spec", ["", "2", "s7"])
@pytest.mark.parametrize("B,IC,H,W,OC,pad,has_bias", S2_SHAPES)
def test_window_conv_stride2(B, IC, H, W, OC, pad, has_bias, spec, monkeypatch):
    if spec:
        monkeypatch.setenv("BAIM_CONV_WIN", spec)
    x, w = gen((B, IC, H, W), 21), gen((OC, IC, 3, 3), 22)
    b = gen((OC,), 23) if has_bias else None
    p = plan(x, w, pad, 1, 2)
    say(f"BAIM_CONV_WIN={spec!r} stride 2 x=[{B},{IC},{H},{W}] OC={OC} p={pad} plan {p}")
    assert p["kernel"] == 1 and (p["bm"], p["bn"], p["kgroups"]) == (64, 64, 4)
    assert p["stream_blocks"] == 0  # no streamed instance at stride 2
    if spec == "2":
        assert p["splits"] == (2 if IC > 16 else 1)
    check_close(run(x, w, b, pad, 1, 2), oracle.conv2d(x, w, b, 2, pad, 1), IC * 9, 1.0,
                f"window s2 {spec}")
    xi, wi, bi = gen((B, IC, H, W), 24, "I"), gen((OC, IC, 3, 3), 25, "I"), gen((OC,), 26, "I")
    check_bitwise(run(xi, wi, bi, pad, 1, 2), oracle.conv2d(xi, wi, bi, 2, pad, 1),
                  f"window s2 integer {spec}")


def test_window_stride2_matches_the_gather_kernel_bitwise(monkeypatch):
    x, w, b = gen((2, 40, 45, 46), 27, "I"), gen((72, 40, 3, 3), 28, "I"), gen((72,), 29, "I")
    assert plan(x, w, 1, 1, 2)["kernel"] == 1
    win = run(x, w, b, 1, 1, 2)
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    assert plan(x, w, 1, 1, 2)["kernel"] == 0
    gat = run(x, w, b, 1, 1, 2)
    assert (win == gat).all()


def test_window_stride2_nonfinite_input_stays_local():
    """Non-finite values in the tail column and the first column reach
    exactly the outputs whose taps read them."""
    import numpy as np
    x, w, b = gen((1, 8, 45, 57), 30), gen((64, 8, 3, 3), 31), gen((64,), 32)
    x[0, 3, 0, 56] = float("inf")    # tail column (W % 4 = 1) of the first row
    x[0, 5, 44, 0] = float("-inf")   # first column of the last row
    x[0, 6, 21, 55] = float("nan")   # last column of the whole quads, an interior row
    assert plan(x, w, 1, 1, 2)["kernel"] == 1
    out = run(x, w, b, 1, 1, 2)
    ref = oracle.conv2d(x, w, b, 2, 1, 1)
    bad = ~np.isfinite(ref.ref)
    assert bad.any() and (~np.isfinite(out) == bad).all()
    finite = np.isfinite(ref.ref)
    assert (np.abs(out[finite] - ref.ref[finite]) <= oracle.tolerance(ref, 72)[finite]).all()
