"""GPU parity of the stem kernel (3-channel 7x7 stride-4 convs) against the
fp64 oracle, through conv2d_gemm_f32 (NCHW) and conv2d_nhwc_f32
(channels-last, where the input columns arrive interleaved with their three
channels and four output channels go out per 16-byte store).

The kernel copies the weights and the input columns a block's 144 output
pixels read into LDS once and runs all of K = 147 from there; what it must
get right is the phase-row layout of the input (columns split by residue
mod 4), pixel runs that continue on the next output row or end past the
image, padding on every side, output channels past a multiple of 128 and
the zero-weight padded tap.  Every case first checks through
baim_conv2d_plan (baim_conv2d_nhwc_plan) that the stem kernel really is
what runs.  Acceptance as
in tests/test_parity.py; integer-valued inputs must match bit for bit.
"""
import numpy as np
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
    print(f"[stem] {msg}", flush=True)


def gen(shape, seed, kind="U"):
    g = torch.Generator("cpu").manual_seed(seed)
    if kind == "U":
        return torch.rand(shape, generator=g) * 2 - 1
    return torch.randint(-4, 5, shape, generator=g).float()


def run(x, w, b, pad):
    import bias_addmm_im2col_amd as baim
    out = baim.conv2d(dev(x), dev(w), dev(b), 4, pad, 1)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [
    # B, H, W, OC, pad, bias
    (1, 600, 580, 128, 3, True),     # OW 145: runs straddle rows; last run of 6 pixels
    (2, 580, 600, 100, (2, 1), True),  # OC below 128 (masked rows), unequal pads, two images
    (1, 583, 580, 260, 0, False),    # three blocks of output channels, no padding, OW = 144
    (1, 777, 768, 64, (3, 5), True), # right pad wider than the kernel's reach past W
]


@pytest.mark.parametrize("B,H,W,OC,pad,has_bias", SHAPES)
def test_stem_conv(B, H, W, OC, pad, has_bias):
    import bias_addmm_im2col_amd as baim
    x, w = gen((B, 3, H, W), 1), gen((OC, 3, 7, 7), 2)
    b = gen((OC,), 3) if has_bias else None
    p = baim.conv2d_plan(tuple(x.shape), tuple(w.shape), 4, pad, 1)
    say(f"x=[{B},3,{H},{W}] OC={OC} p={pad} plan {p}")
    assert p["kernel"] == 3
    check_close(run(x, w, b, pad), oracle.conv2d(x, w, b, 4, pad, 1), 147, 1.0, "stem")
    xi, wi, bi = gen((B, 3, H, W), 4, "I"), gen((OC, 3, 7, 7), 5, "I"), gen((OC,), 6, "I")
    check_bitwise(run(xi, wi, bi, pad), oracle.conv2d(xi, wi, bi, 4, pad, 1), "stem integer")


def test_stem_matches_the_gather_kernel_bitwise(monkeypatch):
    """On integer inputs the stem kernel and the general implicit-im2col
    kernel (BAIM_CONV_WIN=off) both give the exact result."""
    import bias_addmm_im2col_amd as baim
    x, w, b = gen((1, 3, 768, 768), 7, "I"), gen((128, 3, 7, 7), 8, "I"), gen((128,), 9, "I")
    stem = run(x, w, b, 3)
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    assert baim.conv2d_plan(tuple(x.shape), tuple(w.shape), 4, 3, 1)["kernel"] == 0
    gat = run(x, w, b, 3)
    assert (stem == gat).all()


def test_stem_nonfinite_input_stays_local():
    """An Inf in the input reaches exactly the outputs whose taps read it:
    padding slots and the padded tap are zeros times zero weights."""
    x, w, b = gen((1, 3, 600, 580), 10), gen((64, 3, 7, 7), 11), gen((64,), 12)
    x[0, 0, 0, 579] = float("inf")    # last column of the first row
    x[0, 2, 599, 0] = float("-inf")   # first column of the last row
    x[0, 1, 301, 290] = float("nan")  # an interior pixel
    out = run(x, w, b, 3)
    ref = oracle.conv2d(x, w, b, 4, 3, 1)
    bad = ~np.isfinite(ref.ref)
    assert bad.any() and (~np.isfinite(out) == bad).all()
    finite = np.isfinite(ref.ref)
    assert (np.abs(out[finite] - ref.ref[finite]) <= oracle.tolerance(ref, 147)[finite]).all()


def run_nhwc(x, w, b, pad):
    import bias_addmm_im2col_amd as baim
    out = baim.conv2d_nhwc(dev(x), dev(w), dev(b), 4, pad, 1)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,H,W,OC,pad,has_bias", SHAPES)
def test_stem_conv_channels_last(B, H, W, OC, pad, has_bias):
    import bias_addmm_im2col_amd as baim
    x, w = gen((B, H, W, 3), 21), gen((OC, 7, 7, 3), 22)
    b = gen((OC,), 23) if has_bias else None
    p = baim.conv2d_nhwc_plan(tuple(x.shape), tuple(w.shape), 4, pad, 1)
    say(f"nhwc x=[{B},{H},{W},3] OC={OC} p={pad} plan {p}")
    assert p["kernel"] == 3
    check_close(run_nhwc(x, w, b, pad), oracle.conv2d_nhwc(x, w, b, 4, pad, 1), 147, 1.0,
                "stem nhwc")
    xi, wi, bi = gen((B, H, W, 3), 24, "I"), gen((OC, 7, 7, 3), 25, "I"), gen((OC,), 26, "I")
    check_bitwise(run_nhwc(xi, wi, bi, pad), oracle.conv2d_nhwc(xi, wi, bi, 4, pad, 1),
                  "stem nhwc integer")


def test_stem_channels_last_matches_the_im2col_kernel_bitwise(monkeypatch):
    """On integer inputs the channels-last stem and the addmm kernels with an
    im2col A operand (BAIM_CONV_WIN=off) both give the exact result, and it
    is the NCHW stem's result transposed."""
    import bias_addmm_im2col_amd as baim
    x, w, b = gen((1, 768, 768, 3), 27, "I"), gen((128, 7, 7, 3), 28, "I"), gen((128,), 29, "I")
    stem = run_nhwc(x, w, b, 3)
    nchw = run(x.permute(0, 3, 1, 2).contiguous(), w.permute(0, 3, 1, 2).contiguous(), b, 3)
    assert (stem == nchw.transpose(0, 2, 3, 1)).all()
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    assert baim.conv2d_nhwc_plan(tuple(x.shape), tuple(w.shape), 4, 3, 1)["kernel"] == 0
    gat = run_nhwc(x, w, b, 3)
    assert (stem == gat).all()


def test_stem_channels_last_nonfinite_input_stays_local():
    """An Inf or NaN in one channel of one column reaches exactly the
    outputs whose taps read it: the interleaved split puts every input
    float in its own channel's slot."""
    x, w, b = gen((1, 600, 580, 3), 30), gen((64, 7, 7, 3), 31), gen((64,), 32)
    x[0, 0, 579, 0] = float("inf")    # last column of the first row, channel 0
    x[0, 599, 0, 2] = float("-inf")   # first column of the last row, channel 2
    x[0, 301, 290, 1] = float("nan")  # an interior pixel, channel 1
    out = run_nhwc(x, w, b, 3)
    ref = oracle.conv2d_nhwc(x, w, b, 4, 3, 1)
    bad = ~np.isfinite(ref.ref)
    assert bad.any() and (~np.isfinite(out) == bad).all()
    finite = np.isfinite(ref.ref)
    assert (np.abs(out[finite] - ref.ref[finite]) <= oracle.tolerance(ref, 147)[finite]).all()
