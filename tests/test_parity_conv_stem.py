"""GPU parity of the stem kernel (3-channel 7x7 stride-4 convs) against the
fp64 oracle, through conv2d_gemm_f32.

The kernel copies the weights and the input columns a block's 144 output
pixels read into LDS once and runs all of K = 147 from there; what it must
get right is the phase-row layout of the input (columns split by residue
mod 4), pixel runs that continue on the next output row or end past the
image, padding on every side, output channels past a multiple of 128 and
the zero-weight padded tap.  Every case first checks through
baim_conv2d_plan that the stem kernel really is what runs.  Acceptance as
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
