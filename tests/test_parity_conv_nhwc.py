"""GPU parity of the channels-last conv (conv2d_nhwc_f32) against the fp64
oracle.

The conv page ("et_vk conv2d: route standard (groups==1) conv through an
im2col tiled GEMM", Solution/Constraints) computes the conv as a GEMM with
an implicit im2col operand; channels-last tensors (input [B,H,W,IC], weight
[OC,KH,KW,IC], output [B,OH,OW,OC]) make its K dimension contiguous.
Acceptance: |out - ref| <= 4e-6*sqrt(K)*(sum_k|a*b| + |bias|) elementwise,
K = KH*KW*IC; integer-valued inputs must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from bias_addmm_im2col_amd import inputs as I
from tests import _specs
from tests._parity import check_bitwise, check_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def say(msg):
    print(f"[parity] {msg}", flush=True)


def gen(shape, seed, kind="U"):
    g = torch.Generator("cpu").manual_seed(seed)
    if kind == "U":
        return torch.rand(shape, generator=g) * 2 - 1
    return torch.randint(-4, 5, shape, generator=g).float()


def run(x, w, b, stride=1, pad=0, dil=1):
    import bias_addmm_im2col_amd as baim
    out = baim.conv2d_nhwc(dev(x), dev(w), dev(b), stride, pad, dil)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, dil, bias
    (1, 4, 8, 8, 8, 3, 3, 1, 1, 1, True),
    (2, 3, 33, 31, 20, 7, 7, 4, 3, 1, True),        # IC % 4 != 0: 4-byte gathers
    (2, 64, 14, 15, 96, 3, 3, 1, 1, 1, False),
    (1, 32, 20, 20, 64, 3, 3, 2, 1, 1, True),
    (2, 16, 17, 13, 40, 3, 3, 1, 2, 2, True),       # dilation 2
    (1, 8, 9, 10, 33, 5, 3, (2, 1), (2, 0), (1, 2), True),
    (3, 12, 6, 7, 130, 1, 1, 1, 0, 1, True),        # 1x1
    (1, 128, 28, 28, 128, 3, 3, 1, 1, 1, True),     # several k-tiles per tap
    (1, 5, 40, 40, 7, 3, 3, 1, 1, 1, False),        # IC = 5, K = 45
]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,has_bias", SHAPES)
def test_nhwc_conv_small_full(B, IC, H, W, OC, KH, KW, stride, pad, dil, has_bias):
    say(f"conv2d_nhwc_f32 x=[{B},{H},{W},{IC}] w=[{OC},{KH},{KW},{IC}] s={stride} p={pad} d={dil}")
    x, w = gen((B, H, W, IC), 1), gen((OC, KH, KW, IC), 2)
    b = gen((OC,), 3) if has_bias else None
    check_close(run(x, w, b, stride, pad, dil), oracle.conv2d_nhwc(x, w, b, stride, pad, dil),
                KH * KW * IC, 1.0, f"nhwc {IC}x{KH}x{KW}")


@pytest.mark.parametrize("IC,OC,k,stride", [(4, 8, 3, 1), (3, 16, 7, 2), (64, 64, 3, 1),
                                            (20, 130, 3, 2)])
def test_nhwc_conv_integer_bitwise(IC, OC, k, stride):
    say(f"conv2d_nhwc_f32 integer IC={IC} OC={OC} k={k} s={stride}")
    x, w, b = gen((2, 19, 17, IC), 4, "I"), gen((OC, k, k, IC), 5, "I"), gen((OC,), 6, "I")
    check_bitwise(run(x, w, b, stride, k // 2, 1), oracle.conv2d_nhwc(x, w, b, stride, k // 2, 1),
                  "nhwc integer")


TILE_SPECS = _specs.NHWC_SPECS


@pytest.mark.parametrize("spec", TILE_SPECS)
def test_nhwc_conv_forced_tile_configs(spec, monkeypatch):
    monkeypatch.setenv("BAIM_TILE", spec)
    for (IC, k, stride) in _specs.NHWC_SHAPES:
        say(f"BAIM_TILE={spec} conv2d_nhwc_f32 IC={IC} k={k}")
        x, w, b = gen((2, 21, 18, IC), 7), gen((70, k, k, IC), 8), gen((70,), 9)
        check_close(run(x, w, b, stride, 1, 1), oracle.conv2d_nhwc(x, w, b, stride, 1, 1),
                    k * k * IC, 1.0, f"nhwc {spec}")
    B, H, W, IC, OC = _specs.NHWC_INT_SHAPE
    say(f"BAIM_TILE={spec} conv2d_nhwc_f32 integer x=[{B},{H},{W},{IC}] OC={OC}")
    x, w, b = gen((B, H, W, IC), 10, "I"), gen((OC, 3, 3, IC), 11, "I"), gen((OC,), 12, "I")
    check_bitwise(run(x, w, b, 1, 1, 1), oracle.conv2d_nhwc(x, w, b, 1, 1, 1), f"nhwc int {spec}")


def test_nhwc_conv_unaligned_input_uses_4_byte_gathers():
    import bias_addmm_im2col_amd as baim
    say("conv2d_nhwc_f32 unaligned input")
    x, w, b = gen((2, 12, 11, 8), 13), gen((24, 3, 3, 8), 14), gen((24,), 15)
    buf = torch.empty(x.numel() + 1, device="cuda")
    buf[1:] = dev(x).reshape(-1)
    out = baim.conv2d_nhwc(buf[1:].view(x.shape), dev(w), dev(b), 1, 1, 1)
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), oracle.conv2d_nhwc(x, w, b, 1, 1, 1), 72, 1.0, "nhwc unaligned")


def nhwc_sample(B, OH, OW, OC, n_rand=4096, seed=0):
    """Flat NHWC output indices: every channel at the image corners and
    centre, whole planes of a few channels, random points."""
    g = np.random.default_rng(seed)
    P = OH * OW
    idx = []
    for b in sorted({0, B - 1}):
        for pix in (0, OW - 1, P - OW, P - 1, P // 2):
            idx.append((b * P + pix) * OC + np.arange(OC))
    for b, oc in {(0, 0), (B - 1, OC - 1), (0, min(127, OC - 1)), (B - 1, min(128, OC - 1))}:
        idx.append((b * P + np.arange(P)) * OC + oc)
    idx.append(g.integers(0, B * P * OC, n_rand))
    return np.unique(np.concatenate(idx).astype(np.int64))


@pytest.mark.parametrize("name", list(I.NHWC_CASES))
def test_workload_nhwc_conv(name):
    import bias_addmm_im2col_amd as baim
    c = I.NHWC_CASES[name]
    say(f"workload {name}: conv2d_nhwc_f32")
    x, w, b = I.conv_inputs(c)
    out = baim.conv2d_nhwc(dev(x), dev(w), dev(b), c.stride, c.padding, c.dilation)
    torch.cuda.synchronize()
    OH, OW = c.out_hw()
    idx = nhwc_sample(c.B, OH, OW, c.OC)
    got = out.reshape(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()
    res = oracle.conv2d_nhwc_at(x, w, b, c.stride, c.padding, c.dilation, idx)
    check_close(got, res, c.KH * c.KW * c.IC, 1.0, name)
