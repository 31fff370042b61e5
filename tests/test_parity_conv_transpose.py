"""GPU parity of the transposed conv (conv_transpose2d_f32) against the fp64
oracle.

The conv page keeps transposed convs on their own gather kernels; the
operation is the adjoint of conv2d (aten's conv_transpose2d, weight
[IC, OC/groups, KH, KW]).  Acceptance: |out - ref| <=
4e-6*sqrt(K)*(sum|x*w| + |bias|) elementwise with K = (IC/groups)*KH*KW
(an upper bound on the taps of any output); integer-valued inputs must
match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from bias_addmm_im2col_amd import inputs as I
from tests._parity import check_bitwise, check_close, conv_sample, dev

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


def run(x, w, b, stride=1, pad=0, opad=0, groups=1, dil=1):
    import bias_addmm_im2col_amd as baim
    out = baim.conv_transpose2d(dev(x), dev(w), dev(b), stride, pad, opad, groups, dil)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, out_pad, dil, bias
    (1, 4, 5, 5, 8, 3, 3, 1, 0, 0, 1, True),
    (2, 16, 9, 7, 12, 4, 4, 2, 1, 0, 1, True),          # 2x upsampling
    (2, 8, 6, 6, 5, 2, 2, 2, 0, 0, 1, False),           # 2x2 / stride 2: one tap per phase
    (1, 6, 7, 5, 9, 3, 3, 2, 1, 1, 1, True),            # output padding
    (1, 5, 6, 8, 7, 3, 2, (3, 2), (1, 0), (2, 1), (1, 2), True),
    (2, 3, 5, 4, 4, 5, 3, 3, 2, (2, 0), 2, True),       # dilation 2 with stride 3
    (1, 32, 10, 11, 70, 3, 3, 2, 1, 1, 1, True),
    (1, 4, 4, 4, 3, 1, 1, 3, 0, 2, 1, True),            # 1x1 / stride 3: phases with no taps
    (1, 64, 12, 12, 130, 4, 4, 2, 1, 0, 1, True),       # several k-tiles and m-tiles
    (1, 2, 3, 3, 2, 3, 3, 5, 0, 0, 1, True),            # stride 5: 25 phases (two launches)
]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,opad,dil,has_bias", SHAPES)
def test_convt_small_full(B, IC, H, W, OC, KH, KW, stride, pad, opad, dil, has_bias):
    say(f"conv_transpose2d_f32 x=[{B},{IC},{H},{W}] w=[{IC},{OC},{KH},{KW}] s={stride} "
        f"p={pad} op={opad} d={dil}")
    x, w = gen((B, IC, H, W), 1), gen((IC, OC, KH, KW), 2)
    b = gen((OC,), 3) if has_bias else None
    check_close(run(x, w, b, stride, pad, opad, 1, dil),
                oracle.conv_transpose2d(x, w, b, stride, pad, dil, opad), IC * KH * KW, 1.0,
                f"convT {IC}x{KH}x{KW}")


@pytest.mark.parametrize("groups,IC,OC", [(2, 8, 6), (4, 16, 16), (8, 8, 8)])
def test_convt_grouped(groups, IC, OC):
    say(f"conv_transpose2d_f32 groups={groups} IC={IC} OC={OC}")
    x, w, b = gen((2, IC, 7, 6), 4), gen((IC, OC // groups, 3, 3), 5), gen((OC,), 6)
    check_close(run(x, w, b, 2, 1, 1, groups), oracle.conv_transpose2d(x, w, b, 2, 1, 1, 1, groups),
                IC // groups * 9, 1.0, f"convT groups {groups}")


@pytest.mark.parametrize("stride,k", [(1, 3), (2, 4), (2, 2), (3, 3)])
def test_convt_integer_bitwise(stride, k):
    say(f"conv_transpose2d_f32 integer s={stride} k={k}")
    x, w, b = gen((2, 24, 9, 10), 7, "I"), gen((24, 40, k, k), 8, "I"), gen((40,), 9, "I")
    check_bitwise(run(x, w, b, stride, 1 if k > 2 else 0),
                  oracle.conv_transpose2d(x, w, b, stride, 1 if k > 2 else 0, 1, 0),
                  f"convT integer s={stride}")


@pytest.mark.parametrize("spec", ["0", "1", "2", "3", "4", "5", "6", "7", "8"])
def test_convt_forced_tile_configs(spec, monkeypatch):
    monkeypatch.setenv("BAIM_TILE", spec)
    say(f"BAIM_TILE={spec} conv_transpose2d_f32")
    x, w, b = gen((2, 20, 9, 8), 10), gen((20, 70, 4, 4), 11), gen((70,), 12)
    check_close(run(x, w, b, 2, 1, 1), oracle.conv_transpose2d(x, w, b, 2, 1, 1, 1), 20 * 16, 1.0,
                f"convT {spec}")
    x, w, b = gen((1, 16, 6, 7), 13, "I"), gen((16, 33, 3, 3), 14, "I"), gen((33,), 15, "I")
    check_bitwise(run(x, w, b, 2, 1, 1), oracle.conv_transpose2d(x, w, b, 2, 1, 1, 1),
                  f"convT int {spec}")


@pytest.mark.parametrize("spec", ["2,2", "2,3", "0,2", "3,4", "7,2", "8,3"])
def test_convt_k_slices(spec, monkeypatch):
    """K split over blocks that add into an output pre-filled with the bias:
    several phases, a phase with no taps (1x1 kernel, stride 3), groups, and
    more slices than some phases have k-tiles."""
    monkeypatch.setenv("BAIM_TILE", spec)
    for (B, IC, H, W, OC, KH, KW, stride, pad, opad, groups, dil) in [
            (2, 64, 9, 7, 40, 4, 4, 2, 1, 0, 1, 1),
            (1, 48, 5, 6, 33, 3, 3, 2, 1, 1, 1, 1),
            (1, 96, 4, 4, 20, 1, 1, 3, 0, 2, 1, 1),
            (2, 64, 6, 5, 32, 3, 3, 2, 1, 1, 4, 1),
            (1, 40, 7, 7, 24, 3, 3, (3, 2), 2, (2, 1), 1, (1, 2))]:
        say(f"BAIM_TILE={spec} conv_transpose2d_f32 x=[{B},{IC},{H},{W}] OC={OC} k=({KH},{KW}) "
            f"s={stride} p={pad} op={opad} g={groups} d={dil}")
        x, w = gen((B, IC, H, W), 16), gen((IC, OC // groups, KH, KW), 17)
        b = gen((OC,), 18)
        ref = oracle.conv_transpose2d(x, w, b, stride, pad, dil, opad, groups)
        check_close(run(x, w, b, stride, pad, opad, groups, dil), ref, IC // groups * KH * KW, 1.0,
                    f"convT slices {spec}")
        xi, wi = gen((B, IC, H, W), 19, "I"), gen((IC, OC // groups, KH, KW), 20, "I")
        refi = oracle.conv_transpose2d(xi, wi, None, stride, pad, dil, opad, groups)
        check_bitwise(run(xi, wi, None, stride, pad, opad, groups, dil), refi,
                      f"convT slices integer {spec}")


@pytest.mark.parametrize("B,IC,H,OC,k,stride,pad", [(1, 512, 7, 256, 4, 2, 1), (1, 256, 14, 40, 3, 2, 1),
                                                  (2, 1024, 4, 24, 4, 2, 1)])
def test_convt_small_grid_deep_k(B, IC, H, OC, k, stride, pad):
    """Shapes whose tiles leave most CUs idle: the planner splits K itself."""
    say(f"conv_transpose2d_f32 small grid x=[{B},{IC},{H},{H}] OC={OC} k={k} s={stride} p={pad}")
    x, w, b = gen((B, IC, H, H), 21), gen((IC, OC, k, k), 22), gen((OC,), 23)
    check_close(run(x, w, b, stride, pad), oracle.conv_transpose2d(x, w, b, stride, pad, 1, 0),
                IC * k * k, 1.0, "convT small grid")
    xi, wi, bi = gen((B, IC, H, H), 24, "I"), gen((IC, OC, k, k), 25, "I"), gen((OC,), 26, "I")
    check_bitwise(run(xi, wi, bi, stride, pad), oracle.conv_transpose2d(xi, wi, bi, stride, pad, 1, 0),
                  "convT small grid integer")


@pytest.mark.parametrize("name", list(I.CONVT_CASES))
def test_workload_convt(name):
    import bias_addmm_im2col_amd as baim
    c = I.CONVT_CASES[name]
    say(f"workload {name}: conv_transpose2d_f32")
    x, w, b = I.convt_inputs(c)
    out = baim.conv_transpose2d(dev(x), dev(w), dev(b), c.stride, c.padding, c.output_padding, 1,
                                c.dilation)
    torch.cuda.synchronize()
    OH, OW = c.out_hw()
    idx = conv_sample(c.B, c.OC, OH, OW)
    got = out.reshape(-1)[torch.from_numpy(idx).cuda()].cpu().numpy()
    res = oracle.conv_transpose2d_at(x, w, b, c.stride, c.padding, c.dilation, c.output_padding, idx)
    check_close(got, res, c.IC * c.KH * c.KW, 1.0, name)


UNIT_SHAPES = [
    # B, IC, H, W, OC, k, stride, groups: kernel = stride, no padding, H*W % 4 == 0
    (2, 40, 8, 6, 70, 2, 2, 1),     # a partial k-tile (40 = 32 + 8), ragged output channels
    (1, 64, 12, 16, 33, 3, 3, 1),   # 3x3 / stride 3: nine single-tap phases
    (2, 32, 8, 8, 48, 2, 2, 4),     # four groups of 8 -> 12 channels
    (3, 24, 4, 5, 20, 2, 2, 1),     # images of 20 pixels: quads stay inside one image
]


@pytest.mark.parametrize("spec", ["", "0", "2", "3", "7", "8", "2,2", "3,3"])
@pytest.mark.parametrize("B,IC,H,W,OC,k,stride,groups", UNIT_SHAPES)
def test_convt_single_tap_phases(B, IC, H, W, OC, k, stride, groups, spec, monkeypatch):
    """Kernel equal to the stride and no padding: every phase is one tap over
    the input grid, and B loads as 16-byte quads of output pixels.  Checked
    against the oracle, and bit for bit on integers against the table-driven
    gathers (BAIM_CONVT_UNIT=off)."""
    if spec:
        monkeypatch.setenv("BAIM_TILE", spec)
    say(f"BAIM_TILE={spec!r} conv_transpose2d_f32 single-tap x=[{B},{IC},{H},{W}] OC={OC} "
        f"k={k} s={stride} g={groups}")
    x, w, b = gen((B, IC, H, W), 31), gen((IC, OC // groups, k, k), 32), gen((OC,), 33)
    check_close(run(x, w, b, stride, 0, 0, groups),
                oracle.conv_transpose2d(x, w, b, stride, 0, 1, 0, groups), IC // groups * k * k,
                1.0, f"convT single-tap {spec}")
    xi, wi, bi = (gen((B, IC, H, W), 34, "I"), gen((IC, OC // groups, k, k), 35, "I"),
                  gen((OC,), 36, "I"))
    fast = run(xi, wi, bi, stride, 0, 0, groups)
    check_bitwise(fast, oracle.conv_transpose2d(xi, wi, bi, stride, 0, 1, 0, groups),
                  f"convT single-tap integer {spec}")
    monkeypatch.setenv("BAIM_CONVT_UNIT", "off")
    assert (run(xi, wi, bi, stride, 0, 0, groups) == fast).all()


FUSED_SHAPES = [
    # B, IC, H, W, OC, (KH, KW), groups: kernel = stride, no padding, H*W % 128 == 0
    (2, 40, 16, 8, 70, (2, 2), 1),   # M = 280 rows in three 128-row tiles, K = 40
    (1, 96, 8, 32, 48, (2, 2), 2),   # two groups: M = 96 (the 64-row tile), K = 48
    (2, 64, 16, 16, 32, (3, 3), 1),  # 3x3 / stride 3: M = 288
    (1, 24, 32, 8, 20, (2, 4), 1),   # kernel 2x4 / stride (2, 4): the (kh, kw) decode
    (4, 256, 16, 16, 64, (2, 2), 1), # the upsampling's channels at a smaller image
]


@pytest.mark.parametrize("B,IC,H,W,OC,k,groups", FUSED_SHAPES)
def test_convt_fused_phases(B, IC, H, W, OC, k, groups, monkeypatch):
    """Kernel equal to the stride, no padding, whole 128-pixel tiles per
    image: all phases in one GEMM (rows (oc, kh, kw), the weight read as its
    transpose).  Checked against the oracle, and bit for bit on integers
    against the per-phase path (BAIM_CONVT_UNIT=off)."""
    KH, KW = k
    say(f"conv_transpose2d_f32 fused x=[{B},{IC},{H},{W}] OC={OC} k={k} g={groups}")
    x, w, b = gen((B, IC, H, W), 41), gen((IC, OC // groups, KH, KW), 42), gen((OC,), 43)
    check_close(run(x, w, b, k, 0, 0, groups),
                oracle.conv_transpose2d(x, w, b, k, 0, 1, 0, groups), IC // groups * KH * KW,
                1.0, "convT fused")
    xi, wi, bi = (gen((B, IC, H, W), 44, "I"), gen((IC, OC // groups, KH, KW), 45, "I"),
                  gen((OC,), 46, "I"))
    fused = run(xi, wi, bi, k, 0, 0, groups)
    check_bitwise(fused, oracle.conv_transpose2d(xi, wi, bi, k, 0, 1, 0, groups),
                  "convT fused integer")
    monkeypatch.setenv("BAIM_CONVT_UNIT", "off")
    assert (run(xi, wi, bi, k, 0, 0, groups) == fused).all()


def test_convt_fused_output_padding_falls_back():
    """Output padding adds rows that no tap reaches (bias only): such convs
    keep the per-phase path, and still match the oracle."""
    x, w, b = gen((1, 16, 8, 16), 47), gen((16, 12, 2, 2), 48), gen((12,), 49)
    check_close(run(x, w, b, 2, 0, 1), oracle.conv_transpose2d(x, w, b, 2, 0, 1, 1), 16 * 4, 1.0,
                "convT output padding")


def test_convt_fused_with_an_output_off_8_byte_alignment():
    """An output that starts 4 bytes past an 8-byte boundary cannot take the
    fused path's 8-byte stores: the per-phase path runs, with the same
    result."""
    import bias_addmm_im2col_amd as baim
    x, w, b = gen((2, 32, 16, 8), 50, "I"), gen((32, 16, 2, 2), 51, "I"), gen((16,), 52, "I")
    ref = oracle.conv_transpose2d(x, w, b, 2, 0, 1, 0)
    buf = torch.empty(2 * 16 * 32 * 16 + 1, dtype=torch.float32, device="cuda")
    out = buf[1:].view(2, 16, 32, 16)
    assert out.data_ptr() % 8 == 4
    baim.conv_transpose2d_f32(out, dev(x), dev(w), dev(b), 2, 0, 0)
    torch.cuda.synchronize()
    check_bitwise(out.cpu().numpy(), ref, "convT fused, offset output")
    assert (out.cpu().numpy() == run(x, w, b, 2, 0, 0)).all()
