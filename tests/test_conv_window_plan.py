"""Host-side routing of conv2d_gemm_f32 (no GPU): which convs take the
LDS-window kernel, how its tiles map to blocks, and that every window shape
of the GPU parity tests really is planned onto it.

The window kernel holds, per input channel, the input rows that a run of 128
output pixels touches (6 rows for a 3x3 stride-1 kernel, 8 at dilation 2,
when OW >= 43) with every column [-pW, W + pW) in a 64-float LDS row; it
loads whole rows with 16-byte loads (W % 4 == 0) and weight rows
K = IC*9 with 16-byte loads (IC % 4 == 0).  Anything else takes the
general implicit-im2col GEMM (kernel 0) or, for grouped convs, the direct
kernels (kernel 2).
"""
import os

import pytest

from bias_addmm_im2col_amd import _capi


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(_capi.LIB_PATH):
        import bias_addmm_im2col_amd.build as b
        b.build()
    return _capi.lib()


def plan(B, IC, H, W, OC, KH=3, KW=3, s=1, p=1, d=1, groups=1, pH=None):
    st, pl = _capi.conv2d_plan(B, IC, H, W, OC, KH, KW, s, s, p if pH is None else pH, p, d, d,
                               groups)
    assert st == 0, _capi.last_error()
    return pl


def test_mid_stage_convs_take_the_window_kernel():
    # [4,256,56,56] x [256,256,3,3]: 4 x 100 tiles of 64 x 128, streamed
    # over one block per CU
    for d in (1, 2):
        pl = plan(4, 256, 56, 56, 256, p=d, d=d)
        assert pl["kernel"] == 1 and pl["stream_blocks"] == 256 and pl["splits"] == 1
        assert (pl["bm"], pl["bn"], pl["bk"], pl["waves"], pl["kgroups"]) == (64, 128, 144, 16, 2)


def test_other_convs_keep_their_kernels():
    assert plan(4, 256, 57, 57, 256, s=2, d=2, p=2)["kernel"] == 0  # stride 2 dilation 2
    assert plan(1, 3, 768, 768, 128, 7, 7, 4, 3)["kernel"] == 3     # the 7x7 stem: its own kernel
    assert plan(2, 16, 40, 42, 64)["kernel"] == 0                   # OW = 42: runs touch 5 rows
    assert plan(2, 16, 40, 44, 64)["kernel"] == 1                   # OW = 44: at most 4
    assert plan(2, 16, 40, 46, 64)["kernel"] == 0                   # W % 4 != 0
    assert plan(2, 18, 40, 48, 64)["kernel"] == 0                   # IC % 4 != 0
    assert plan(2, 16, 40, 64, 64, p=0)["kernel"] == 0              # W + 4 > 64 floats
    assert plan(2, 16, 40, 60, 64, p=0)["kernel"] == 1              # W + 4 = 64: fits
    assert plan(2, 16, 40, 60, 64, p=1)["kernel"] == 0              # W + pW + 4 > 64
    assert plan(2, 16, 40, 48, 64, p=5)["kernel"] == 0              # pW above the 4 pad columns
    assert plan(2, 16, 40, 48, 64, 1, 1, 1, 0)["kernel"] == 0       # 1x1 (not compiled)
    assert plan(2, 16, 40, 48, 64, groups=2)["kernel"] == 0         # grouped: per-group GEMM
    assert plan(2, 16, 40, 48, 16, groups=16)["kernel"] == 2        # depthwise: direct
    assert plan(2, 16, 40, 48, 64, d=3, p=3)["kernel"] == 0         # dilation 3


def test_window_schedules(monkeypatch):
    # few tiles: one per block; 257..511 tiles: stream over 256 blocks
    assert plan(1, 64, 48, 48, 128)["stream_blocks"] == 0           # 2 x 18 tiles
    assert plan(1, 64, 56, 56, 256)["stream_blocks"] == 0           # 4 x 25 tiles
    assert plan(3, 64, 56, 56, 256)["stream_blocks"] == 256         # 4 x 75 tiles
    assert plan(6, 64, 56, 56, 256)["stream_blocks"] == 0           # 4 x 150 tiles
    assert plan(3, 16, 56, 56, 256)["stream_blocks"] == 0           # one k-tile: nothing to split
    monkeypatch.setenv("BAIM_CONV_WIN", "2")
    assert plan(1, 64, 48, 48, 128)["splits"] == 2
    assert plan(1, 16, 48, 48, 128)["splits"] == 1                  # one k-tile
    monkeypatch.setenv("BAIM_CONV_WIN", "s7")
    assert plan(1, 64, 48, 48, 128)["stream_blocks"] == 7
    monkeypatch.setenv("BAIM_CONV_WIN", "s36")                      # not below the 36 tiles
    assert plan(1, 64, 48, 48, 128)["stream_blocks"] == 0
    monkeypatch.setenv("BAIM_CONV_WIN", "tile")
    pl = plan(4, 256, 56, 56, 256)
    assert pl["kernel"] == 1 and pl["stream_blocks"] == 0 and pl["splits"] == 1
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    assert plan(4, 256, 56, 56, 256)["kernel"] == 0


def test_stem_routing(monkeypatch):
    pl = plan(1, 3, 768, 768, 128, 7, 7, 4, 3)
    assert (pl["kernel"], pl["bm"], pl["bn"], pl["bk"], pl["waves"]) == (3, 128, 144, 147, 16)
    assert plan(1, 3, 580, 572, 128, 7, 7, 4, 3)["kernel"] == 0     # OW = 143 < 144
    assert plan(1, 3, 580, 580, 128, 7, 7, 4, 3)["kernel"] == 3     # OW = 145
    assert plan(1, 3, 768, 766, 128, 7, 7, 4, 3)["kernel"] == 0     # W % 4 != 0
    assert plan(1, 3, 768, 768, 126, 7, 7, 4, 3)["kernel"] == 0     # OC % 4 != 0
    assert plan(1, 4, 768, 768, 128, 7, 7, 4, 3)["kernel"] == 0     # 4 channels
    assert plan(1, 3, 768, 768, 128, 7, 7, 2, 3)["kernel"] == 0     # stride 2
    assert plan(1, 3, 768, 768, 128, 5, 5, 4, 2)["kernel"] == 0     # 5x5
    assert plan(1, 3, 768, 768, 128, 7, 7, 4, 3, d=2)["kernel"] == 0
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    assert plan(1, 3, 768, 768, 128, 7, 7, 4, 3)["kernel"] == 0


def test_gpu_stem_shapes_are_planned_onto_the_stem_kernel():
    from tests.test_parity_conv_stem import SHAPES
    for B, H, W, OC, pad, _ in SHAPES:
        pH, pW = (pad, pad) if isinstance(pad, int) else pad
        st, pl = _capi.conv2d_plan(B, 3, H, W, OC, 7, 7, 4, 4, pH, pW, 1, 1, 1)
        assert st == 0 and pl["kernel"] == 3, (B, H, W, OC, pad)


def test_gpu_window_shapes_are_planned_onto_the_window_kernel():
    from tests.test_parity_conv_window import SHAPES
    for B, IC, H, W, OC, pad, dil, _ in SHAPES:
        pH, pW = (pad, pad) if isinstance(pad, int) else pad
        st, pl = _capi.conv2d_plan(B, IC, H, W, OC, 3, 3, 1, 1, pH, pW, dil, dil, 1)
        assert st == 0 and pl["kernel"] == 1, (B, IC, H, W, OC, pad, dil)


def test_invalid_sizes_are_rejected_like_the_op():
    st, _ = _capi.conv2d_plan(1, 4, 5, 5, 8, 7, 7, 1, 1, 0, 0, 1, 1, 1)   # kernel larger than input
    assert st == 2
    st, _ = _capi.conv2d_plan(1, 6, 5, 5, 8, 3, 3, 1, 1, 0, 0, 1, 1, 4)   # groups do not divide
    assert st == 2


def test_stride2_convs_take_the_window_kernel(monkeypatch):
    # [4,256,57,57] s2: OW = 29, runs of 64 pixels touch 4 output rows = 9
    # input rows; 4 x 56 tiles of 64 x 64, one per block
    pl = plan(4, 256, 57, 57, 256, s=2)
    assert pl["kernel"] == 1 and pl["stream_blocks"] == 0 and pl["splits"] == 1
    assert (pl["bm"], pl["bn"], pl["bk"], pl["waves"], pl["kgroups"]) == (64, 64, 144, 16, 4)
    for W in (44, 45, 46, 47, 57, 59):                              # any W % 4 up to 14 quads
        assert plan(1, 16, 40, W, 64, s=2)["kernel"] == 1, W
    assert plan(1, 16, 40, 60, 64, s=2, p=0)["kernel"] == 0         # 15 quads: not compiled
    assert plan(1, 16, 43, 42, 64, s=2)["kernel"] == 1              # OW = 21: 4 output rows
    assert plan(1, 16, 41, 40, 64, s=2)["kernel"] == 0              # OW = 20: 5 rows
    assert plan(1, 18, 40, 57, 64, s=2)["kernel"] == 0              # IC % 4 != 0
    assert plan(4, 256, 57, 57, 256, 1, 1, 2, 0)["kernel"] == 0     # 1x1 stride 2
    # no streamed instance: 257..511 tiles still run one per block
    assert plan(5, 256, 57, 57, 256, s=2)["stream_blocks"] == 0     # 4 x 70 tiles
    monkeypatch.setenv("BAIM_CONV_WIN", "s7")
    assert plan(4, 256, 57, 57, 256, s=2)["stream_blocks"] == 0
    monkeypatch.setenv("BAIM_CONV_WIN", "2")
    assert plan(4, 256, 57, 57, 256, s=2)["splits"] == 2


def nhwc_plan(B, H, W, IC, OC, K=7, s=4, p=3, d=1):
    st, pl = _capi.conv2d_nhwc_plan(B, IC, H, W, OC, K, K, s, s, p, p, d, d)
    assert st == 0, _capi.last_error()
    return pl["kernel"]


def test_channels_last_stem_routing(monkeypatch):
    """conv2d_nhwc_f32 takes the stem kernel under the NCHW stem's
    conditions, and the im2col addmm kernels otherwise."""
    assert nhwc_plan(1, 768, 768, 3, 128) == 3
    assert nhwc_plan(1, 580, 580, 3, 128) == 3      # OW = 145
    assert nhwc_plan(1, 580, 572, 3, 128) == 0      # OW = 143 < 144
    assert nhwc_plan(1, 768, 766, 3, 128) == 0      # W % 4 != 0
    assert nhwc_plan(1, 768, 768, 3, 126) == 0      # OC % 4 != 0
    assert nhwc_plan(1, 768, 768, 4, 128) == 0      # 4 channels
    assert nhwc_plan(1, 768, 768, 3, 128, s=2) == 0
    assert nhwc_plan(1, 768, 768, 3, 128, d=2) == 0
    assert nhwc_plan(2, 21, 18, 16, 70, K=3, s=1, p=1) == 0
    monkeypatch.setenv("BAIM_CONV_WIN", "off")
    assert nhwc_plan(1, 768, 768, 3, 128) == 0


def test_gpu_channels_last_stem_shapes_are_planned_onto_the_stem_kernel():
    from tests.test_parity_conv_stem import SHAPES
    for B, H, W, OC, pad, _ in SHAPES:
        pH, pW = (pad, pad) if isinstance(pad, int) else pad
        st, pl = _capi.conv2d_nhwc_plan(B, 3, H, W, OC, 7, 7, 4, 4, pH, pW, 1, 1)
        assert st == 0 and pl["kernel"] == 3, (B, H, W, OC, pad)


def test_channels_last_plan_rejects_like_the_op():
    st, _ = _capi.conv2d_nhwc_plan(1, 4, 5, 5, 8, 7, 7, 1, 1, 0, 0, 1, 1)  # kernel larger than input
    assert st == 2
    st, _ = _capi.conv2d_nhwc_plan(0, 3, 768, 768, 128, 7, 7, 4, 4, 3, 3, 1, 1)
    assert st == 2
    import ctypes
    assert _capi.lib().baim_conv2d_nhwc_plan(1, 3, 768, 768, 128, 7, 7, 4, 4, 3, 3, 1, 1,
                                             ctypes.cast(None, ctypes.POINTER(ctypes.c_int))) == 1
