"""Every forced tile spec the GPU parity tests use changes what the library
runs on at least one of that test's shapes (host only: the library's own
planner through ``baim_gemm_plan``).

A spec the planner cannot honour (a schedule not compiled for that
configuration, a worker count not below the tile count, more slices than
k-tiles) falls back to something else; a spec that falls back on every
shape of its test would add no coverage.  The launchers change a plan in two
documented ways, which the check applies too: the stream schedule needs
16-byte operand loads, and the channels-last conv runs the 16-wave 128x128
tile's 4-byte gathers on the 8-wave 128x128 tile.
"""
import os

import pytest

from bias_addmm_im2col_amd import _capi
from tests import _specs

CFG = {  # bm, bn, bk, waves
    0: (128, 128, 32, 8), 1: (128, 64, 32, 8), 2: (64, 128, 32, 8), 3: (64, 64, 32, 4),
    4: (128, 128, 64, 16), 5: (128, 64, 64, 16), 6: (64, 64, 64, 8), 7: (64, 64, 128, 16),
    8: (32, 128, 32, 4), 9: (256, 256, 16, 8)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_capi.LIB_PATH):
        import bias_addmm_im2col_amd.build as b
        b.build()
    return _capi.lib()


def parse(spec):
    cfg, _, rest = spec.partition(",")
    if not rest:
        return int(cfg), "tile", 1
    if rest.startswith("s"):
        return int(cfg), "stream", int(rest[1:])
    return int(cfg), "slices", int(rest)


def effective(spec, M, N, K, vec, nhwc, monkeypatch):
    """(cfg tuple, splits, stream blocks) the launcher runs for this call."""
    monkeypatch.setenv("BAIM_TILE", spec)
    st, p = _capi.gemm_plan(M, N, K)
    assert st == 0
    tile = (p["bm"], p["bn"], p["bk"], p["waves"])
    splits, stream = p["splits"], p["stream_blocks"]
    if stream and not vec:
        splits, stream = 1, 0
    if nhwc and not vec and tile == CFG[4]:
        monkeypatch.setenv("BAIM_TILE", "0")
        st, p = _capi.gemm_plan(M, N, K)
        tile, splits, stream = (p["bm"], p["bn"], p["bk"], p["waves"]), p["splits"], p["stream_blocks"]
    return tile, splits, stream


CASES = ([("addmm", s) for s in _specs.ADDMM_SPECS] + [("linear", s) for s in _specs.GEMM_SPECS] +
         [("conv", s) for s in _specs.GEMM_SPECS] + [("nhwc", s) for s in _specs.NHWC_SPECS])
GEMMS = {"addmm": _specs.addmm_gemms, "linear": _specs.linear_gemms, "conv": _specs.conv_gemms,
         "nhwc": _specs.nhwc_gemms}


@pytest.mark.parametrize("op,spec", CASES)
def test_forced_spec_takes_effect(lib, op, spec, monkeypatch):
    cfg, mode, n = parse(spec)
    runs = [effective(spec, M, N, K, vec, op == "nhwc", monkeypatch)
            for M, N, K, vec in GEMMS[op]()]
    ok = [r for r in runs if r[0] == CFG[cfg]]
    assert ok, f"{op} {spec}: configuration {cfg} never runs: {runs}"
    if mode == "stream":
        assert any(r[2] == n for r in ok), f"{op} {spec}: never streamed over {n} blocks: {runs}"
    elif mode == "slices":
        assert any(r[1] == min(n, 8) or (n > 8 and r[1] >= 2) for r in ok), \
            f"{op} {spec}: never split into {n} slices: {runs}"
    else:
        assert any(r[1] == 1 and r[2] == 0 for r in ok)


def test_spec_lists_hold_the_dominant_conv_instance():
    # the 3x3 mid-stage convs stream configuration 5 over 256 blocks; its
    # split forms must be in both lists
    for lst in (_specs.GEMM_SPECS, _specs.NHWC_SPECS):
        for s in ("5,s7", "5,s13", "5,2", "5,3"):
            assert s in lst


def plan_tile(M, N, K):
    st, p = _capi.gemm_plan(M, N, K)
    assert st == 0
    return p["bm"], p["bn"], p["bk"], p["waves"]


def test_large_gemms_take_the_256_tile(lib, monkeypatch):
    monkeypatch.delenv("BAIM_TILE", raising=False)
    big = CFG[9]
    assert plan_tile(4096, 4096, 1024) == big       # up-proj: 256 tiles, one per CU
    assert plan_tile(4096, 4096, 4096) == big
    assert plan_tile(8192, 8192, 512) == big        # 1024 tiles
    assert plan_tile(4000, 4096, 1024) == big       # ragged rows: still 256 tiles
    assert plan_tile(4096, 1024, 4096) != big       # down-proj: 64 tiles
    assert plan_tile(4096, 4096, 256) != big        # K below 512
    assert plan_tile(4096, 4352, 1024) != big       # 272 tiles: a second round mostly idle
    assert plan_tile(2048, 3072, 768) != big        # FFN: 96 tiles


def test_conv_paths_never_run_the_256_tile(lib, monkeypatch):
    """The im2col conv kernels are not compiled with the 256x256 tile: a
    plan (or a forced spec) for it becomes the 128x128 tile."""
    for spec in ("", "9"):
        monkeypatch.setenv("BAIM_TILE", spec)
        # a 1x1 conv with M = 512, N = 64*56*56, K = 512: 1568 tiles of 256x256
        st, p = _capi.conv2d_plan(64, 512, 56, 56, 512, 1, 1, 1, 1, 0, 0, 1, 1, 1)
        assert st == 0 and p["kernel"] == 0
        assert (p["bm"], p["bn"], p["bk"], p["waves"]) == CFG[0]


def test_forced_256_tile_respects_its_32_bit_offsets(lib, monkeypatch):
    """The 256x256 kernel addresses all of mat2 [K, N] and a 256-row panel
    of mat1 with 32-bit offsets: forced where K*N or 256*K reaches 2^29,
    the plan (as addmm_f32 launches it) is the 128x128 tile instead."""
    monkeypatch.setenv("BAIM_TILE", "9")
    assert plan_tile(512, 4096, 1024) == CFG[9]
    assert plan_tile(512, 4096, 1 << 17) == CFG[0]          # K*N = 2^29
    assert plan_tile(512, 64, 1 << 21) == CFG[0]            # 256*K = 2^29
