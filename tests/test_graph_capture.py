"""GPU: the C-ABI entry points can be captured in a HIP graph.

None of the kernels allocates or clears memory with a memset: the split
schedules initialise `out` with a kernel of their own.  The test captures
one call of each op (including a two-piece stream plan, whose init kernel
is part of the capture, the LDS-window conv and the stem in both layouts), replays the graph three times with eager work and
synchronisations in between, and requires every replay to reproduce the
eager results bit for bit (every path here is deterministic).
"""
import numpy as np
import pytest
import torch

from tests._parity import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def gen(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g)


def test_graph_replays_match_eager():
    import bias_addmm_im2col_amd as baim
    print("[graph] building inputs", flush=True)
    # addmm on the 3x3 conv's GEMM shape: planned as stream pieces with the
    # two-piece exchange (init kernel + GEMM kernel)
    a, b, s = dev(gen((256, 2304), 1)), dev(gen((2304, 12544), 2)), dev(gen((12544,), 3))
    plan = baim.gemm_plan(256, 12544, 2304)
    assert plan["stream_blocks"] > 0, plan
    x, w, bias = dev(gen((2, 64, 28, 28), 4)), dev(gen((64, 64, 3, 3), 5)), dev(gen((64,), 6))
    xd, wd = dev(gen((2, 64, 28, 28), 7)), dev(gen((64, 1, 3, 3), 8))
    lx, lw = dev(gen((300, 128), 9)), dev(gen((96, 128), 10))
    q, k, v = dev(gen((2, 4, 100, 64), 11)), dev(gen((2, 4, 150, 64), 12)), dev(gen((2, 4, 150, 64), 13))
    tx, tw = dev(gen((2, 32, 10, 10), 14)), dev(gen((32, 16, 4, 4), 15))
    # the LDS-window conv (3x3, OW 44), the stem in both layouts
    wx, ww = dev(gen((1, 16, 40, 44), 16)), dev(gen((64, 16, 3, 3), 17))
    sx, sw, sb = dev(gen((1, 3, 600, 580), 18)), dev(gen((64, 3, 7, 7), 19)), dev(gen((64,), 20))
    nx, nw = dev(gen((1, 600, 580, 3), 21)), dev(gen((64, 7, 7, 3), 22))
    assert baim.conv2d_plan(tuple(wx.shape), tuple(ww.shape), 1, 1, 1)["kernel"] == 1
    assert baim.conv2d_plan(tuple(sx.shape), tuple(sw.shape), 4, 3, 1)["kernel"] == 3
    assert baim.conv2d_nhwc_plan(tuple(nx.shape), tuple(nw.shape), 4, 3, 1)["kernel"] == 3
    outs = [torch.empty(256, 12544, device="cuda"), torch.empty(2, 64, 28, 28, device="cuda"),
            torch.empty(2, 64, 28, 28, device="cuda"), torch.empty(300, 96, device="cuda"),
            torch.empty(2, 4, 100, 64, device="cuda"), torch.empty(2, 16, 20, 20, device="cuda"),
            torch.empty(1, 64, 40, 44, device="cuda"), torch.empty(1, 64, 150, 145, device="cuda"),
            torch.empty(1, 150, 145, 64, device="cuda")]

    def ops():
        baim.addmm_f32(outs[0], s, a, b, 0.5, 2.0)
        baim.conv2d_gemm_f32(outs[1], x, w, bias, 1, 1, 1, 1)
        baim.conv2d_gemm_f32(outs[2], xd, wd, bias, 1, 1, 1, 64)
        baim.linear_f32(outs[3], lx, lw, None)
        baim.sdpa_f32(outs[4], q, k, v)
        baim.conv_transpose2d_f32(outs[5], tx, tw, None, 2, 1)
        baim.conv2d_gemm_f32(outs[6], wx, ww, None, 1, 1, 1, 1)
        baim.conv2d_gemm_f32(outs[7], sx, sw, sb, 4, 3, 1, 1)
        baim.conv2d_nhwc_f32(outs[8], nx, nw, sb, 4, 3, 1)

    print(f"[graph] eager (addmm plan {plan})", flush=True)
    ops()
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().copy() for o in outs]
    for o in outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()

    print("[graph] capture", flush=True)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ops()
    torch.cuda.synchronize()
    for r in range(3):
        print(f"[graph] replay {r}", flush=True)
        for o in outs:
            o.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda") * 2.0  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del scratch
        for i, (o, e) in enumerate(zip(outs, eager)):
            got = o.cpu().numpy()
            assert (got.view(np.uint32) == e.view(np.uint32)).all(), f"replay {r}, op {i} differs"
