"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Acceptance: |out - ref| <= 4e-6*sqrt(K)*(|alpha|*sum_k|a*b| + |beta*self|)
elementwise; integer-valued inputs (every partial sum an integer below
2^24, so every fp32 summation order is exact) must match bit for bit.
Definitions: "[ExecuTorch][WebGPU] Add optimized addmm op" (Solution) and
"et_vk conv2d: route standard (groups==1) conv through an im2col tiled GEMM"
(Solution/Implementation).
"""
import numpy as np
import pytest
import torch

import oracle
from bias_addmm_im2col_amd import inputs as I
from tests import _specs
from tests._parity import addmm_sample, check_bitwise, check_close, conv_sample, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    import bias_addmm_im2col_amd  # noqa: F401  (fails loudly if not built)
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def say(msg):
    print(f"[parity] {msg}", flush=True)


def gen(shape, seed, kind="U"):
    g = torch.Generator("cpu").manual_seed(seed)
    if kind == "U":
        return torch.rand(shape, generator=g) * 2 - 1
    if kind == "I":
        return torch.randint(-4, 5, shape, generator=g).float()
    raise ValueError(kind)


def run_addmm(a, b, s, beta, alpha):
    import bias_addmm_im2col_amd as baim
    out = baim.addmm(dev(s), dev(a), dev(b), beta=beta, alpha=alpha)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_conv(x, w, bias, stride, pad, dil):
    import bias_addmm_im2col_amd as baim
    out = baim.conv2d(dev(x), dev(w), dev(bias), stride, pad, dil)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ------------------------------------------------------------ addmm, small

ADDMM_SHAPES = [
    # M, K, N, self_2d, beta, alpha
    (1, 1, 1, False, 1.0, 1.0),
    (3, 5, 7, True, 0.5, 2.0),
    (64, 96, 80, False, 1.0, 1.0),
    (128, 32, 128, False, 1.0, 1.0),
    (127, 33, 129, True, 1.0, -1.0),
    (129, 31, 257, False, 2.0, 0.5),
    (257, 64, 130, True, -0.5, 1.5),
    (200, 300, 300, False, 1.0, 1.0),
    (131, 1, 67, False, 1.0, 1.0),
    (300, 517, 100, True, 0.25, 1.0),
    (256, 256, 512, False, 1.0, 1.0),
    (37, 1000, 41, True, 1.0, 1.0),
    (32, 600, 1000, True, 1.0, 1.0),     # M <= 32: 32-row tiles
    (7, 4096, 300, False, 1.0, 2.0),     # M <= 32, deep K: 32-row tiles in K slices
]


@pytest.mark.parametrize("M,K,N,self_2d,beta,alpha", ADDMM_SHAPES)
def test_addmm_small_full(M, K, N, self_2d, beta, alpha):
    say(f"addmm_f32 M={M} K={K} N={N} self_2d={self_2d} beta={beta} alpha={alpha}")
    a, b = gen((M, K), 1), gen((K, N), 2)
    s = gen((M, N) if self_2d else (N,), 3)
    out = run_addmm(a, b, s, beta, alpha)
    res = oracle.addmm(a, b, s, self_2d, beta, alpha)
    check_close(out, res, K, alpha, f"addmm {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,self_2d", [(64, 96, 80, False), (129, 257, 131, True),
                                           (256, 1024, 384, False), (77, 4096, 65, True)])
def test_addmm_integer_bitwise(M, K, N, self_2d):
    """P-7: small-integer inputs, power-of-two alpha/beta: bit-exact."""
    say(f"addmm_f32 integer M={M} K={K} N={N}")
    a, b = gen((M, K), 4, "I"), gen((K, N), 5, "I")
    s = gen((M, N) if self_2d else (N,), 6, "I")
    out = run_addmm(a, b, s, 0.5, 2.0)
    check_bitwise(out, oracle.addmm(a, b, s, self_2d, 0.5, 2.0), "addmm integer")


def test_addmm_alpha_zero_is_beta_self_exactly():
    say("addmm_f32 alpha=0")
    a, b, s = gen((70, 50), 7), gen((50, 90), 8), gen((70, 90), 9)
    out = run_addmm(a, b, s, 0.75, 0.0)
    check_bitwise(out, oracle.addmm(a, b, s, True, 0.75, 0.0), "alpha=0")


def test_addmm_identity_mat2():
    say("addmm_f32 identity mat2")
    a, s = gen((100, 64), 10), gen((64,), 11)
    out = run_addmm(a, torch.eye(64), s, 0.5, 4.0)
    check_bitwise(out, oracle.addmm(a, torch.eye(64), s, False, 0.5, 4.0), "identity")


def test_addmm_beta_zero_ignores_nan_self():
    import bias_addmm_im2col_amd as baim
    say("addmm_f32 beta=0, NaN self")
    a, b = gen((40, 24), 12), gen((24, 36), 13)
    s = torch.full((36,), float("nan"))
    out = baim.addmm(dev(s), dev(a), dev(b), beta=0, alpha=1.5).cpu().numpy()
    assert np.isfinite(out).all()
    check_close(out, oracle.addmm(a, b, s, False, 0.0, 1.5), 24, 1.5, "beta=0")
    out2 = baim.addmm(None, dev(a), dev(b), beta=0, alpha=1.5).cpu().numpy()
    assert np.array_equal(out, out2)


def test_addmm_k0_and_empty():
    import bias_addmm_im2col_amd as baim
    say("addmm_f32 K=0 / M=0 / N=0")
    s = gen((5, 6), 14)
    out = baim.addmm(dev(s), torch.zeros(5, 0).cuda(), torch.zeros(0, 6).cuda(), beta=2.0)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), 2.0 * s.numpy())
    e = baim.addmm(torch.zeros(6).cuda(), torch.zeros(0, 3).cuda(), torch.zeros(3, 6).cuda())
    assert tuple(e.shape) == (0, 6)
    e = baim.addmm(torch.zeros(0).cuda(), torch.zeros(4, 3).cuda(), torch.zeros(3, 0).cuda())
    assert tuple(e.shape) == (4, 0)


def test_addmm_self_row_shape_and_unaligned_operands():
    """self given as [1,N]; mat1/mat2 starting 4 bytes into an allocation
    (forces the scalar-load variant)."""
    import bias_addmm_im2col_amd as baim
    say("addmm_f32 self [1,N], unaligned operands")
    M, K, N = 150, 68, 132
    a, b, s = gen((M, K), 15), gen((K, N), 16), gen((1, N), 17)
    abuf = torch.empty(M * K + 1, device="cuda")
    abuf[1:] = dev(a).reshape(-1)
    bbuf = torch.empty(K * N + 1, device="cuda")
    bbuf[1:] = dev(b).reshape(-1)
    out = baim.addmm(dev(s), abuf[1:].view(M, K), bbuf[1:].view(K, N))
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), oracle.addmm(a, b, s.reshape(-1), False), K, 1.0, "unaligned")


# ----------------------------------------------------------- conv, small

CONV_SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, dil, bias
    (1, 1, 5, 5, 1, 3, 3, 1, 0, 1, True),
    (2, 3, 17, 19, 8, 3, 3, 1, 1, 1, True),
    (1, 3, 64, 64, 16, 7, 7, 4, 3, 1, True),
    (2, 16, 14, 14, 32, 3, 3, 1, 2, 2, False),
    (2, 16, 15, 15, 24, 3, 3, 2, 1, 1, True),
    (3, 5, 11, 13, 130, 2, 3, (2, 1), (0, 2), (1, 2), True),
    (1, 64, 9, 9, 129, 1, 1, 1, 0, 1, True),
    (2, 32, 20, 12, 64, 5, 5, (1, 2), (2, 1), (2, 1), True),
    (1, 8, 40, 40, 200, 3, 3, 3, 1, 1, True),
]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,has_bias", CONV_SHAPES)
def test_conv_small_full(B, IC, H, W, OC, KH, KW, stride, pad, dil, has_bias):
    say(f"conv2d_gemm_f32 x=[{B},{IC},{H},{W}] w=[{OC},{IC},{KH},{KW}] s={stride} p={pad} d={dil}")
    x, w = gen((B, IC, H, W), 20), gen((OC, IC, KH, KW), 21)
    bias = gen((OC,), 22) if has_bias else None
    out = run_conv(x, w, bias, stride, pad, dil)
    res = oracle.conv2d(x, w, bias, stride, pad, dil)
    check_close(out, res, IC * KH * KW, 1.0, "conv")


@pytest.mark.parametrize("stride,pad,dil", [(1, 1, 1), (1, 2, 2), (2, 1, 1), (4, 3, 1)])
def test_conv_integer_bitwise(stride, pad, dil):
    say(f"conv2d_gemm_f32 integer s={stride} p={pad} d={dil}")
    x, w, bias = gen((2, 24, 23, 21), 23, "I"), gen((136, 24, 3, 3), 24, "I"), gen((136,), 25, "I")
    out = run_conv(x, w, bias, stride, pad, dil)
    check_bitwise(out, oracle.conv2d(x, w, bias, stride, pad, dil), "conv integer")


# Output rows a multiple of 4 wide (whole 16-byte groups of output columns),
# pads up to 6 on 4-wide rows, one-row inputs and a 64-float input, where
# every tap row is the first or last row of the tensor.
ROW4_SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, dil, bias
    (1, 4, 4, 4, 3, 3, 3, 1, 1, 1, True),
    (2, 8, 12, 16, 40, 3, 3, 1, 1, 1, True),
    (1, 4, 6, 8, 9, 3, 3, 1, 2, 2, False),
    (2, 12, 9, 20, 70, 5, 5, 1, 2, 1, True),
    (1, 16, 7, 4, 33, 1, 7, 1, (0, 3), 1, True),
    (3, 20, 5, 12, 136, 3, 5, 1, (1, 2), 1, True),
    (1, 4, 1, 8, 5, 1, 3, 1, (0, 1), 1, True),
    (2, 8, 15, 12, 24, 3, 3, (2, 1), 1, 1, True),
    (1, 4, 3, 4, 8, 1, 9, 1, (0, 6), 1, True),
]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,has_bias", ROW4_SHAPES)
def test_conv_rows_of_four(B, IC, H, W, OC, KH, KW, stride, pad, dil, has_bias):
    say(f"conv2d_gemm_f32 x=[{B},{IC},{H},{W}] w=[{OC},{IC},{KH},{KW}] s={stride} p={pad} d={dil}")
    x, w = gen((B, IC, H, W), 60), gen((OC, IC, KH, KW), 61)
    bias = gen((OC,), 62) if has_bias else None
    out = run_conv(x, w, bias, stride, pad, dil)
    check_close(out, oracle.conv2d(x, w, bias, stride, pad, dil), IC * KH * KW, 1.0, "conv rows of 4")
    xi, wi, bi = gen((B, IC, H, W), 63, "I"), gen((OC, IC, KH, KW), 64, "I"), gen((OC,), 65, "I")
    check_bitwise(run_conv(xi, wi, bi, stride, pad, dil), oracle.conv2d(xi, wi, bi, stride, pad, dil),
                  "conv rows of 4 integer")


def test_conv_1x1_equals_addmm():
    """P-4 on the GPU: a 1x1 conv and addmm(W, x[b]) agree bit for bit on
    integer inputs."""
    import bias_addmm_im2col_amd as baim
    say("conv 1x1 vs addmm")
    B, IC, H, W, OC = 2, 40, 12, 13, 72
    x, w = gen((B, IC, H, W), 26, "I"), gen((OC, IC, 1, 1), 27, "I")
    bias = gen((OC,), 28, "I")
    out = run_conv(x, w, bias, 1, 0, 1)
    for b in range(B):
        mm = baim.addmm(dev(bias.view(OC, 1).expand(OC, H * W).contiguous()),
                        dev(w.view(OC, IC)), dev(x[b].reshape(IC, H * W))).cpu().numpy()
        assert np.array_equal(mm, out[b].reshape(OC, H * W))


def test_conv_delta_kernel_shift():
    """P-5 on the GPU: delta weights shift the input (exact)."""
    say("conv delta kernel")
    C = 8
    x = gen((2, C, 19, 17), 29)
    w = torch.zeros(C, C, 3, 3)
    for c in range(C):
        w[c, c, 2, 0] = 1.0
    out = run_conv(x, w, None, 1, (1, 1), (2, 1))
    check_bitwise(out, oracle.conv2d(x, w, None, 1, (1, 1), (2, 1)), "delta")


# ------------------------------------------------------- full workloads
# Every output of every workload case is compared with the oracle (the
# largest, 4096 x 4096 x 1024, is a few seconds of fp64 work on the host).

@pytest.mark.parametrize("name", [n for n, c in I.CASES.items() if c.kind == "addmm"])
def test_workload_addmm(name):
    import bias_addmm_im2col_amd as baim
    c = I.CASES[name]
    say(f"workload {name}: addmm_f32 M={c.M} K={c.K} N={c.N} self_2d={c.self_2d}")
    a, b, s = I.addmm_inputs(c)
    out = baim.addmm(dev(s), dev(a), dev(b), beta=c.beta, alpha=c.alpha)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    res = oracle.addmm(a, b, s, c.self_2d, c.beta, c.alpha)
    ratio = check_close(out, res, c.K, c.alpha, name)
    say(f"{name}: all {out.size} outputs, max err/tol = {ratio:.3f}")


@pytest.mark.parametrize("name", [n for n, c in I.CASES.items() if c.kind == "conv"])
def test_workload_conv(name):
    import bias_addmm_im2col_amd as baim
    c = I.CASES[name]
    say(f"workload {name}: conv2d_gemm_f32 x=[{c.B},{c.IC},{c.H},{c.W}] "
        f"w=[{c.OC},{c.IC},{c.KH},{c.KW}] s={c.stride} p={c.padding} d={c.dilation}")
    x, w, bias = I.conv_inputs(c)
    out = baim.conv2d(dev(x), dev(w), dev(bias), c.stride, c.padding, c.dilation)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    OH, OW = c.out_hw()
    assert out.shape == (c.B, c.OC, OH, OW)
    res = oracle.conv2d(x, w, bias, c.stride, c.padding, c.dilation)
    ratio = check_close(out, res, c.IC * c.KH * c.KW, 1.0, name)
    say(f"{name}: all {out.size} outputs, max err/tol = {ratio:.3f}")


# Integer-valued inputs at the workload shapes: every partial sum is an
# integer below 2^24 (K * 16 <= 65536), so every fp32 summation order is
# exact and the whole output must equal the oracle bit for bit, in the
# launch configuration the workload runs in.
@pytest.mark.parametrize("name", ["conv3x3_56_s1", "conv3x3_56_d2", "conv3x3_57_s2",
                                  "stem_conv7x7_s4_768"])
def test_workload_conv_integer_bitwise(name):
    import bias_addmm_im2col_amd as baim
    c = I.CASES[name]
    say(f"integer workload {name}: conv2d_gemm_f32")
    x, w, bias = (gen((c.B, c.IC, c.H, c.W), 60, "I"), gen((c.OC, c.IC, c.KH, c.KW), 61, "I"),
                  gen((c.OC,), 62, "I"))
    out = baim.conv2d(dev(x), dev(w), dev(bias), c.stride, c.padding, c.dilation)
    torch.cuda.synchronize()
    check_bitwise(out.cpu().numpy(), oracle.conv2d(x, w, bias, c.stride, c.padding, c.dilation),
                  f"integer {name}")


@pytest.mark.parametrize("name", ["down_proj_4096x4096x1024", "up_proj_4096x1024x4096",
                                  "ragged_577x1024x4096_full_self"])
def test_workload_addmm_integer_bitwise(name):
    import bias_addmm_im2col_amd as baim
    c = I.CASES[name]
    say(f"integer workload {name}: addmm_f32 M={c.M} K={c.K} N={c.N}")
    a, b = gen((c.M, c.K), 63, "I"), gen((c.K, c.N), 64, "I")
    s = gen((c.M, c.N) if c.self_2d else (c.N,), 65, "I")
    out = baim.addmm(dev(s), dev(a), dev(b), beta=2.0, alpha=0.5)
    torch.cuda.synchronize()
    check_bitwise(out.cpu().numpy(), oracle.addmm(a, b, s, c.self_2d, 2.0, 0.5), f"integer {name}")


@pytest.mark.parametrize("self_2d", [False, True])
def test_addmm_256_tile_ragged_full_output(self_2d):
    """The planner's 256x256 kernel on a shape with ragged M (4000 = 15*256
    + 160) and K (520 = 32*16 + 8): whole tiles (the untested store loop
    with self [N]), edge tiles and the partial last k-tile, every output
    against the oracle.  Uniform inputs to the bound with alpha/beta;
    integer inputs (every partial sum exact) bit for bit."""
    import bias_addmm_im2col_amd as baim
    M, K, N = 4000, 520, 4096
    p = baim.gemm_plan(M, N, K)
    say(f"addmm 256x256 tile M={M} K={K} N={N} self_2d={self_2d} plan {p}")
    assert (p["bm"], p["bn"], p["bk"], p["waves"]) == (256, 256, 16, 8)
    a, b = gen((M, K), 70), gen((K, N), 71)
    s = gen((M, N) if self_2d else (N,), 72)
    out = run_addmm(a, b, s, 0.5, 2.0)
    check_close(out, oracle.addmm(a, b, s, self_2d, 0.5, 2.0), K, 2.0, "256 tile")
    ai, bi = gen((M, K), 73, "I"), gen((K, N), 74, "I")
    si = gen((M, N) if self_2d else (N,), 75, "I")
    check_bitwise(run_addmm(ai, bi, si, 2.0, 0.5), oracle.addmm(ai, bi, si, self_2d, 2.0, 0.5),
                  "256 tile integer")


def test_repeated_launches_are_deterministic():
    """The same call twice gives the same bits (no cross-launch state)."""
    import bias_addmm_im2col_amd as baim
    say("determinism")
    a, b, s = gen((300, 200), 30), gen((200, 260), 31), gen((260,), 32)
    o1 = baim.addmm(dev(s), dev(a), dev(b)).cpu()
    o2 = baim.addmm(dev(s), dev(a), dev(b)).cpu()
    assert torch.equal(o1, o2)


# ------------------------------------------- every tile config and K split
# BAIM_TILE forces the host's choice; the specs and the shapes they run on
# are in tests/_specs.py, which explains the notation.  Each spec changes the
# launched plan on at least one shape (checked on the CPU in
# tests/test_forced_specs.py).
TILE_SPECS = _specs.GEMM_SPECS


@pytest.mark.parametrize("spec", _specs.ADDMM_SPECS)
def test_addmm_forced_tile_configs(spec, monkeypatch):
    monkeypatch.setenv("BAIM_TILE", spec)
    for M, K, N, self_2d, beta, alpha in _specs.ADDMM_SHAPES:
        say(f"BAIM_TILE={spec} addmm_f32 M={M} K={K} N={N} self_2d={self_2d}")
        a, b = gen((M, K), 40), gen((K, N), 41)
        s = gen((M, N) if self_2d else (N,), 42)
        out = run_addmm(a, b, s, beta, alpha)
        check_close(out, oracle.addmm(a, b, s, self_2d, beta, alpha), K, alpha, f"addmm {spec}")
    M, K, N = _specs.ADDMM_INT_SHAPE
    say(f"BAIM_TILE={spec} addmm_f32 integer M={M} K={K} N={N}")
    a, b, s = gen((M, K), 43, "I"), gen((K, N), 44, "I"), gen((N,), 45, "I")
    out = run_addmm(a, b, s, 2.0, 0.5)
    check_bitwise(out, oracle.addmm(a, b, s, False, 2.0, 0.5), f"addmm integer {spec}")


@pytest.mark.parametrize("spec", TILE_SPECS)
def test_conv_forced_tile_configs(spec, monkeypatch):
    monkeypatch.setenv("BAIM_TILE", spec)
    for B, IC, H, W, OC, KH, KW, stride, pad, dil, has_bias in _specs.CONV_SHAPES:
        say(f"BAIM_TILE={spec} conv2d_gemm_f32 x=[{B},{IC},{H},{W}] w=[{OC},{IC},{KH},{KW}] "
            f"s={stride} p={pad} d={dil}")
        x, w = gen((B, IC, H, W), 46), gen((OC, IC, KH, KW), 47)
        bias = gen((OC,), 48) if has_bias else None
        out = run_conv(x, w, bias, stride, pad, dil)
        check_close(out, oracle.conv2d(x, w, bias, stride, pad, dil), IC * KH * KW, 1.0,
                    f"conv {spec}")
    B, IC, H, W, OC = _specs.CONV_INT_SHAPE
    say(f"BAIM_TILE={spec} conv2d_gemm_f32 integer x=[{B},{IC},{H},{W}] OC={OC}")
    x, w, bias = gen((B, IC, H, W), 49, "I"), gen((OC, IC, 3, 3), 50, "I"), gen((OC,), 51, "I")
    out = run_conv(x, w, bias, 1, 1, 1)
    check_bitwise(out, oracle.conv2d(x, w, bias, 1, 1, 1), f"conv integer {spec}")
    say(f"BAIM_TILE={spec} conv2d_gemm_f32 rows of 4")
    x, w, bias = gen((2, 24, 13, 20), 52), gen((136, 24, 3, 3), 53), gen((136,), 54)
    check_close(run_conv(x, w, bias, 1, 1, 1), oracle.conv2d(x, w, bias, 1, 1, 1), 24 * 9, 1.0,
                f"conv rows of 4 {spec}")
    x, w, bias = gen((2, 24, 13, 20), 55, "I"), gen((136, 24, 3, 3), 56, "I"), gen((136,), 57, "I")
    check_bitwise(run_conv(x, w, bias, 1, 2, 2), oracle.conv2d(x, w, bias, 1, 2, 2),
                  f"conv rows of 4 integer {spec}")


@pytest.mark.parametrize("spec", ["3,s7", "0,2", "6,s5", "1,s4"])
def test_two_piece_paths_are_bit_reproducible(spec, monkeypatch):
    """Stream pieces and 2-slice splits combine with an order-free sum: the
    same call gives the same bits every time."""
    import bias_addmm_im2col_amd as baim
    monkeypatch.setenv("BAIM_TILE", spec)
    say(f"BAIM_TILE={spec} reproducibility")
    a, b, s = gen((300, 700), 52), gen((700, 260), 53), gen((300, 260), 54)
    outs = [baim.addmm(dev(s), dev(a), dev(b), beta=0.5, alpha=2.0).cpu() for _ in range(4)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    x, w, bias = gen((2, 40, 19, 17), 55), gen((72, 40, 3, 3), 56), gen((72,), 57)
    outs = [baim.conv2d(dev(x), dev(w), dev(bias), 1, 1, 1).cpu() for _ in range(4)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


@pytest.mark.parametrize("spec", ["3,s7", "1,2", "7,3"])
def test_split_paths_with_unaligned_out(spec, monkeypatch):
    """The output-initialisation kernels handle an out that starts 4 bytes
    past a 16-byte boundary and whose size is not a multiple of 4."""
    import bias_addmm_im2col_amd as baim
    monkeypatch.setenv("BAIM_TILE", spec)
    say(f"BAIM_TILE={spec} unaligned out")
    M, K, N = 131, 600, 197
    a, b, s = gen((M, K), 58), gen((K, N), 59), gen((N,), 60)
    buf = torch.full((M * N + 1,), 7.0, device="cuda")
    out = buf[1:].view(M, N)
    baim.addmm_f32(out, dev(s), dev(a), dev(b), 1.0, 1.0)
    torch.cuda.synchronize()
    assert float(buf[0]) == 7.0
    check_close(out.cpu().numpy(), oracle.addmm(a, b, s, False, 1.0, 1.0), K, 1.0, f"addmm {spec}")
    x, w, bias = gen((2, 24, 21, 19), 61), gen((70, 24, 3, 3), 62), gen((70,), 63)
    OH, OW = baim.conv2d_out_hw(21, 19, 3, 3, 1, 1, 1)
    cbuf = torch.full((2 * 70 * OH * OW + 1,), 7.0, device="cuda")
    cout = cbuf[1:].view(2, 70, OH, OW)
    baim.conv2d_gemm_f32(cout, dev(x), dev(w), dev(bias), 1, 1, 1)
    torch.cuda.synchronize()
    assert float(cbuf[0]) == 7.0
    check_close(cout.cpu().numpy(), oracle.conv2d(x, w, bias, 1, 1, 1), 24 * 9, 1.0, f"conv {spec}")


# ------------------------------------------------------------------ linear
# out = x @ weight^T + bias, weight [N,K] (the linear_fp32 form the addmm
# page shares its GEMM skeleton with).

def run_linear(x, w, b):
    import bias_addmm_im2col_amd as baim
    out = baim.linear(dev(x), dev(w), dev(b))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("M,K,N,has_bias", [
    (1, 1, 1, True), (3, 5, 7, False), (64, 96, 80, True), (127, 33, 129, True),
    (129, 31, 257, False), (257, 64, 130, True), (300, 517, 100, True), (37, 1000, 41, False)])
def test_linear_small_full(M, K, N, has_bias):
    say(f"linear_f32 M={M} K={K} N={N} bias={has_bias}")
    x, w = gen((M, K), 80), gen((N, K), 81)
    b = gen((N,), 82) if has_bias else None
    check_close(run_linear(x, w, b), oracle.linear(x, w, b), K, 1.0, f"linear {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(64, 96, 80), (129, 257, 131), (256, 1024, 384)])
def test_linear_integer_bitwise(M, K, N):
    say(f"linear_f32 integer M={M} K={K} N={N}")
    x, w, b = gen((M, K), 83, "I"), gen((N, K), 84, "I"), gen((N,), 85, "I")
    check_bitwise(run_linear(x, w, b), oracle.linear(x, w, b), "linear integer")


@pytest.mark.parametrize("spec", TILE_SPECS)
def test_linear_forced_tile_configs(spec, monkeypatch):
    monkeypatch.setenv("BAIM_TILE", spec)
    for M, K, N in _specs.LINEAR_SHAPES:
        say(f"BAIM_TILE={spec} linear_f32 M={M} K={K} N={N}")
        x, w, b = gen((M, K), 86), gen((N, K), 87), gen((N,), 88)
        check_close(run_linear(x, w, b), oracle.linear(x, w, b), K, 1.0, f"linear {spec}")
    M, K, N = _specs.LINEAR_INT_SHAPE
    say(f"BAIM_TILE={spec} linear_f32 integer M={M} K={K} N={N}")
    x, w, b = gen((M, K), 89, "I"), gen((N, K), 90, "I"), gen((N,), 91, "I")
    check_bitwise(run_linear(x, w, b), oracle.linear(x, w, b), f"linear integer {spec}")


def test_linear_leading_dims_and_unaligned():
    """x [..., K] is flattened; operands 4 bytes off a 16-byte boundary use
    the 4-byte-load variant."""
    import bias_addmm_im2col_amd as baim
    say("linear_f32 leading dims / unaligned")
    x, w, b = gen((2, 3, 50, 68), 92), gen((90, 68), 93), gen((90,), 94)
    out = baim.linear(dev(x), dev(w), dev(b))
    assert tuple(out.shape) == (2, 3, 50, 90)
    check_close(out.reshape(-1, 90).cpu().numpy(), oracle.linear(x.reshape(-1, 68), w, b), 68, 1.0,
                "linear leading dims")
    xb = torch.empty(300 * 68 + 1, device="cuda")
    xb[1:] = dev(x).reshape(-1)
    out = torch.empty(300, 90, device="cuda")
    baim.linear_f32(out, xb[1:].view(300, 68), dev(w), dev(b))
    torch.cuda.synchronize()
    check_close(out.cpu().numpy(), oracle.linear(x.reshape(-1, 68), w, b), 68, 1.0, "linear unaligned")


@pytest.mark.parametrize("name", list(I.LINEAR_CASES))
def test_workload_linear(name):
    import bias_addmm_im2col_amd as baim
    c = I.LINEAR_CASES[name]
    say(f"workload {name}: linear_f32 M={c.M} K={c.K} N={c.N}")
    x, w, b = I.linear_inputs(c)
    out = baim.linear(dev(x), dev(w), dev(b))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    rows, cols = addmm_sample(c.M, c.N)
    ratio = check_close(out[rows, cols], oracle.linear_at(x, w, b, rows, cols), c.K, 1.0, name)
    say(f"{name}: {rows.size} sampled outputs, max err/tol = {ratio:.3f}")


# ------------------------------------------------------------ grouped conv
# Per-group GEMM when a group has >= 32 output channels and >= 32 taps,
# else the direct kernel (depthwise and other small groups).

def run_gconv(x, w, bias, stride, pad, dil, groups):
    import bias_addmm_im2col_amd as baim
    out = baim.conv2d(dev(x), dev(w), dev(bias), stride, pad, dil, groups)
    torch.cuda.synchronize()
    return out.cpu().numpy()


GCONV_SHAPES = [
    # B, IC, H, W, OC, KH, KW, stride, pad, dil, groups, bias   (path)
    (2, 64, 17, 19, 128, 3, 3, 1, 1, 1, 2, True),     # GEMM, 64 out ch / group
    (2, 128, 15, 13, 128, 3, 3, 2, 1, 1, 4, True),    # GEMM, 32 / group, stride 2
    (1, 96, 14, 14, 96, 3, 3, 1, 2, 2, 3, False),     # GEMM, dilation 2
    (2, 64, 12, 16, 128, 3, 3, 1, 1, 1, 4, True),     # GEMM, rows of 16
    (2, 32, 17, 19, 32, 3, 3, 1, 1, 1, 32, True),     # depthwise: direct
    (2, 8, 21, 20, 16, 3, 3, 1, 1, 1, 8, True),       # channel multiplier 2: direct
    (1, 16, 30, 31, 24, 5, 5, (2, 1), 2, (1, 2), 4, True),  # small groups: direct
    (2, 12, 9, 9, 12, 1, 1, 1, 0, 1, 3, True),        # grouped 1x1: direct
    (1, 8, 70, 70, 8, 3, 3, 8, 1, 1, 8, True),        # stride 8: window > LDS, plain direct
    (2, 16, 70, 130, 16, 3, 3, 1, 1, 1, 16, False),   # depthwise, width 130: LDS tiles
    (1, 8, 130, 130, 8, 3, 3, 1, 1, 1, 4, True),      # 2 channels per group: LDS tiles
    (1, 4, 140, 140, 4, 3, 3, 8, 1, 1, 4, True),      # stride 8 on a large plane: plain direct
    (1, 2, 6, 1100, 2, 3, 3, 1, 1, 1, 2, True),       # depthwise 3x3 "same", width % 4 == 0:
    (2, 24, 13, 16, 24, 5, 5, 1, 2, 1, 24, True),     #   4x4 output blocks in registers
    (1, 8, 21, 28, 16, 7, 7, 1, 3, 1, 8, False),      #   (5x5, 7x7 with channel multiplier 2)
]


@pytest.mark.parametrize("B,IC,H,W,OC,KH,KW,stride,pad,dil,groups,has_bias", GCONV_SHAPES)
def test_grouped_conv_full(B, IC, H, W, OC, KH, KW, stride, pad, dil, groups, has_bias):
    say(f"conv2d_gemm_f32 groups={groups} x=[{B},{IC},{H},{W}] w=[{OC},{IC // groups},{KH},{KW}]")
    x, w = gen((B, IC, H, W), 95), gen((OC, IC // groups, KH, KW), 96)
    bias = gen((OC,), 97) if has_bias else None
    out = run_gconv(x, w, bias, stride, pad, dil, groups)
    check_close(out, oracle.conv2d_grouped(x, w, bias, stride, pad, dil, groups),
                IC // groups * KH * KW, 1.0, f"grouped conv g={groups}")


@pytest.mark.parametrize("groups,OC,W", [(2, 128, 14), (8, 256, 14), (64, 64, 14), (16, 32, 14),
                                          (32, 32, 16)])
def test_grouped_conv_integer_bitwise(groups, OC, W):
    say(f"conv2d_gemm_f32 integer groups={groups} W={W}")
    IC = 64 if groups <= 8 else groups
    x, w, bias = gen((2, IC, 15, W), 98, "I"), gen((OC, IC // groups, 3, 3), 99, "I"), gen((OC,), 100, "I")
    out = run_gconv(x, w, bias, 1, 1, 1, groups)
    check_bitwise(out, oracle.conv2d_grouped(x, w, bias, 1, 1, 1, groups), f"grouped integer g={groups}")


@pytest.mark.parametrize("spec", ["1", "3", "6,2", "3,s7", "7,3", "8", "8,2"])
def test_grouped_gemm_forced_tile_configs(spec, monkeypatch):
    monkeypatch.setenv("BAIM_TILE", spec)
    say(f"BAIM_TILE={spec} grouped conv")
    x, w, bias = gen((2, 64, 13, 12), 101), gen((96, 32, 3, 3), 102), gen((96,), 103)
    out = run_gconv(x, w, bias, 1, 1, 1, 2)
    check_close(out, oracle.conv2d_grouped(x, w, bias, 1, 1, 1, 2), 32 * 9, 1.0, f"grouped {spec}")


@pytest.mark.parametrize("name", list(I.GROUPED_CASES))
def test_workload_grouped_conv(name):
    import bias_addmm_im2col_amd as baim
    c = I.GROUPED_CASES[name]
    say(f"workload {name}: conv2d_gemm_f32 groups={c.groups}")
    x, w, bias = I.conv_inputs(c)
    out = baim.conv2d(dev(x), dev(w), dev(bias), c.stride, c.padding, c.dilation, c.groups)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    OH, OW = c.out_hw()
    idx = conv_sample(c.B, c.OC, OH, OW)
    res = oracle.conv2d_grouped_at(x, w, bias, c.stride, c.padding, c.dilation, c.groups, idx)
    ratio = check_close(out.reshape(-1)[idx], res, c.IC // c.groups * c.KH * c.KW, 1.0, name)
    say(f"{name}: {idx.size} sampled outputs, max err/tol = {ratio:.3f}")
