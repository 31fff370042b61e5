"""GPU parity of the fused attention kernel (sdpa_f32) against the fp64 oracle.

Definition: "[ExecuTorch][WebGPU] Add optimized SDPA op", Problem/Solution:
out = softmax(q @ k^T * scale + attn_mask) @ v, softmax over the keys, an
optional additive [B,H,Sq,Skv] mask, Sq != Skv allowed, scale 1/sqrt(D) by
default.  Acceptance: |out - ref| <= 4e-6 * err elementwise, err being the
oracle's first-order error scale of an fp32 evaluation (in fp32 rounding
units: the logits' dot products, the exponent arguments, the key count);
rows the definition leaves without a softmax (every key masked) must be NaN.
Cases built so that every softmax weight is 0 or 1/2^n and every sum is
exact (zero scale, 0/-inf masks, integer values) must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from bias_addmm_im2col_amd import inputs as I
from tests._parity import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    from bias_addmm_im2col_amd import _capi
    _capi.lib()


def say(msg):
    print(f"[parity] {msg}", flush=True)


def gen(shape, seed, sigma=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g) * sigma


def run_sdpa(q, k, v, mask=None, scale=None):
    import bias_addmm_im2col_amd as baim
    out = baim.sdpa(dev(q), dev(k), dev(v), dev(mask), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_sdpa(out, res, what=""):
    out = np.asarray(out, dtype=np.float64)
    assert out.shape == res.ref.shape, (out.shape, res.ref.shape)
    nan_ref = np.isnan(res.ref)
    assert (np.isnan(out) == nan_ref).all(), f"{what}: NaN pattern differs from the oracle"
    err = np.abs(np.where(nan_ref, 0.0, out - res.ref))
    tol = np.where(nan_ref, 0.0, oracle.sdpa_tolerance(res))
    bad = ~(err <= tol)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} outputs outside tolerance; worst at {idx}: "
            f"out={out[idx]!r} ref={res.ref[idx]!r} err={err[idx]:.3e} tol={tol[idx]:.3e}")


SHAPES = [
    # B, H, Sq, Skv, D, mask, scale
    (1, 1, 1, 1, 4, False, None),
    (2, 3, 33, 65, 32, False, None),
    (1, 2, 129, 64, 64, True, None),       # mask rows 16-byte aligned
    (2, 2, 127, 63, 64, True, 0.2),        # mask with the 4-byte-load path
    (1, 4, 200, 300, 36, True, None),      # D padded to 64
    (2, 1, 64, 129, 72, False, None),      # D padded to 96
    (1, 2, 130, 70, 96, True, None),
    (1, 1, 45, 257, 100, False, 0.05),     # D padded to 128
    (2, 2, 128, 128, 128, True, None),
    (1, 3, 5, 1000, 64, True, None),       # few queries, many keys
    (1, 1, 600, 3, 16, False, None),       # many queries, few keys
]


@pytest.mark.parametrize("B,H,Sq,Skv,D,masked,scale", SHAPES)
def test_sdpa_small_full(B, H, Sq, Skv, D, masked, scale):
    say(f"sdpa_f32 B={B} H={H} Sq={Sq} Skv={Skv} D={D} mask={masked} scale={scale}")
    q, k, v = gen((B, H, Sq, D), 1), gen((B, H, Skv, D), 2), gen((B, H, Skv, D), 3)
    m = gen((B, H, Sq, Skv), 4, 2.0) if masked else None
    check_sdpa(run_sdpa(q, k, v, m, scale), oracle.sdpa(q, k, v, m, scale),
               f"sdpa {B}x{H}x{Sq}x{Skv}x{D}")


CFG_SHAPES = [
    # BH, Sq, Skv, D, mask
    (3, 33, 65, 32, True), (2, 130, 200, 64, False), (2, 70, 129, 64, True),
    (1, 100, 300, 96, True), (2, 65, 257, 128, False), (1, 5, 1000, 64, True),
    (2, 40, 31, 128, True),
]


@pytest.mark.parametrize("cfg", ["0", "1", "2", "3"])
def test_sdpa_forced_block_shapes(cfg, monkeypatch):
    """Every block shape (query groups x key groups) on ragged sizes, forced
    through BAIM_SDPA: 128 query rows; 64 rows with two key groups; 32 rows
    with four key groups merged at the end; 32 rows with eight key groups in
    eight waves (D <= 64; the larger D fall back to the plan)."""
    monkeypatch.setenv("BAIM_SDPA", cfg)
    for i, (BH, Sq, Skv, D, masked) in enumerate(CFG_SHAPES):
        say(f"BAIM_SDPA={cfg} sdpa_f32 BH={BH} Sq={Sq} Skv={Skv} D={D} mask={masked}")
        q, k, v = gen((BH, Sq, D), 30 + i), gen((BH, Skv, D), 40 + i), gen((BH, Skv, D), 50 + i)
        m = gen((BH, Sq, Skv), 60 + i, 2.0) if masked else None
        if masked:
            m[:, 1, :] = float("-inf")          # a row with no keys
            m[:, 2, : Skv // 2] = float("-inf")  # leading keys dropped
        check_sdpa(run_sdpa(q, k, v, m), oracle.sdpa(q, k, v, m), f"cfg {cfg} shape {i}")
    # exact case: zero scale, one key kept per row (out = that value row)
    BH, Sq, Skv, D = 2, 50, 300, 64
    pick = np.random.default_rng(int(cfg)).integers(0, Skv, size=(BH, Sq))
    mask = np.full((BH, Sq, Skv), -np.inf, np.float32)
    for b in range(BH):
        mask[b, np.arange(Sq), pick[b]] = 0.0
    q, k, v = gen((BH, Sq, D), 70), gen((BH, Skv, D), 71), gen((BH, Skv, D), 72)
    out = run_sdpa(q, k, v, torch.from_numpy(mask), 0.0)
    assert (out == np.stack([v.numpy()[b][pick[b]] for b in range(BH)])).all()


@pytest.mark.parametrize("Skv,D", [(64, 64), (100, 32), (333, 128), (8, 96)])
def test_sdpa_uniform_weights_bitwise(Skv, D):
    """Zero scale and a 0/-inf mask leaving 2^n keys per row: every weight
    is exactly 1/2^n, and with small integer values every sum is exact."""
    say(f"sdpa_f32 uniform weights Skv={Skv} D={D}")
    BH, Sq = 3, 70
    rng = np.random.default_rng(Skv + D)
    mask = np.full((BH, Sq, Skv), -np.inf, np.float32)
    for b in range(BH):
        for i in range(Sq):
            n = 2 ** int(rng.integers(0, int(np.log2(Skv)) + 1))
            mask[b, i, rng.choice(Skv, n, replace=False)] = 0.0
    q, k = gen((BH, Sq, D), 5), gen((BH, Skv, D), 6)
    v = torch.randint(-8, 9, (BH, Skv, D), generator=torch.Generator().manual_seed(7)).float()
    mask_t = torch.from_numpy(mask)
    out = run_sdpa(q, k, v, mask_t, 0.0)
    ref = oracle.sdpa(q, k, v, mask_t, 0.0).ref.astype(np.float32)
    assert (out.view(np.uint32) == ref.view(np.uint32)).all()


def test_sdpa_one_hot_mask_copies_value_rows():
    say("sdpa_f32 one-hot mask")
    BH, Sq, Skv, D = 4, 150, 190, 64
    pick = np.random.default_rng(8).integers(0, Skv, size=(BH, Sq))
    mask = np.full((BH, Sq, Skv), -np.inf, np.float32)
    for b in range(BH):
        mask[b, np.arange(Sq), pick[b]] = 0.0
    q, k, v = gen((BH, Sq, D), 9), gen((BH, Skv, D), 10), gen((BH, Skv, D), 11)
    out = run_sdpa(q, k, v, torch.from_numpy(mask))
    want = np.stack([v.numpy()[b][pick[b]] for b in range(BH)])
    assert (out == want).all()


def test_sdpa_masked_rows_and_leading_tiles():
    """A row with every key masked is NaN; rows whose first key tiles are
    all masked (the running maximum starts at -inf) are still exact."""
    say("sdpa_f32 masked rows")
    BH, Sq, Skv, D = 2, 40, 300, 64
    q, k, v = gen((BH, Sq, D), 12), gen((BH, Skv, D), 13), gen((BH, Skv, D), 14)
    m = gen((BH, Sq, Skv), 15).numpy()
    m[0, 3, :] = -np.inf
    m[1, 39, :] = -np.inf
    m[0, 5, :200] = -np.inf   # first three 64-key tiles and part of the fourth
    m[1, 7, 64:] = -np.inf    # only the first tile
    m[1, 8, :-1] = -np.inf    # only the last key
    mt = torch.from_numpy(m)
    out = run_sdpa(q, k, v, mt)
    res = oracle.sdpa(q, k, v, mt)
    assert np.isnan(out[0, 3]).all() and np.isnan(out[1, 39]).all()
    check_sdpa(out, res, "masked rows")
    assert (out[1, 8] == v.numpy()[1, -1]).all()


def test_sdpa_leading_dims():
    import bias_addmm_im2col_amd as baim
    say("sdpa_f32 rank 3 and rank 5")
    q, k, v = gen((6, 50, 32), 16), gen((6, 70, 32), 17), gen((6, 70, 32), 18)
    check_sdpa(run_sdpa(q, k, v), oracle.sdpa(q, k, v), "rank 3")
    q, k, v = gen((2, 2, 3, 17, 64), 19), gen((2, 2, 3, 9, 64), 20), gen((2, 2, 3, 9, 64), 21)
    m = gen((2, 2, 3, 17, 9), 22)
    out = baim.sdpa(dev(q), dev(k), dev(v), dev(m))
    torch.cuda.synchronize()
    assert tuple(out.shape) == (2, 2, 3, 17, 64)
    check_sdpa(out.cpu().numpy(), oracle.sdpa(q, k, v, m), "rank 5")


def test_sdpa_is_deterministic():
    say("sdpa_f32 run-to-run")
    q, k, v, m = gen((3, 4, 300, 64), 23), gen((3, 4, 500, 64), 24), gen((3, 4, 500, 64), 25), \
        gen((3, 4, 300, 500), 26)
    a = run_sdpa(q, k, v, m)
    b = run_sdpa(q, k, v, m)
    assert (a.view(np.uint32) == b.view(np.uint32)).all()


def test_sdpa_rejects_unaligned_inputs():
    import bias_addmm_im2col_amd as baim
    say("sdpa_f32 unaligned q")
    buf = torch.zeros(2 * 8 * 16 + 1, device="cuda")
    q = buf[1:].view(2, 8, 16)
    k = torch.zeros(2, 8, 16, device="cuda")
    with pytest.raises(NotImplementedError):
        baim.sdpa(q, k, k)


def _rows_sample(BH, Sq, n_rand=48, seed=0):
    g = np.random.default_rng(seed)
    rows = {0, Sq - 1, min(127, Sq - 1), min(128, Sq - 1), BH * Sq - 1, (BH - 1) * Sq,
            (BH // 2) * Sq + Sq // 2}
    rows |= set(g.integers(0, BH * Sq, n_rand).tolist())
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", list(I.SDPA_CASES))
def test_workload_sdpa(name):
    """Workload size, sampled query rows (whole output rows of D values)."""
    import bias_addmm_im2col_amd as baim
    c = I.SDPA_CASES[name]
    say(f"workload {name}: sdpa_f32 B={c.B} H={c.H} Sq={c.Sq} Skv={c.Skv} D={c.D}")
    q, k, v, m = I.sdpa_inputs(c)
    out = baim.sdpa(dev(q), dev(k), dev(v), dev(m), c.scale)
    torch.cuda.synchronize()
    rows = _rows_sample(c.B * c.H, c.Sq)
    got = out.reshape(-1, c.D)[torch.from_numpy(rows).cuda()].cpu().numpy()
    check_sdpa(got, oracle.sdpa_rows(q, k, v, m, c.scale, rows), name)
