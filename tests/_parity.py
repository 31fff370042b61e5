"""Shared helpers for the GPU parity tests: device transfer, sampling of
outputs that the oracle computes one by one, and the acceptance check."""
import numpy as np
import torch

import oracle


def dev(t):
    return None if t is None else t.contiguous().cuda()


def check_close(out, res, K, alpha=1.0, what=""):
    """|out - ref| <= 4e-6*sqrt(K)*(|alpha|*sabs + |beta*self|) elementwise."""
    out = np.asarray(out, dtype=np.float64)
    assert out.shape == res.ref.shape, (out.shape, res.ref.shape)
    err = np.abs(out - res.ref)
    tol = oracle.tolerance(res, K, alpha)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {err.size} outputs outside tolerance; worst at {idx}: "
            f"out={out[idx]!r} ref={res.ref[idx]!r} err={err[idx]:.3e} tol={tol[idx]:.3e}")
    return float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0


def check_bitwise(out, res, what=""):
    """out equals the fp32 rounding of the exact result, bit for bit."""
    out = np.asarray(out, dtype=np.float32)
    ref32 = res.ref.astype(np.float32)
    same = (out.view(np.uint32) == ref32.view(np.uint32))
    if not same.all():
        idx = np.argwhere(~same)[0]
        raise AssertionError(f"{what}: {int((~same).sum())} outputs differ bitwise; first at "
                             f"{tuple(idx)}: out={out[tuple(idx)]!r} ref={ref32[tuple(idx)]!r}")


def addmm_sample(M, N, tile=128, n_rand=4096, seed=0):
    """Output coordinates: whole rows and columns at the edges and at tile
    boundaries, plus random points."""
    g = np.random.default_rng(seed)
    edge_rows = sorted({0, 1, M - 1, min(tile - 1, M - 1), min(tile, M - 1), M // 2} |
                       set(g.integers(0, M, 3).tolist()))
    edge_cols = sorted({0, 1, N - 1, min(tile - 1, N - 1), min(tile, N - 1), N // 2} |
                       set(g.integers(0, N, 3).tolist()))
    rows = [np.full(N, r) for r in edge_rows] + [np.arange(M) for _ in edge_cols]
    cols = [np.arange(N) for _ in edge_rows] + [np.full(M, c) for c in edge_cols]
    rows.append(g.integers(0, M, n_rand))
    cols.append(g.integers(0, N, n_rand))
    return np.concatenate(rows).astype(np.int64), np.concatenate(cols).astype(np.int64)


def conv_sample(B, OC, OH, OW, n_rand=4096, seed=0):
    """Flat NCHW output indices: full output planes of a few (b, oc) pairs
    (first, last, tile edges), full channel columns at the image corners,
    and random points."""
    g = np.random.default_rng(seed)
    P = OH * OW
    planes = {(0, 0), (B - 1, OC - 1), (0, min(127, OC - 1)), (B - 1, min(128, OC - 1)),
              (int(g.integers(0, B)), int(g.integers(0, OC)))}
    idx = [np.arange(P) + (b * OC + oc) * P for b, oc in sorted(planes)]
    for b in sorted({0, B - 1}):
        for pix in (0, OW - 1, P - OW, P - 1, P // 2):
            idx.append((b * OC + np.arange(OC)) * P + pix)
    idx.append(g.integers(0, B * OC * P, n_rand))
    return np.unique(np.concatenate(idx).astype(np.int64))
