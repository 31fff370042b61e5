"""fp64 CPU oracle for the fp32 bias-addmm and implicit-im2col conv2d path.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``; never by the
product package.  It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain loops, fp64 accumulation, sum over
k in increasing order); this module only builds/loads that library and
marshals numpy arrays.  Definitions followed:

* addmm -- "[ExecuTorch][WebGPU] Add optimized addmm op" (PR #20855),
  Solution/Implementation: ``out = beta*self + alpha*(mat1 @ mat2)``,
  self broadcast from [N] or full [M,N].
* linear -- the same page, Implementation: the GEMM skeleton shared with
  linear_fp32, which reads a transposed [N,K] weight:
  ``out = x @ weight^T + bias``.
* conv2d -- "et_vk conv2d: route standard (groups==1) conv through an im2col
  tiled GEMM" (PR #20873), Solution/Implementation: direct sum over
  (ic, kh, kw) taps at ih = oh*sH - pH + kh*dH (and the W analogue),
  out-of-range taps read 0, per-OC bias, NCHW output.
* conv2d_nhwc -- the same conv page, Constraints paragraph (the NCHW channel
  stride is not contiguous, so K cannot be read four at a time): the conv
  with channels-last tensors, input [B,H,W,IC], weight [OC,KH,KW,IC],
  output [B,OH,OW,OC], taps summed in (kh, kw, ic) order.
* conv_transpose2d -- the conv page routes transposed convs to their own
  gather kernels and defines nothing more, so the standard definition (the
  adjoint of conv2d, weight [IC,OC,KH,KW]): each input element scatters
  x*w into out[b, oc, ih*sH - pH + kh*dH, iw*sW - pW + kw*dW].
* sdpa -- "[ExecuTorch][WebGPU] Add optimized SDPA op" (PR #20851),
  Problem/Solution: non-causal ``softmax(q @ k^T * scale + mask) @ v`` over
  [B,H,S,D] tensors, optional additive mask [B,H,Sq,Skv], Sq may differ from
  Skv, scale 1/sqrt(D) when not given.

Acceptance bound used by the parity tests (stated with the workload):
``|out - ref| <= 4e-6 * sqrt(K) * (|alpha|*sabs + |beta*self|)`` where
``sabs = sum_k |a_ik * b_kj|``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from collections import namedtuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# BAIM_ORACLE_LIB lets the oracle's own tests load a deliberately broken build
# (planted mistakes) to show that the pins catch them.
_LIB = os.environ.get("BAIM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

Result = namedtuple("Result", ["ref", "sabs", "selfabs"])
SdpaResult = namedtuple("SdpaResult", ["ref", "err"])

_i64 = ctypes.c_int64
_fp = ctypes.POINTER(ctypes.c_float)
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_addmm.argtypes = [_i64, _i64, _i64, _fp, _fp, _fp, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_float, _dp, _dp]
    lib.oracle_addmm.restype = None
    lib.oracle_addmm_at.argtypes = [_i64, _i64, _i64, _fp, _fp, _fp, ctypes.c_int,
                                    ctypes.c_float, ctypes.c_float, _i64, _lp, _lp,
                                    _dp, _dp]
    lib.oracle_addmm_at.restype = None
    lib.oracle_linear.argtypes = [_i64, _i64, _i64, _fp, _fp, _fp, _dp, _dp]
    lib.oracle_linear.restype = None
    lib.oracle_linear_at.argtypes = [_i64, _i64, _i64, _fp, _fp, _fp, _i64, _lp, _lp, _dp, _dp]
    lib.oracle_linear_at.restype = None
    lib.oracle_conv_out_size.argtypes = [_i64] * 5
    lib.oracle_conv_out_size.restype = _i64
    lib.oracle_conv2d.argtypes = [_i64] * 13 + [_fp, _fp, _fp, _dp, _dp]
    lib.oracle_conv2d.restype = ctypes.c_int
    lib.oracle_conv2d_at.argtypes = [_i64] * 13 + [_fp, _fp, _fp, _i64, _lp, _dp, _dp]
    lib.oracle_conv2d_at.restype = ctypes.c_int
    lib.oracle_conv2d_grouped.argtypes = [_i64] * 14 + [_fp, _fp, _fp, _dp, _dp]
    lib.oracle_conv2d_grouped.restype = ctypes.c_int
    lib.oracle_conv2d_grouped_at.argtypes = [_i64] * 14 + [_fp, _fp, _fp, _i64, _lp, _dp, _dp]
    lib.oracle_conv2d_grouped_at.restype = ctypes.c_int
    lib.oracle_conv2d_nhwc.argtypes = [_i64] * 13 + [_fp, _fp, _fp, _dp, _dp]
    lib.oracle_conv2d_nhwc.restype = ctypes.c_int
    lib.oracle_conv2d_nhwc_at.argtypes = [_i64] * 13 + [_fp, _fp, _fp, _i64, _lp, _dp, _dp]
    lib.oracle_conv2d_nhwc_at.restype = ctypes.c_int
    lib.oracle_convt_out_size.argtypes = [_i64] * 6
    lib.oracle_convt_out_size.restype = _i64
    lib.oracle_conv_transpose2d.argtypes = [_i64] * 16 + [_fp, _fp, _fp, _dp, _dp]
    lib.oracle_conv_transpose2d.restype = ctypes.c_int
    lib.oracle_conv_transpose2d_at.argtypes = [_i64] * 16 + [_fp, _fp, _fp, _i64, _lp, _dp, _dp]
    lib.oracle_conv_transpose2d_at.restype = ctypes.c_int
    lib.oracle_sdpa.argtypes = [_i64] * 4 + [_fp] * 4 + [ctypes.c_float, _dp, _dp]
    lib.oracle_sdpa.restype = ctypes.c_int
    lib.oracle_sdpa_rows.argtypes = [_i64] * 4 + [_fp] * 4 + [ctypes.c_float, _i64, _lp, _dp, _dp]
    lib.oracle_sdpa_rows.restype = ctypes.c_int
    lib.oracle_im2col.argtypes = [_i64] * 12 + [_fp, _dp]
    lib.oracle_im2col.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def _f32(a):
    if a is None:
        return None
    if hasattr(a, "numpy"):  # a CPU torch tensor
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle inputs are the fp32 values the kernels see")
    return a


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _pair(v):
    return (int(v), int(v)) if np.isscalar(v) else (int(v[0]), int(v[1]))


def _selfabs_addmm(self, self_2d, beta, M, N, rows=None, cols=None):
    if beta == 0.0:
        shape = (M, N) if rows is None else (len(rows),)
        return np.zeros(shape)
    s = self.astype(np.float64)
    if rows is None:
        full = s.reshape(M, N) if self_2d else np.broadcast_to(s, (M, N))
    else:
        full = s.reshape(M, N)[rows, cols] if self_2d else s[cols]
    return np.abs(np.float64(np.float32(beta)) * full)


def addmm(mat1, mat2, self, self_2d: bool, beta: float = 1.0, alpha: float = 1.0) -> Result:
    """Full [M,N] reference of beta*self + alpha*(mat1 @ mat2) in fp64."""
    mat1, mat2, self = _f32(mat1), _f32(mat2), _f32(self)
    M, K = mat1.shape
    K2, N = mat2.shape
    assert K == K2
    ref = np.empty((M, N), np.float64)
    sabs = np.empty((M, N), np.float64)
    _load().oracle_addmm(M, N, K, _ptr(mat1, _fp), _ptr(mat2, _fp), _ptr(self, _fp),
                         int(bool(self_2d)), beta, alpha, _ptr(ref, _dp), _ptr(sabs, _dp))
    return Result(ref, sabs, _selfabs_addmm(self, self_2d, beta, M, N))


def addmm_at(mat1, mat2, self, self_2d: bool, beta, alpha, rows, cols) -> Result:
    """Reference at sampled outputs (rows[s], cols[s])."""
    mat1, mat2, self = _f32(mat1), _f32(mat2), _f32(self)
    M, K = mat1.shape
    N = mat2.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert (rows >= 0).all() and (rows < M).all() and (cols >= 0).all() and (cols < N).all()
    n = rows.size
    ref = np.empty(n, np.float64)
    sabs = np.empty(n, np.float64)
    _load().oracle_addmm_at(M, N, K, _ptr(mat1, _fp), _ptr(mat2, _fp), _ptr(self, _fp),
                            int(bool(self_2d)), beta, alpha, n, _ptr(rows, _lp),
                            _ptr(cols, _lp), _ptr(ref, _dp), _ptr(sabs, _dp))
    return Result(ref, sabs, _selfabs_addmm(self, self_2d, beta, M, N, rows, cols))


def _selfabs_bias(bias, M, N, rows=None, cols=None):
    if bias is None:
        return np.zeros((M, N) if rows is None else (len(rows),))
    b = np.abs(bias.astype(np.float64))
    return np.broadcast_to(b, (M, N)) if rows is None else b[cols]


def linear(x, weight, bias=None) -> Result:
    """Full [M,N] reference of x[M,K] @ weight[N,K]^T + bias[N] in fp64."""
    x, weight, bias = _f32(x), _f32(weight), _f32(bias)
    M, K = x.shape
    N, K2 = weight.shape
    assert K == K2
    ref = np.empty((M, N), np.float64)
    sabs = np.empty((M, N), np.float64)
    _load().oracle_linear(M, N, K, _ptr(x, _fp), _ptr(weight, _fp), _ptr(bias, _fp),
                          _ptr(ref, _dp), _ptr(sabs, _dp))
    return Result(ref, sabs, _selfabs_bias(bias, M, N))


def linear_at(x, weight, bias, rows, cols) -> Result:
    """Linear reference at sampled outputs (rows[s], cols[s])."""
    x, weight, bias = _f32(x), _f32(weight), _f32(bias)
    M, K = x.shape
    N = weight.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert (rows >= 0).all() and (rows < M).all() and (cols >= 0).all() and (cols < N).all()
    n = rows.size
    ref = np.empty(n, np.float64)
    sabs = np.empty(n, np.float64)
    _load().oracle_linear_at(M, N, K, _ptr(x, _fp), _ptr(weight, _fp), _ptr(bias, _fp), n,
                             _ptr(rows, _lp), _ptr(cols, _lp), _ptr(ref, _dp), _ptr(sabs, _dp))
    return Result(ref, sabs, _selfabs_bias(bias, M, N, rows, cols))


def conv_out_size(size, k, stride, pad, dil) -> int:
    return int(_load().oracle_conv_out_size(size, k, stride, pad, dil))


def _conv_args(x, w, stride, padding, dilation, groups=1):
    B, IC, H, W = x.shape
    OC, IC2, KH, KW = w.shape
    assert IC == IC2 * groups, "weight must be [OC, IC/groups, KH, KW]"
    (sH, sW), (pH, pW), (dH, dW) = _pair(stride), _pair(padding), _pair(dilation)
    return (B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW)


def conv2d(x, w, bias=None, stride=1, padding=0, dilation=1) -> Result:
    """Full NCHW reference of the direct conv (groups == 1) plus bias[oc]."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _conv_args(x, w, stride, padding, dilation)
    B, OC = a[0], a[4]
    OH = conv_out_size(a[2], a[5], a[7], a[9], a[11])
    OW = conv_out_size(a[3], a[6], a[8], a[10], a[12])
    if OH <= 0 or OW <= 0:
        raise ValueError("empty conv output")
    ref = np.empty((B, OC, OH, OW), np.float64)
    sabs = np.empty((B, OC, OH, OW), np.float64)
    rc = _load().oracle_conv2d(*a, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp),
                               _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    bb = np.zeros(OC) if bias is None else np.abs(bias.astype(np.float64))
    return Result(ref, sabs, np.broadcast_to(bb[None, :, None, None], ref.shape))


def conv2d_at(x, w, bias, stride, padding, dilation, idx) -> Result:
    """Reference at sampled flat NCHW output indices."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _conv_args(x, w, stride, padding, dilation)
    B, OC = a[0], a[4]
    OH = conv_out_size(a[2], a[5], a[7], a[9], a[11])
    OW = conv_out_size(a[3], a[6], a[8], a[10], a[12])
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert (idx >= 0).all() and (idx < B * OC * OH * OW).all()
    n = idx.size
    ref = np.empty(n, np.float64)
    sabs = np.empty(n, np.float64)
    rc = _load().oracle_conv2d_at(*a, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp), n,
                                  _ptr(idx, _lp), _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    oc = (idx // (OH * OW)) % OC
    bb = np.zeros(n) if bias is None else np.abs(bias.astype(np.float64)[oc])
    return Result(ref, sabs, bb)


def conv2d_grouped(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1) -> Result:
    """Full NCHW reference of the grouped direct conv plus bias[oc]."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _conv_args(x, w, stride, padding, dilation, groups)
    B, OC = a[0], a[4]
    OH = conv_out_size(a[2], a[5], a[7], a[9], a[11])
    OW = conv_out_size(a[3], a[6], a[8], a[10], a[12])
    if OH <= 0 or OW <= 0:
        raise ValueError("empty conv output")
    ref = np.empty((B, OC, OH, OW), np.float64)
    sabs = np.empty((B, OC, OH, OW), np.float64)
    rc = _load().oracle_conv2d_grouped(*a, groups, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp),
                                       _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    bb = np.zeros(OC) if bias is None else np.abs(bias.astype(np.float64))
    return Result(ref, sabs, np.broadcast_to(bb[None, :, None, None], ref.shape))


def conv2d_grouped_at(x, w, bias, stride, padding, dilation, groups, idx) -> Result:
    """Grouped conv reference at sampled flat NCHW output indices."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _conv_args(x, w, stride, padding, dilation, groups)
    B, OC = a[0], a[4]
    OH = conv_out_size(a[2], a[5], a[7], a[9], a[11])
    OW = conv_out_size(a[3], a[6], a[8], a[10], a[12])
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert (idx >= 0).all() and (idx < B * OC * OH * OW).all()
    n = idx.size
    ref = np.empty(n, np.float64)
    sabs = np.empty(n, np.float64)
    rc = _load().oracle_conv2d_grouped_at(*a, groups, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp),
                                          n, _ptr(idx, _lp), _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    oc = (idx // (OH * OW)) % OC
    bb = np.zeros(n) if bias is None else np.abs(bias.astype(np.float64)[oc])
    return Result(ref, sabs, bb)


def _nhwc_args(x, w, stride, padding, dilation):
    B, H, W, IC = x.shape
    OC, KH, KW, IC2 = w.shape
    assert IC == IC2, "weight must be [OC, KH, KW, IC]"
    (sH, sW), (pH, pW), (dH, dW) = _pair(stride), _pair(padding), _pair(dilation)
    return (B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW)


def conv2d_nhwc(x, w, bias=None, stride=1, padding=0, dilation=1) -> Result:
    """Full [B,OH,OW,OC] reference of the channels-last conv: x [B,H,W,IC],
    w [OC,KH,KW,IC], bias [OC]."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _nhwc_args(x, w, stride, padding, dilation)
    B, OC = a[0], a[4]
    OH = conv_out_size(a[2], a[5], a[7], a[9], a[11])
    OW = conv_out_size(a[3], a[6], a[8], a[10], a[12])
    if OH <= 0 or OW <= 0:
        raise ValueError("empty conv output")
    ref = np.empty((B, OH, OW, OC), np.float64)
    sabs = np.empty((B, OH, OW, OC), np.float64)
    rc = _load().oracle_conv2d_nhwc(*a, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp),
                                    _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    bb = np.zeros(OC) if bias is None else np.abs(bias.astype(np.float64))
    return Result(ref, sabs, np.broadcast_to(bb, ref.shape))


def conv2d_nhwc_at(x, w, bias, stride, padding, dilation, idx) -> Result:
    """Channels-last conv reference at sampled flat NHWC output indices."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _nhwc_args(x, w, stride, padding, dilation)
    B, OC = a[0], a[4]
    OH = conv_out_size(a[2], a[5], a[7], a[9], a[11])
    OW = conv_out_size(a[3], a[6], a[8], a[10], a[12])
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert (idx >= 0).all() and (idx < B * OH * OW * OC).all()
    n = idx.size
    ref = np.empty(n, np.float64)
    sabs = np.empty(n, np.float64)
    rc = _load().oracle_conv2d_nhwc_at(*a, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp), n,
                                       _ptr(idx, _lp), _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    bb = np.zeros(n) if bias is None else np.abs(bias.astype(np.float64)[idx % OC])
    return Result(ref, sabs, bb)


def convt_out_size(size, k, stride, pad, dil, out_pad) -> int:
    return int(_load().oracle_convt_out_size(size, k, stride, pad, dil, out_pad))


def _convt_args(x, w, stride, padding, dilation, output_padding, groups):
    B, IC, H, W = x.shape
    IC2, OCg, KH, KW = w.shape
    assert IC == IC2, "weight must be [IC, OC/groups, KH, KW]"
    assert groups >= 1 and IC % groups == 0
    (sH, sW), (pH, pW), (dH, dW) = _pair(stride), _pair(padding), _pair(dilation)
    opH, opW = _pair(output_padding)
    return (B, IC, H, W, OCg * groups, KH, KW, sH, sW, pH, pW, dH, dW, opH, opW, groups)


def conv_transpose2d(x, w, bias=None, stride=1, padding=0, dilation=1, output_padding=0,
                     groups=1) -> Result:
    """Full [B,OC,OH,OW] reference of the transposed conv (scatter form):
    x [B,IC,H,W], w [IC,OC/groups,KH,KW], bias [OC].  Input channel ic only
    feeds the output channels of its group ic // (IC/groups)."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _convt_args(x, w, stride, padding, dilation, output_padding, groups)
    B, OC = a[0], a[4]
    OH = convt_out_size(a[2], a[5], a[7], a[9], a[11], a[13])
    OW = convt_out_size(a[3], a[6], a[8], a[10], a[12], a[14])
    if OH <= 0 or OW <= 0:
        raise ValueError("empty transposed-conv output")
    ref = np.empty((B, OC, OH, OW), np.float64)
    sabs = np.empty((B, OC, OH, OW), np.float64)
    rc = _load().oracle_conv_transpose2d(*a, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp),
                                         _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    bb = np.zeros(OC) if bias is None else np.abs(bias.astype(np.float64))
    return Result(ref, sabs, np.broadcast_to(bb[None, :, None, None], ref.shape))


def conv_transpose2d_at(x, w, bias, stride, padding, dilation, output_padding, idx,
                        groups=1) -> Result:
    """Transposed-conv reference (gather form) at sampled flat NCHW indices."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    a = _convt_args(x, w, stride, padding, dilation, output_padding, groups)
    B, OC = a[0], a[4]
    OH = convt_out_size(a[2], a[5], a[7], a[9], a[11], a[13])
    OW = convt_out_size(a[3], a[6], a[8], a[10], a[12], a[14])
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert (idx >= 0).all() and (idx < B * OC * OH * OW).all()
    n = idx.size
    ref = np.empty(n, np.float64)
    sabs = np.empty(n, np.float64)
    rc = _load().oracle_conv_transpose2d_at(*a, _ptr(x, _fp), _ptr(w, _fp), _ptr(bias, _fp), n,
                                            _ptr(idx, _lp), _ptr(ref, _dp), _ptr(sabs, _dp))
    assert rc == 0
    oc = (idx // (OH * OW)) % OC
    bb = np.zeros(n) if bias is None else np.abs(bias.astype(np.float64)[oc])
    return Result(ref, sabs, bb)


def im2col(x, KH, KW, stride=1, padding=0, dilation=1):
    """Explicit [IC*KH*KW, B*OH*OW] im2col matrix in fp64 (0 for padding taps)."""
    x = _f32(x)
    B, IC, H, W = x.shape
    (sH, sW), (pH, pW), (dH, dW) = _pair(stride), _pair(padding), _pair(dilation)
    OH = conv_out_size(H, KH, sH, pH, dH)
    OW = conv_out_size(W, KW, sW, pW, dW)
    col = np.empty((IC * KH * KW, B * OH * OW), np.float64)
    rc = _load().oracle_im2col(B, IC, H, W, KH, KW, sH, sW, pH, pW, dH, dW,
                               _ptr(x, _fp), _ptr(col, _dp))
    assert rc == 0
    return col


def tolerance(res: Result, K: int, alpha: float = 1.0):
    """Elementwise acceptance bound 4e-6*sqrt(K)*(|alpha|*sabs + |beta*self|)."""
    return 4e-6 * np.sqrt(K) * (abs(float(np.float32(alpha))) * res.sabs + res.selfabs)


def _sdpa_args(q, k, v, mask, scale):
    q, k, v, mask = _f32(q), _f32(k), _f32(v), _f32(mask)
    assert q.ndim >= 3 and k.ndim == q.ndim and v.shape == k.shape
    assert q.shape[:-2] == k.shape[:-2] and q.shape[-1] == k.shape[-1]
    Sq, D = q.shape[-2:]
    Skv = k.shape[-2]
    BH = int(np.prod(q.shape[:-2]))
    if mask is not None:
        assert mask.shape == q.shape[:-1] + (Skv,), "mask must be [..., Sq, Skv]"
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    return q, k, v, mask, float(np.float32(scale)), BH, Sq, Skv, D


def sdpa(q, k, v, mask=None, scale=None) -> SdpaResult:
    """Full reference of softmax(q @ k^T * scale + mask) @ v in fp64.

    q [..., Sq, D], k and v [..., Skv, D], mask [..., Sq, Skv] or None;
    scale None means 1/sqrt(D) (rounded to fp32, the value a kernel sees).
    """
    q, k, v, mask, scale, BH, Sq, Skv, D = _sdpa_args(q, k, v, mask, scale)
    ref = np.empty(q.shape, np.float64)
    err = np.empty(q.shape, np.float64)
    rc = _load().oracle_sdpa(BH, Sq, Skv, D, _ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp),
                             _ptr(mask, _fp), scale, _ptr(ref, _dp), _ptr(err, _dp))
    if rc != 0:
        raise ValueError("attention over an empty key set")
    return SdpaResult(ref, err)


def sdpa_rows(q, k, v, mask, scale, rows) -> SdpaResult:
    """Reference at sampled query rows (flat index bh*Sq + i): [n, D]."""
    q, k, v, mask, scale, BH, Sq, Skv, D = _sdpa_args(q, k, v, mask, scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.ndim == 1 and (rows >= 0).all() and (rows < BH * Sq).all()
    n = rows.size
    ref = np.empty((n, D), np.float64)
    err = np.empty((n, D), np.float64)
    rc = _load().oracle_sdpa_rows(BH, Sq, Skv, D, _ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp),
                                  _ptr(mask, _fp), scale, n, _ptr(rows, _lp), _ptr(ref, _dp),
                                  _ptr(err, _dp))
    if rc != 0:
        raise ValueError("attention over an empty key set")
    return SdpaResult(ref, err)


def sdpa_tolerance(res: SdpaResult):
    """Elementwise acceptance bound 4e-6 * err (err in fp32 rounding units)."""
    return 4e-6 * res.err
