"""ctypes view of libbaim.so: the C ABI declared in include/baim.h.

Argument marshalling only.  There is no fallback: if the library is missing
the first call raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbaim.so")

BAIM_OK = 0
BAIM_ERR_NULL = 1
BAIM_ERR_SHAPE = 2
BAIM_ERR_UNSUPPORTED = 3
BAIM_ERR_TOO_LARGE = 4
BAIM_ERR_ALIAS = 5
BAIM_ERR_LAUNCH = 6

STATUS_NAMES = {
    0: "BAIM_OK", 1: "BAIM_ERR_NULL", 2: "BAIM_ERR_SHAPE", 3: "BAIM_ERR_UNSUPPORTED",
    4: "BAIM_ERR_TOO_LARGE", 5: "BAIM_ERR_ALIAS", 6: "BAIM_ERR_LAUNCH",
}

# Every symbol include/baim.h declares.
EXPORTS = ("addmm_f32", "linear_f32", "conv2d_gemm_f32", "conv2d_nhwc_f32",
           "conv_transpose2d_f32", "sdpa_f32", "baim_conv2d_out_hw", "baim_conv_transpose2d_out_hw",
           "baim_gemm_plan", "baim_conv2d_plan", "baim_conv2d_nhwc_plan", "baim_last_error",
           "baim_version")

_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def lib():
    """Load libbaim.so once and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m bias_addmm_im2col_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    L = ctypes.CDLL(LIB_PATH)
    L.addmm_f32.argtypes = [_vp, _vp, ctypes.c_int, _vp, _vp, _i64, _i64, _i64,
                            ctypes.c_float, ctypes.c_float, _vp]
    L.addmm_f32.restype = ctypes.c_int
    L.linear_f32.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
    L.linear_f32.restype = ctypes.c_int
    L.conv2d_gemm_f32.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 14 + [_vp]
    L.conv2d_gemm_f32.restype = ctypes.c_int
    L.conv2d_nhwc_f32.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 13 + [_vp]
    L.conv2d_nhwc_f32.restype = ctypes.c_int
    L.conv_transpose2d_f32.argtypes = [_vp, _vp, _vp, _vp] + [_i64] * 16 + [_vp]
    L.conv_transpose2d_f32.restype = ctypes.c_int
    L.baim_conv_transpose2d_out_hw.argtypes = [_i64] * 12 + [ctypes.POINTER(_i64)] * 2
    L.baim_conv_transpose2d_out_hw.restype = ctypes.c_int
    L.sdpa_f32.argtypes = [_vp] * 5 + [_i64] * 4 + [ctypes.POINTER(ctypes.c_float), _vp]
    L.sdpa_f32.restype = ctypes.c_int
    L.baim_conv2d_out_hw.argtypes = [_i64] * 10 + [ctypes.POINTER(_i64)] * 2
    L.baim_conv2d_out_hw.restype = ctypes.c_int
    L.baim_gemm_plan.argtypes = [_i64] * 3 + [ctypes.POINTER(ctypes.c_int)] * 7
    L.baim_gemm_plan.restype = ctypes.c_int
    L.baim_conv2d_plan.argtypes = [_i64] * 14 + [ctypes.POINTER(ctypes.c_int)] * 8
    L.baim_conv2d_plan.restype = ctypes.c_int
    L.baim_conv2d_nhwc_plan.argtypes = [_i64] * 13 + [ctypes.POINTER(ctypes.c_int)]
    L.baim_conv2d_nhwc_plan.restype = ctypes.c_int
    L.baim_last_error.argtypes = []
    L.baim_last_error.restype = ctypes.c_char_p
    L.baim_version.argtypes = []
    L.baim_version.restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().baim_last_error().decode()


def addmm_f32(out, self, self_2d, mat1, mat2, M, N, K, beta, alpha, stream) -> int:
    return lib().addmm_f32(out, self, self_2d, mat1, mat2, M, N, K, beta, alpha, stream)


def linear_f32(out, x, w, bias, M, N, K, stream) -> int:
    return lib().linear_f32(out, x, w, bias, M, N, K, stream)


def conv2d_nhwc_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW,
                    stream) -> int:
    return lib().conv2d_nhwc_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH,
                                 dW, stream)


def conv_transpose2d_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW,
                         opH, opW, groups, stream) -> int:
    return lib().conv_transpose2d_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW,
                                      dH, dW, opH, opW, groups, stream)


def conv_transpose2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, opH, opW):
    oh, ow = _i64(0), _i64(0)
    st = lib().baim_conv_transpose2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, opH, opW,
                                            ctypes.byref(oh), ctypes.byref(ow))
    return st, oh.value, ow.value


def sdpa_f32(out, q, k, v, mask, BH, Sq, Skv, D, scale, stream) -> int:
    sc = None if scale is None else ctypes.byref(ctypes.c_float(scale))
    return lib().sdpa_f32(out, q, k, v, mask, BH, Sq, Skv, D, sc, stream)


def conv2d_gemm_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW,
                    groups, stream) -> int:
    return lib().conv2d_gemm_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW,
                                 dH, dW, groups, stream)


def gemm_plan(M, N, K):
    """(status, dict) with the tile the library picks for an M x N x K GEMM."""
    outs = [ctypes.c_int(0) for _ in range(7)]
    st = lib().baim_gemm_plan(M, N, K, *[ctypes.byref(o) for o in outs])
    keys = ("bm", "bn", "bk", "waves", "kgroups", "splits", "stream_blocks")
    return st, {k: o.value for k, o in zip(keys, outs)}


def conv2d_plan(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, groups):
    """(status, dict) with the kernel and tile conv2d_gemm_f32 uses."""
    outs = [ctypes.c_int(0) for _ in range(8)]
    st = lib().baim_conv2d_plan(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, groups,
                                *[ctypes.byref(o) for o in outs])
    keys = ("kernel", "bm", "bn", "bk", "waves", "kgroups", "splits", "stream_blocks")
    return st, {k: o.value for k, o in zip(keys, outs)}


def conv2d_nhwc_plan(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW):
    """(status, dict) with the kernel conv2d_nhwc_f32 uses."""
    k = ctypes.c_int(0)
    st = lib().baim_conv2d_nhwc_plan(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW,
                                     ctypes.byref(k))
    return st, {"kernel": k.value}


def conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW):
    oh, ow = _i64(0), _i64(0)
    st = lib().baim_conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW,
                                  ctypes.byref(oh), ctypes.byref(ow))
    return st, oh.value, ow.value
