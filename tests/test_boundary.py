"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol include/baim.h declares, and rejects every invalid call before
anything is enqueued.

No case here reaches a kernel launch: every call either fails validation or
has an empty output.  Pointers are fake, non-NULL addresses that are never
dereferenced.
"""
import os
import re

import pytest

from bias_addmm_im2col_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x10000000  # fake device addresses, 256 MiB apart
A, Bp, S, O = P, 2 * P, 3 * P, 4 * P


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_capi.LIB_PATH):
        import bias_addmm_im2col_amd.build as b
        b.build()
    return _capi.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "baim.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_capi.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"libbaim.so does not export {n}"
    assert lib.baim_version() >= 100


def addmm(out=O, self=S, self_2d=0, a=A, b=Bp, M=8, N=8, K=8, beta=1.0, alpha=1.0):
    return _capi.addmm_f32(out, self, self_2d, a, b, M, N, K, beta, alpha, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), _capi.BAIM_ERR_SHAPE),
    (dict(N=-3), _capi.BAIM_ERR_SHAPE),
    (dict(K=-1), _capi.BAIM_ERR_SHAPE),
    (dict(self_2d=2), _capi.BAIM_ERR_SHAPE),
    (dict(out=None), _capi.BAIM_ERR_NULL),
    (dict(self=None), _capi.BAIM_ERR_NULL),
    (dict(a=None), _capi.BAIM_ERR_NULL),
    (dict(b=None), _capi.BAIM_ERR_NULL),
    (dict(M=1 << 16, K=1 << 15), _capi.BAIM_ERR_TOO_LARGE),
    (dict(M=1 << 16, N=1 << 15), _capi.BAIM_ERR_TOO_LARGE),
    (dict(M=1, N=1, K=1 << 21), _capi.BAIM_ERR_TOO_LARGE),
    (dict(M=1, K=1, N=1 << 23), _capi.BAIM_ERR_TOO_LARGE),
    (dict(M=1 << 40, N=1 << 40), _capi.BAIM_ERR_TOO_LARGE),
    (dict(out=A + 4), _capi.BAIM_ERR_ALIAS),          # out inside mat1
    (dict(out=Bp - 16), _capi.BAIM_ERR_ALIAS),        # out runs into mat2
    (dict(out=S, self_2d=1), _capi.BAIM_ERR_ALIAS),   # in-place on self
])
def test_addmm_rejects(lib, kw, status):
    st = addmm(**kw)
    assert st == status, (st, _capi.last_error())
    assert _capi.last_error()


def test_addmm_beta_zero_needs_no_self_and_checks_no_self_alias(lib):
    # beta == 0: self may be NULL and may even alias out; still rejected here
    # only because of an unrelated problem (NULL mat1), never because of self.
    assert addmm(self=None, beta=0.0, a=None) == _capi.BAIM_ERR_NULL
    assert "mat1" in _capi.last_error()
    assert addmm(self=O, beta=0.0, a=None) == _capi.BAIM_ERR_NULL


def test_addmm_empty_output_is_ok_without_launch(lib):
    assert addmm(M=0) == _capi.BAIM_OK
    assert addmm(N=0, out=None, self=None, a=None, b=None) == _capi.BAIM_OK
    assert _capi.last_error() == ""


def linear(out=O, x=A, w=Bp, bias=S, M=8, N=8, K=8):
    return _capi.linear_f32(out, x, w, bias, M, N, K, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), _capi.BAIM_ERR_SHAPE),
    (dict(K=-2), _capi.BAIM_ERR_SHAPE),
    (dict(out=None), _capi.BAIM_ERR_NULL),
    (dict(x=None), _capi.BAIM_ERR_NULL),
    (dict(w=None), _capi.BAIM_ERR_NULL),
    (dict(M=1 << 16, K=1 << 15), _capi.BAIM_ERR_TOO_LARGE),
    (dict(N=1 << 16, K=1 << 15), _capi.BAIM_ERR_TOO_LARGE),
    (dict(M=1, N=1, K=1 << 21), _capi.BAIM_ERR_TOO_LARGE),
    (dict(out=A + 4), _capi.BAIM_ERR_ALIAS),
    (dict(out=Bp - 8), _capi.BAIM_ERR_ALIAS),
    (dict(out=S - 4), _capi.BAIM_ERR_ALIAS),
])
def test_linear_rejects(lib, kw, status):
    st = linear(**kw)
    assert st == status, (st, _capi.last_error())
    assert _capi.last_error()


def test_linear_null_bias_and_empty_are_fine_to_validate(lib):
    assert linear(M=0) == _capi.BAIM_OK
    assert linear(N=0, out=None, x=None, w=None) == _capi.BAIM_OK


def conv(out=O, x=A, w=Bp, bias=S, B=1, IC=3, H=8, W=8, OC=4, KH=3, KW=3, sH=1, sW=1, pH=1,
         pW=1, dH=1, dW=1, groups=1):
    return _capi.conv2d_gemm_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH,
                                 dW, groups, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), _capi.BAIM_ERR_SHAPE),
    (dict(IC=0), _capi.BAIM_ERR_SHAPE),
    (dict(OC=0), _capi.BAIM_ERR_SHAPE),
    (dict(H=0), _capi.BAIM_ERR_SHAPE),
    (dict(KW=0), _capi.BAIM_ERR_SHAPE),
    (dict(sH=0), _capi.BAIM_ERR_SHAPE),
    (dict(dW=0), _capi.BAIM_ERR_SHAPE),
    (dict(pH=-1), _capi.BAIM_ERR_SHAPE),
    (dict(H=2, KH=5, pH=0), _capi.BAIM_ERR_SHAPE),      # kernel larger than input
    (dict(H=5, KH=3, dH=3, pH=0), _capi.BAIM_ERR_SHAPE),  # dilated kernel too large
    (dict(groups=0), _capi.BAIM_ERR_SHAPE),
    (dict(groups=3), _capi.BAIM_ERR_SHAPE),          # 3 does not divide OC = 4
    (dict(groups=2, IC=3, OC=4), _capi.BAIM_ERR_SHAPE),  # 2 does not divide IC = 3
    (dict(groups=70000, IC=70000, OC=70000, KH=1, KW=1, pH=0, pW=0, H=1, W=1),
     _capi.BAIM_ERR_TOO_LARGE),
    (dict(out=None), _capi.BAIM_ERR_NULL),
    (dict(x=None), _capi.BAIM_ERR_NULL),
    (dict(w=None), _capi.BAIM_ERR_NULL),
    (dict(B=1 << 12, IC=1 << 10, H=1 << 9, W=1), _capi.BAIM_ERR_TOO_LARGE),
    (dict(IC=1 << 20, KH=3, KW=3, H=3, W=3), _capi.BAIM_ERR_TOO_LARGE),
    (dict(H=40000, W=40000, pH=1, pW=1, IC=1), _capi.BAIM_ERR_TOO_LARGE),
    (dict(out=A + 8), _capi.BAIM_ERR_ALIAS),
    (dict(out=S - 4), _capi.BAIM_ERR_ALIAS),  # out runs into bias
])
def test_conv_rejects(lib, kw, status):
    st = conv(**kw)
    assert st == status, (st, _capi.last_error())
    assert _capi.last_error()


def test_conv_out_hw(lib):
    assert _capi.conv2d_out_hw(768, 768, 7, 7, 4, 4, 3, 3, 1, 1) == (0, 192, 192)
    assert _capi.conv2d_out_hw(56, 56, 3, 3, 1, 1, 2, 2, 2, 2) == (0, 56, 56)
    assert _capi.conv2d_out_hw(57, 57, 3, 3, 2, 2, 1, 1, 1, 1) == (0, 29, 29)
    assert _capi.conv2d_out_hw(10, 7, 3, 2, 3, 1, 0, 2, 1, 3) == (0, 3, 8)  # (7+4-3-1)//1+1
    st, oh, ow = _capi.conv2d_out_hw(2, 2, 5, 5, 1, 1, 0, 0, 1, 1)
    assert st == _capi.BAIM_ERR_SHAPE and (oh, ow) == (0, 0)
    assert lib.baim_conv2d_out_hw(1, 1, 1, 1, 1, 1, 0, 0, 1, 1, None, None) == _capi.BAIM_ERR_NULL


def test_gemm_plan(lib, monkeypatch):
    import bias_addmm_im2col_amd as baim
    monkeypatch.delenv("BAIM_TILE", raising=False)
    p = baim.gemm_plan(4096, 4096, 1024)
    assert (p["bm"], p["bn"], p["bk"], p["waves"], p["kgroups"], p["splits"]) == (256, 256, 16, 8, 1, 1)
    p = baim.gemm_plan(8192, 4096, 256)  # K below 512: the 128x128 tile
    assert (p["bm"], p["bn"], p["bk"], p["waves"], p["kgroups"], p["splits"]) == (128, 128, 32, 8, 1, 1)
    # every workload shape is planned without a cross-block K split
    from bias_addmm_im2col_amd import inputs as I
    for c in I.CASES.values():
        M, N, K = (c.M, c.N, c.K) if c.kind != "conv" else c.gemm_mnk
        assert baim.gemm_plan(M, N, K)["splits"] <= 2, c.name
    monkeypatch.setenv("BAIM_TILE", "7,3")
    p = baim.gemm_plan(300, 300, 30000)
    assert (p["bm"], p["bn"], p["bk"], p["waves"], p["kgroups"], p["splits"]) == (64, 64, 128, 16, 4, 3)
    st, _ = _capi.gemm_plan(-1, 2, 3)
    assert st == _capi.BAIM_ERR_SHAPE
    assert lib.baim_gemm_plan(1, 1, 1, None, None, None, None, None, None, None) == \
        _capi.BAIM_ERR_NULL
    monkeypatch.setenv("BAIM_TILE", "1,s256")
    p = baim.gemm_plan(256, 12544, 2304)
    assert (p["bm"], p["bn"], p["splits"], p["stream_blocks"]) == (128, 64, 1, 256)


def conv_nhwc(out=O, x=A, w=Bp, bias=S, B=1, IC=3, H=8, W=8, OC=4, KH=3, KW=3, sH=1, sW=1,
              pH=1, pW=1, dH=1, dW=1):
    return _capi.conv2d_nhwc_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH,
                                 dW, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), _capi.BAIM_ERR_SHAPE),
    (dict(IC=0), _capi.BAIM_ERR_SHAPE),
    (dict(sH=0), _capi.BAIM_ERR_SHAPE),
    (dict(pW=-1), _capi.BAIM_ERR_SHAPE),
    (dict(KH=20), _capi.BAIM_ERR_SHAPE),                   # empty output
    (dict(out=None), _capi.BAIM_ERR_NULL),
    (dict(w=None), _capi.BAIM_ERR_NULL),
    (dict(B=1, H=1 << 14, W=1 << 13, IC=4), _capi.BAIM_ERR_TOO_LARGE),   # input 2^29
    (dict(IC=1 << 18, KH=3, KW=3), _capi.BAIM_ERR_TOO_LARGE),            # K >= 2^21
    (dict(OC=1 << 23, H=1, W=1, KH=1, KW=1, pH=0, pW=0), _capi.BAIM_ERR_TOO_LARGE),
    (dict(out=A + 8), _capi.BAIM_ERR_ALIAS),
    (dict(out=S - 4), _capi.BAIM_ERR_ALIAS),
])
def test_conv_nhwc_rejects(lib, kw, status):
    st = conv_nhwc(**kw)
    assert st == status, (st, _capi.last_error())
    assert _capi.last_error()


def convt(out=O, x=A, w=Bp, bias=S, B=1, IC=4, H=8, W=8, OC=4, KH=3, KW=3, sH=2, sW=2, pH=1,
          pW=1, dH=1, dW=1, opH=0, opW=0, groups=1):
    return _capi.conv_transpose2d_f32(out, x, w, bias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW,
                                      dH, dW, opH, opW, groups, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), _capi.BAIM_ERR_SHAPE),
    (dict(groups=3), _capi.BAIM_ERR_SHAPE),             # does not divide IC
    (dict(groups=0), _capi.BAIM_ERR_SHAPE),
    (dict(sW=0), _capi.BAIM_ERR_SHAPE),
    (dict(opH=2), _capi.BAIM_ERR_SHAPE),                # output padding >= max(stride, dilation)
    (dict(opW=-1), _capi.BAIM_ERR_SHAPE),
    (dict(H=1, KH=1, pH=1, sH=1), _capi.BAIM_ERR_SHAPE),  # empty output
    (dict(out=None), _capi.BAIM_ERR_NULL),
    (dict(x=None), _capi.BAIM_ERR_NULL),
    (dict(IC=1 << 20, H=32, W=32), _capi.BAIM_ERR_TOO_LARGE),   # input 2^30
    (dict(IC=1 << 18, OC=2, KH=3, KW=3, H=1, W=1), _capi.BAIM_ERR_TOO_LARGE),  # K >= 2^21
    (dict(out=A + 8), _capi.BAIM_ERR_ALIAS),
    (dict(out=S - 4), _capi.BAIM_ERR_ALIAS),
])
def test_conv_transpose_rejects(lib, kw, status):
    st = convt(**kw)
    assert st == status, (st, _capi.last_error())
    assert _capi.last_error()


def test_conv_transpose_out_hw(lib):
    assert _capi.conv_transpose2d_out_hw(28, 28, 4, 4, 2, 2, 1, 1, 1, 1, 0, 0) == (0, 56, 56)
    assert _capi.conv_transpose2d_out_hw(64, 64, 2, 2, 2, 2, 0, 0, 1, 1, 0, 0) == (0, 128, 128)
    assert _capi.conv_transpose2d_out_hw(4, 5, 3, 3, 2, 2, 1, 1, 2, 2, 1, 0) == (0, 10, 11)
    st, oh, ow = _capi.conv_transpose2d_out_hw(4, 4, 3, 3, 2, 2, 1, 1, 1, 1, 2, 0)
    assert st == _capi.BAIM_ERR_SHAPE and (oh, ow) == (0, 0)


M5 = 5 * P  # fake mask address


def sdpa(out=O, q=A, k=Bp, v=S, mask=None, BH=2, Sq=8, Skv=8, D=16, scale=None):
    return _capi.sdpa_f32(out, q, k, v, mask, BH, Sq, Skv, D, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(BH=-1), _capi.BAIM_ERR_SHAPE),
    (dict(Skv=-3), _capi.BAIM_ERR_SHAPE),
    (dict(Skv=0), _capi.BAIM_ERR_SHAPE),
    (dict(D=6), _capi.BAIM_ERR_UNSUPPORTED),
    (dict(D=132), _capi.BAIM_ERR_UNSUPPORTED),
    (dict(out=None), _capi.BAIM_ERR_NULL),
    (dict(v=None), _capi.BAIM_ERR_NULL),
    (dict(q=A + 4), _capi.BAIM_ERR_UNSUPPORTED),   # not on a 16-byte boundary
    (dict(k=Bp + 8), _capi.BAIM_ERR_UNSUPPORTED),
    (dict(out=A + 64), _capi.BAIM_ERR_ALIAS),      # out inside q
    (dict(out=S - 4), _capi.BAIM_ERR_ALIAS),       # out runs into v
    (dict(mask=M5, out=M5 + 4), _capi.BAIM_ERR_ALIAS),
    (dict(BH=1 << 20, Sq=1 << 11, D=8), _capi.BAIM_ERR_TOO_LARGE),
    (dict(BH=1, Sq=1 << 27, D=4), _capi.BAIM_ERR_TOO_LARGE),       # Sq*D = 2^29
    (dict(BH=1, Sq=1 << 15, Skv=1 << 14, D=4, mask=M5), _capi.BAIM_ERR_TOO_LARGE),
])
def test_sdpa_rejects(lib, kw, status):
    st = sdpa(**kw)
    assert st == status, (st, _capi.last_error())
    assert _capi.last_error()


def test_sdpa_empty_output_is_ok_without_launch(lib):
    assert sdpa(Sq=0) == _capi.BAIM_OK
    assert sdpa(BH=0, Skv=0) == _capi.BAIM_OK
    assert sdpa(D=0, out=None, q=None, k=None, v=None) == _capi.BAIM_OK
    # a large mask is fine when no mask is passed
    assert sdpa(BH=1, Sq=1 << 15, Skv=1 << 14, D=4, out=None) == _capi.BAIM_ERR_NULL


def test_python_layer_checks_before_the_library():
    """Dtype/device/shape errors of the torch wrapper, raised on the CPU."""
    import torch
    import bias_addmm_im2col_amd as baim
    with pytest.raises(TypeError):
        baim.addmm(torch.zeros(3), torch.zeros(2, 3, dtype=torch.float64), torch.zeros(3, 3))
    with pytest.raises(ValueError):
        baim.addmm(torch.zeros(3), torch.zeros(2, 3), torch.zeros(3, 3))  # CPU tensors
    with pytest.raises(ValueError):  # CPU tensors
        baim.conv2d(torch.zeros(1, 4, 5, 5), torch.zeros(4, 2, 3, 3), groups=2)
    with pytest.raises(TypeError):
        baim.sdpa(torch.zeros(1, 2, 4, dtype=torch.float64), torch.zeros(1, 2, 4), torch.zeros(1, 2, 4))
    with pytest.raises(ValueError):  # CPU tensors
        baim.sdpa(torch.zeros(1, 2, 4), torch.zeros(1, 2, 4), torch.zeros(1, 2, 4))
