"""fp32 tiled GEMM with a fused epilogue for AMD MI355X (gfx950).

Two operations, both computed by the hand-written HIP kernels in
``libbaim.so`` (C ABI in include/baim.h); this package only marshals
arguments and allocates outputs with torch:

* ``addmm(self, mat1, mat2, *, beta=1, alpha=1)`` --
  ``beta*self + alpha*(mat1 @ mat2)`` with self ``[N]`` (or ``[1,N]``) or
  ``[M,N]`` ("[ExecuTorch][WebGPU] Add optimized addmm op", Solution).
* ``linear(x, weight, bias=None)`` -- ``x @ weight^T + bias`` with weight
  ``[N,K]``, the linear_fp32 form the addmm page shares its GEMM with.
* ``conv2d(input, weight, bias=None, stride=1, padding=0, dilation=1,
  groups=1)`` -- NCHW convolution; groups==1 as an implicit-im2col GEMM
  ("et_vk conv2d: route standard (groups==1) conv through an im2col tiled
  GEMM", Solution/Implementation), grouped convs as one such GEMM per group
  or, when the groups are small (e.g. depthwise), on a direct kernel.

* ``conv2d_nhwc(input, weight, bias=None, stride=1, padding=0, dilation=1)``
  -- the same conv (groups == 1) on channels-last tensors: input [B,H,W,IC],
  weight [OC,KH,KW,IC], output [B,OH,OW,OC]; the implicit im2col then reads
  K (a tap's input channels) contiguously.
* ``conv_transpose2d(input, weight, bias=None, stride=1, padding=0,
  output_padding=0, groups=1, dilation=1)`` -- the transposed conv (weight
  [IC, OC/groups, KH, KW], aten's argument order), as one dense implicit
  GEMM per output phase.
* ``sdpa(q, k, v, attn_mask=None, scale=None)`` -- non-causal attention
  ``softmax(q @ k^T * scale + attn_mask) @ v`` over [..., S, D] tensors
  ("[ExecuTorch][WebGPU] Add optimized SDPA op", Problem/Solution), in one
  fused pass.

``addmm_f32``, ``linear_f32``, ``conv2d_gemm_f32``, ``conv2d_nhwc_f32``,
``conv_transpose2d_f32`` and ``sdpa_f32`` are the
same-named entry points of the C ABI taking caller-allocated tensors.  Tensors must be fp32, contiguous and
on the same ROCm device; work is enqueued on the current torch stream.
"""
from __future__ import annotations

from . import _capi

__all__ = ["addmm", "linear", "conv2d", "conv2d_nhwc", "conv_transpose2d", "sdpa", "addmm_f32",
           "linear_f32", "conv2d_gemm_f32", "conv2d_nhwc_f32", "conv_transpose2d_f32", "sdpa_f32",
           "conv_transpose2d_out_hw", "conv2d_out_hw", "gemm_plan", "conv2d_plan", "conv2d_nhwc_plan",
           "BaimError", "library_path"]


class BaimError(RuntimeError):
    """A non-OK status from libbaim.so."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_capi.STATUS_NAMES.get(status, status)}: {message}")


class BaimValueError(BaimError, ValueError):
    pass


class BaimUnsupportedError(BaimError, NotImplementedError):
    pass


def library_path() -> str:
    return _capi.LIB_PATH


def _check(status: int):
    if status == _capi.BAIM_OK:
        return
    msg = _capi.last_error()
    if status == _capi.BAIM_ERR_UNSUPPORTED:
        raise BaimUnsupportedError(status, msg)
    if status == _capi.BAIM_ERR_LAUNCH:
        raise BaimError(status, msg)
    raise BaimValueError(status, msg)


def _pair(v, name):
    if isinstance(v, int):
        return v, v
    v = tuple(int(a) for a in v)
    if len(v) != 2:
        raise ValueError(f"{name} must be an int or a pair")
    return v


def _scalar(v, name) -> float:
    # Double, Int or None accepted, None meaning 1 (the page's scalar_or).
    if v is None:
        return 1.0
    if isinstance(v, bool) or not isinstance(v, (int, float)):
        raise TypeError(f"{name} must be an int or float")
    return float(v)


def _dev_f32(t, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32 (got {t.dtype})")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(dev):
    import torch
    return torch.cuda.current_stream(dev).cuda_stream


def _on(dev):
    """Make `dev` the current device for the call, unless it already is."""
    import contextlib
    import torch
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def addmm_f32(out, self, mat1, mat2, beta=1.0, alpha=1.0):
    """out[M,N] = beta*self + alpha*(mat1 @ mat2), written into ``out``.

    self is [N], [1,N] or [M,N]; it may be None when beta == 0."""
    import torch
    beta, alpha = _scalar(beta, "beta"), _scalar(alpha, "alpha")
    out, mat1, mat2 = _dev_f32(out, "out"), _dev_f32(mat1, "mat1"), _dev_f32(mat2, "mat2")
    if mat1.dim() != 2 or mat2.dim() != 2 or out.dim() != 2:
        raise ValueError("mat1, mat2 and out must be 2-D")
    M, K = mat1.shape
    if mat2.shape[0] != K:
        raise ValueError(f"mat2 must be [K={K}, N], got {list(mat2.shape)}")
    N = mat2.shape[1]
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}], got {list(out.shape)}")
    devs = {t.device for t in (out, mat1, mat2)}
    self_ptr, self_2d = None, 0
    if self is not None:
        self = _dev_f32(self, "self")
        devs.add(self.device)
        if tuple(self.shape) in ((N,), (1, N)):
            self_2d = 0
        elif tuple(self.shape) == (M, N):
            self_2d = 1
        else:
            raise ValueError(f"self must be [N], [1,N] or [M,N] with M={M}, N={N}; "
                             f"got {list(self.shape)}")
        self_ptr = self.data_ptr()
    elif beta != 0.0:
        raise ValueError("self is required unless beta == 0")
    if len(devs) != 1:
        raise ValueError("all tensors must be on the same device")
    dev = out.device
    with _on(dev):
        st = _capi.addmm_f32(out.data_ptr(), self_ptr, self_2d, mat1.data_ptr(),
                             mat2.data_ptr(), M, N, K, beta, alpha, _stream(dev))
    _check(st)
    return out


def addmm(self, mat1, mat2, *, beta=1, alpha=1):
    """beta*self + alpha*(mat1 @ mat2) as a new [M,N] fp32 tensor."""
    import torch
    _dev_f32(mat1, "mat1")
    _dev_f32(mat2, "mat2")
    out = torch.empty((mat1.shape[0], mat2.shape[1]), dtype=torch.float32, device=mat1.device)
    return addmm_f32(out, self, mat1, mat2, beta, alpha)


def linear_f32(out, x, weight, bias=None):
    """out[M,N] = x[M,K] @ weight[N,K]^T + bias[N], written into ``out``."""
    import torch
    out, x, weight = _dev_f32(out, "out"), _dev_f32(x, "x"), _dev_f32(weight, "weight")
    if x.dim() != 2 or weight.dim() != 2 or out.dim() != 2:
        raise ValueError("x, weight and out must be 2-D")
    M, K = x.shape
    N, K2 = weight.shape
    if K2 != K:
        raise ValueError(f"weight must be [N, K={K}], got {list(weight.shape)}")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}], got {list(out.shape)}")
    devs = {out.device, x.device, weight.device}
    bias_ptr = None
    if bias is not None:
        bias = _dev_f32(bias, "bias")
        if tuple(bias.shape) != (N,):
            raise ValueError(f"bias must be [{N}]")
        bias_ptr = bias.data_ptr()
        devs.add(bias.device)
    if len(devs) != 1:
        raise ValueError("all tensors must be on the same device")
    dev = out.device
    with _on(dev):
        st = _capi.linear_f32(out.data_ptr(), x.data_ptr(), weight.data_ptr(), bias_ptr, M, N, K,
                              _stream(dev))
    _check(st)
    return out


def linear(x, weight, bias=None):
    """x[..., K] @ weight[N, K]^T + bias[N] as a new [..., N] fp32 tensor."""
    import torch
    x, weight = _dev_f32(x, "x"), _dev_f32(weight, "weight")
    if weight.dim() != 2 or x.dim() < 1:
        raise ValueError("weight must be 2-D and x at least 1-D")
    lead = tuple(x.shape[:-1])
    x2 = x.reshape(-1, x.shape[-1])
    out = torch.empty((x2.shape[0], weight.shape[0]), dtype=torch.float32, device=x.device)
    linear_f32(out, x2, weight, bias)
    return out.reshape(lead + (weight.shape[0],))


def gemm_plan(M, N, K):
    """How the library computes an M x N x K GEMM (dict with bm, bn, bk,
    waves, kgroups, splits, stream_blocks).  Host-only."""
    st, plan = _capi.gemm_plan(M, N, K)
    _check(st)
    return plan


def conv2d_nhwc_plan(input_shape, weight_shape, stride=1, padding=0, dilation=1):
    """Which kernel conv2d_nhwc_f32 runs for these shapes (input [B,H,W,IC],
    weight [OC,KH,KW,IC]): dict with kernel (0 the addmm kernels with an
    im2col A operand, 3 the stem kernel).  Host-only."""
    B, H, W, IC = (int(v) for v in input_shape)
    OC, KH, KW, _ = (int(v) for v in weight_shape)
    (sH, sW), (pH, pW), (dH, dW) = (_pair(stride, "stride"), _pair(padding, "padding"),
                                    _pair(dilation, "dilation"))
    st, plan = _capi.conv2d_nhwc_plan(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW)
    _check(st)
    return plan


def conv2d_plan(input_shape, weight_shape, stride=1, padding=0, dilation=1, groups=1):
    """How conv2d_gemm_f32 computes a conv of these shapes (input [B,IC,H,W],
    weight [OC,IC/groups,KH,KW]): dict with kernel (0 implicit-im2col GEMM,
    1 LDS-window kernel, 2 direct grouped kernel), bm, bn, bk, waves,
    kgroups, splits, stream_blocks.  Host-only."""
    B, IC, H, W = (int(v) for v in input_shape)
    OC, _, KH, KW = (int(v) for v in weight_shape)
    (sH, sW), (pH, pW), (dH, dW) = (_pair(stride, "stride"), _pair(padding, "padding"),
                                    _pair(dilation, "dilation"))
    st, plan = _capi.conv2d_plan(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, int(groups))
    _check(st)
    return plan


def conv2d_out_hw(H, W, KH, KW, stride=1, padding=0, dilation=1):
    (sH, sW), (pH, pW), (dH, dW) = (_pair(stride, "stride"), _pair(padding, "padding"),
                                    _pair(dilation, "dilation"))
    st, oh, ow = _capi.conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW)
    _check(st)
    return oh, ow


def conv2d_gemm_f32(out, input, weight, bias=None, stride=1, padding=0, dilation=1, groups=1):
    """NCHW conv2d (groups == 1) written into ``out`` [B, OC, OH, OW]."""
    import torch
    out, x, w = _dev_f32(out, "out"), _dev_f32(input, "input"), _dev_f32(weight, "weight")
    if x.dim() != 4 or w.dim() != 4 or out.dim() != 4:
        raise ValueError("input, weight and out must be 4-D (NCHW / OIHW)")
    B, IC, H, W = x.shape
    OC, ICg, KH, KW = w.shape
    if int(groups) < 1 or ICg * int(groups) != IC:
        raise ValueError(f"weight has {ICg} input channels per group; input has {IC}, "
                         f"groups={groups}")
    (sH, sW), (pH, pW), (dH, dW) = (_pair(stride, "stride"), _pair(padding, "padding"),
                                    _pair(dilation, "dilation"))
    bias_ptr = None
    devs = {out.device, x.device, w.device}
    if bias is not None:
        bias = _dev_f32(bias, "bias")
        if tuple(bias.shape) != (OC,):
            raise ValueError(f"bias must be [{OC}]")
        bias_ptr = bias.data_ptr()
        devs.add(bias.device)
    if len(devs) != 1:
        raise ValueError("all tensors must be on the same device")
    st, OH, OW = _capi.conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW)
    _check(st)
    if tuple(out.shape) != (B, OC, OH, OW):
        raise ValueError(f"out must be [{B}, {OC}, {OH}, {OW}], got {list(out.shape)}")
    dev = out.device
    with _on(dev):
        st = _capi.conv2d_gemm_f32(out.data_ptr(), x.data_ptr(), w.data_ptr(), bias_ptr,
                                   B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW,
                                   int(groups), _stream(dev))
    _check(st)
    return out


def conv2d(input, weight, bias=None, stride=1, padding=0, dilation=1, groups=1):
    """NCHW conv2d (weight [OC, IC/groups, KH, KW]) as a new output."""
    import torch
    x, w = _dev_f32(input, "input"), _dev_f32(weight, "weight")
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("input and weight must be 4-D")
    OH, OW = conv2d_out_hw(x.shape[2], x.shape[3], w.shape[2], w.shape[3], stride, padding,
                           dilation)
    out = torch.empty((x.shape[0], w.shape[0], OH, OW), dtype=torch.float32, device=x.device)
    return conv2d_gemm_f32(out, x, w, bias, stride, padding, dilation, groups)


def sdpa_f32(out, q, k, v, attn_mask=None, scale=None):
    """out = softmax(q @ k^T * scale + attn_mask) @ v, written into ``out``.

    q [..., Sq, D]; k, v [..., Skv, D] with the same leading dims; attn_mask
    [..., Sq, Skv] or None; scale None means 1/sqrt(D).  out is like q."""
    import torch
    out, q, k, v = (_dev_f32(out, "out"), _dev_f32(q, "q"), _dev_f32(k, "k"), _dev_f32(v, "v"))
    if q.dim() < 3:
        raise ValueError("q must have rank >= 3 ([..., S, D])")
    if k.shape != v.shape or k.dim() != q.dim():
        raise ValueError("k and v must have the same shape and q's rank")
    if k.shape[:-2] != q.shape[:-2] or k.shape[-1] != q.shape[-1]:
        raise ValueError("q, k and v must share leading dims and D")
    if out.shape != q.shape:
        raise ValueError(f"out must be {list(q.shape)}")
    Sq, D = q.shape[-2], q.shape[-1]
    Skv = k.shape[-2]
    BH = 1
    for n in q.shape[:-2]:
        BH *= int(n)
    devs = {out.device, q.device, k.device, v.device}
    mask_ptr = None
    if attn_mask is not None:
        attn_mask = _dev_f32(attn_mask, "attn_mask")
        if attn_mask.shape != q.shape[:-1] + (Skv,):
            raise ValueError(f"attn_mask must be {list(q.shape[:-1]) + [Skv]}")
        mask_ptr = attn_mask.data_ptr()
        devs.add(attn_mask.device)
    if len(devs) != 1:
        raise ValueError("all tensors must be on the same device")
    sc = None if scale is None else float(scale)
    dev = out.device
    with _on(dev):
        st = _capi.sdpa_f32(out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), mask_ptr,
                            BH, Sq, Skv, D, sc, _stream(dev))
    _check(st)
    return out


def sdpa(q, k, v, attn_mask=None, scale=None):
    """Non-causal scaled-dot-product attention as a new tensor shaped like q."""
    import torch
    q = _dev_f32(q, "q")
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    return sdpa_f32(out, q, k, v, attn_mask, scale)


def conv2d_nhwc_f32(out, input, weight, bias=None, stride=1, padding=0, dilation=1):
    """Channels-last conv2d written into ``out`` [B, OH, OW, OC]: input
    [B, H, W, IC], weight [OC, KH, KW, IC], bias [OC] or None."""
    import torch
    out, x, w = _dev_f32(out, "out"), _dev_f32(input, "input"), _dev_f32(weight, "weight")
    if x.dim() != 4 or w.dim() != 4 or out.dim() != 4:
        raise ValueError("input, weight and out must be 4-D (NHWC / OHWI)")
    B, H, W, IC = x.shape
    OC, KH, KW, IC2 = w.shape
    if IC2 != IC:
        raise ValueError(f"weight must be [OC, KH, KW, IC={IC}], got {list(w.shape)}")
    (sH, sW), (pH, pW), (dH, dW) = (_pair(stride, "stride"), _pair(padding, "padding"),
                                    _pair(dilation, "dilation"))
    bias_ptr = None
    devs = {out.device, x.device, w.device}
    if bias is not None:
        bias = _dev_f32(bias, "bias")
        if tuple(bias.shape) != (OC,):
            raise ValueError(f"bias must be [{OC}]")
        bias_ptr = bias.data_ptr()
        devs.add(bias.device)
    if len(devs) != 1:
        raise ValueError("all tensors must be on the same device")
    st, OH, OW = _capi.conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW)
    _check(st)
    if tuple(out.shape) != (B, OH, OW, OC):
        raise ValueError(f"out must be [{B}, {OH}, {OW}, {OC}], got {list(out.shape)}")
    dev = out.device
    with _on(dev):
        st = _capi.conv2d_nhwc_f32(out.data_ptr(), x.data_ptr(), w.data_ptr(), bias_ptr,
                                   B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, _stream(dev))
    _check(st)
    return out


def conv2d_nhwc(input, weight, bias=None, stride=1, padding=0, dilation=1):
    """Channels-last conv2d (input [B,H,W,IC], weight [OC,KH,KW,IC]) as a new
    [B, OH, OW, OC] tensor."""
    import torch
    x, w = _dev_f32(input, "input"), _dev_f32(weight, "weight")
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("input and weight must be 4-D")
    OH, OW = conv2d_out_hw(x.shape[1], x.shape[2], w.shape[1], w.shape[2], stride, padding,
                           dilation)
    out = torch.empty((x.shape[0], OH, OW, w.shape[0]), dtype=torch.float32, device=x.device)
    return conv2d_nhwc_f32(out, x, w, bias, stride, padding, dilation)


def conv_transpose2d_out_hw(H, W, KH, KW, stride=1, padding=0, dilation=1, output_padding=0):
    (sH, sW), (pH, pW), (dH, dW), (oH, oW) = (
        _pair(stride, "stride"), _pair(padding, "padding"), _pair(dilation, "dilation"),
        _pair(output_padding, "output_padding"))
    st, oh, ow = _capi.conv_transpose2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, oH, oW)
    _check(st)
    return oh, ow


def conv_transpose2d_f32(out, input, weight, bias=None, stride=1, padding=0, output_padding=0,
                         groups=1, dilation=1):
    """Transposed conv2d written into ``out`` [B, OC, OH, OW]: input
    [B, IC, H, W], weight [IC, OC/groups, KH, KW], bias [OC] or None."""
    import torch
    out, x, w = _dev_f32(out, "out"), _dev_f32(input, "input"), _dev_f32(weight, "weight")
    if x.dim() != 4 or w.dim() != 4 or out.dim() != 4:
        raise ValueError("input, weight and out must be 4-D")
    B, IC, H, W = x.shape
    IC2, OCg, KH, KW = w.shape
    if IC2 != IC or int(groups) < 1:
        raise ValueError(f"weight must be [IC={IC}, OC/groups, KH, KW], got {list(w.shape)}")
    OC = OCg * int(groups)
    (sH, sW), (pH, pW), (dH, dW), (oH, oW) = (
        _pair(stride, "stride"), _pair(padding, "padding"), _pair(dilation, "dilation"),
        _pair(output_padding, "output_padding"))
    bias_ptr = None
    devs = {out.device, x.device, w.device}
    if bias is not None:
        bias = _dev_f32(bias, "bias")
        if tuple(bias.shape) != (OC,):
            raise ValueError(f"bias must be [{OC}]")
        bias_ptr = bias.data_ptr()
        devs.add(bias.device)
    if len(devs) != 1:
        raise ValueError("all tensors must be on the same device")
    st, OH, OW = _capi.conv_transpose2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, oH, oW)
    _check(st)
    if tuple(out.shape) != (B, OC, OH, OW):
        raise ValueError(f"out must be [{B}, {OC}, {OH}, {OW}], got {list(out.shape)}")
    dev = out.device
    with _on(dev):
        st = _capi.conv_transpose2d_f32(out.data_ptr(), x.data_ptr(), w.data_ptr(), bias_ptr,
                                        B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, oH, oW,
                                        int(groups), _stream(dev))
    _check(st)
    return out


def conv_transpose2d(input, weight, bias=None, stride=1, padding=0, output_padding=0, groups=1,
                     dilation=1):
    """Transposed conv2d (weight [IC, OC/groups, KH, KW]) as a new tensor."""
    import torch
    x, w = _dev_f32(input, "input"), _dev_f32(weight, "weight")
    if x.dim() != 4 or w.dim() != 4:
        raise ValueError("input and weight must be 4-D")
    OH, OW = conv_transpose2d_out_hw(x.shape[2], x.shape[3], w.shape[2], w.shape[3], stride,
                                     padding, dilation, output_padding)
    out = torch.empty((x.shape[0], w.shape[1] * int(groups), OH, OW), dtype=torch.float32,
                      device=x.device)
    return conv_transpose2d_f32(out, x, w, bias, stride, padding, output_padding, groups, dilation)
