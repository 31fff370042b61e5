"""Seeded synthetic inputs for the addmm and conv2d workloads.

This module only draws random numbers and describes workload shapes; it holds
none of the method's arithmetic, so both the HIP path and the CPU oracle can
be fed from it.  Everything is generated on the CPU with a
``torch.Generator('cpu')`` seeded per case (seed 0 unless stated), in the
draw order mat1, mat2, self (addmm) or input, weight, bias (conv), as fp32
contiguous tensors.

Distributions: ``("U", a, b)`` is uniform on [a, b) (``rand*(b-a)+a``);
``("N", sigma)`` is normal with mean 0 (``randn*sigma``); ``("I", lo, hi)`` is
integer-valued in [lo, hi] (used for order-independent, exact cases).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class AddmmCase:
    name: str
    M: int
    K: int
    N: int
    mat1: tuple
    mat2: tuple
    self: tuple
    self_2d: bool
    beta: float = 1.0
    alpha: float = 1.0
    seed: int = 0
    kind: str = field(default="addmm", init=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


@dataclass(frozen=True)
class ConvCase:
    name: str
    B: int
    IC: int
    H: int
    W: int
    OC: int
    KH: int
    KW: int
    stride: tuple
    padding: tuple
    dilation: tuple
    x: tuple
    w: tuple
    bias: tuple | None
    seed: int = 0
    groups: int = 1
    channels_last: bool = False  # x [B,H,W,IC], w [OC,KH,KW,IC], out [B,OH,OW,OC]
    kind: str = field(default="conv", init=False)

    def out_hw(self):
        """Output size with floor((H + 2p - d(k-1) - 1)/s) + 1 per axis."""
        def one(n, k, s, p, d):
            return (n + 2 * p - d * (k - 1) - 1) // s + 1
        return (one(self.H, self.KH, self.stride[0], self.padding[0], self.dilation[0]),
                one(self.W, self.KW, self.stride[1], self.padding[1], self.dilation[1]))

    @property
    def gemm_mnk(self):
        """Per-group GEMM: (OC/G, B*OH*OW, (IC/G)*KH*KW)."""
        OH, OW = self.out_hw()
        return (self.OC // self.groups, self.B * OH * OW,
                self.IC // self.groups * self.KH * self.KW)

    @property
    def flops(self) -> int:
        M, N, K = self.gemm_mnk
        return 2 * M * N * K * self.groups


@dataclass(frozen=True)
class LinearCase:
    name: str
    M: int
    K: int
    N: int
    x: tuple
    w: tuple
    bias: tuple | None
    seed: int = 0
    kind: str = field(default="linear", init=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


@dataclass(frozen=True)
class ConvTCase:
    """Transposed conv: x [B,IC,H,W], weight [IC,OC,KH,KW], bias [OC]."""
    name: str
    B: int
    IC: int
    H: int
    W: int
    OC: int
    KH: int
    KW: int
    stride: tuple
    padding: tuple
    dilation: tuple
    output_padding: tuple
    x: tuple
    w: tuple
    bias: tuple | None
    seed: int = 0
    kind: str = field(default="convt", init=False)

    def out_hw(self):
        """(H-1)*s - 2p + d(k-1) + output_padding + 1 per axis."""
        def one(n, k, s, p, d, op):
            return (n - 1) * s - 2 * p + d * (k - 1) + op + 1
        return (one(self.H, self.KH, self.stride[0], self.padding[0], self.dilation[0],
                    self.output_padding[0]),
                one(self.W, self.KW, self.stride[1], self.padding[1], self.dilation[1],
                    self.output_padding[1]))

    @property
    def flops(self) -> int:
        """Every input element meets every (oc, kh, kw): 2*B*IC*H*W*OC*KH*KW
        (taps that fall outside the output are few and not subtracted)."""
        return 2 * self.B * self.IC * self.H * self.W * self.OC * self.KH * self.KW


@dataclass(frozen=True)
class SdpaCase:
    """Non-causal attention: q [B,H,Sq,D], k and v [B,H,Skv,D], optional
    additive mask [B,H,Sq,Skv].  ``key_pad`` gives each batch entry b a
    valid key length L_b drawn uniformly from [Skv/2, Skv]; mask entries for
    keys >= L_b are -inf (padding of a variable-length key sequence)."""
    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    D: int
    q: tuple
    k: tuple
    v: tuple
    mask: tuple | None = None
    key_pad: bool = False
    scale: float | None = None  # None: 1/sqrt(D)
    seed: int = 0
    kind: str = field(default="sdpa", init=False)

    @property
    def flops(self) -> int:
        """q @ k^T and p @ v: 4*B*H*Sq*Skv*D (the softmax is not counted)."""
        return 4 * self.B * self.H * self.Sq * self.Skv * self.D


U11 = ("U", -1.0, 1.0)
U01 = ("U", 0.0, 1.0)


def N(sigma):
    return ("N", float(sigma))


# The workloads: a small addmm, a transformer FFN linear (bias [N] and full
# self [M,N]), a 7x7/s4 patch-embed stem conv, a 3x3 mid-stage conv (base,
# dilation 2, stride 2 on 57x57) and large / ragged projection addmms.
CASES = {c.name: c for c in [
    AddmmCase("addmm_small_64x96x80", 64, 96, 80, U11, U11, U11, False),
    AddmmCase("ffn_2048x768x3072_bias", 2048, 768, 3072, N(1), N(0.02), N(0.02), False),
    AddmmCase("ffn_2048x768x3072_full_self", 2048, 768, 3072, N(1), N(0.02), N(1), True,
              beta=0.5, alpha=2.0),
    ConvCase("stem_conv7x7_s4_768", 1, 3, 768, 768, 128, 7, 7, (4, 4), (3, 3), (1, 1),
             U01, N(0.05), N(0.02)),
    ConvCase("conv3x3_56_s1", 4, 256, 56, 56, 256, 3, 3, (1, 1), (1, 1), (1, 1),
             N(1), N(0.02), N(0.02)),
    ConvCase("conv3x3_56_d2", 4, 256, 56, 56, 256, 3, 3, (1, 1), (2, 2), (2, 2),
             N(1), N(0.02), N(0.02)),
    ConvCase("conv3x3_57_s2", 4, 256, 57, 57, 256, 3, 3, (2, 2), (1, 1), (1, 1),
             N(1), N(0.02), N(0.02)),
    AddmmCase("up_proj_4096x1024x4096", 4096, 1024, 4096, N(1), N(0.02), N(0.02), False),
    AddmmCase("down_proj_4096x4096x1024", 4096, 4096, 1024, N(1), N(0.02), N(0.02), False),
    AddmmCase("ragged_577x1024x4096_full_self", 577, 1024, 4096, N(1), N(0.02), N(1), True),
]}

# linear (x @ weight^T + bias, weight [N,K]): the FFN projection shape with
# the weight stored as [out_features, in_features].
LINEAR_CASES = {c.name: c for c in [
    LinearCase("linear_ffn_2048x768x3072", 2048, 768, 3072, N(1), N(0.02), N(0.02)),
    LinearCase("linear_ragged_577x1024x4096_nobias", 577, 1024, 4096, N(1), N(0.02), None),
]}

# Grouped convs on the 3x3 mid-stage shape: 8 groups of 32 channels (one
# GEMM per group) and depthwise (the direct kernel).
GROUPED_CASES = {c.name: c for c in [
    ConvCase("conv3x3_56_g8", 4, 256, 56, 56, 256, 3, 3, (1, 1), (1, 1), (1, 1),
             N(1), N(0.05), N(0.02), groups=8),
    ConvCase("dwconv3x3_56", 4, 256, 56, 56, 256, 3, 3, (1, 1), (1, 1), (1, 1),
             N(1), N(0.2), N(0.02), groups=256),
]}

# Channels-last (NHWC) convs: the 3x3 mid-stage shape and the 3-channel stem.
NHWC_CASES = {c.name: c for c in [
    ConvCase("conv3x3_56_s1_nhwc", 4, 256, 56, 56, 256, 3, 3, (1, 1), (1, 1), (1, 1),
             N(1), N(0.02), N(0.02), channels_last=True),
    ConvCase("stem_conv7x7_s4_768_nhwc", 1, 3, 768, 768, 128, 7, 7, (4, 4), (3, 3), (1, 1),
             U01, N(0.05), N(0.02), channels_last=True),
]}

# Transposed convs of decoders: a 4x4 / stride-2 2x upsampling (256 -> 128
# channels, 28 -> 56) and the 2x2 / stride-2 upscaling of a mask decoder
# (256 -> 64 channels, 64 -> 128).
CONVT_CASES = {c.name: c for c in [
    ConvTCase("convt4x4_s2_28_to_56", 4, 256, 28, 28, 128, 4, 4, (2, 2), (1, 1), (1, 1), (0, 0),
              N(1), N(0.02), N(0.02)),
    ConvTCase("convt2x2_s2_64_to_128", 4, 256, 64, 64, 64, 2, 2, (2, 2), (0, 0), (1, 1), (0, 0),
              N(1), N(0.05), N(0.02)),
]}

# Non-causal attention in vision encoders and cross-attention: ViT-B/16 at
# 224 px (196 patches + class token, 12 heads of 64), a 1024-token encoder
# with 16 heads of 128, cross-attention from 64 queries to 577 image tokens
# with an additive mask and padded keys, and pooled-query attention
# (Sq = Skv/4).  q and k ~ N(0,1), so with scale 1/sqrt(D) the logits are
# about N(0,1); v ~ N(0,1).
SDPA_CASES = {c.name: c for c in [
    SdpaCase("sdpa_vit_b32_h12_s197_d64", 32, 12, 197, 197, 64, N(1), N(1), N(1)),
    SdpaCase("sdpa_b4_h16_s1024_d128", 4, 16, 1024, 1024, 128, N(1), N(1), N(1)),
    SdpaCase("sdpa_xattn_b8_h12_q64_kv577_d64_mask", 8, 12, 64, 577, 64, N(1), N(1), N(1),
             mask=N(1), key_pad=True),
    SdpaCase("sdpa_pooled_b1_h8_q1024_kv4096_d64", 1, 8, 1024, 4096, 64, N(1), N(1), N(1)),
]}

# Groups of cases as the workload list states them (small / FFN / stem /
# 3x3 mid-stage / large and ragged projections).
GROUPS = {
    "addmm_small": ["addmm_small_64x96x80"],
    "ffn": ["ffn_2048x768x3072_bias", "ffn_2048x768x3072_full_self"],
    "stem": ["stem_conv7x7_s4_768"],
    "conv3x3": ["conv3x3_56_s1", "conv3x3_56_d2", "conv3x3_57_s2"],
    "proj": ["up_proj_4096x1024x4096", "down_proj_4096x4096x1024",
             "ragged_577x1024x4096_full_self"],
}


def draw(shape, dist, gen: torch.Generator) -> torch.Tensor:
    """One fp32 CPU tensor of ``shape`` from ``dist`` using ``gen``."""
    kind = dist[0]
    if kind == "U":
        lo, hi = dist[1], dist[2]
        return torch.rand(shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo
    if kind == "N":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * dist[1]
    if kind == "I":
        lo, hi = int(dist[1]), int(dist[2])
        return torch.randint(lo, hi + 1, shape, generator=gen).to(torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def addmm_inputs(case: AddmmCase):
    """(mat1 [M,K], mat2 [K,N], self [N] or [M,N]) as fp32 CPU tensors."""
    g = torch.Generator("cpu").manual_seed(case.seed)
    mat1 = draw((case.M, case.K), case.mat1, g)
    mat2 = draw((case.K, case.N), case.mat2, g)
    self = draw((case.M, case.N) if case.self_2d else (case.N,), case.self, g)
    return mat1, mat2, self


def conv_inputs(case: ConvCase):
    """(input [B,IC,H,W], weight [OC,IC/groups,KH,KW], bias [OC] or None);
    channels-last cases draw input [B,H,W,IC] and weight [OC,KH,KW,IC]."""
    g = torch.Generator("cpu").manual_seed(case.seed)
    if case.channels_last:
        x = draw((case.B, case.H, case.W, case.IC), case.x, g)
        w = draw((case.OC, case.KH, case.KW, case.IC // case.groups), case.w, g)
        b = None if case.bias is None else draw((case.OC,), case.bias, g)
        return x, w, b
    x = draw((case.B, case.IC, case.H, case.W), case.x, g)
    w = draw((case.OC, case.IC // case.groups, case.KH, case.KW), case.w, g)
    b = None if case.bias is None else draw((case.OC,), case.bias, g)
    return x, w, b


def linear_inputs(case: LinearCase):
    """(x [M,K], weight [N,K], bias [N] or None)."""
    g = torch.Generator("cpu").manual_seed(case.seed)
    x = draw((case.M, case.K), case.x, g)
    w = draw((case.N, case.K), case.w, g)
    b = None if case.bias is None else draw((case.N,), case.bias, g)
    return x, w, b


def sdpa_inputs(case: SdpaCase):
    """(q, k, v, mask or None) as fp32 CPU tensors, drawn in that order; the
    key lengths (with key_pad) are drawn last."""
    g = torch.Generator("cpu").manual_seed(case.seed)
    q = draw((case.B, case.H, case.Sq, case.D), case.q, g)
    k = draw((case.B, case.H, case.Skv, case.D), case.k, g)
    v = draw((case.B, case.H, case.Skv, case.D), case.v, g)
    mask = None
    if case.mask is not None:
        mask = draw((case.B, case.H, case.Sq, case.Skv), case.mask, g)
        if case.key_pad:
            lens = torch.randint(case.Skv // 2, case.Skv + 1, (case.B,), generator=g)
            for b in range(case.B):
                mask[b, :, :, int(lens[b]):] = float("-inf")
    return q, k, v, mask


def convt_inputs(case: ConvTCase):
    """(input [B,IC,H,W], weight [IC,OC,KH,KW], bias [OC] or None)."""
    g = torch.Generator("cpu").manual_seed(case.seed)
    x = draw((case.B, case.IC, case.H, case.W), case.x, g)
    w = draw((case.IC, case.OC, case.KH, case.KW), case.w, g)
    b = None if case.bias is None else draw((case.OC,), case.bias, g)
    return x, w, b


def inputs(case):
    if case.kind == "convt":
        return convt_inputs(case)
    if case.kind == "sdpa":
        return sdpa_inputs(case)
    if case.kind == "addmm":
        return addmm_inputs(case)
    if case.kind == "linear":
        return linear_inputs(case)
    return conv_inputs(case)
