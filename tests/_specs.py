"""Forced tile configurations for the parity tests, and the problem shapes
they run on.

``BAIM_TILE`` overrides the library's plan: "cfg" (one tile per block),
"cfg,S" (S K slices on separate blocks: S == 2 is the two-piece exchange,
S > 2 atomic adds) or "cfg,sP" (P blocks stream over the (tile, k-tile)
units; two-piece exchange).  Configurations (bm x bn x bk, waves):
0 = 128x128x32 (8), 1 = 128x64x32 (8), 2 = 64x128x32 (8), 3 = 64x64x32 (4),
4 = 128x128x64 (16), 5 = 128x64x64 (16), 6 = 64x64x64 (8),
7 = 64x64x128 (16), 8 = 32x128x32 (4), 9 = 256x256x16 (8; addmm only: linear
and the im2col conv paths run configuration 0 for it).

Configuration 5 streamed over P blocks carries the 3x3 mid-stage convs; its
specs ("5,sP", "5,2", "5,3") are here on purpose.  Every spec must change
what the library runs on at least one of its test's shapes:
``tests/test_forced_specs.py`` checks that on the CPU with the library's own
planner, so a spec that silently falls back to one tile per block cannot
hide in these lists.
"""

GEMM_SPECS = ["0", "1", "2", "3", "4", "5", "6", "7", "8",
              "0,3", "1,2", "2,4", "3,5", "0,64", "5,2", "5,3", "6,3", "7,2", "7,3", "8,2", "8,3",
              "3,s7", "0,s2", "5,s7", "5,s13", "6,s5", "2,s9", "1,s4", "8,s5"]

# addmm also forces the 256x256 tile
ADDMM_SPECS = GEMM_SPECS + ["9"]

NHWC_SPECS = ["0", "1", "2", "3", "4", "5", "6", "7", "8",
              "0,3", "2,3", "5,2", "5,3", "7,2",
              "3,s7", "1,s4", "6,s5", "8,s3", "5,s7", "5,s13"]

# addmm: (M, K, N, self_2d, beta, alpha); the integer case is (M, K, N)
ADDMM_SHAPES = [(130, 300, 257, True, 0.5, 2.0), (77, 1000, 65, False, 1.0, 1.0),
                (256, 64, 128, False, 0.0, -1.0), (33, 45, 70, True, 1.0, 1.0)]
ADDMM_INT_SHAPE = (260, 520, 700)

# linear: (M, K, N); integer (M, K, N)
LINEAR_SHAPES = [(130, 300, 257), (77, 1000, 65), (33, 45, 70)]
LINEAR_INT_SHAPE = (260, 520, 300)

# NCHW conv: (B, IC, H, W, OC, KH, KW, stride, pad, dil, has_bias); integer
# case (B, IC, H, W, OC) with a 3x3 kernel, stride 1, pad 1
CONV_SHAPES = [(2, 24, 23, 21, 136, 3, 3, 1, 1, 1, True),
               (1, 3, 40, 44, 70, 7, 7, 4, 3, 1, False),
               (2, 16, 15, 15, 24, 3, 3, 2, 1, 2, True)]
CONV_INT_SHAPE = (2, 40, 27, 29, 72)

# channels-last conv: (IC, k, stride) on x [2, 21, 18, IC], OC 70, pad 1;
# integer case (B, H, W, IC, OC) with a 3x3 kernel, stride 1, pad 1
NHWC_SHAPES = [(16, 3, 1), (3, 5, 2)]
NHWC_INT_SHAPE = (2, 23, 24, 32, 66)


def _out(n, k, s, p, d=1):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def addmm_gemms():
    """(M, N, K, 16-byte loads possible) of every forced-spec addmm call."""
    out = [(M, N, K, K % 4 == 0 and N % 4 == 0) for M, K, N, *_ in ADDMM_SHAPES]
    M, K, N = ADDMM_INT_SHAPE
    return out + [(M, N, K, K % 4 == 0 and N % 4 == 0)]


def linear_gemms():
    out = [(M, N, K, K % 4 == 0) for M, K, N in LINEAR_SHAPES]
    M, K, N = LINEAR_INT_SHAPE
    return out + [(M, N, K, K % 4 == 0)]


def conv_gemms():
    """NCHW conv as a GEMM: M = OC, N = B*OH*OW, K = IC*KH*KW; the stream
    schedule needs 16-byte weight loads (K % 4 == 0)."""
    out = []
    for B, IC, H, W, OC, KH, KW, s, p, d, _ in CONV_SHAPES:
        K = IC * KH * KW
        out.append((OC, B * _out(H, KH, s, p, d) * _out(W, KW, s, p, d), K, K % 4 == 0))
    B, IC, H, W, OC = CONV_INT_SHAPE
    out.append((OC, B * H * W, IC * 9, True))
    out.append((136, 2 * 13 * 20, 24 * 9, True))   # the rows-of-four case
    return out


def nhwc_gemms():
    """Channels-last conv as a GEMM: M = B*OH*OW, N = OC, K = KH*KW*IC; the
    16-byte gathers need IC % 4 == 0."""
    out = []
    for IC, k, s in NHWC_SHAPES:
        OH, OW = _out(21, k, s, 1), _out(18, k, s, 1)
        out.append((2 * OH * OW, 70, k * k * IC, IC % 4 == 0))
    B, H, W, IC, OC = NHWC_INT_SHAPE
    out.append((B * H * W, OC, 9 * IC, True))
    return out
