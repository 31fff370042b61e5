// conv_window.hip -- groups==1 NCHW conv2d with a small kernel as an
// implicit GEMM whose B operand is read from an input window held in LDS
// ("et_vk conv2d: route standard (groups==1) conv through an im2col tiled
// GEMM", Solution and Implementation paragraphs: M = OC, N = B*OH*OW,
// K = IC*KH*KW, B[kk, n] = x[b, ic, oh*sH - pH + kh*dH, ow*sW - pW + kw*dW]
// or 0 outside the input, bias per OC, NCHW output).
//
// The general conv kernel (conv2d_gemm.hip) gathers every im2col element
// B[kk, n] with its own 4-byte load.  For a 3x3 kernel the nine taps of one
// input channel read the same few input rows, shifted; here a block instead
// copies, for each k-tile of CI input channels, the input rows its output
// pixels touch (all W columns, zero rows above and below the image, zero
// columns left and right) into LDS with 16-byte loads, and every MFMA step
// reads its B value from that window at a compile-time offset from a
// per-lane base: one `ds_read_b32 v, base offset:imm`, no index arithmetic.
// A 3x3 stride-1 k-tile of 16 channels and 128 pixels then costs 21 window
// loads per block instead of 288 gathers.
//
// At stride 2 each input element serves about 2.25 outputs instead of 9, so
// the window saves fewer loads, but it still replaces one 4-byte gather per
// im2col element by 16-byte row copies: per k-tile of 16 channels and 64
// pixels a block issues about 4 loads per thread (weights and window)
// against 10 for the gather kernel's 128-deep k-tile.  Stride-2 rows need
// not be a multiple of 4 floats (57 x 57 feature maps); their whole quads
// load 16 bytes at a time from the 4-byte-aligned row start and the last
// W % 4 columns 4 bytes at a time.
//
// Block tile: BM output channels x BN consecutive output pixels of one
// image (a run of (oh, ow) in row-major order; 128 pixels touch at most four
// output rows when OW >= 43).  16 waves: WM x WN waves of 32 x 32 outputs,
// and WK wave groups that split each k-tile by input channel (group g takes
// channels [g*CI/WK, (g+1)*CI/WK) of the k-tile); the groups' partial tiles
// are summed through LDS in group order.  The 64 x 128 block with 16
// channels per k-tile measured faster than 128 x 64 with 8 (3x3 s1:
// 139.5 -> 136.1 us; in steady state 72% -> 77% of the fp32 peak): half the
// barriers per flop, fewer weight loads per flop, and lane-half weight runs
// of 36 (a whole number of float4s, so 16-byte LDS writes).
//
// K order inside a wave group.  v_mfma_f32_32x32x2_f32 takes k = h from
// lane-half h (lanes 32h..32h+31).  Step s (0 <= s < CH*TAPS) of half h uses
// channel g*CI/WK + h*CH + s/TAPS of the k-tile and tap s%TAPS, CH being the
// channels per lane-half.  The two halves' B addresses then differ by the
// constant CH channel planes, which folds into the per-lane base, and each
// half's A values for consecutive steps are consecutive weights of one row
// (weight k = ic*TAPS + tap), read 16 bytes at a time from a segment of the
// A tile.  Any fp32 summation order is acceptable.
#include <stdlib.h>

#include "conv_window_plan.hpp"
#include "gemm_core.hpp"
#include "launch.hpp"
#include "tile_select.hpp"

namespace baim {

template <int KH_, int KW_, int SH_, int SW_, int DH_, int DW_, int WR_, int BM_ = 128,
          int BN_ = 64, int CI_ = 8, int WM_ = 4, int WN_ = 2, int WK_ = 2, bool TAIL_ = false,
          int MAXQ_ = 15>
struct WinCfg {
  static constexpr int KH = KH_, KW = KW_, SH = SH_, SW = SW_, DH = DH_, DW = DW_;
  static constexpr int TAPS = KH * KW;
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int CI = CI_;         // input channels per k-tile
  static constexpr int BK = CI * TAPS;   // k per k-tile
  static constexpr int WM = WM_, WN = WN_, WK = WK_;
  static constexpr int NT = 64 * WM * WN * WK;
  static constexpr int WTM = BM / WM, WTN = BN / WN, FM = 1, FN = 1;
  static_assert(WTM == 32 && WTN == 32, "one 32 x 32 block per wave");
  static constexpr int BKW = BK / WK;
  // Channels of one lane-half: wave group g takes channels
  // [g*CI/WK, (g+1)*CI/WK) of the k-tile, lane-half h the h-th half of them.
  static constexpr int CH = CI / (2 * WK);
  // A tile in LDS: per row 2*WK segments (wave group g, lane-half h at
  // segment 2g + h) of HALF = CH*TAPS weights, each padded to a multiple of
  // four floats so that every segment starts 16-byte aligned.  The row
  // stride is an odd multiple of 4 floats (mod 32): the 16-byte reads of 8
  // consecutive rows cover all 32 banks.
  static constexpr int HALF = CH * TAPS;
  static constexpr int SEG = (HALF + 3) / 4 * 4;
  static constexpr int AS = 2 * WK * SEG + 4;
  // Input window in LDS: per channel WR rows of RS floats; input column iw
  // sits at CL + iw, so columns [CL - pW, CL) and [CL + W, RS) hold zeros.
  static constexpr int RS = 64, CL = 4, WR = WR_;
  static constexpr int PS = WR * RS;
  static constexpr int A_FLOATS = BM * AS;
  static constexpr int B_FLOATS = CI * PS;
  static constexpr int STAGE = A_FLOATS + B_FLOATS;
  static constexpr int SMEM_FLOATS = 2 * STAGE;
  static constexpr int A_ITEMS = BM * BK / 4;  // float4 loads of one A tile
  static constexpr int A_NQ = (A_ITEMS + NT - 1) / NT;
  // Input rows: W / 4 <= MAXQ whole quads each; with TAIL, also W % 4 != 0,
  // the last W % 4 columns then taking one 4-byte load per thread.
  static constexpr bool TAIL = TAIL_;
  static constexpr int MAXQ = MAXQ_;
  static constexpr int B_ITEMS = CI * WR * MAXQ;  // upper bound
  static constexpr int B_NQ = (B_ITEMS + NT - 1) / NT;
  static_assert(CL + 4 * MAXQ <= RS, "whole quads fit a window row");
  static_assert(!TAIL || CI * WR * 3 <= NT, "one tail column per thread");
  static_assert(CI % (2 * WK) == 0 && HALF % 2 == 0 && BKW == 2 * HALF, "lane-half channels");
  static_assert(AS % 8 == 4, "A rows must start an odd multiple of 4 floats apart (mod 32)");
  static_assert((WK - 1) * BM * BN <= SMEM_FLOATS, "k-group reduction must fit in LDS");
  static_assert(SMEM_FLOATS * 4 <= 160 * 1024, "LDS budget");
};

struct WinArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int IC, H, W, OC, pH, pW, OH, OW;
  int P;       // OH*OW
  int tpi;     // BN-pixel tiles per image
  int K;       // IC*TAPS
  int x_elems;
  Sched sched;
};

// One BM x BK tile of the weight [OC, IC*TAPS] per k-tile: float4 loads
// along K, written to LDS as two 8-byte halves into their segments.
template <class C>
struct WinALoader {
  const float* base;
  int K, rows_left;
  f32x4 reg[2][C::A_NQ];

  __device__ void init(const float* w, int m0, int M, int K_) {
    base = w + (size_t)m0 * K_;
    K = K_;
    rows_left = M - m0;
  }
  template <int S>
  __device__ void load(int t) {
    const int k0 = t * C::BK;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0, (int64_t)rows_left * K - k0);
#pragma unroll
    for (int q = 0; q < C::A_NQ; ++q) {
      const int i = threadIdx.x + C::NT * q;
      const int r = i / (C::BK / 4), c = (i % (C::BK / 4)) * 4;
      const bool ok = i < C::A_ITEMS && r < rows_left && k0 + c < K;
      reg[S][q] = Vec<4>::load(rs, ok ? (uint32_t)(r * K + c) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* As) const {
#pragma unroll
    for (int q = 0; q < C::A_NQ; ++q) {
      const int i = threadIdx.x + C::NT * q;
      if (C::A_ITEMS % C::NT != 0 && i >= C::A_ITEMS) continue;
      const int r = i / (C::BK / 4), c = (i % (C::BK / 4)) * 4;
      if constexpr (C::HALF % 4 == 0) {
        // segments hold whole float4s
        *reinterpret_cast<f32x4*>(&As[r * C::AS + (c / C::HALF) * C::SEG + c % C::HALF]) = reg[S][q];
      } else {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const int k0 = c, k1 = c + 2;  // even, so each pair stays in one segment
        *reinterpret_cast<f32x2*>(&As[r * C::AS + (k0 / C::HALF) * C::SEG + k0 % C::HALF]) =
            f32x2{reg[S][q][0], reg[S][q][1]};
        *reinterpret_cast<f32x2*>(&As[r * C::AS + (k1 / C::HALF) * C::SEG + k1 % C::HALF]) =
            f32x2{reg[S][q][2], reg[S][q][3]};
      }
    }
  }
};

// The input window of one k-tile: channels CI*t .. CI*t + CI-1 of image b,
// input rows ih_first .. ih_first + WR - 1, all W columns.  Columns
// [0, 4*(W/4)) load as float4s; a row starts 16 bytes aligned when W % 4 == 0
// and the input is, and 4 bytes aligned otherwise, which buffer loads
// accept.  With TAIL the last W % 4 columns load 4 bytes at a time.  Which
// (channel, row, column quad) a thread copies is fixed for the whole piece;
// rows outside the image and channels past IC load as 0 (out-of-range
// offset).
template <class C>
struct WinBLoader {
  int goff[C::B_NQ];  // float offset of the item in channel CI*t + icl at t = 0
  int ldst[C::B_NQ];  // LDS float offset in the window (-1: no item)
  int icl[C::B_NQ];
  bool rok[C::B_NQ];
  int tgoff, tldst, ticl;  // the thread's tail column (TAIL; tldst -1: none)
  bool trok;
  const WinArgs* a;
  f32x4 reg[2][C::B_NQ];
  float treg[2];

  __device__ void init(const WinArgs& args, int b, int ih_first) {
    a = &args;
    const int W4 = args.W >> 2;
    tgoff = ticl = 0;
    tldst = -1;
    trok = false;
    if constexpr (C::TAIL) {
      const int tw = args.W & 3, i = threadIdx.x;
      if (i < C::CI * C::WR * tw) {
        const int ch = i / (C::WR * tw), rem = i - ch * (C::WR * tw);
        const int wr = rem / tw, col = 4 * W4 + rem - wr * tw;
        const int ih = ih_first + wr;
        ticl = ch;
        trok = ih >= 0 && ih < args.H;
        tgoff = ((b * args.IC + ch) * args.H + ih) * args.W + col;
        tldst = ch * C::PS + wr * C::RS + C::CL + col;
      }
    }
    const int items = C::CI * C::WR * W4;
#pragma unroll
    for (int q = 0; q < C::B_NQ; ++q) {
      const int i = threadIdx.x + C::NT * q;
      ldst[q] = -1;
      goff[q] = 0;
      icl[q] = 0;
      rok[q] = false;
      if (i < items) {
        const int ch = i / (C::WR * W4), rem = i - ch * (C::WR * W4);
        const int wr = rem / W4, c4 = rem - wr * W4;
        const int ih = ih_first + wr;
        icl[q] = ch;
        rok[q] = ih >= 0 && ih < args.H;
        goff[q] = ((b * args.IC + ch) * args.H + ih) * args.W + 4 * c4;
        ldst[q] = ch * C::PS + wr * C::RS + C::CL + 4 * c4;
      }
    }
  }
  template <int S>
  __device__ void load(int t) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a->x, a->x_elems);
    const int ic0 = t * C::CI;
    const int step = ic0 * a->H * a->W;
#pragma unroll
    for (int q = 0; q < C::B_NQ; ++q) {
      const bool ok = rok[q] && ic0 + icl[q] < a->IC;
      reg[S][q] = Vec<4>::load(rs, ok ? (uint32_t)(goff[q] + step) * 4u : kOOB);
    }
    if constexpr (C::TAIL) {
      const bool ok = trok && ic0 + ticl < a->IC;
      treg[S] = Vec<1>::load(rs, ok ? (uint32_t)(tgoff + step) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* Bs) const {
#pragma unroll
    for (int q = 0; q < C::B_NQ; ++q)
      if (ldst[q] >= 0) *reinterpret_cast<f32x4*>(&Bs[ldst[q]]) = reg[S][q];
    if constexpr (C::TAIL)
      if (tldst >= 0) Bs[tldst] = treg[S];
  }
};

// LDS offset (floats) of the B value of MFMA step s relative to the lane's
// base: the step's channel within the lane-half's pair and its tap.
template <class C>
__device__ constexpr int win_off(int s) {
  return (s / C::TAPS) * C::PS + ((s % C::TAPS) / C::KW) * C::DH * C::RS +
         ((s % C::TAPS) % C::KW) * C::DW;
}

template <class C, int S0, int NS>
__device__ __forceinline__ void win_steps(f32x16& acc, const float* Aw, const float* Bw) {
  f32x4 av;
  if constexpr (NS == 4) {
    av = *reinterpret_cast<const f32x4*>(Aw + S0);
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 a2 = *reinterpret_cast<const f32x2*>(Aw + S0);
    av[0] = a2[0];
    av[1] = a2[1];
  }
  float bv[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) bv[u] = Bw[win_off<C>(S0 + u)];
#pragma unroll
  for (int u = 0; u < NS; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], acc, 0, 0, 0);
}

template <class C, int S0>
__device__ __forceinline__ void win_mma_from(f32x16& acc, const float* Aw, const float* Bw) {
  if constexpr (S0 + 4 <= C::HALF) {
    win_steps<C, S0, 4>(acc, Aw, Bw);
    win_mma_from<C, S0 + 4>(acc, Aw, Bw);
  } else if constexpr (S0 < C::HALF) {
    static_assert(C::HALF - S0 == 2, "HALF is even");
    win_steps<C, S0, 2>(acc, Aw, Bw);
  }
}

// The k loop over k-tiles [tb, te) with a two-deep register prefetch and
// double-buffered LDS (one barrier per k-tile), as the GEMM main loop.
// Loads of a range's last two iterations fetch tile te - 1 again into a slot
// never written to LDS, so no branch skips a load and the wait before each
// LDS write covers only the loads issued an iteration earlier.
template <class C>
struct WinLoop {
  WinALoader<C>& al;
  WinBLoader<C>& bl;
  f32x16& acc;
  float* smem;
  int aoff, boff;  // the lane's A and B read offsets within a stage
  int te;

  template <int S>
  __device__ __forceinline__ void fetch(int t) {
    al.template load<S>(t);
    bl.template load<S>(t);
  }
  template <int S>
  __device__ __forceinline__ void put(float* buf) {
    al.template store<S>(buf);
    bl.template store<S>(buf + C::A_FLOATS);
  }
  template <int S>
  __device__ __forceinline__ void step(int t, int i) {
    float* cur = smem + (i & 1) * C::STAGE;
    float* nxt = smem + ((i + 1) & 1) * C::STAGE;
    fetch<S>(t + 2 < te ? t + 2 : te - 1);
    win_mma_from<C, 0>(acc, cur + aoff, cur + C::A_FLOATS + boff);
    if (t + 1 < te) put<1 - S>(nxt);
    __syncthreads();
  }
};

// Zero the window columns outside the input (both stages): the loads only
// ever write columns [CL, CL + W).
template <class C>
__device__ __forceinline__ void win_zero_pads(float* smem, int W) {
  const int padw = C::RS - W;  // CL on the left, RS - CL - W on the right
  const int n = 2 * C::CI * C::WR * padw;
  for (int i = threadIdx.x; i < n; i += C::NT) {
    const int row = i / padw, j = i - row * padw;
    const int stage = row / (C::CI * C::WR), r = row - stage * (C::CI * C::WR);
    const int col = j < C::CL ? j : W + j;
    smem[stage * C::STAGE + C::A_FLOATS + r * C::RS + col] = 0.0f;
  }
}

// BIAS_AHEAD: a whole block of output channels loads its 16 bias values
// per lane before storing (the stride-2 conv 47.9 -> 46.8 us); the
// streamed instances have no registers to spare for it.
template <class C, bool BIAS_AHEAD>
__device__ __forceinline__ void win_piece(const WinArgs& p, float* smem, int m0, int n0, int tb,
                                          int te, int epi) {
  const int lane = threadIdx.x & 63, c = lane & 31, h = lane >> 5;
  const WaveSlot ws = wave_slot<C>();
  const int tn = n0 / C::BN;
  const int b = tn / p.tpi, p0 = (tn - b * p.tpi) * C::BN;
  const int oh_first = p0 / p.OW;
  const int ih_first = oh_first * C::SH - p.pH;

  WinALoader<C> al;
  al.init(p.w, m0, p.OC, p.K);
  WinBLoader<C> bl;
  bl.init(p, b, ih_first);

  // The lane's output pixel, and where its taps start in the window.
  const int pix = p0 + ws.wn0 + c;
  int boff = (2 * ws.kgroup + h) * C::CH * C::PS + C::CL;
  if (pix < p.P) {
    const int oh = pix / p.OW, ow = pix - oh * p.OW;
    boff += (oh - oh_first) * C::SH * C::RS + ow * C::SW - p.pW;
  }
  const int aoff = (ws.wm0 + c) * C::AS + (2 * ws.kgroup + h) * C::SEG;

  win_zero_pads<C>(smem, p.W);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  if (tb < te) {
    WinLoop<C> ml{al, bl, acc, smem, aoff, boff, te};
    ml.template fetch<0>(tb);
    ml.template fetch<1>(tb + 1 < te ? tb + 1 : tb);
    ml.template put<0>(smem);
    __syncthreads();
    for (int t = tb; t < te; t += 2) {
      ml.template step<0>(t, t - tb);
      if (t + 1 < te) ml.template step<1>(t + 1, t + 1 - tb);
    }
  }
  Accum<C> accs;
  accs.c[0][0] = acc;
  if (!reduce_k_groups<C>(accs, smem, ws, lane)) return;
  acc = accs.c[0][0];

  // Epilogue: + bias[oc], NCHW store out[b, oc, pix].  A two-piece tile is
  // combined first (the exchange described in gemm_core.hpp).
  const bool pok = pix < p.P;
  float* ob = p.out + (size_t)b * p.OC * p.P + pix;
  if (epi == EPI_EXCHANGE) {
    uint32_t other[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int oc = m0 + ws.wm0 + acc_row(r, lane);
      other[r] = kPieceSentinel;
      if (pok && oc < p.OC)
        other[r] = atomicExch(reinterpret_cast<unsigned int*>(&ob[(size_t)oc * p.P]),
                              __float_as_uint(acc[r]));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int oc = m0 + ws.wm0 + acc_row(r, lane);
      if (!pok || oc >= p.OC || other[r] == kPieceSentinel) continue;
      const float v = __uint_as_float(other[r]) + acc[r];
      ob[(size_t)oc * p.P] = v + (p.bias ? p.bias[oc] : 0.0f);
    }
    return;
  }
  if (!pok) return;
  if (BIAS_AHEAD && m0 + C::BM <= p.OC) {
    float bv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) bv[r] = p.bias ? p.bias[m0 + ws.wm0 + acc_row(r, lane)] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ob[(size_t)(m0 + ws.wm0 + acc_row(r, lane)) * p.P] = acc[r] + bv[r];
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int oc = m0 + ws.wm0 + acc_row(r, lane);
    if (oc < p.OC) ob[(size_t)oc * p.P] = acc[r] + (p.bias ? p.bias[oc] : 0.0f);
  }
}

template <class C, int MODE>
__global__ __launch_bounds__(C::NT) void conv_window_kernel(WinArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[C::SMEM_FLOATS];
  for_each_piece<MODE>(p.sched, C::BM, C::BN, [&](int m0, int n0, int tb, int te, int epi)
                                                  __attribute__((always_inline)) {
    win_piece<C, MODE != MODE_STREAM>(p, smem, m0, n0, tb, te, epi);
  });
}

// Compiled geometries (the host plan's table, conv_window_plan.hpp).
typedef WinCfg<3, 3, 1, 1, 1, 1, 6, 64, 128, 16, 2, 4, 2> Win3x3S1D1;
typedef WinCfg<3, 3, 1, 1, 2, 2, 8, 64, 128, 16, 2, 4, 2> Win3x3S1D2;
typedef WinCfg<3, 3, 2, 2, 1, 1, 9, 64, 64, 16, 2, 2, 4, true, 14> Win3x3S2D1;

template <class C>
constexpr bool same_geom(int g) {
  return C::KH == kWinKH[g] && C::KW == kWinKW[g] && C::SH == kWinSH[g] && C::SW == kWinSW[g] &&
         C::DH == kWinDH[g] && C::DW == kWinDW[g] && C::WR == kWinWR[g] && C::BM == kWinBM[g] &&
         C::BN == kWinBN[g] && C::CI == kWinCI && C::RS == kWinRS && C::CL == kWinCL &&
         C::NT == 64 * kWinWaves && C::WK == kWinKGroups[g] && C::TAIL == kWinTail[g] &&
         C::MAXQ == kWinMaxQ[g];
}
static_assert(same_geom<Win3x3S1D1>(WIN_3x3_S1_D1) && same_geom<Win3x3S1D2>(WIN_3x3_S1_D2) &&
                  same_geom<Win3x3S2D1>(WIN_3x3_S2_D1),
              "window geometry table out of sync with the compiled kernels");

template <class C, int MODE>
static hipError_t win_launch(const WinArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((conv_window_kernel<C, MODE>), dim3(nblocks), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

template <class C, bool STREAM>
static hipError_t win_run(const ConvProblem& q, const WinPlan& pl, hipStream_t stream) {
  WinArgs a;
  a.out = q.out;
  a.x = q.x;
  a.w = q.w;
  a.bias = q.bias;
  a.IC = q.IC;
  a.H = q.H;
  a.W = q.W;
  a.OC = q.OC;
  a.pH = q.pH;
  a.pW = q.pW;
  a.OH = q.OH;
  a.OW = q.OW;
  a.P = q.OH * q.OW;
  a.tpi = pl.tpi;
  a.K = q.IC * C::TAPS;
  a.x_elems = q.B * q.IC * q.H * q.W;
  a.sched = Sched{pl.tiles_m, pl.tiles_n, 8, pl.nkt, pl.splits, pl.kt_per_split};
  if (pl.mode != MODE_TILE) {
    // split tiles (two pieces each) meet through the sentinel exchange
    const hipError_t e = launch_conv_out_init(q.out, q.bias, true, (uint32_t)q.OC * q.B * a.P,
                                              (uint32_t)a.P, (uint32_t)q.OC, stream);
    if (e != hipSuccess) return e;
  }
  const int nblocks = (int)win_plan_blocks(pl);
  switch (pl.mode) {
    case MODE_STREAM:
      if constexpr (STREAM) return win_launch<C, MODE_STREAM>(a, nblocks, stream);
      return hipErrorInvalidValue;
    case MODE_SLICES:
      return win_launch<C, MODE_SLICES>(a, nblocks, stream);
    default:
      return win_launch<C, MODE_TILE>(a, nblocks, stream);
  }
}

hipError_t launch_conv2d_window(const ConvProblem& q, const WinPlan& pl, hipStream_t stream) {
  // the two-piece exchange needs exactly two slices (the plan makes no more)
  if (pl.mode == MODE_SLICES && pl.splits != 2) return hipErrorInvalidValue;
  switch (pl.geom) {
    case WIN_3x3_S1_D1:
      return win_run<Win3x3S1D1, kWinStream[WIN_3x3_S1_D1]>(q, pl, stream);
    case WIN_3x3_S1_D2:
      return win_run<Win3x3S1D2, kWinStream[WIN_3x3_S1_D2]>(q, pl, stream);
    case WIN_3x3_S2_D1:
      return win_run<Win3x3S2D1, kWinStream[WIN_3x3_S2_D1]>(q, pl, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace baim
