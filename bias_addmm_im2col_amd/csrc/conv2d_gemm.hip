// conv2d_gemm.hip -- groups==1 NCHW conv2d as a GEMM with an implicit
// im2col B operand ("et_vk conv2d: route standard (groups==1) conv through
// an im2col tiled GEMM", Solution and Implementation paragraphs):
// M = OC, N = B*OH*OW, K = IC*KH*KW; A is the weight viewed as [OC, K];
// B[kk, n] is the input at (b, ic, oh*sH - pH + kh*dH, ow*sW - pW + kw*dW)
// for n = (b, oh, ow) and kk = (ic, kh, kw), or 0 outside the input; the
// epilogue adds bias[oc] and stores NCHW.
//
// The im2col matrix is never formed: each B tile is gathered from the
// input straight into LDS.  The column decode n -> (b, oh, ow) is done once
// per thread; the row decode kk -> (ic, kh, kw) is uniform across a wave
// (a wave loads 64 consecutive columns of one row) and runs on the scalar
// unit with multiply-high division.
#include <stdlib.h>

#include "gemm_core.hpp"
#include "launch.hpp"
#include "tile_select.hpp"

namespace baim {

struct ConvArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW;
  int M, N, K;  // per group: OC/G, B*OH*OW, (IC/G)*KH*KW
  int x_elems;  // B*IC*H*W
  int groups, ICg, OCg;  // groups, channels per group
  FastDiv div_khw, div_kw, div_p, div_ow;
  Sched sched;
};

// B operand: the implicit im2col tile B[kk, n] for kk in [k0, k0+BK),
// n in [n0, n0+BN).
//  * Column side (per thread, once): n -> (b, oh, ow), the input offset of
//    the tap (kh, kw) = (0, 0) and its coordinates ih0 = oh*sH - pH,
//    iw0 = ow*sW - pW.  Columns past N get iw0 = -(dW*(KW-1)) - 1, so
//    every tap of theirs reads as out of range.
//  * Row side (per k-tile, in LDS): kk -> (ic, kh, kw) gives the offset
//    ic*H*W + kh*dH*W + kw*dW and the tap shifts dh = kh*dH, dw = kw*dW.
//    Rows past K get dh = -(H + 2*pH) - 1, so they read as out of range.
//    BK threads decode one row each, ahead of use (see mainloop).
//  * Element: valid iff 0 <= ih0+dh < H and 0 <= iw0+dw < W; invalid
//    elements load from an out-of-range offset and read 0 (the padding).
// A wave loads 64 consecutive columns of one row per instruction, so every
// lane of a wave reads the same table entry (an LDS broadcast).  Each lane
// gathers four consecutive rows of its column and stores them with one
// 16-byte write into the transposed tile [BN][BK+4].
template <class T>
struct ImColTileLoader {
  static constexpr bool kHasMeta = true;
  static constexpr bool kBTransposed = true;
  static constexpr int RPP = T::NT / T::BN;  // row quads covered per pass
  static constexpr int NP = T::BK * T::BN / T::NT;  // elements per thread
  static constexpr int NQ = NP / 4;                 // quads per thread
  static_assert(T::NT % T::BN == 0 && NP % 4 == 0 && T::BK == 4 * RPP * NQ, "im2col tile split");
  static_assert(T::NT >= T::BK, "one thread per table row");
  const ConvArgs* a;
  int4* tbl;  // [META_SLOTS][BK] {offset, dh, dw, unused}
  int q0, col, cbase, ih0, iw0;
  f32x4 reg[2][NQ];  // two register slots (prefetch depth up to 2)

  __device__ void init(const ConvArgs& args, int n0, int4* table, int g) {
    a = &args;
    tbl = table;
    col = threadIdx.x % T::BN;
    q0 = threadIdx.x / T::BN;
    const int n = n0 + col;
    const bool cok = n < args.N;
    const uint32_t nn = cok ? (uint32_t)n : 0u;
    const uint32_t b = fdiv(nn, args.div_p);
    const uint32_t pix = nn - b * args.div_p.d;
    const uint32_t oh = fdiv(pix, args.div_ow);
    const uint32_t ow = pix - oh * args.div_ow.d;
    ih0 = (int)oh * args.sH - args.pH;
    iw0 = cok ? (int)ow * args.sW - args.pW : -(args.dW * (args.KW - 1)) - 1;
    // image b, first input channel of group g
    cbase = ((int)b * args.IC + g * args.ICg) * args.H * args.W + ih0 * args.W + iw0;
  }
  __device__ void meta(int t) {
    if (threadIdx.x < T::BK) {
      const int kk = t * T::BK + (int)threadIdx.x;
      int4 e;
      if (kk < a->K) {
        const uint32_t ic = fdiv((uint32_t)kk, a->div_khw);
        const uint32_t rem = (uint32_t)kk - ic * a->div_khw.d;
        const uint32_t kh = fdiv(rem, a->div_kw);
        const uint32_t kw = rem - kh * a->div_kw.d;
        e.y = (int)kh * a->dH;
        e.z = (int)kw * a->dW;
        e.x = (int)ic * a->H * a->W + e.y * a->W + e.z;
      } else {
        e.x = 0;
        e.y = -(a->H + 2 * a->pH) - 1;
        e.z = 0;
      }
      e.w = 0;
      tbl[(t % T::META_SLOTS) * T::BK + threadIdx.x] = e;
    }
  }
  template <int S>
  __device__ void load(int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a->x, a->x_elems);
    const int4* slot = tbl + ((k0 / T::BK) % T::META_SLOTS) * T::BK;
    // All table reads first, then branch-free address selection, so the
    // NP global loads issue back to back.
    int4 e[NP];
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) e[4 * i + s] = slot[4 * (q0 + RPP * i) + s];
#pragma unroll
    for (int i = 0; i < NQ; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int4 v = e[4 * i + s];
        const unsigned ok = (unsigned)((unsigned)(ih0 + v.y) < (unsigned)a->H) &
                            (unsigned)((unsigned)(iw0 + v.z) < (unsigned)a->W);
        reg[S][i][s] = Vec<1>::load(rs, ok ? (uint32_t)(cbase + v.x) * 4u : kOOB);
      }
  }
  template <int S>
  __device__ void store(float* Bt) const {
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      *reinterpret_cast<f32x4*>(&Bt[col * T::BTS + 4 * (q0 + RPP * i)]) = reg[S][i];
  }
};

// A grouped conv runs one GEMM per group g = blockIdx.y: rows m of the
// group's weight slice, input channels g*IC/G.., output channels g*OC/G...
template <class T, int VA>
__device__ __forceinline__ void conv_piece(const ConvArgs& p, float* smem, int m0, int n0, int tb, int te,
                                  int epi) {
  const int lane = threadIdx.x & 63;
  const WaveSlot ws = wave_slot<T>();
  const int g = blockIdx.y;
  RowTileLoader<T, VA> al;
  al.init(p.w + (size_t)g * p.OCg * p.K, m0, p.M, p.K);
  ImColTileLoader<T> bl;
  bl.init(p, n0, reinterpret_cast<int4*>(smem + 2 * T::STAGE), g);
  Accum<T> acc;
  mainloop<T>(acc, al, bl, tb, te, smem, ws, lane);
  if (!reduce_k_groups<T>(acc, smem, ws, lane)) return;

  // Epilogue: + bias[oc], NCHW store: column n = (b, pix) goes to
  // out[b, oc, pix] = out[(b*OC + oc)*P + pix], P = OH*OW.  A split tile's
  // pieces are combined first (see the two-piece exchange and the atomic
  // K slices in gemm_core.hpp).
  const int c = lane & 31;
  const uint32_t P = p.div_p.d;
  size_t obase[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n0 + ws.wn0 + 32 * j + c;
    const uint32_t b = fdiv((uint32_t)(n < p.N ? n : 0), p.div_p);
    obase[j] = (size_t)b * p.OC * P + ((uint32_t)n - b * P);
  }
  if (epi == EPI_EXCHANGE) {
    // Two-piece tile: swap every partial in first (all swaps in flight at
    // once), then finish the elements whose other piece had already landed.
    uint32_t other[T::FM][T::FN][16];
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = n0 + ws.wn0 + 32 * j + c, oc = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          other[i][j][r] = kPieceSentinel;
          if (n < p.N && oc < p.M)
            other[i][j][r] = atomicExch(
                reinterpret_cast<unsigned int*>(&p.out[obase[j] + (size_t)(g * p.OCg + oc) * P]),
                __float_as_uint(acc.c[i][j][r]));
        }
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = n0 + ws.wn0 + 32 * j + c, oc = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          if (n >= p.N || oc >= p.M || other[i][j][r] == kPieceSentinel) continue;
          const int ocx = g * p.OCg + oc;
          const float v = __uint_as_float(other[i][j][r]) + acc.c[i][j][r];
          p.out[obase[j] + (size_t)ocx * P] = v + (p.bias ? p.bias[ocx] : 0.0f);
        }
    return;
  }
  if (epi == EPI_STORE && m0 + T::BM <= p.M && n0 + T::BN <= p.N) {
    // A whole tile: per 32-row block the bias values first, then stores
    // without tests (the grouped 3x3 conv with 8 groups of 32 channels:
    // 42.4 -> 39.5 us), non-temporal since nothing reads them back (38.9 ->
    // 37.8 us).
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      float bv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        bv[r] = p.bias ? p.bias[g * p.OCg + m0 + ws.wm0 + 32 * i + acc_row(r, lane)] : 0.0f;
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ocx = g * p.OCg + m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          __builtin_nontemporal_store(acc.c[i][j][r] + bv[r], &p.out[obase[j] + (size_t)ocx * P]);
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n0 + ws.wn0 + 32 * j + c;
    if (n >= p.N) continue;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int oc = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
        if (oc >= p.M) continue;
        const int ocx = g * p.OCg + oc;
        float* o = &p.out[obase[j] + (size_t)ocx * P];
        if (epi == EPI_ATOMIC)
          unsafeAtomicAdd(o, acc.c[i][j][r]);
        else
          *o = acc.c[i][j][r] + (p.bias ? p.bias[ocx] : 0.0f);
      }
  }
}

template <class T, int VA, int MODE>
__global__ __launch_bounds__(T::NT) void conv2d_gemm_kernel(ConvArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[T::SMEM_FLOATS];
  for_each_piece<MODE>(p.sched, T::BM, T::BN, [&](int m0, int n0, int tb, int te, int epi) __attribute__((always_inline)) {
    conv_piece<T, VA>(p, smem, m0, n0, tb, te, epi);
  });
}

// Output initialisation before a split tile's pieces land: the sentinel
// (two-piece combine, 16-byte stores) or bias[oc] / 0 (atomic K slices).
__global__ __launch_bounds__(256) void conv_init_kernel(float* out, const float* bias,
                                                        int sentinel, uint32_t total,
                                                        FastDiv div_p, uint32_t OC) {
  const uint32_t stride = gridDim.x * 256u;
  if (sentinel) {
    const float s = __uint_as_float(kPieceSentinel);
    const f32x4 s4 = {s, s, s, s};
    const uint32_t head = (uint32_t)((16u - ((uintptr_t)out & 15u)) & 15u) / 4u;
    const uint32_t h = head < total ? head : total;
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < h; i += stride) out[i] = s;
    const uint32_t nvec = (total - h) / 4u;
    f32x4* o4 = reinterpret_cast<f32x4*>(out + h);
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < nvec; i += stride) o4[i] = s4;
    for (uint32_t i = h + nvec * 4u + blockIdx.x * 256u + threadIdx.x; i < total; i += stride)
      out[i] = s;
    return;
  }
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += stride)
    out[i] = bias ? bias[fdiv(i, div_p) % OC] : 0.0f;
}

typedef Tile<128, 128, 32, 2, 4, 1, 2> T128x128;
typedef Tile<128, 64, 32, 4, 2, 1, 2> T128x64;
typedef Tile<64, 128, 32, 2, 4, 1, 2> T64x128;
typedef Tile<64, 64, 32, 2, 2, 1, 2> T64x64;
// The 16-wave 128x128 tile keeps a one-tile prefetch here: the im2col
// loader's extra registers would not fit a second slot in its budget.
typedef Tile<128, 128, 64, 2, 4, 2, 1> T128x128K2;
typedef Tile<128, 64, 64, 4, 2, 2, 2> T128x64K2;
typedef Tile<64, 64, 64, 2, 2, 2, 2> T64x64K2;
typedef Tile<64, 64, 128, 2, 2, 4, 2> T64x64K4;
typedef Tile<32, 128, 32, 1, 4, 1, 2> T32x128;

// The host planner's table must describe exactly these tiles.
template <class T>
constexpr bool same_tile(int cfg) {
  return T::BM == kTileBM[cfg] && T::BN == kTileBN[cfg] && T::BK == kTileBK[cfg] &&
         T::NT == 64 * kTileWaves[cfg] && T::WK == kTileKGroups[cfg];
}
static_assert(same_tile<T128x128>(TILE_128x128) && same_tile<T128x64>(TILE_128x64) &&
                  same_tile<T64x128>(TILE_64x128) && same_tile<T64x64>(TILE_64x64) &&
                  same_tile<T128x128K2>(TILE_128x128_K2) && same_tile<T128x64K2>(TILE_128x64_K2) &&
                  same_tile<T64x64K2>(TILE_64x64_K2) && same_tile<T64x64K4>(TILE_64x64_K4) &&
                  same_tile<T32x128>(TILE_32x128),
              "tile table out of sync with the compiled tiles");

template <class T, int VA, int MODE>
static hipError_t launch_t(const ConvArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((conv2d_gemm_kernel<T, VA, MODE>), dim3(nblocks, a.groups), dim3(T::NT), 0, s,
                     a);
  return hipGetLastError();
}

// Stream pieces are compiled for 16-byte weight loads only (the launcher
// falls back to one tile per block otherwise).
template <class T, int CFG, int MODE>
static hipError_t launch_vec(const ConvArgs& a, int nblocks, bool va, hipStream_t s) {
  if constexpr (MODE == MODE_STREAM) {
    if constexpr (kTileStream[CFG]) return launch_t<T, 4, MODE_STREAM>(a, nblocks, s);
    return hipErrorInvalidValue;  // never planned
  } else if constexpr (MODE == MODE_SLICES && !kTileSlices[CFG]) {
    return hipErrorInvalidValue;  // never planned
  } else {
    return va ? launch_t<T, 4, MODE>(a, nblocks, s) : launch_t<T, 1, MODE>(a, nblocks, s);
  }
}

template <int MODE>
static hipError_t launch_cfg(int cfg, const ConvArgs& a, int nblocks, bool va, hipStream_t s) {
  switch (cfg) {
    case TILE_128x64:
      return launch_vec<T128x64, TILE_128x64, MODE>(a, nblocks, va, s);
    case TILE_64x128:
      return launch_vec<T64x128, TILE_64x128, MODE>(a, nblocks, va, s);
    case TILE_64x64:
      return launch_vec<T64x64, TILE_64x64, MODE>(a, nblocks, va, s);
    case TILE_128x128_K2:
      return launch_vec<T128x128K2, TILE_128x128_K2, MODE>(a, nblocks, va, s);
    case TILE_128x64_K2:
      return launch_vec<T128x64K2, TILE_128x64_K2, MODE>(a, nblocks, va, s);
    case TILE_64x64_K2:
      return launch_vec<T64x64K2, TILE_64x64_K2, MODE>(a, nblocks, va, s);
    case TILE_64x64_K4:
      return launch_vec<T64x64K4, TILE_64x64_K4, MODE>(a, nblocks, va, s);
    case TILE_256x256:
      return hipErrorInvalidValue;  // not compiled here (plan_core_tile)
    case TILE_32x128:
      return launch_vec<T32x128, TILE_32x128, MODE>(a, nblocks, va, s);
    default:
      return launch_vec<T128x128, TILE_128x128, MODE>(a, nblocks, va, s);
  }
}

hipError_t launch_conv_out_init(float* out, const float* bias, bool sentinel, uint32_t total,
                                uint32_t P, uint32_t OC, hipStream_t stream) {
  const int gb = (int)((total + 255u) / 256u < 4096u ? (total + 255u) / 256u : 4096u);
  hipLaunchKernelGGL(conv_init_kernel, dim3(gb), dim3(256), 0, stream, out, bias, sentinel ? 1 : 0,
                     total, make_fastdiv(P), OC);
  return hipGetLastError();
}

hipError_t launch_conv2d(const ConvProblem& q, hipStream_t stream) {
  const bool aligned = ((uintptr_t)q.x & 15) == 0 && ((uintptr_t)q.w & 15) == 0;
  const char* wspec = getenv("BAIM_CONV_WIN");
  const WinPlan wp = plan_conv_window(win_shape(q), aligned, wspec);
  if (wp.geom >= 0) return launch_conv2d_window(q, wp, stream);
  if (plan_conv_stem(win_shape(q), aligned, wspec)) return launch_conv2d_stem(q, false, stream);
  ConvArgs a;
  a.out = q.out;
  a.x = q.x;
  a.w = q.w;
  a.bias = q.bias;
  a.IC = q.IC;
  a.H = q.H;
  a.W = q.W;
  a.OC = q.OC;
  a.KH = q.KH;
  a.KW = q.KW;
  a.sH = q.sH;
  a.sW = q.sW;
  a.pH = q.pH;
  a.pW = q.pW;
  a.dH = q.dH;
  a.dW = q.dW;
  a.OH = q.OH;
  a.OW = q.OW;
  a.groups = q.groups;
  a.ICg = q.IC / q.groups;
  a.OCg = q.OC / q.groups;
  a.M = a.OCg;
  a.N = q.B * q.OH * q.OW;
  a.K = a.ICg * q.KH * q.KW;
  a.x_elems = q.B * q.IC * q.H * q.W;
  a.div_khw = make_fastdiv((uint32_t)(q.KH * q.KW));
  a.div_kw = make_fastdiv((uint32_t)q.KW);
  a.div_p = make_fastdiv((uint32_t)(q.OH * q.OW));
  a.div_ow = make_fastdiv((uint32_t)q.OW);
  const bool va = a.K % 4 == 0 && ((uintptr_t)q.w & 15) == 0;
  GemmPlan plan = plan_core_tile(plan_gemm(a.M, a.N, a.K, getenv("BAIM_TILE")), a.M, a.N, a.K);
  if (plan.mode == MODE_STREAM && !va) plan = plan_tiles_only(plan, a.M, a.N, a.K);
  a.sched = Sched{plan.tiles_m, plan.tiles_n, 8, plan.nkt, plan.splits, plan.kt_per_split};
  const int nblocks = (int)plan_blocks(plan);
  if (plan_needs_init(plan)) {
    const hipError_t e = launch_conv_out_init(q.out, q.bias, plan_uses_exchange(plan),
                                              (uint32_t)q.OC * (uint32_t)a.N, a.div_p.d,
                                              (uint32_t)q.OC, stream);
    if (e != hipSuccess) return e;
  }
  switch (plan.mode) {
    case MODE_SLICES:
      return launch_cfg<MODE_SLICES>(plan.cfg, a, nblocks, va, stream);
    case MODE_STREAM:
      return launch_cfg<MODE_STREAM>(plan.cfg, a, nblocks, va, stream);
    default:
      return launch_cfg<MODE_TILE>(plan.cfg, a, nblocks, va, stream);
  }
}

}  // namespace baim
