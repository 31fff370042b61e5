// conv_transpose.hip -- transposed conv2d (NCHW, weight [IC, OC/G, KH, KW])
// as implicit GEMMs on the fp32 matrix cores.
//
// The conv page routes transposed convs to their own gather kernels ("et_vk
// conv2d: route standard (groups==1) conv through an im2col tiled GEMM",
// Solution paragraph); the operation is the adjoint of conv2d: input element
// (ih, iw) meets weight tap (kh, kw) at output (ih*sH - pH + kh*dH,
// iw*sW - pW + kw*dW).  Gathered per output, a tap contributes only when
// oh + pH - kh*dH is a multiple of sH, which depends on oh only through
// its phase rh = oh % sH.  So the outputs split into sH*sW phases
// (rh, rw), and on phase (rh, rw) the valid taps form a fixed arithmetic
// progression kh = kh0 + i*step (step = sH / gcd(sH, dH)) with input row
//   ih = t + c0h - i*dlh     (oh = rh + sH*t, dlh = dH / gcd(sH, dH)),
// and likewise along W.  Each phase is then a dense GEMM without wasted
// taps:
//   M = OC/G, N = B * Th * Tw (the phase's outputs), K = IC/G * nh * nw,
//   A[oc, kk] = w[ic, oc, kh_i, kw_j], B[kk, n] = x[b, ic, ih, iw] (0 outside),
// with kk = (ic*nh + i)*nw + j.  One launch runs all phases (blockIdx.y,
// up to 16 per launch) and groups (blockIdx.z); the per-phase geometry is
// computed on the host.
//
// Both operands are gathered through a per-k-tile LDS table (as in the
// conv's im2col loader): row kk -> {input offset, ih shift, iw shift,
// weight offset}.  The weight is small and cache-resident, so its A tile
// uses 4-byte loads; the input gather writes the transposed B tile with
// 16-byte LDS stores.  The epilogue adds bias[oc] and stores to
// out[b, oc, rh + sH*t, rw + sW*u].  When the tiles of all phases would
// leave most CUs idle and K is deep, K is split over blocks instead: an
// initialisation kernel writes bias[oc] into the output and each slice adds
// its partial sums atomically (the summation order then varies run to run).
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "gemm_core.hpp"
#include "launch.hpp"
#include "tile_select.hpp"

namespace baim {

namespace {

constexpr int kMaxPhases = 16;  // phases per launch

struct ConvTPhase {
  int rh, rw;                      // output phase
  int Th, Tw;                      // outputs of the phase per image: rows, columns
  int N, K;                        // B*Th*Tw, ICg*nh*nw
  int tiles_n, nkt;
  int kps;                         // k-tiles per K slice
  int nw;                          // valid taps along W
  int kh0, kw0, step_h, step_w;    // valid taps kh = kh0 + i*step_h, kw = kw0 + j*step_w
  int c0h, c0w, dlh, dlw;          // input row of tap i: t + c0h - i*dlh (same along W)
  FastDiv div_p, div_tw, div_taps, div_nw;
};

struct ConvTArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int IC, H, W, OC, KH, KW, sH, sW, OH, OW;
  int ICg, OCg;
  int x_elems, w_elems;
  int tiles_m;
  int splits;     // K slices per tile; above 1 they add into an output holding the bias
  int slice_row;  // blocks per slice in a grid row: tiles_m * (largest phase's tiles_n)
  ConvTPhase ph[kMaxPhases];
};

// Entry e of the table for row kk: {input offset, ih shift, iw shift,
// weight offset}; rows past K get an ih shift that fails every bounds test
// and weight offset -1.
template <class T>
struct TImColLoader {
  static constexpr bool kHasMeta = true;
  static constexpr bool kBTransposed = true;
  static constexpr int RPP = T::NT / T::BN;
  static constexpr int NP = T::BK * T::BN / T::NT;
  static constexpr int NQ = NP / 4;
  static_assert(T::NT % T::BN == 0 && NP % 4 == 0 && T::BK == 4 * RPP * NQ, "gather tile split");
  static_assert(T::NT >= T::BK, "one thread per table row");
  int4* tbl;
  __amdgpu_buffer_rsrc_t rs;
  int q0, col, cbase, ih0, iw0, H, W;
  // table construction
  int K, HW, OCKK, KW, kh0, kw0, step_h, step_w, c0h, c0w, dlh, dlw, nw;
  FastDiv div_taps, div_nw;
  f32x4 reg[2][NQ];

  __device__ void init(const ConvTArgs& a, const ConvTPhase& P, int n0, int4* table, int g) {
    tbl = table;
    rs = make_rsrc(a.x, a.x_elems);
    H = a.H;
    W = a.W;
    K = P.K;
    HW = a.H * a.W;
    OCKK = a.OCg * a.KH * a.KW;
    KW = a.KW;
    kh0 = P.kh0;
    kw0 = P.kw0;
    step_h = P.step_h;
    step_w = P.step_w;
    c0h = P.c0h;
    c0w = P.c0w;
    dlh = P.dlh;
    dlw = P.dlw;
    nw = P.nw;
    div_taps = P.div_taps;
    div_nw = P.div_nw;
    col = threadIdx.x % T::BN;
    q0 = threadIdx.x / T::BN;
    const int n = n0 + col;
    const bool cok = n < P.N;
    const uint32_t nn = cok ? (uint32_t)n : 0u;
    const uint32_t b = fdiv(nn, P.div_p);
    const uint32_t pix = nn - b * P.div_p.d;
    const uint32_t t = fdiv(pix, P.div_tw);
    const uint32_t u = pix - t * P.div_tw.d;
    ih0 = (int)t;
    iw0 = cok ? (int)u : -(1 << 29);
    cbase = ((int)b * a.IC + g * a.ICg) * HW + (int)t * W + (int)u;
  }
  __device__ void meta(int tt) {
    if (threadIdx.x < T::BK) {
      const int kk = tt * T::BK + (int)threadIdx.x;
      int4 e;
      if (kk < K) {
        const uint32_t ic = fdiv((uint32_t)kk, div_taps);
        const uint32_t rem = (uint32_t)kk - ic * div_taps.d;
        const uint32_t i = fdiv(rem, div_nw);
        const int j = (int)rem - (int)i * nw;
        e.y = c0h - (int)i * dlh;
        e.z = c0w - j * dlw;
        e.x = (int)ic * HW + e.y * W + e.z;
        e.w = (int)ic * OCKK + (kh0 + (int)i * step_h) * KW + kw0 + j * step_w;
      } else {
        e.x = 0;
        e.y = -(1 << 29);
        e.z = 0;
        e.w = -1;
      }
      tbl[(tt % T::META_SLOTS) * T::BK + threadIdx.x] = e;
    }
  }
  template <int S>
  __device__ void load(int k0) {
    const int4* slot = tbl + ((k0 / T::BK) % T::META_SLOTS) * T::BK;
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
        const unsigned ok = (unsigned)((unsigned)(ih0 + v.y) < (unsigned)H) &
                            (unsigned)((unsigned)(iw0 + v.z) < (unsigned)W);
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

// A tile [BM][BK+4] of the phase's weight matrix A[oc, kk] =
// w[ic, oc, kh_i, kw_j]: a thread keeps one k column (its table entry) and
// loads NCH rows oc with 4-byte loads.
template <class T>
struct TWeightLoader {
  static constexpr int NCH = T::BM * T::BK / T::NT;
  static_assert((T::BM * T::BK) % T::NT == 0 && T::NT % T::BK == 0, "weight tile split");
  const int4* tbl;
  __amdgpu_buffer_rsrc_t rs;
  int col, r0, rows_left, khw;
  float reg[2][NCH];

  __device__ void init(const ConvTArgs& a, int m0, const int4* table, int g) {
    tbl = table;
    khw = a.KH * a.KW;
    // group g: weight rows g*ICg.. (the table's offsets are local to them),
    // and the block's first output channel m0 folded into the base
    const int64_t base = ((int64_t)g * a.ICg * a.OCg + m0) * khw;
    rs = make_rsrc(a.w + base, a.w_elems - base);
    col = threadIdx.x % T::BK;
    r0 = threadIdx.x / T::BK;
    rows_left = a.OCg - m0;
  }
  template <int S>
  __device__ void load(int k0) {
    const int4 e = tbl[((k0 / T::BK) % T::META_SLOTS) * T::BK + col];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = r0 + i * (T::NT / T::BK);
      const bool ok = e.w >= 0 && r < rows_left;
      reg[S][i] = Vec<1>::load(rs, ok ? (uint32_t)(e.w + r * khw) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* As) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) As[(r0 + i * (T::NT / T::BK)) * T::AS + col] = reg[S][i];
  }
  __device__ void meta(int) {}
};

// Phases with a single tap and the input grid as their output grid (kernel
// equal to the stride, no padding: the 2x2 stride-2 upsampling): B[kk, n]
// = x[b, g*ICg + kk, t, u] is a plain row-major [K, N] matrix per image, so
// B tiles load as 16-byte quads of four output pixels (H*W % 4 == 0 keeps a
// quad inside one image) into the [BK][BN+8] layout, and A[oc, kk] =
// w[g*ICg + kk, oc, kh0, kw0] needs no table.
template <class T>
struct TUnitColLoader {
  static constexpr bool kHasMeta = false;
  static constexpr bool kBTransposed = false;
  static constexpr int QPR = T::BN / 4;                  // quads per tile row
  static constexpr int NI = T::BK * QPR / T::NT;         // quads per thread
  static_assert((T::BK * QPR) % T::NT == 0, "tile splits evenly");
  __amdgpu_buffer_rsrc_t rs;
  int HW, K;
  int base[NI], kk[NI], n4[NI];
  bool nok[NI];
  f32x4 reg[2][NI];

  __device__ void init(const ConvTArgs& a, const ConvTPhase& P, int n0, int4*, int g) {
    rs = make_rsrc(a.x, a.x_elems);
    HW = a.H * a.W;
    K = P.K;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = (int)threadIdx.x + T::NT * i;
      kk[i] = idx / QPR;
      n4[i] = idx - kk[i] * QPR;
      const int n = n0 + 4 * n4[i];
      nok[i] = n < P.N;
      const uint32_t nn = nok[i] ? (uint32_t)n : 0u;
      const uint32_t b = fdiv(nn, P.div_p);
      base[i] = ((int)b * a.IC + g * a.ICg) * HW + (int)(nn - b * P.div_p.d);
    }
  }
  __device__ void meta(int) {}
  template <int S>
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = k0 + kk[i];
      reg[S][i] = Vec<4>::load(rs, (nok[i] && k < K) ? (uint32_t)(base[i] + k * HW) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* Bs) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<f32x4*>(&Bs[kk[i] * T::BS + 4 * n4[i]]) = reg[S][i];
  }
};

template <class T>
struct TUnitWeightLoader {
  static constexpr int NCH = T::BM * T::BK / T::NT;
  static_assert((T::BM * T::BK) % T::NT == 0 && T::NT % T::BK == 0, "weight tile split");
  __amdgpu_buffer_rsrc_t rs;
  int col, r0, rows_left, khw, ockk, tap0, K;
  float reg[2][NCH];

  __device__ void init(const ConvTArgs& a, const ConvTPhase& P, int m0, int g) {
    khw = a.KH * a.KW;
    const int64_t base = ((int64_t)g * a.ICg * a.OCg + m0) * khw;
    rs = make_rsrc(a.w + base, a.w_elems - base);
    col = threadIdx.x % T::BK;
    r0 = threadIdx.x / T::BK;
    rows_left = a.OCg - m0;
    ockk = a.OCg * khw;
    tap0 = P.kh0 * a.KW + P.kw0;
    K = P.K;
  }
  template <int S>
  __device__ void load(int k0) {
    const int k = k0 + col;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = r0 + i * (T::NT / T::BK);
      const bool ok = k < K && r < rows_left;
      reg[S][i] = Vec<1>::load(rs, ok ? (uint32_t)(k * ockk + tap0 + r * khw) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* As) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) As[(r0 + i * (T::NT / T::BK)) * T::AS + col] = reg[S][i];
  }
  __device__ void meta(int) {}
};

// UNIT: every phase has one tap and the input grid as its output grid
// (TUnitColLoader); else the table-driven gathers.
template <class T, bool UNIT>
__global__ __launch_bounds__(T::NT) void conv_transpose_kernel(ConvTArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[T::SMEM_FLOATS];
  const ConvTPhase& P = a.ph[blockIdx.y];
  const int g = blockIdx.z;
  const int ntiles = a.tiles_m * P.tiles_n;
  const int lid = xcd_linear(blockIdx.x, gridDim.x);
  const int z = lid / a.slice_row, tile = lid - z * a.slice_row;
  if (tile >= ntiles) return;  // this phase has fewer tiles than the grid row
  const int tb = z * P.kps;
  const int te = P.nkt < tb + P.kps ? P.nkt : tb + P.kps;
  if (a.splits > 1 && tb >= te) return;  // empty slice: the output already holds the bias
  int tm, tn;
  grouped_tile(tile, a.tiles_m, P.tiles_n, 8, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int lane = threadIdx.x & 63;
  const WaveSlot ws = wave_slot<T>();
  Accum<T> acc;
  if constexpr (UNIT) {
    TUnitWeightLoader<T> al;
    al.init(a, P, m0, g);
    TUnitColLoader<T> bl;
    bl.init(a, P, n0, nullptr, g);
    mainloop<T>(acc, al, bl, tb, te, smem, ws, lane);
  } else {
    int4* table = reinterpret_cast<int4*>(smem + 2 * T::STAGE);
    TWeightLoader<T> al;
    al.init(a, m0, table, g);
    TImColLoader<T> bl;
    bl.init(a, P, n0, table, g);
    // the unpeeled k loop: 62.4 against 65.0 us peeled on the 4x4 stride-2 case
    mainloop<T, decltype(al), decltype(bl), false>(acc, al, bl, tb, te, smem, ws, lane);
  }
  if (!reduce_k_groups<T>(acc, smem, ws, lane)) return;

  // + bias[oc]; column n = (b, t, u) goes to out[b, oc, rh + sH*t, rw + sW*u].
  const int c = lane & 31;
  const size_t plane = (size_t)a.OH * a.OW;
  size_t obase[T::FN];
  bool nok[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n0 + ws.wn0 + 32 * j + c;
    nok[j] = n < P.N;
    const uint32_t nn = nok[j] ? (uint32_t)n : 0u;
    const uint32_t b = fdiv(nn, P.div_p);
    const uint32_t pix = nn - b * P.div_p.d;
    const uint32_t t = fdiv(pix, P.div_tw);
    const uint32_t u = pix - t * P.div_tw.d;
    obase[j] = (size_t)b * a.OC * plane + (size_t)(P.rh + a.sH * (int)t) * a.OW +
               (size_t)(P.rw + a.sW * (int)u);
  }
  if (a.splits == 1 && m0 + T::BM <= a.OCg && n0 + T::BN <= P.N) {
    // A whole tile: per 32-row block the bias values first, then stores
    // without tests (the 4x4 stride-2 upsampling 62.3 -> 60.9 us).
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      float bv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        bv[r] = a.bias ? a.bias[g * a.OCg + m0 + ws.wm0 + 32 * i + acc_row(r, lane)] : 0.0f;
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ocx = g * a.OCg + m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          a.out[obase[j] + (size_t)ocx * plane] = acc.c[i][j][r] + bv[r];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    if (!nok[j]) continue;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int oc = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
        if (oc >= a.OCg) continue;
        const int ocx = g * a.OCg + oc;
        float* o = &a.out[obase[j] + (size_t)ocx * plane];
        if (a.splits > 1)
          unsafeAtomicAdd(o, acc.c[i][j][r]);
        else
          *o = acc.c[i][j][r] + (a.bias ? a.bias[ocx] : 0.0f);
      }
  }
}

// bias[oc] (or 0) into every output before K slices add their partial sums.
__global__ __launch_bounds__(256) void convt_init_kernel(float* out, const float* bias, uint32_t total,
                                                         FastDiv div_plane, uint32_t OC) {
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += stride)
    out[i] = bias ? bias[fdiv(i, div_plane) % OC] : 0.0f;
}

typedef Tile<128, 128, 32, 2, 4, 1, 2> T128x128;
typedef Tile<128, 64, 32, 4, 2, 1, 2> T128x64;
typedef Tile<64, 128, 32, 2, 4, 1, 2> T64x128;
typedef Tile<64, 64, 32, 2, 2, 1, 2> T64x64;
typedef Tile<128, 128, 64, 2, 4, 2, 1> T128x128K2;
typedef Tile<128, 64, 64, 4, 2, 2, 2> T128x64K2;
typedef Tile<64, 64, 64, 2, 2, 2, 2> T64x64K2;
typedef Tile<64, 64, 128, 2, 2, 4, 2> T64x64K4;
typedef Tile<32, 128, 32, 1, 4, 1, 2> T32x128;

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

// Valid taps of one axis on output phase r: k in [0, KK) with
// r + p - k*d a multiple of s, as k0 + i*step for i < n.
struct AxisTaps {
  int k0, step, n, c0, dl;
};

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

AxisTaps axis_taps(int r, int s, int p, int d, int KK) {
  AxisTaps t{0, s / gcd_int(s, d), 0, 0, d / gcd_int(s, d)};
  for (int k = 0; k < KK; ++k)
    if ((r + p - k * d) % s == 0) {
      t.k0 = k;
      t.n = (KK - 1 - k) / t.step + 1;
      t.c0 = (r + p - k * d) / s;  // exact
      return t;
    }
  return t;
}

template <class T>
hipError_t launch_phases(const ConvTArgs& a, int nph, int groups, bool unit, hipStream_t s) {
  const dim3 grid(a.slice_row * a.splits, nph, groups);
  if (unit)
    hipLaunchKernelGGL((conv_transpose_kernel<T, true>), grid, dim3(T::NT), 0, s, a);
  else
    hipLaunchKernelGGL((conv_transpose_kernel<T, false>), grid, dim3(T::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cfg(int cfg, const ConvTArgs& a, int nph, int groups, bool unit,
                      hipStream_t s) {
  switch (cfg) {
    case TILE_128x64: return launch_phases<T128x64>(a, nph, groups, unit, s);
    case TILE_64x128: return launch_phases<T64x128>(a, nph, groups, unit, s);
    case TILE_64x64: return launch_phases<T64x64>(a, nph, groups, unit, s);
    case TILE_128x128_K2: return launch_phases<T128x128K2>(a, nph, groups, unit, s);
    case TILE_128x64_K2: return launch_phases<T128x64K2>(a, nph, groups, unit, s);
    case TILE_64x64_K2: return launch_phases<T64x64K2>(a, nph, groups, unit, s);
    case TILE_64x64_K4: return launch_phases<T64x64K4>(a, nph, groups, unit, s);
    case TILE_32x128: return launch_phases<T32x128>(a, nph, groups, unit, s);
    case TILE_256x256: return hipErrorInvalidValue;  // not compiled here (plan_core_tile)
    default: return launch_phases<T128x128>(a, nph, groups, unit, s);
  }
}

// ------------------------------------------------ kernel = stride, no pad
//
// When the kernel equals the stride and there is no padding (the 2x2
// stride-2 upsampling), every output pixel takes exactly one tap, and all
// phases read the same input pixel: out[b, oc, sH*t + kh, sW*u + kw] =
// bias[oc] + sum_ic x[b, ic, t, u] * w[ic, oc, kh, kw].  So the phases fuse
// into one GEMM per group, M = OCg*KH*KW rows m = (oc, kh, kw), N = B*H*W,
// K = ICg: A[m, ic] = w[ic, m] (the weight viewed [ICg, M], row-major: A
// transposed), B[ic, n] = x[b, ic, t, u] (row-major [K, H*W] per image),
// each B tile loaded once for all phases.  A's tiles load as 16-byte quads
// along m and go to LDS transposed, lanes along k (conflict-free 4-byte
// stores); a B tile lies inside one image (H*W % BN == 0).  With KW == 2 a
// lane holds both kw of an output pair and stores them as 8 bytes.

// A tile [BM][BK+4] from a row-major [K][M] matrix (A transposed).
template <class T>
struct TColALoader {
  static constexpr int CPR = T::BM / 4;  // quads per k row
  static constexpr int NCH = T::BK * CPR / T::NT;
  static_assert((T::BK * CPR) % T::NT == 0 && T::NT % T::BK == 0, "A tile split");
  const float* base;  // column m0 of row 0
  int M, K, cols_left;
  f32x4 reg[2][NCH];

  __device__ void init(const float* At, int m0, int M_, int K_) {
    base = At + m0;
    M = M_;
    K = K_;
    cols_left = M_ - m0;
  }
  // item q: k row q % BK (consecutive lanes, consecutive rows), quad q / BK
  template <int S>
  __device__ void load(int k0) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (size_t)k0 * M, (int64_t)(K - k0) * M - (M - cols_left));
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q % T::BK, c = (q / T::BK) * 4;
      const bool ok = k0 + r < K && c < cols_left;  // M % 4 == 0: whole quads
      reg[S][i] = Vec<4>::load(rs, ok ? (uint32_t)(r * M + c) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* As) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q % T::BK, c = (q / T::BK) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) As[(c + e) * T::AS + r] = reg[S][i][e];
    }
  }
  __device__ void meta(int) {}
};

struct ConvTFusedArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int IC, ICg, OC, OCg, KH, KW, W, OH, OW;
  int M, HW, tiles_m, tiles_n;
  FastDiv div_khw, div_kw, div_w;
};

template <class T>
__global__ __launch_bounds__(T::NT) void convt_fused_kernel(ConvTFusedArgs a) {
  __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];
  const int g = blockIdx.z;
  const int lid = xcd_linear(blockIdx.x, gridDim.x);
  int tm, tn;
  grouped_tile(lid, a.tiles_m, a.tiles_n, 8, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int b = n0 / a.HW, p0 = n0 - b * a.HW;  // the tile lies in image b
  const int lane = threadIdx.x & 63;
  const WaveSlot ws = wave_slot<T>();
  TColALoader<T> al;
  al.init(a.w + (size_t)g * a.ICg * a.M, m0, a.M, a.ICg);
  ColTileLoader<T, 4> bl;
  bl.init(a.x + ((size_t)b * a.IC + (size_t)g * a.ICg) * a.HW, p0, a.HW, a.ICg);
  Accum<T> acc;
  mainloop<T>(acc, al, bl, 0, (a.ICg + T::BK - 1) / T::BK, smem, ws, lane);
  if (!reduce_k_groups<T>(acc, smem, ws, lane)) return;

  // row m = (oc, kh, kw), column p = (t, u) of image b
  const int c = lane & 31;
  const size_t plane = (size_t)a.OH * a.OW;
  float* ob = a.out + ((size_t)b * a.OC + (size_t)g * a.OCg) * plane;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const uint32_t pix = (uint32_t)(p0 + ws.wn0 + 32 * j + c);
    const uint32_t t = fdiv(pix, a.div_w), u = pix - t * a.div_w.d;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      if (a.KW == 2) {
        // rows m (kw = 0) and m + 1 (kw = 1) sit in registers r and r + 1
        // of the lane: one 8-byte store of two neighbouring outputs, marked
        // non-temporal (the 2x2 upsampling 24.4 -> 22.3 us; the phase
        // kernel's half-line stride-2 stores got slower that way, 61.0 ->
        // 63.3 us on the 4x4 case, and keep plain stores)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int m = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          if (m0 + T::BM > a.M && m >= a.M) continue;  // only an edge tile tests
          const uint32_t oc = fdiv((uint32_t)m, a.div_khw), kh = ((uint32_t)m - oc * a.div_khw.d) >> 1;
          const float bv = a.bias ? a.bias[g * a.OCg + oc] : 0.0f;
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(
              f32x2{acc.c[i][j][r] + bv, acc.c[i][j][r + 1] + bv},
              reinterpret_cast<f32x2*>(&ob[oc * plane + (size_t)(a.KH * t + kh) * a.OW + 2 * u]));
        }
        continue;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
        if (m0 + T::BM > a.M && m >= a.M) continue;  // only an edge tile tests
        const uint32_t oc = fdiv((uint32_t)m, a.div_khw), tap = (uint32_t)m - oc * a.div_khw.d;
        const uint32_t kh = fdiv(tap, a.div_kw), kw = tap - kh * a.div_kw.d;
        ob[oc * plane + (size_t)(a.KH * t + kh) * a.OW + a.KW * u + kw] =
            acc.c[i][j][r] + (a.bias ? a.bias[g * a.OCg + oc] : 0.0f);
      }
    }
  }
}

// Whether q takes the fused path, and with which tile (64 x 128 below 128
// rows, else 128 x 128; both 128 pixels wide).
int convt_fused_cfg(const ConvTProblem& q) {
  const int ICg = q.IC / q.groups, OCg = q.OC / q.groups;
  const int64_t M = (int64_t)OCg * q.KH * q.KW;
  if (q.KH != q.sH || q.KW != q.sW || q.pH != 0 || q.pW != 0) return -1;
  if (q.OH != q.sH * q.H || q.OW != q.sW * q.W) return -1;  // no output padding
  if ((q.H * q.W) % 128 != 0 || M % 4 != 0 || ICg < 1) return -1;
  if (((uintptr_t)q.x & 15) != 0 || ((uintptr_t)q.w & 15) != 0) return -1;
  if (((uintptr_t)q.out & 7) != 0) return -1;  // the 8-byte output stores
  if (q.groups > 65535) return -1;
  return M >= 128 ? TILE_128x128 : TILE_64x128;
}

template <class T>
hipError_t launch_fused(const ConvTProblem& q, hipStream_t s) {
  ConvTFusedArgs a;
  a.out = q.out;
  a.x = q.x;
  a.w = q.w;
  a.bias = q.bias;
  a.IC = q.IC;
  a.ICg = q.IC / q.groups;
  a.OC = q.OC;
  a.OCg = q.OC / q.groups;
  a.KH = q.KH;
  a.KW = q.KW;
  a.W = q.W;
  a.OH = q.OH;
  a.OW = q.OW;
  a.M = a.OCg * q.KH * q.KW;
  a.HW = q.H * q.W;
  a.tiles_m = (a.M + T::BM - 1) / T::BM;
  a.tiles_n = q.B * (a.HW / T::BN);
  a.div_khw = make_fastdiv((uint32_t)(q.KH * q.KW));
  a.div_kw = make_fastdiv((uint32_t)q.KW);
  a.div_w = make_fastdiv((uint32_t)q.W);
  const dim3 grid(a.tiles_m * a.tiles_n, 1, q.groups);
  hipLaunchKernelGGL((convt_fused_kernel<T>), grid, dim3(T::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_transpose2d(const ConvTProblem& q, hipStream_t stream) {
  const char* fspec = getenv("BAIM_CONVT_UNIT");
  const int fcfg = fspec && strcmp(fspec, "off") == 0 ? -1 : convt_fused_cfg(q);
  if (fcfg == TILE_128x128) return launch_fused<T128x128>(q, stream);
  if (fcfg == TILE_64x128) return launch_fused<T64x128>(q, stream);
  ConvTArgs a;
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
  a.OH = q.OH;
  a.OW = q.OW;
  a.ICg = q.IC / q.groups;
  a.OCg = q.OC / q.groups;
  a.x_elems = q.B * q.IC * q.H * q.W;
  a.w_elems = q.IC * a.OCg * q.KH * q.KW;

  // Phases with outputs, and the GEMM the tile choice is made for: all of
  // them side by side (they run in one launch).
  int64_t n_sum = 0;
  int k_max = 0;
  std::vector<ConvTPhase> all;
  static_assert(kTileBM[TILE_64x128] == 64 && kTileBN[TILE_64x128] == 128, "64x128 tile id");
  for (int rh = 0; rh < q.sH; ++rh)
    for (int rw = 0; rw < q.sW; ++rw) {
      ConvTPhase P{};
      P.rh = rh;
      P.rw = rw;
      P.Th = rh < q.OH ? (q.OH - rh + q.sH - 1) / q.sH : 0;
      P.Tw = rw < q.OW ? (q.OW - rw + q.sW - 1) / q.sW : 0;
      if (P.Th == 0 || P.Tw == 0) continue;
      const AxisTaps th = axis_taps(rh, q.sH, q.pH, q.dH, q.KH);
      const AxisTaps tw = axis_taps(rw, q.sW, q.pW, q.dW, q.KW);
      P.N = q.B * P.Th * P.Tw;
      P.K = a.ICg * th.n * tw.n;
      P.nw = tw.n;
      P.kh0 = th.k0;
      P.kw0 = tw.k0;
      P.step_h = th.step;
      P.step_w = tw.step;
      P.c0h = th.c0;
      P.c0w = tw.c0;
      P.dlh = th.dl;
      P.dlw = tw.dl;
      P.div_p = make_fastdiv((uint32_t)(P.Th * P.Tw));
      P.div_tw = make_fastdiv((uint32_t)P.Tw);
      P.div_taps = make_fastdiv((uint32_t)(th.n * tw.n > 0 ? th.n * tw.n : 1));
      P.div_nw = make_fastdiv((uint32_t)(tw.n > 0 ? tw.n : 1));
      n_sum += P.N;
      if (P.K > k_max) k_max = P.K;
      all.push_back(P);
    }
  const int nall = (int)all.size();
  // Single-tap phases over the input grid: the 16-byte B loads
  bool unit = (q.H * q.W) % 4 == 0 && ((uintptr_t)q.x & 15) == 0 && nall > 0;
  for (const ConvTPhase& P : all)
    unit = unit && P.K == a.ICg && P.c0h == 0 && P.c0w == 0 && P.Th == q.H && P.Tw == q.W;
  if (getenv("BAIM_CONVT_UNIT") && strcmp(getenv("BAIM_CONVT_UNIT"), "off") == 0) unit = false;
  // Tile choice for all phases side by side.  Both operands are 4-byte
  // gathers here, so the 8-wave 64x128 tile (a 64-row weight tile against
  // 128 output pixels) is preferred while it still gives half the CUs a
  // block: on the 4x4 and 2x2 stride-2 upsamplings it beat the GEMM
  // planner's choice by 1.3-1.5x.  Smaller problems keep the GEMM plan.
  const int n_all = (int)(n_sum < 0x7FFFFFFF ? n_sum : 0x7FFFFFFF);
  const char* spec = getenv("BAIM_TILE");
  const bool forced = spec && *spec;
  GemmPlan plan = plan_core_tile(plan_gemm(a.OCg, n_all, k_max, spec), a.OCg, n_all, k_max);
  // K slices only from a "cfg,S" override here; the automatic choice follows.
  int splits = forced && plan.mode == MODE_SLICES ? plan.splits : 1;
  const int64_t t64x128 = (int64_t)((a.OCg + 63) / 64) * ((n_all + 127) / 128);
  if (!forced && t64x128 >= kNumCUs / 2) plan = plan_gemm(a.OCg, n_all, k_max, "2");
  plan = plan_tiles_only(plan, a.OCg, n_all, k_max);
  // Tiles of all phases and groups, and the deepest phase's k-tiles.
  auto count = [&](int cfg, int64_t* tiles, int* nkt_max) {
    const int bm = kTileBM[cfg], bn = kTileBN[cfg], bk = kTileBK[cfg];
    *tiles = 0;
    *nkt_max = 0;
    for (const ConvTPhase& P : all) {
      *tiles += (int64_t)((a.OCg + bm - 1) / bm) * ((P.N + bn - 1) / bn);
      const int nkt = (P.K + bk - 1) / bk;
      if (nkt > *nkt_max) *nkt_max = nkt;
    }
    *tiles *= q.groups;
  };
  int64_t tiles;
  int nkt_max;
  count(plan.cfg, &tiles, &nkt_max);
  // Too few tiles to give half the CUs a block, and deep K: split K over
  // 2..8 slices towards two blocks per CU, on the 8-wave 64x128 tile when
  // there are more than 32 output channels per group (measured 3-5x faster
  // than whole tiles on 7x7 -> 14x14 and 4x4 -> 8x8 upsamplings with
  // K = 2048-4096).  The 200-tile 4x4 upsampling of 28x28 stays whole:
  // there two slices measured 6% slower.
  if (!forced && tiles < kNumCUs / 2 && nkt_max >= 16) {
    if (a.OCg > 32) {
      plan = plan_tiles_only(plan_gemm(a.OCg, n_all, k_max, "2"), a.OCg, n_all, k_max);
      count(plan.cfg, &tiles, &nkt_max);
    }
    const int64_t want = (2 * kNumCUs + tiles - 1) / tiles;
    splits = want < 2 ? 2 : (want > 8 ? 8 : (int)want);
  }
  const int BN = kTileBN[plan.cfg], BK = kTileBK[plan.cfg];
  a.tiles_m = (a.OCg + kTileBM[plan.cfg] - 1) / kTileBM[plan.cfg];
  a.splits = splits;
  if (splits > 1) {
    const uint32_t total = (uint32_t)((int64_t)q.B * q.OC * q.OH * q.OW);
    const uint32_t gb = (total + 255u) / 256u < 4096u ? (total + 255u) / 256u : 4096u;
    hipLaunchKernelGGL(convt_init_kernel, dim3(gb), dim3(256), 0, stream, q.out, q.bias, total,
                       make_fastdiv((uint32_t)(q.OH * q.OW)), (uint32_t)q.OC);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t err = hipSuccess;
  for (int first = 0; first < nall && err == hipSuccess; first += kMaxPhases) {
    const int nph = nall - first < kMaxPhases ? nall - first : kMaxPhases;
    int max_tiles_n = 0;
    for (int i = 0; i < nph; ++i) {
      ConvTPhase P = all[first + i];
      P.tiles_n = (P.N + BN - 1) / BN;
      P.nkt = (P.K + BK - 1) / BK;
      P.kps = (P.nkt + splits - 1) / splits;
      if (P.tiles_n > max_tiles_n) max_tiles_n = P.tiles_n;
      a.ph[i] = P;
    }
    a.slice_row = a.tiles_m * max_tiles_n;
    err = launch_cfg(plan.cfg, a, nph, q.groups, unit, stream);
  }
  return err;
}

}  // namespace baim
