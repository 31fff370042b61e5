// conv_stem.hip -- the 3-channel patch-embed stem: groups==1 NCHW conv2d
// with a 7x7 kernel at stride 4 on an image of few channels ("et_vk conv2d:
// route standard (groups==1) conv through an im2col tiled GEMM", Problem
// paragraph: the direct kernel re-reads the input for every output, which
// the im2col GEMM fixes; Solution/Implementation: M = OC, N = B*OH*OW,
// K = IC*KH*KW, B[kk, n] = x[b, ic, oh*s - pH + kh, ow*s - pW + kw] or 0,
// bias per OC, NCHW output).
//
// K = 3*7*7 = 147 is too short for the k-tile pipeline of the GEMM kernels:
// a block there spends most of its time filling and draining.  Here one
// block computes 128 output channels x 144 consecutive output pixels of one
// image (the stem's 192 x 192 x 128 output is exactly 256 such tiles, one
// per CU) in a single pass over K:
//   1. issue the loads of the weights and of the input columns the tile
//      reads;
//   2. write them to LDS, one barrier, then all 37 MFMA steps from LDS;
//   3. add the bias and store NCHW.
// (Writing channel 0 first and running its steps while channels 1 and 2
// were still in flight, with a barrier per channel, measured 1% slower.)
// LDS layouts, chosen so that every MFMA operand is one LDS read:
//  * weights as they are in memory, [oc][ic][kh][kw] (147 floats a row, an
//    odd stride: the 16 rows a lane group reads fall in 16 banks), copied
//    with 16-byte stores;
//  * input "phase rows": for each (ic, kh), input column u - pW (u the
//    column in the padded image) is stored in phase row u % 4 at index
//    u / 4, so tap (ic, kh, kw) of 16 consecutive pixels is 16 consecutive
//    floats.  A run of 144 pixels covers at most two output rows (OW >=
//    144); each phase row holds both segments back to back, and rows are
//    16 (mod 32) floats long so that neighbouring taps' rows sit 16 banks
//    apart.  Input positions outside the image are zeros; one extra zero
//    row serves the padding tap.
// MFMA: v_mfma_f32_16x16x4_f32 (A 16x4, B 4x16, C 16x16; lane l supplies
// A[l%16][l/16] and B[l/16][l%16], and holds C[4*(l/16) + r][l%16] in
// register r).  Step s takes taps k = 4s .. 4s+3 (k = (ic*7 + kh)*7 + kw in
// memory order), lane group j = l/16 tap 4s + j: its weight is at a
// compile-time offset from its row, and the window offset of its tap comes
// from a 148-entry table in LDS.  K = 147 is 37 steps; the padding tap
// k = 147 reads the next weight row (or zeroed slack) against the zero
// row, adding exactly 0 for finite weights; an Inf or NaN in the input
// reaches only the outputs that read it.  Each of the 16 waves owns 16
// output channels and 5 or 4 of the 9 blocks of 16 pixels: four waves to a
// SIMD, independent accumulators.  The window sits first in LDS.
//
// Channels-last (x [B,H,W,IC], w [OC,KH,KW,IC], out [B,OH,OW,OC]) runs the
// same kernel with three changes: the input columns of a row arrive
// interleaved (IC floats per column), so each 16-byte load is split into
// its (column, channel) slots of the same phase rows; the weight rows hold
// the taps in (kh, kw, ic) order, which the tap table maps onto the window;
// and a lane's four consecutive output channels of one pixel go out as one
// 16-byte store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.hpp"
#include "launch.hpp"

namespace baim {

template <int IC_, int KH_, int KW_, int S_>
struct StemCfg {
  static constexpr int IC = IC_, KH = KH_, KW = KW_, S = S_;
  static constexpr int K = IC * KH * KW;         // taps, weight floats per oc
  static constexpr int KSTEPS = (K + 3) / 4;     // MFMA steps of 4 taps
  static constexpr int BM = 128, BN = 144, NPB = BN / 16;
  // 16 waves: wave w owns output channels 16*(w % 8) .. +15 and pixel
  // blocks [0, PBH) (w < 8) or [PBH, NPB) (w >= 8)
  static constexpr int PBH = (NPB + 1) / 2;
  static constexpr int WAVES = 2 * (BM / 16), NT = 64 * WAVES;
  static constexpr int E = (KW - 1) / S;  // extra phase slots per segment
  // phase-row length: two segments of n1 + E and n2 + E slots, rounded to
  // 16 (mod 32) floats so that neighbouring taps' rows sit 16 banks apart
  static constexpr int Q = ((BN + 2 * E + 16) / 32) * 32 + 16;
  static constexpr int AS = K;  // weight rows as in memory (odd)
  // slack past the last row: the padding tap k = K of the last row
  static constexpr int A_FLOATS = BM * AS + 16;
  // window: [ic][kh][phase][Q], then one zero row for the padding tap
  static constexpr int X_ROWS = IC * KH * S;
  static constexpr int X_FLOATS = (X_ROWS + 1) * Q;
  static constexpr int T_INTS = 4 * KSTEPS;  // per-tap window offsets
  static constexpr int SMEM_FLOATS = X_FLOATS + A_FLOATS + T_INTS;
  static constexpr int W_ITEMS = (BM * K + 3) / 4;  // float4s of the block's weights
  static constexpr int W_NQ = (W_ITEMS + NT - 1) / NT;
  // input float4s per (ic, kh, segment): the segment's columns span
  // S*(n-1) + KW floats, at most S*BN + KW - S, plus one for alignment
  static constexpr int X_F4 = (S * BN + KW - S + 3) / 4 + 1;
  static constexpr int X_NQI = (KH * 2 * X_F4 + NT - 1) / NT;  // per thread and channel
  static_assert(Q >= BN + 2 * E && Q % 32 == 16 && (S * Q) % 4 == 0, "stem layout");
  static_assert(AS % 2 == 1 && (BM * AS) % 4 == 0 && (X_FLOATS + A_FLOATS) % 4 == 0,
                "odd weight rows, 16-byte copies");
  static_assert(T_INTS - K <= 16, "padding taps stay in the slack");
  static_assert(SMEM_FLOATS * 4 <= 160 * 1024, "LDS budget");
};

// Window offset of tap k = (ic*KH + kh)*KW + kw: phase row (ic, kh, kw % S)
// at index kw / S; the padding taps (k >= K) read the zero row.
template <class C>
__host__ __device__ constexpr int stem_tap_off(int k) {
  return k >= C::K ? C::X_ROWS * C::Q
                   : (((k / C::KW) * C::S + (k % C::KW) % C::S) * C::Q + (k % C::KW) / C::S);
}

// The same for a channels-last weight row, tap k = (kh*KW + kw)*IC + ic.
template <class C>
__host__ __device__ constexpr int stem_tap_off_nhwc(int k) {
  return k >= C::K ? C::X_ROWS * C::Q
                   : stem_tap_off<C>(((k % C::IC) * C::KH + (k / C::IC) / C::KW) * C::KW +
                                     (k / C::IC) % C::KW);
}

struct StemArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int H, W, OC, pH, pW, OH, OW, P, tpi;
  int x_elems, w_elems;
};

// One tile's input columns for one channel: item i covers float4 f of
// the column span of (kh, segment g), row = kh*2 + g.  Items outside the
// image (rows or columns) load zeros, which fill their window slots.
template <class C>
struct StemXItems {
  f32x4 v[C::X_NQI];
  int row[C::X_NQI];  // kh*2 + g, or -1 (no item)
  int col[C::X_NQI];  // first input column of the float4

  __device__ void load(const StemArgs& p, __amdgpu_buffer_rsrc_t xr, int b, int ic, int oh1,
                       int n1, int n2, int f0_1, int f0_2, int colA1, int colA2) {
#pragma unroll
    for (int q = 0; q < C::X_NQI; ++q) {
      const int i = threadIdx.x + C::NT * q;
      const int r = i / C::X_F4, f = i - r * C::X_F4;
      const int g = r & 1, kh = r >> 1;
      const int n = g ? n2 : n1;
      const int ih = (oh1 + g) * C::S - p.pH + kh;
      const int c = ((g ? f0_2 : f0_1) + f) * 4;
      const int colA = g ? colA2 : colA1;
      const int colB = colA + C::S * (n - 1) + C::KW;  // one past the last column
      const bool cover = kh < C::KH && n > 0 && c < colB && c + 4 > colA;
      const bool ok = cover && ih >= 0 && ih < p.H && c >= 0 && c < p.W;
      row[q] = cover ? r : -1;
      col[q] = c;
      // a float4 lies wholly inside the row (W % 4 == 0, aligned columns)
      const int off = ((b * C::IC + ic) * p.H + ih) * p.W + c;
      v[q] = Vec<4>::load(xr, ok ? (uint32_t)off * 4u : kOOB);
    }
  }
  __device__ void store(float* Xs, int ic, int pW, int ow1, int n1, int n2, int seg2) const {
#pragma unroll
    for (int q = 0; q < C::X_NQI; ++q) {
      if (row[q] < 0) continue;
      const int g = row[q] & 1, kh = row[q] >> 1;
      const int n = g ? n2 : n1;
      const int owA = g ? 0 : ow1;
      const int base = ((ic * C::KH + kh) * C::S) * C::Q + (g ? seg2 : 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = col[q] + e + pW;  // column in the padded image
        const int rel = u - C::S * owA;  // within the segment's span
        if (rel < 0 || rel >= C::S * (n - 1) + C::KW) continue;
        Xs[base + (u % C::S) * C::Q + rel / C::S] = v[q][e];
      }
    }
  }
};

// Channels-last input: item i covers float4 f of the interleaved span of
// (kh, segment g), whose floats iw*IC + ic run over the segment's columns
// [colA, colB) and every channel; row = kh*2 + g.  Rows W*IC floats long
// (W % 4 == 0) start on 16-byte boundaries, so a float4 lies wholly inside
// or wholly outside the row; outside ones load zeros.
template <class C>
struct StemXItemsNhwc {
  static constexpr int F4 = (C::IC * (C::S * C::BN + C::KW - C::S) + 3) / 4 + 1;
  static constexpr int NQ = (C::KH * 2 * F4 + C::NT - 1) / C::NT;
  f32x4 v[NQ];
  int row[NQ];  // kh*2 + g, or -1 (no item)
  int fl[NQ];   // first float of the float4 within its input row

  __device__ void load(const StemArgs& p, __amdgpu_buffer_rsrc_t xr, int b, int oh1, int n1,
                       int n2, int colA1, int colA2) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = threadIdx.x + C::NT * q;
      const int r = i / F4, f = i - r * F4;
      const int g = r & 1, kh = r >> 1;
      const int n = g ? n2 : n1;
      const int ih = (oh1 + g) * C::S - p.pH + kh;
      const int colA = g ? colA2 : colA1;
      const int fA = colA * C::IC, fB = (colA + C::S * (n - 1) + C::KW) * C::IC;
      const int f0 = fA >= 0 ? fA >> 2 : -((-fA + 3) >> 2);
      const int c = (f0 + f) * 4;
      const bool cover = kh < C::KH && n > 0 && c < fB && c + 4 > fA;
      const bool ok = cover && ih >= 0 && ih < p.H && c >= 0 && c < p.W * C::IC;
      row[q] = cover ? r : -1;
      fl[q] = c;
      const int off = ((b * p.H + ih) * p.W) * C::IC + c;
      v[q] = Vec<4>::load(xr, ok ? (uint32_t)off * 4u : kOOB);
    }
  }
  __device__ void store(float* Xs, int pW, int ow1, int n1, int n2, int seg2) const {
    // a multiple of IC that makes every float index of the span >= 0
    const int shift = C::IC * (pW + 4);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (row[q] < 0) continue;
      const int g = row[q] & 1, kh = row[q] >> 1;
      const int n = g ? n2 : n1;
      const int owA = g ? 0 : ow1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int fs = fl[q] + e + shift;
        const int ic = fs % C::IC;
        const int u = fs / C::IC - 4;    // column in the padded image
        const int rel = u - C::S * owA;  // within the segment's span
        if (rel < 0 || rel >= C::S * (n - 1) + C::KW) continue;
        Xs[((ic * C::KH + kh) * C::S + u % C::S) * C::Q + (g ? seg2 : 0) + rel / C::S] = v[q][e];
      }
    }
  }
};

// Steps [S0, S1) for the wave's NB pixel blocks: lane group j takes tap
// k = 4s + j, whose window offset it reads from the tap table.
template <class C, int S0, int S1, int NB>
__device__ __forceinline__ void stem_mma(f32x4* acc, const float* Aw, const int* Tj,
                                         const float* Xs, const int* boff) {
#pragma unroll
  for (int s = S0; s < S1; ++s) {
    const float av = Aw[4 * s];
    const int t = Tj[4 * s];
    float bv[NB];
#pragma unroll
    for (int pb = 0; pb < NB; ++pb) bv[pb] = Xs[boff[pb] + t];
#pragma unroll
    for (int pb = 0; pb < NB; ++pb)
      acc[pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[pb], acc[pb], 0, 0, 0);
  }
}

template <class C, bool NHWC>
__global__ __launch_bounds__(C::NT) void conv_stem_kernel(StemArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[C::SMEM_FLOATS];
  float* Xs = smem;
  float* As = smem + C::X_FLOATS;
  int* Ts = reinterpret_cast<int*>(smem + C::X_FLOATS + C::A_FLOATS);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // consecutive tiles (which share input rows) on the same XCD's L2
  const int tm = blockIdx.y, tn = xcd_linear(blockIdx.x, gridDim.x);
  const int m0 = tm * C::BM;
  const int b = tn / p.tpi, p0 = (tn - b * p.tpi) * C::BN;
  // the tile's pixels: segment 1 on output row oh1 from ow1, segment 2 on
  // the next row from column 0
  const int oh1 = p0 / p.OW, ow1 = p0 - oh1 * p.OW;
  const int left = p.P - p0;
  const int n1 = min(min(C::BN, p.OW - ow1), left);
  const int n2 = min(C::BN - n1, left - n1);
  const int seg2 = n1 + C::E;  // phase-row index where segment 2 starts

  // 1. loads in flight: the block's weight rows (flat, 16-byte aligned),
  // then the input columns
  const int wrows = min(C::BM, p.OC - m0);
  const int wcount = wrows * C::K;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (size_t)m0 * C::K, wcount);
  f32x4 wv[C::W_NQ];
#pragma unroll
  for (int q = 0; q < C::W_NQ; ++q) {
    const int i = tid + C::NT * q;
    wv[q] = Vec<4>::load(wr, i * 4 < wcount ? (uint32_t)i * 16u : kOOB);
  }
  const int colA1 = C::S * ow1 - p.pW, colA2 = -p.pW;  // first input column of each segment
  const int f0_1 = colA1 >= 0 ? colA1 >> 2 : -((-colA1 + 3) >> 2);
  const int f0_2 = colA2 >= 0 ? colA2 >> 2 : -((-colA2 + 3) >> 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, p.x_elems);
  StemXItems<C> xi[NHWC ? 1 : C::IC];
  StemXItemsNhwc<C> xn;
  if constexpr (NHWC) {
    xn.load(p, xr, b, oh1, n1, n2, colA1, colA2);
  } else {
#pragma unroll
    for (int ic = 0; ic < C::IC; ++ic)
      xi[ic].load(p, xr, b, ic, oh1, n1, n2, f0_1, f0_2, colA1, colA2);
  }

  // 2. what no load writes: the zero row, the weight rows past OC with the
  // slack after the last row, and the tap table
  {
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = tid; i < C::Q / 4; i += C::NT)
      reinterpret_cast<f32x4*>(Xs + C::X_ROWS * C::Q)[i] = z;
    const int za = ((C::BM - wrows) * C::AS + 16) / 4;
    for (int i = tid; i < za; i += C::NT) reinterpret_cast<f32x4*>(As + wrows * C::AS)[i] = z;
    if (tid < C::T_INTS) Ts[tid] = NHWC ? stem_tap_off_nhwc<C>(tid) : stem_tap_off<C>(tid);
  }
  // 3. weights and input into LDS
#pragma unroll
  for (int q = 0; q < C::W_NQ; ++q) {
    const int i = tid + C::NT * q;
    if (i * 4 < wcount) reinterpret_cast<f32x4*>(As)[i] = wv[q];
  }
  if constexpr (NHWC) {
    xn.store(Xs, p.pW, ow1, n1, n2, seg2);
  } else {
#pragma unroll
    for (int ic = 0; ic < C::IC; ++ic) xi[ic].store(Xs, ic, p.pW, ow1, n1, n2, seg2);
  }
  __syncthreads();

  // 4. all of K: wave w computes pixel blocks [0, PBH) (w < 8) or [PBH, NPB)
  const int m = lane & 15, j = lane >> 4;
  const int ocb = wave % (C::BM / 16), half = wave / (C::BM / 16);
  const int pb0 = half ? C::PBH : 0, nb = half ? C::NPB - C::PBH : C::PBH;
  const float* Aw = As + (ocb * 16 + m) * C::AS + j;  // tap k = 4s + j at Aw[4s]
  const int* Tj = Ts + j;
  int boff[C::PBH];
#pragma unroll
  for (int pb = 0; pb < C::PBH; ++pb) {
    const int t = 16 * (pb0 + pb) + m;  // pixel within the tile
    boff[pb] = t < n1 ? t : (t < n1 + n2 ? seg2 + (t - n1) : 0);
  }
  f32x4 acc[C::PBH];
#pragma unroll
  for (int pb = 0; pb < C::PBH; ++pb) acc[pb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (half == 0)
    stem_mma<C, 0, C::KSTEPS, C::PBH>(acc, Aw, Tj, Xs, boff);
  else
    stem_mma<C, 0, C::KSTEPS, C::NPB - C::PBH>(acc, Aw, Tj, Xs, boff);

  // 5. + bias, store: lane (pixel m, group j) holds output channels
  // 4j .. 4j+3 of the wave's 16
  const int npix = n1 + n2;
  if constexpr (NHWC) {
    // [B, OH, OW, OC]: the four channels of one pixel are one 16-byte
    // store (OC % 4 == 0: they are all inside or all past OC), marked
    // non-temporal like the NCHW stores (21.5 -> 20.2 us on the 768 x 768
    // stem; staging the tile through LDS for whole-pixel runs of lanes
    // measured 22.7)
    const int oc0 = m0 + ocb * 16 + 4 * j;
    if (oc0 >= p.OC) return;
    f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.bias) {
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = p.bias[oc0 + r];
    }
    float* obn = p.out + ((size_t)b * p.P + p0) * p.OC + oc0;
#pragma unroll
    for (int pb = 0; pb < C::PBH; ++pb) {
      const int t = 16 * (pb0 + pb) + m;
      if (pb < nb && (npix == C::BN || t < npix))
        __builtin_nontemporal_store(acc[pb] + bv, reinterpret_cast<f32x4*>(obn + (size_t)t * p.OC));
    }
    return;
  }
  float* ob = p.out + (size_t)b * p.OC * p.P + p0;
  if (m0 + C::BM <= p.OC && npix == C::BN) {
    // A whole tile: the four bias values first, then stores without the
    // per-element channel and pixel tests (22.9 -> 21.3 us on the
    // 768 x 768 stem, whose 256 tiles are all whole), marked non-temporal:
    // the output is written once, all tiles at the end (19.9 -> 19.0 us).
    float bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) bv[r] = p.bias ? p.bias[m0 + ocb * 16 + 4 * j + r] : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* orow = ob + (size_t)(m0 + ocb * 16 + 4 * j + r) * p.P + 16 * pb0 + m;
#pragma unroll
      for (int pb = 0; pb < C::PBH; ++pb)
        if (pb < nb) __builtin_nontemporal_store(acc[pb][r] + bv[r], &orow[16 * pb]);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int oc = m0 + ocb * 16 + 4 * j + r;
    if (oc >= p.OC) continue;
    const float bv = p.bias ? p.bias[oc] : 0.0f;
#pragma unroll
    for (int pb = 0; pb < C::PBH; ++pb) {
      const int t = 16 * (pb0 + pb) + m;
      if (pb < nb && t < npix) ob[(size_t)oc * p.P + t] = acc[pb][r] + bv;
    }
  }
}

typedef StemCfg<3, 7, 7, 4> Stem3x7x7S4;

hipError_t launch_conv2d_stem(const ConvProblem& q, bool nhwc, hipStream_t stream) {
  typedef Stem3x7x7S4 C;
  static_assert(C::IC == kStemIC && C::KH == kStemK && C::KW == kStemK && C::S == kStemS &&
                    C::BM == kStemBM && C::BN == kStemBN && C::NT == 64 * kStemWaves,
                "stem table out of sync with the compiled kernel");
  StemArgs a;
  a.out = q.out;
  a.x = q.x;
  a.w = q.w;
  a.bias = q.bias;
  a.H = q.H;
  a.W = q.W;
  a.OC = q.OC;
  a.pH = q.pH;
  a.pW = q.pW;
  a.OH = q.OH;
  a.OW = q.OW;
  a.P = q.OH * q.OW;
  a.tpi = (a.P + C::BN - 1) / C::BN;
  a.x_elems = q.B * q.IC * q.H * q.W;
  a.w_elems = q.OC * C::K;
  const dim3 grid(q.B * a.tpi, (q.OC + C::BM - 1) / C::BM);
  if (nhwc)
    hipLaunchKernelGGL((conv_stem_kernel<C, true>), grid, dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((conv_stem_kernel<C, false>), grid, dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace baim
