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
#include "gemm_core.hpp"
#include "launch.hpp"

namespace baim {

struct ConvArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW;
  int M, N, K;
  int x_elems;  // B*IC*H*W
  FastDiv div_khw, div_kw, div_p, div_ow;
  int tiles_m, tiles_n, group_m;
};

template <class T>
struct ImColTileLoader {
  static constexpr int RPP = T::NT / T::BN;  // tile rows covered per pass
  static constexpr int NP = T::BK / RPP;     // passes per k-tile
  static_assert(T::NT % T::BN == 0 && T::BK % RPP == 0, "im2col tile split");
  static_assert(T::BN % 64 == 0, "a wave must cover columns of a single row");
  int row0, col, cbase, ih0, iw0;
  bool cok;
  float reg[NP];

  __device__ void init(const ConvArgs& a, int n0) {
    col = threadIdx.x % T::BN;
    row0 = __builtin_amdgcn_readfirstlane(threadIdx.x / T::BN);
    const int n = n0 + col;
    cok = n < a.N;
    const uint32_t nn = cok ? (uint32_t)n : 0u;
    const uint32_t b = fdiv(nn, a.div_p);
    const uint32_t pix = nn - b * a.div_p.d;
    const uint32_t oh = fdiv(pix, a.div_ow);
    const uint32_t ow = pix - oh * a.div_ow.d;
    ih0 = (int)oh * a.sH - a.pH;
    iw0 = (int)ow * a.sW - a.pW;
    cbase = (int)b * a.IC * a.H * a.W + ih0 * a.W + iw0;
  }
  __device__ void load(const ConvArgs& a, int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.x, a.x_elems);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int kk = k0 + row0 + RPP * i;
      const uint32_t ic = fdiv((uint32_t)kk, a.div_khw);
      const uint32_t rem = (uint32_t)kk - ic * a.div_khw.d;
      const uint32_t kh = fdiv(rem, a.div_kw);
      const uint32_t kw = rem - kh * a.div_kw.d;
      const int dh = (int)kh * a.dH, dw = (int)kw * a.dW;
      const int off = (int)ic * a.H * a.W + dh * a.W + dw;
      const bool ok = cok && kk < a.K && (unsigned)(ih0 + dh) < (unsigned)a.H &&
                      (unsigned)(iw0 + dw) < (unsigned)a.W;
      reg[i] = Vec<1>::load(rs, ok ? (uint32_t)(cbase + off) * 4u : kOOB);
    }
  }
  __device__ void store(float* Bs) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) Bs[(row0 + RPP * i) * T::BS + col] = reg[i];
  }
};

// Adapts the im2col loader to the (load(k0), store(buf)) shape of mainloop.
template <class T>
struct ImColBound {
  ImColTileLoader<T> ld;
  const ConvArgs* a;
  __device__ void load(int k0) { ld.load(*a, k0); }
  __device__ void store(float* Bs) const { ld.store(Bs); }
};

template <class T, int VA>
__global__ __launch_bounds__(T::NT) void conv2d_gemm_kernel(ConvArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave / T::WN) * T::WTM, wn0 = (wave % T::WN) * T::WTN;

  RowTileLoader<T, VA> al;
  al.init(p.w, m0, p.M, p.K);
  ImColBound<T> bl;
  bl.a = &p;
  bl.ld.init(p, n0);
  Accum<T> acc;
  mainloop<T>(acc, al, bl, p.K, smem, wm0, wn0, lane);

  // Epilogue: + bias[oc], NCHW store: column n = (b, pix) goes to
  // out[b, oc, pix] = out[(b*OC + oc)*P + pix], P = OH*OW.
  const int c = lane & 31;
  const uint32_t P = p.div_p.d;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n0 + wn0 + 32 * j + c;
    if (n >= p.N) continue;
    const uint32_t b = fdiv((uint32_t)n, p.div_p);
    const size_t obase = (size_t)b * p.OC * P + ((uint32_t)n - b * P);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int oc = m0 + wm0 + 32 * i + acc_row(r, lane);
        if (oc >= p.M) continue;
        const float bv = p.bias ? p.bias[oc] : 0.0f;
        p.out[obase + (size_t)oc * P] = acc.c[i][j][r] + bv;
      }
  }
}

typedef Tile<128, 128, 32, 2, 2> ConvTile;

template <class T, int VA>
static hipError_t launch_t(const ConvArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((conv2d_gemm_kernel<T, VA>), dim3(nblocks), dim3(T::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_conv2d(const ConvProblem& q, hipStream_t stream) {
  typedef ConvTile T;
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
  a.M = q.OC;
  a.N = q.B * q.OH * q.OW;
  a.K = q.IC * q.KH * q.KW;
  a.x_elems = q.B * q.IC * q.H * q.W;
  a.div_khw = make_fastdiv((uint32_t)(q.KH * q.KW));
  a.div_kw = make_fastdiv((uint32_t)q.KW);
  a.div_p = make_fastdiv((uint32_t)(q.OH * q.OW));
  a.div_ow = make_fastdiv((uint32_t)q.OW);
  a.tiles_m = (a.M + T::BM - 1) / T::BM;
  a.tiles_n = (a.N + T::BN - 1) / T::BN;
  a.group_m = 8;
  const int nblocks = a.tiles_m * a.tiles_n;
  const bool va = a.K % 4 == 0 && ((uintptr_t)q.w & 15) == 0;
  if (va) return launch_t<T, 4>(a, nblocks, stream);
  return launch_t<T, 1>(a, nblocks, stream);
}

}  // namespace baim
