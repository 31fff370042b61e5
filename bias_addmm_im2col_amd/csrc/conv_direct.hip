// conv_direct.hip -- grouped / depthwise NCHW conv whose per-group GEMM is
// too small for the matrix cores (fewer than 32 output channels or 32 taps
// per group, e.g. depthwise), computed directly, each output summing the
// IC/G input channels of its group over the (kh, kw) taps.  The conv page
// keeps grouped and depthwise convs on direct kernels ("et_vk conv2d: route
// standard (groups==1) conv through an im2col tiled GEMM", Solution
// paragraph); this is that path on gfx950.  Memory-bound; three kernels:
//  * conv_dw_rows_kernel -- one input channel per output channel, odd
//    K x K with same padding at stride 1, rows of 4k <= 256 floats: 2 x 4
//    output blocks per thread from registers, halo columns by lane
//    shuffles, no LDS (see the kernel);
//  * conv_direct_tiled_kernel -- otherwise: a block owns a 32-row x
//    64-column tile of one (image, output channel) plane; for each input
//    channel of the group it stages the input rows and columns the tile's
//    taps touch (with the halo, zero-filled outside the input) in LDS with
//    coalesced loads all in flight at once, then each thread sums its
//    outputs' taps from LDS; the weights are uniform across the block;
//  * conv_direct_kernel -- one thread per output reading the input
//    directly, for tiles whose input window would exceed 64 KB of LDS
//    (large strides or dilations).
// The fp32 sum runs in (ic, kh, kw) order with fused multiply-adds.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.hpp"
#include "index_math.hpp"
#include "launch.hpp"

namespace baim {

struct ConvDirectArgs {
  float* out;
  const float* x;
  const float* w;
  const float* bias;
  int IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW;
  int ICg, OCg;
  FastDiv div_ow;
};

constexpr int kTileW = 64, kTileH = 32;  // outputs per block tile (8 per thread)
constexpr int kMaxWindow = 16384;        // floats of LDS for the input window

__global__ __launch_bounds__(256) void conv_direct_tiled_kernel(ConvDirectArgs p, int tiles_w,
                                                                int win_h, int win_w) {
  extern __shared__ float win[];  // win_h x win_w floats
  const int oc = blockIdx.y, b = blockIdx.z;
  const int th = blockIdx.x / tiles_w, tw = blockIdx.x - th * tiles_w;
  const int oy0 = th * kTileH, ox0 = tw * kTileW;
  const int iy0 = oy0 * p.sH - p.pH, ix0 = ox0 * p.sW - p.pW;  // window origin
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;         // column, row group
  const int g = oc / p.OCg;
  const float* xg = p.x + ((size_t)b * p.IC + (size_t)g * p.ICg) * p.H * p.W;
  const float* wo = p.w + (size_t)oc * p.ICg * p.KH * p.KW;
  float acc[kTileH / 4] = {};
  for (int icl = 0; icl < p.ICg; ++icl) {
    const float* xc = xg + (size_t)icl * p.H * p.W;
    for (int wy = ty; wy < win_h; wy += 4) {
      const int iy = iy0 + wy;
      const bool yok = (unsigned)iy < (unsigned)p.H;
      for (int wx = tx; wx < win_w; wx += 64) {
        const int ix = ix0 + wx;
        win[wy * win_w + wx] = (yok && (unsigned)ix < (unsigned)p.W) ? xc[iy * p.W + ix] : 0.0f;
      }
    }
    __syncthreads();
    // tap-major: one weight load per tap feeds the thread's 8 outputs
    // (rows ty, ty+4, ..., ty+28 of the tile), independent FMAs
    const float* wc = wo + icl * p.KH * p.KW;
    const float* base = win + (ty * p.sH) * win_w + tx * p.sW;
    const int rstep = 4 * p.sH * win_w;
    for (int kh = 0; kh < p.KH; ++kh)
      for (int kw = 0; kw < p.KW; ++kw) {
        const float wv = wc[kh * p.KW + kw];
        const float* r = base + kh * p.dH * win_w + kw * p.dW;
#pragma unroll
        for (int i = 0; i < kTileH / 4; ++i) acc[i] = fmaf(wv, r[i * rstep], acc[i]);
      }
    __syncthreads();
  }
  const int P = p.OH * p.OW;
  const float bv = p.bias ? p.bias[oc] : 0.0f;
  float* o = p.out + ((size_t)b * p.OC + oc) * P;
  const int ox = ox0 + tx;
#pragma unroll
  for (int i = 0; i < kTileH / 4; ++i) {
    const int oy = oy0 + ty + 4 * i;
    if (ox < p.OW && oy < p.OH) o[oy * p.OW + ox] = acc[i] + bv;
  }
}

// Depthwise K x K, stride 1, "same" padding (K odd, pad (K-1)/2), width a
// multiple of 4 and at most 256: no LDS and no barriers.  A thread computes
// an OR x 4 output block.  The threads of an output row band sit in
// consecutive lanes, one per 4-column chunk, in groups of TWP lanes (the
// chunk count rounded up to a power of two, so a group never straddles a
// wave).  Each thread loads its chunk of the K+OR-1 input rows with one
// 16-byte load per row, and takes the (K-1)/2 columns on either side from
// its neighbours' chunks by lane shuffles; the lanes at the row ends (and
// the idle lanes past the last chunk) supply the zero padding.  So every
// input element is loaded about (K+OR-1)/OR times and never across lanes.
template <int K, int OR>
__global__ __launch_bounds__(256) void conv_dw_rows_kernel(ConvDirectArgs p, uint32_t nthreads,
                                                           int twp, FastDiv div_plane,
                                                           FastDiv div_twp) {
  constexpr int PADK = (K - 1) / 2;
  static_assert(K % 2 == 1 && PADK <= 4, "odd K up to 9");
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  // Threads past the end still take part in the shuffles (their lanes
  // carry zeros) and simply store nothing.
  const uint32_t g = gid < nthreads ? gid : nthreads - 1;
  const uint32_t plane = fdiv(g, div_plane);  // (b, oc)
  const uint32_t t = g - plane * div_plane.d;
  const uint32_t ty = fdiv(t, div_twp);
  const int tx = (int)(t - ty * div_twp.d);
  const int oh0 = OR * (int)ty, ow0 = 4 * tx;
  const bool live = gid < nthreads && ow0 < p.OW;
  const int oc = (int)(plane % (uint32_t)p.OC);
  const int b = (int)(plane / (uint32_t)p.OC);
  const int c = oc / p.OCg;  // the one input channel of this output channel
  const int H = p.H, W = p.W;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.x + ((size_t)b * p.IC + c) * H * W, (int64_t)H * W);
  float wk[K * K];
#pragma unroll
  for (int i = 0; i < K * K; ++i) wk[i] = p.w[(size_t)oc * K * K + i];
  float acc[OR][4] = {};
#pragma unroll
  for (int r = 0; r < K + OR - 1; ++r) {
    const int iy = oh0 - PADK + r;
    const bool ok = live && (unsigned)iy < (unsigned)H;
    const f32x4 q = Vec<4>::load(rs, ok ? (uint32_t)(iy * W + ow0) * 4u : kOOB);
    // row[i] is input column ow0 - PADK + i
    float row[4 + 2 * PADK];
#pragma unroll
    for (int e = 0; e < 4; ++e) row[PADK + e] = q[e];
#pragma unroll
    for (int e = 0; e < PADK; ++e) {
      const float left = __shfl_up(q[4 - PADK + e], 1, twp);
      const float right = __shfl_down(q[e], 1, twp);
      row[e] = tx > 0 ? left : 0.0f;
      row[4 + PADK + e] = tx < twp - 1 ? right : 0.0f;
    }
    // input row r feeds output rows oy = r - kh for kh = 0..K-1
#pragma unroll
    for (int kh = 0; kh < K; ++kh) {
      const int oy = r - kh;
      if (oy < 0 || oy >= OR) continue;
#pragma unroll
      for (int kw = 0; kw < K; ++kw)
#pragma unroll
        for (int ox = 0; ox < 4; ++ox)
          acc[oy][ox] = fmaf(wk[kh * K + kw], row[ox + kw], acc[oy][ox]);
    }
  }
  if (!live) return;
  const float bv = p.bias ? p.bias[oc] : 0.0f;
  float* o = p.out + (size_t)plane * p.OH * p.OW;
  // the output is written once and not read back here: non-temporal
  // stores (5.97 -> 5.42 us on [4,256,56,56]; four output rows per thread
  // instead of two measured 6.6)
#pragma unroll
  for (int oy = 0; oy < OR; ++oy)
    if (oh0 + oy < p.OH) {
      const f32x4 v = {acc[oy][0] + bv, acc[oy][1] + bv, acc[oy][2] + bv, acc[oy][3] + bv};
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o + (oh0 + oy) * p.OW + ow0));
    }
}

__global__ __launch_bounds__(256) void conv_direct_kernel(ConvDirectArgs p) {
  const int P = p.OH * p.OW;
  const int pix = blockIdx.x * 256 + threadIdx.x;
  const int oc = blockIdx.y, b = blockIdx.z;
  if (pix >= P) return;
  const int oh = (int)fdiv((uint32_t)pix, p.div_ow);
  const int ow = pix - oh * p.OW;
  const int g = oc / p.OCg;
  const int ih0 = oh * p.sH - p.pH, iw0 = ow * p.sW - p.pW;
  const float* xg = p.x + ((size_t)b * p.IC + (size_t)g * p.ICg) * p.H * p.W;
  const float* wo = p.w + (size_t)oc * p.ICg * p.KH * p.KW;
  float acc = 0.0f;
  for (int icl = 0; icl < p.ICg; ++icl) {
    const float* xc = xg + (size_t)icl * p.H * p.W;
    const float* wc = wo + icl * p.KH * p.KW;
    for (int kh = 0; kh < p.KH; ++kh) {
      const int ih = ih0 + kh * p.dH;
      if ((unsigned)ih >= (unsigned)p.H) continue;
      for (int kw = 0; kw < p.KW; ++kw) {
        const int iw = iw0 + kw * p.dW;
        if ((unsigned)iw >= (unsigned)p.W) continue;
        acc = fmaf(wc[kh * p.KW + kw], xc[ih * p.W + iw], acc);
      }
    }
  }
  p.out[((size_t)b * p.OC + oc) * P + pix] = acc + (p.bias ? p.bias[oc] : 0.0f);
}

hipError_t launch_conv2d_direct(const ConvProblem& q, hipStream_t stream) {
  ConvDirectArgs a;
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
  a.ICg = q.IC / q.groups;
  a.OCg = q.OC / q.groups;
  a.div_ow = make_fastdiv((uint32_t)q.OW);
  // one input channel per output channel, K x K odd with "same" padding,
  // stride and dilation 1, width a multiple of 4 up to 256, aligned tensors
  const int K = q.KH;
  if (a.ICg == 1 && q.KW == K && (K == 3 || K == 5 || K == 7) && q.pH == (K - 1) / 2 &&
      q.pW == (K - 1) / 2 && q.sH == 1 && q.sW == 1 && q.dH == 1 && q.dW == 1 && q.W % 4 == 0 &&
      q.W <= 256 && (((uintptr_t)q.x | (uintptr_t)q.out) & 15) == 0) {
    constexpr int OR = 2;  // output rows per thread
    int twp = 1;
    while (twp < q.OW / 4) twp *= 2;
    const uint32_t th = ((uint32_t)q.OH + OR - 1) / OR;
    const uint32_t n = (uint32_t)q.B * (uint32_t)q.OC * th * (uint32_t)twp;
    const dim3 grid((n + 255) / 256);
    const FastDiv dp = make_fastdiv(th * (uint32_t)twp), dt = make_fastdiv((uint32_t)twp);
    if (K == 3)
      hipLaunchKernelGGL((conv_dw_rows_kernel<3, OR>), grid, dim3(256), 0, stream, a, n, twp, dp, dt);
    else if (K == 5)
      hipLaunchKernelGGL((conv_dw_rows_kernel<5, OR>), grid, dim3(256), 0, stream, a, n, twp, dp, dt);
    else
      hipLaunchKernelGGL((conv_dw_rows_kernel<7, OR>), grid, dim3(256), 0, stream, a, n, twp, dp, dt);
    return hipGetLastError();
  }
  // input window of one output tile: rows / columns its taps touch
  const int64_t win_h = (int64_t)(kTileH - 1) * q.sH + (int64_t)(q.KH - 1) * q.dH + 1;
  const int64_t win_w = (int64_t)(kTileW - 1) * q.sW + (int64_t)(q.KW - 1) * q.dW + 1;
  if (win_h * win_w <= kMaxWindow) {
    const int tiles_w = (q.OW + kTileW - 1) / kTileW, tiles_h = (q.OH + kTileH - 1) / kTileH;
    hipLaunchKernelGGL(conv_direct_tiled_kernel, dim3(tiles_w * tiles_h, q.OC, q.B), dim3(256),
                       (size_t)(win_h * win_w) * sizeof(float), stream, a, tiles_w, (int)win_h,
                       (int)win_w);
    return hipGetLastError();
  }
  const int P = q.OH * q.OW;
  hipLaunchKernelGGL(conv_direct_kernel, dim3((P + 255) / 256, q.OC, q.B), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace baim
