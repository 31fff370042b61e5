// im2col_nhwc.hpp -- A-operand loader of the channels-last conv GEMM.
//
// With input x [B,H,W,IC], weight [OC,KH,KW,IC] and output [B,OH,OW,OC],
// the conv is the GEMM  out[m, oc] = sum_kk A[m, kk] * w[oc, kk] + bias[oc]
// with m = (b*OH + oh)*OW + ow, kk = (kh*KW + kw)*IC + ic and
// A[m, kk] = x[b, oh*sH - pH + kh*dH, ow*sW - pW + kw*dW, ic] (0 outside
// the input).  The weight is already the K-contiguous [N,K] B operand of
// linear, and the output is the row-major [M,N] tile of addmm, so only the
// A tile is new: the rows of the implicit im2col matrix, gathered straight
// into the [BM][BK+4] LDS tile.  "et_vk conv2d: route standard (groups==1)
// conv through an im2col tiled GEMM", Constraints paragraph: in NCHW the
// channel stride is not contiguous, so K cannot be read four at a time;
// here K runs along the input channels of one tap, so with IC % 4 == 0 a
// 16-byte load takes four consecutive k.
//
// Decode: a thread keeps the same k column of the tile for all its rows,
// so per k-tile it decodes one kk -> (kh, kw, ic) (two multiply-high
// divisions) and per row, once, m -> (b, oh, ow).  An element is read when
// 0 <= ih0 + kh*dH < H and 0 <= iw0 + kw*dW < W and kk < K; otherwise the
// load takes the out-of-range offset and returns 0 (padding, ragged K and
// rows past M, whose ih0 is a large negative sentinel).  Offsets are 32-bit
// modular sums, exact whenever the element is in range (the input has
// fewer than 2^29 elements).
#pragma once

#include "gemm_core.hpp"
#include "index_math.hpp"

namespace baim {

struct NhwcGeom {
  int H, W, IC, KW, OH, OW;
  int sH, sW, pH, pW, dH, dW;
  int x_elems;
  FastDiv div_ow, div_oh, div_ic, div_kw;
};

template <class T, int VEC>
struct NhwcRowLoader {
  static constexpr int CPR = T::BK / VEC;
  static constexpr int NCH = T::BM * CPR / T::NT;
  static_assert((T::BM * CPR) % T::NT == 0, "A tile must split evenly over threads");
  static_assert(T::NT % CPR == 0, "a thread keeps one k column");
  typedef typename Vec<VEC>::T V;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t rowbase[NCH];
  int ih0[NCH], iw0[NCH];
  int K, H, W, IC, KW, dH, dW;
  FastDiv div_ic, div_kw;
  V reg[2][NCH];

  __device__ void init(const float* x, const NhwcGeom& g, int m0, int M, int K_) {
    rs = make_rsrc(x, g.x_elems);
    K = K_;
    H = g.H;
    W = g.W;
    IC = g.IC;
    KW = g.KW;
    dH = g.dH;
    dW = g.dW;
    div_ic = g.div_ic;
    div_kw = g.div_kw;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int m = m0 + (int)(threadIdx.x + T::NT * i) / CPR;
      if (m < M) {
        const uint32_t t = fdiv((uint32_t)m, g.div_ow);
        const int ow = m - (int)t * g.OW;
        const uint32_t b = fdiv(t, g.div_oh);
        const int oh = (int)t - (int)b * g.OH;
        ih0[i] = oh * g.sH - g.pH;
        iw0[i] = ow * g.sW - g.pW;
        rowbase[i] = (((uint32_t)b * (uint32_t)g.H + (uint32_t)ih0[i]) * (uint32_t)g.W +
                      (uint32_t)iw0[i]) * (uint32_t)g.IC;
      } else {
        ih0[i] = -(1 << 30);  // fails every row test
        iw0[i] = 0;
        rowbase[i] = 0;
      }
    }
  }
  template <int S>
  __device__ void load(int k0) {
    const int kk = k0 + (int)(threadIdx.x % CPR) * VEC;
    const uint32_t tap = fdiv((uint32_t)kk, div_ic);
    const uint32_t kh = fdiv(tap, div_kw);
    const int ic = kk - (int)tap * IC, kw = (int)tap - (int)kh * KW;
    const int dh = (int)kh * dH, dw = kw * dW;
    const uint32_t tapoff = ((uint32_t)dh * (uint32_t)W + (uint32_t)dw) * (uint32_t)IC + (uint32_t)ic;
    const bool kok = kk < K;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const bool ok = kok && (unsigned)(ih0[i] + dh) < (unsigned)H &&
                      (unsigned)(iw0[i] + dw) < (unsigned)W;
      reg[S][i] = Vec<VEC>::load(rs, ok ? (rowbase[i] + tapoff) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* dst) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q / CPR, c = (q % CPR) * VEC;
      *reinterpret_cast<V*>(&dst[r * T::AS + c]) = reg[S][i];
    }
  }
  __device__ void meta(int) {}
};

}  // namespace baim
