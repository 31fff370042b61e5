// launch.hpp -- host-side interface between the C ABI (api.cpp) and the
// kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "conv_window_plan.hpp"

namespace baim {

struct AddmmProblem {
  float* out;
  const float* self;  // read only when self_mode != 0
  const float* mat1;
  const float* mat2;  // [K,N]; or, with weight_nk, a [N,K] weight (linear)
  bool weight_nk;
  int M, N, K;
  int self_mode;  // 0: beta == 0, self not read; 1: self [N]; 2: self [M,N]
  float beta, alpha;
};

struct ConvProblem {
  float* out;
  const float* x;
  const float* w;
  const float* bias;  // may be NULL
  int B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW;
  int groups;  // >= 1, dividing IC and OC; weight is [OC, IC/groups, KH, KW]
};

struct SdpaProblem {
  float* out;          // [BH, Sq, D]
  const float* q;      // [BH, Sq, D]
  const float* k;      // [BH, Skv, D]
  const float* v;      // [BH, Skv, D]
  const float* mask;   // [BH, Sq, Skv] additive, or NULL
  int BH, Sq, Skv, D;  // D % 4 == 0, D <= 128; Skv >= 1
  float scale;
};

struct ConvTProblem {
  float* out;         // [B, OC, OH, OW]
  const float* x;     // [B, IC, H, W]
  const float* w;     // [IC, OC/groups, KH, KW]
  const float* bias;  // may be NULL
  int B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW;
  int groups;
};

// Whether a grouped conv runs as one implicit-im2col GEMM per group (true)
// or on the direct kernel (per-group GEMMs too small for the matrix cores).
inline bool conv_uses_gemm(const ConvProblem& q) {
  const int icg = q.IC / q.groups, ocg = q.OC / q.groups;
  return q.groups == 1 || (ocg >= 32 && icg * q.KH * q.KW >= 32);
}

hipError_t launch_addmm(const AddmmProblem& p, hipStream_t stream);
// Output initialisation before split conv tiles land: the two-piece
// sentinel, or bias[oc] (0 without a bias) for atomic K slices.  out is
// [B, OC, P] with total = B*OC*P elements.
hipError_t launch_conv_out_init(float* out, const float* bias, bool sentinel, uint32_t total,
                                uint32_t P, uint32_t OC, hipStream_t stream);
// groups == 1 convs with a compiled small-kernel geometry (3x3 at stride 1,
// dilation 1 or 2) whose input rows fit the LDS window: the implicit GEMM
// with the B operand read from an LDS copy of the input rows.
inline WinShape win_shape(const ConvProblem& q) {
  return WinShape{q.B, q.IC, q.H, q.W, q.OC, q.KH, q.KW, q.sH, q.sW, q.pH, q.pW, q.dH, q.dW,
                  q.OH, q.OW, q.groups};
}
hipError_t launch_conv2d_window(const ConvProblem& p, const WinPlan& plan, hipStream_t stream);
// The 3-channel 7x7 stride-4 stem (plan_conv_stem): one pass over K per
// block of 128 output channels x 144 output pixels; NCHW, or channels-last
// (nhwc: x [B,H,W,IC], w [OC,KH,KW,IC], out [B,OH,OW,OC], out 16-byte
// aligned).
hipError_t launch_conv2d_stem(const ConvProblem& p, bool nhwc, hipStream_t stream);
hipError_t launch_conv2d(const ConvProblem& p, hipStream_t stream);
hipError_t launch_conv2d_direct(const ConvProblem& p, hipStream_t stream);
hipError_t launch_sdpa(const SdpaProblem& p, hipStream_t stream);
hipError_t launch_conv_transpose2d(const ConvTProblem& p, hipStream_t stream);
// Channels-last conv (groups == 1): x [B,H,W,IC], w [OC,KH,KW,IC],
// out [B,OH,OW,OC]; the stem kernel where plan_conv_stem takes the shape
// (input, weight and out 16-byte aligned), else the addmm kernels with an
// im2col A operand.
hipError_t launch_conv2d_nhwc(const ConvProblem& p, hipStream_t stream);

}  // namespace baim
