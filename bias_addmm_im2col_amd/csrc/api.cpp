// api.cpp -- the C ABI of libbaim.so (declared in include/baim.h).
//
// Every check runs on the host before anything is enqueued, so an invalid
// call launches nothing and leaves `out` untouched (the conv page computes
// both dispatch grids before any buffer is allocated so that a throw cannot
// leak; here nothing is allocated at all).  Validation makes no HIP call,
// which keeps it testable on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>

#include "baim.h"
#include "launch.hpp"
#include "tile_select.hpp"

namespace {

thread_local std::string g_err;

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // exclusive
// Byte offsets inside one tile of the operands are 32-bit: a block's A tile
// spans at most 128 rows of K floats, and the conv gather addresses the
// whole input.  A B tile of mat2 [K, N] spans BK rows of N floats: 64 rows
// fit any N below 2^23, and the launcher moves a plan whose tile has 128
// rows to a 64-row tile when (127 * N + BN) floats would pass 2^31 bytes.
constexpr int64_t kMaxK = (int64_t)1 << 21;
constexpr int64_t kMaxAddmmN = (int64_t)1 << 23;
constexpr int64_t kMaxConvInput = (int64_t)1 << 29;
// Attention addresses one (batch, head) slice of each tensor with 32-bit
// byte offsets.
constexpr int64_t kMaxSlice = (int64_t)1 << 29;

baim_status fail(baim_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

// Number of elements of a product of sizes, or -1 on overflow.
int64_t elems(std::initializer_list<int64_t> dims) {
  int64_t n = 1;
  for (int64_t d : dims)
    if (!mul_ok(n, d, &n)) return -1;
  return n;
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  const uintptr_t a1 = a0 + (uintptr_t)na * 4u, b1 = b0 + (uintptr_t)nb * 4u;
  return a0 < b1 && b0 < a1;
}

baim_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BAIM_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return BAIM_OK;
}

}  // namespace

extern "C" {

int baim_version(void) { return 100; }

const char* baim_last_error(void) { return g_err.c_str(); }

baim_status baim_gemm_plan(int64_t M, int64_t N, int64_t K, int* bm, int* bn, int* bk,
                           int* waves, int* kgroups, int* splits, int* stream_blocks) {
  g_err.clear();
  if (!bm || !bn || !bk || !waves || !kgroups || !splits || !stream_blocks)
    return fail(BAIM_ERR_NULL, "baim_gemm_plan: output pointers must not be NULL");
  if (M < 0 || N < 0 || K < 0) return fail(BAIM_ERR_SHAPE, "baim_gemm_plan: sizes must be >= 0");
  if (M >= kMaxElems || N >= kMaxElems || K >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "baim_gemm_plan: size too large");
  baim::GemmPlan p = baim::plan_gemm((int)M, (int)N, (int)K, getenv("BAIM_TILE"));
  // as addmm_f32 launches it
  if (!baim::plan_big_fits((int)N, (int)K)) p = baim::plan_core_tile(p, (int)M, (int)N, (int)K);
  *bm = baim::kTileBM[p.cfg];
  *bn = baim::kTileBN[p.cfg];
  *bk = baim::kTileBK[p.cfg];
  *waves = baim::kTileWaves[p.cfg];
  *kgroups = baim::kTileKGroups[p.cfg];
  *splits = p.mode == baim::MODE_SLICES ? p.splits : 1;
  *stream_blocks = p.mode == baim::MODE_STREAM ? p.workers : 0;
  return BAIM_OK;
}

baim_status baim_conv2d_out_hw(int64_t H, int64_t W, int64_t KH, int64_t KW, int64_t sH,
                               int64_t sW, int64_t pH, int64_t pW, int64_t dH, int64_t dW,
                               int64_t* OH, int64_t* OW) {
  g_err.clear();
  if (!OH || !OW) return fail(BAIM_ERR_NULL, "baim_conv2d_out_hw: OH/OW must not be NULL");
  *OH = *OW = 0;
  if (H < 1 || W < 1 || KH < 1 || KW < 1)
    return fail(BAIM_ERR_SHAPE, "conv2d: input and kernel sizes must be >= 1");
  if (sH < 1 || sW < 1) return fail(BAIM_ERR_SHAPE, "conv2d: stride must be >= 1");
  if (dH < 1 || dW < 1) return fail(BAIM_ERR_SHAPE, "conv2d: dilation must be >= 1");
  if (pH < 0 || pW < 0) return fail(BAIM_ERR_SHAPE, "conv2d: padding must be >= 0");
  if (H > kMaxElems || W > kMaxElems || KH > kMaxElems || KW > kMaxElems || pH > kMaxElems ||
      pW > kMaxElems || dH > kMaxElems || dW > kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "conv2d: size argument too large");
  const int64_t spanH = H + 2 * pH - dH * (KH - 1) - 1;
  const int64_t spanW = W + 2 * pW - dW * (KW - 1) - 1;
  if (spanH < 0 || spanW < 0)
    return fail(BAIM_ERR_SHAPE, "conv2d: dilated kernel (%lld x %lld) larger than padded input",
                (long long)(dH * (KH - 1) + 1), (long long)(dW * (KW - 1) + 1));
  *OH = spanH / sH + 1;
  *OW = spanW / sW + 1;
  return BAIM_OK;
}

baim_status addmm_f32(float* out, const float* self, int self_2d, const float* mat1,
                      const float* mat2, int64_t M, int64_t N, int64_t K, float beta, float alpha,
                      void* stream) {
  g_err.clear();
  if (M < 0 || N < 0 || K < 0)
    return fail(BAIM_ERR_SHAPE, "addmm: sizes must be >= 0 (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (self_2d != 0 && self_2d != 1)
    return fail(BAIM_ERR_SHAPE, "addmm: self_2d must be 0 (self [N]) or 1 (self [M,N])");
  const int64_t n_out = elems({M, N}), n_a = elems({M, K}), n_b = elems({K, N});
  if (n_out < 0 || n_a < 0 || n_b < 0 || n_out >= kMaxElems || n_a >= kMaxElems ||
      n_b >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "addmm: every tensor must have fewer than 2^31 elements");
  if (K >= kMaxK) return fail(BAIM_ERR_TOO_LARGE, "addmm: K must be below 2^21");
  if (N >= kMaxAddmmN) return fail(BAIM_ERR_TOO_LARGE, "addmm: N must be below 2^23");
  if (M == 0 || N == 0) return BAIM_OK;  // empty output: nothing to do
  const bool reads_self = beta != 0.0f;
  if (!out) return fail(BAIM_ERR_NULL, "addmm: out is NULL");
  if (reads_self && !self) return fail(BAIM_ERR_NULL, "addmm: self is NULL but beta != 0");
  if (K > 0 && (!mat1 || !mat2)) return fail(BAIM_ERR_NULL, "addmm: mat1/mat2 is NULL");
  const int64_t n_self = self_2d ? n_out : N;
  if ((K > 0 && (overlap(out, n_out, mat1, n_a) || overlap(out, n_out, mat2, n_b))) ||
      (reads_self && overlap(out, n_out, self, n_self)))
    return fail(BAIM_ERR_ALIAS, "addmm: out overlaps an input");

  baim::AddmmProblem p;
  p.out = out;
  p.self = reads_self ? self : nullptr;
  p.mat1 = mat1;
  p.mat2 = mat2;
  p.weight_nk = false;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.self_mode = reads_self ? (self_2d ? 2 : 1) : 0;
  p.beta = beta;
  p.alpha = alpha;
  return launched(baim::launch_addmm(p, (hipStream_t)stream), "addmm_f32");
}

baim_status linear_f32(float* out, const float* x, const float* weight, const float* bias,
                       int64_t M, int64_t N, int64_t K, void* stream) {
  g_err.clear();
  if (M < 0 || N < 0 || K < 0)
    return fail(BAIM_ERR_SHAPE, "linear: sizes must be >= 0 (M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  const int64_t n_out = elems({M, N}), n_x = elems({M, K}), n_w = elems({N, K});
  if (n_out < 0 || n_x < 0 || n_w < 0 || n_out >= kMaxElems || n_x >= kMaxElems ||
      n_w >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "linear: every tensor must have fewer than 2^31 elements");
  if (K >= kMaxK) return fail(BAIM_ERR_TOO_LARGE, "linear: K must be below 2^21");
  if (N >= kMaxAddmmN) return fail(BAIM_ERR_TOO_LARGE, "linear: N must be below 2^23");
  if (M == 0 || N == 0) return BAIM_OK;
  if (!out) return fail(BAIM_ERR_NULL, "linear: out is NULL");
  if (K > 0 && (!x || !weight)) return fail(BAIM_ERR_NULL, "linear: x/weight is NULL");
  if ((K > 0 && (overlap(out, n_out, x, n_x) || overlap(out, n_out, weight, n_w))) ||
      overlap(out, n_out, bias, N))
    return fail(BAIM_ERR_ALIAS, "linear: out overlaps an input");

  baim::AddmmProblem p;
  p.out = out;
  p.self = bias;
  p.mat1 = x;
  p.mat2 = weight;
  p.weight_nk = true;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.self_mode = bias ? 1 : 0;
  p.beta = 1.0f;
  p.alpha = 1.0f;
  return launched(baim::launch_addmm(p, (hipStream_t)stream), "linear_f32");
}

}  // extern "C"

namespace {

// The size checks of conv2d_gemm_f32 (everything but pointers); fills the
// sizes of `q` and the element counts of input, weight and output.
baim_status conv_sizes(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC, int64_t KH,
                       int64_t KW, int64_t sH, int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                       int64_t dW, int64_t groups, baim::ConvProblem* q, int64_t* n_x,
                       int64_t* n_w, int64_t* n_out) {
  if (B < 1 || IC < 1 || OC < 1)
    return fail(BAIM_ERR_SHAPE, "conv2d: B, IC and OC must be >= 1");
  if (groups < 1) return fail(BAIM_ERR_SHAPE, "conv2d: groups must be >= 1");
  int64_t OH = 0, OW = 0;
  const baim_status hs = baim_conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, &OH, &OW);
  if (hs != BAIM_OK) return hs;  // message already set
  if (IC % groups != 0 || OC % groups != 0)
    return fail(BAIM_ERR_SHAPE, "conv2d: groups=%lld must divide IC=%lld and OC=%lld",
                (long long)groups, (long long)IC, (long long)OC);
  const int64_t icg = IC / groups;
  *n_x = elems({B, IC, H, W});
  *n_w = elems({OC, icg, KH, KW});
  *n_out = elems({B, OC, OH, OW});
  const int64_t K = elems({icg, KH, KW});
  if (*n_x < 0 || *n_w < 0 || *n_out < 0 || *n_x >= kMaxElems || *n_w >= kMaxElems ||
      *n_out >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "conv2d: every tensor must have fewer than 2^31 elements");
  if (*n_x >= kMaxConvInput) return fail(BAIM_ERR_TOO_LARGE, "conv2d: input must have fewer than 2^29 elements");
  if (K >= kMaxK) return fail(BAIM_ERR_TOO_LARGE, "conv2d: (IC/groups)*KH*KW must be below 2^21");
  if (groups > 65535 || OC > 65535 || B > 65535)
    return fail(BAIM_ERR_TOO_LARGE, "conv2d: groups, OC and B must be at most 65535");
  // In-kernel tap offsets (ih*W + iw over the padded plane) are 32-bit.
  const int64_t n_pad = elems({H + 2 * pH, W + 2 * pW});
  if (n_pad < 0 || n_pad >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "conv2d: padded input plane must have fewer than 2^31 elements");
  q->B = (int)B;
  q->IC = (int)IC;
  q->H = (int)H;
  q->W = (int)W;
  q->OC = (int)OC;
  q->KH = (int)KH;
  q->KW = (int)KW;
  q->sH = (int)sH;
  q->sW = (int)sW;
  q->pH = (int)pH;
  q->pW = (int)pW;
  q->dH = (int)dH;
  q->dW = (int)dW;
  q->OH = (int)OH;
  q->OW = (int)OW;
  q->groups = (int)groups;
  return BAIM_OK;
}

}  // namespace

extern "C" {

baim_status conv2d_gemm_f32(float* out, const float* input, const float* weight,
                            const float* bias, int64_t B, int64_t IC, int64_t H, int64_t W,
                            int64_t OC, int64_t KH, int64_t KW, int64_t sH, int64_t sW,
                            int64_t pH, int64_t pW, int64_t dH, int64_t dW, int64_t groups,
                            void* stream) {
  g_err.clear();
  baim::ConvProblem q;
  int64_t n_x = 0, n_w = 0, n_out = 0;
  const baim_status st =
      conv_sizes(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, groups, &q, &n_x, &n_w, &n_out);
  if (st != BAIM_OK) return st;
  if (!out || !input || !weight) return fail(BAIM_ERR_NULL, "conv2d: out/input/weight is NULL");
  if (overlap(out, n_out, input, n_x) || overlap(out, n_out, weight, n_w) ||
      overlap(out, n_out, bias, OC))
    return fail(BAIM_ERR_ALIAS, "conv2d: out overlaps an input");
  q.out = out;
  q.x = input;
  q.w = weight;
  q.bias = bias;
  if (!baim::conv_uses_gemm(q))
    return launched(baim::launch_conv2d_direct(q, (hipStream_t)stream), "conv2d_gemm_f32");
  return launched(baim::launch_conv2d(q, (hipStream_t)stream), "conv2d_gemm_f32");
}

baim_status baim_conv2d_plan(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC,
                             int64_t KH, int64_t KW, int64_t sH, int64_t sW, int64_t pH,
                             int64_t pW, int64_t dH, int64_t dW, int64_t groups, int* kernel,
                             int* bm, int* bn, int* bk, int* waves, int* kgroups, int* splits,
                             int* stream_blocks) {
  g_err.clear();
  if (!kernel || !bm || !bn || !bk || !waves || !kgroups || !splits || !stream_blocks)
    return fail(BAIM_ERR_NULL, "baim_conv2d_plan: output pointers must not be NULL");
  baim::ConvProblem q;
  int64_t n_x = 0, n_w = 0, n_out = 0;
  const baim_status st =
      conv_sizes(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, groups, &q, &n_x, &n_w, &n_out);
  if (st != BAIM_OK) return st;
  *bm = *bn = *bk = *waves = *kgroups = *stream_blocks = 0;
  *splits = 1;
  if (!baim::conv_uses_gemm(q)) {
    *kernel = 2;
    return BAIM_OK;
  }
  const baim::WinPlan wp = baim::plan_conv_window(baim::win_shape(q), true, getenv("BAIM_CONV_WIN"));
  if (wp.geom >= 0) {
    *kernel = 1;
    *bm = baim::kWinBM[wp.geom];
    *bn = baim::kWinBN[wp.geom];
    *bk = baim::kWinCI * q.KH * q.KW;
    *waves = baim::kWinWaves;
    *kgroups = baim::kWinKGroups[wp.geom];
    *splits = wp.mode == baim::MODE_SLICES ? wp.splits : 1;
    *stream_blocks = wp.mode == baim::MODE_STREAM ? wp.workers : 0;
    return BAIM_OK;
  }
  if (baim::plan_conv_stem(baim::win_shape(q), true, getenv("BAIM_CONV_WIN"))) {
    *kernel = 3;
    *bm = baim::kStemBM;
    *bn = baim::kStemBN;
    *bk = q.IC * q.KH * q.KW;
    *waves = baim::kStemWaves;
    *kgroups = 1;
    return BAIM_OK;
  }
  *kernel = 0;
  const int M = q.OC / q.groups, N = q.B * q.OH * q.OW, K = q.IC / q.groups * q.KH * q.KW;
  baim::GemmPlan p = baim::plan_core_tile(baim::plan_gemm(M, N, K, getenv("BAIM_TILE")), M, N, K);
  if (p.mode == baim::MODE_STREAM && K % 4 != 0) p = baim::plan_tiles_only(p, M, N, K);
  *bm = baim::kTileBM[p.cfg];
  *bn = baim::kTileBN[p.cfg];
  *bk = baim::kTileBK[p.cfg];
  *waves = baim::kTileWaves[p.cfg];
  *kgroups = baim::kTileKGroups[p.cfg];
  *splits = p.mode == baim::MODE_SLICES ? p.splits : 1;
  *stream_blocks = p.mode == baim::MODE_STREAM ? p.workers : 0;
  return BAIM_OK;
}

}  // extern "C"

extern "C" baim_status sdpa_f32(float* out, const float* q, const float* k, const float* v,
                                const float* attn_mask, int64_t BH, int64_t Sq, int64_t Skv,
                                int64_t D, const float* scale, void* stream) {
  g_err.clear();
  if (BH < 0 || Sq < 0 || Skv < 0 || D < 0)
    return fail(BAIM_ERR_SHAPE, "sdpa: sizes must be >= 0 (BH=%lld Sq=%lld Skv=%lld D=%lld)",
                (long long)BH, (long long)Sq, (long long)Skv, (long long)D);
  const int64_t n_q = elems({BH, Sq, D}), n_kv = elems({BH, Skv, D});
  const int64_t n_m = elems({BH, Sq, Skv});
  if (n_q < 0 || n_kv < 0 || n_m < 0 || n_q >= kMaxElems || n_kv >= kMaxElems ||
      (attn_mask && n_m >= kMaxElems))
    return fail(BAIM_ERR_TOO_LARGE, "sdpa: every tensor must have fewer than 2^31 elements");
  if (elems({Sq, D}) >= kMaxSlice || elems({Skv, D}) >= kMaxSlice ||
      (attn_mask && elems({Sq, Skv}) >= kMaxSlice))
    return fail(BAIM_ERR_TOO_LARGE, "sdpa: Sq*D, Skv*D and Sq*Skv must be below 2^29");
  if (n_q == 0) return BAIM_OK;
  if (Skv == 0) return fail(BAIM_ERR_SHAPE, "sdpa: Skv must be >= 1 (no softmax over no keys)");
  if (D % 4 != 0 || D > 128)
    return fail(BAIM_ERR_UNSUPPORTED, "sdpa: D=%lld must be a multiple of 4 and at most 128",
                (long long)D);
  if (!out || !q || !k || !v) return fail(BAIM_ERR_NULL, "sdpa: out/q/k/v is NULL");
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15) != 0)
    return fail(BAIM_ERR_UNSUPPORTED, "sdpa: q, k and v must start on 16-byte boundaries");
  if (overlap(out, n_q, q, n_q) || overlap(out, n_q, k, n_kv) || overlap(out, n_q, v, n_kv) ||
      overlap(out, n_q, attn_mask, n_m))
    return fail(BAIM_ERR_ALIAS, "sdpa: out overlaps an input");

  baim::SdpaProblem p;
  p.out = out;
  p.q = q;
  p.k = k;
  p.v = v;
  p.mask = attn_mask;
  p.BH = (int)BH;
  p.Sq = (int)Sq;
  p.Skv = (int)Skv;
  p.D = (int)D;
  p.scale = scale ? *scale : (float)(1.0 / sqrt((double)D));
  return launched(baim::launch_sdpa(p, (hipStream_t)stream), "sdpa_f32");
}

// Size checks of a channels-last conv (as conv2d_nhwc_f32 applies them)
// and its problem description without pointers.
static baim_status nhwc_sizes(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC, int64_t KH,
                              int64_t KW, int64_t sH, int64_t sW, int64_t pH, int64_t pW,
                              int64_t dH, int64_t dW, baim::ConvProblem* q, int64_t* n_x,
                              int64_t* n_w, int64_t* n_out) {
  if (B < 1 || IC < 1 || OC < 1)
    return fail(BAIM_ERR_SHAPE, "conv2d_nhwc: B, IC and OC must be >= 1");
  int64_t OH = 0, OW = 0;
  const baim_status hs = baim_conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, &OH, &OW);
  if (hs != BAIM_OK) return hs;  // message already set
  *n_x = elems({B, H, W, IC});
  *n_w = elems({OC, KH, KW, IC});
  *n_out = elems({B, OH, OW, OC});
  const int64_t K = elems({KH, KW, IC});
  if (*n_x < 0 || *n_w < 0 || *n_out < 0 || *n_x >= kMaxElems || *n_w >= kMaxElems ||
      *n_out >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "conv2d_nhwc: every tensor must have fewer than 2^31 elements");
  if (*n_x >= kMaxConvInput)
    return fail(BAIM_ERR_TOO_LARGE, "conv2d_nhwc: input must have fewer than 2^29 elements");
  if (K >= kMaxK) return fail(BAIM_ERR_TOO_LARGE, "conv2d_nhwc: KH*KW*IC must be below 2^21");
  if (OC >= kMaxAddmmN) return fail(BAIM_ERR_TOO_LARGE, "conv2d_nhwc: OC must be below 2^23");
  q->out = nullptr;
  q->x = nullptr;
  q->w = nullptr;
  q->bias = nullptr;
  q->B = (int)B;
  q->IC = (int)IC;
  q->H = (int)H;
  q->W = (int)W;
  q->OC = (int)OC;
  q->KH = (int)KH;
  q->KW = (int)KW;
  q->sH = (int)sH;
  q->sW = (int)sW;
  q->pH = (int)pH;
  q->pW = (int)pW;
  q->dH = (int)dH;
  q->dW = (int)dW;
  q->OH = (int)OH;
  q->OW = (int)OW;
  q->groups = 1;
  return BAIM_OK;
}

extern "C" baim_status conv2d_nhwc_f32(float* out, const float* input, const float* weight,
                                       const float* bias, int64_t B, int64_t IC, int64_t H,
                                       int64_t W, int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                                       int64_t sW, int64_t pH, int64_t pW, int64_t dH, int64_t dW,
                                       void* stream) {
  g_err.clear();
  baim::ConvProblem q;
  int64_t n_x = 0, n_w = 0, n_out = 0;
  const baim_status st =
      nhwc_sizes(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, &q, &n_x, &n_w, &n_out);
  if (st != BAIM_OK) return st;
  if (!out || !input || !weight) return fail(BAIM_ERR_NULL, "conv2d_nhwc: out/input/weight is NULL");
  if (overlap(out, n_out, input, n_x) || overlap(out, n_out, weight, n_w) ||
      overlap(out, n_out, bias, OC))
    return fail(BAIM_ERR_ALIAS, "conv2d_nhwc: out overlaps an input");
  q.out = out;
  q.x = input;
  q.w = weight;
  q.bias = bias;
  return launched(baim::launch_conv2d_nhwc(q, (hipStream_t)stream), "conv2d_nhwc_f32");
}

extern "C" baim_status baim_conv2d_nhwc_plan(int64_t B, int64_t IC, int64_t H, int64_t W,
                                             int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                                             int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                                             int64_t dW, int* kernel) {
  g_err.clear();
  if (!kernel) return fail(BAIM_ERR_NULL, "baim_conv2d_nhwc_plan: kernel must not be NULL");
  baim::ConvProblem q;
  int64_t n_x = 0, n_w = 0, n_out = 0;
  const baim_status st =
      nhwc_sizes(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, &q, &n_x, &n_w, &n_out);
  if (st != BAIM_OK) return st;
  *kernel = baim::plan_conv_stem(baim::win_shape(q), true, getenv("BAIM_CONV_WIN")) ? 3 : 0;
  return BAIM_OK;
}

extern "C" baim_status baim_conv_transpose2d_out_hw(int64_t H, int64_t W, int64_t KH, int64_t KW,
                                                    int64_t sH, int64_t sW, int64_t pH,
                                                    int64_t pW, int64_t dH, int64_t dW,
                                                    int64_t opH, int64_t opW, int64_t* OH,
                                                    int64_t* OW) {
  g_err.clear();
  if (!OH || !OW)
    return fail(BAIM_ERR_NULL, "baim_conv_transpose2d_out_hw: OH/OW must not be NULL");
  *OH = *OW = 0;
  if (H < 1 || W < 1 || KH < 1 || KW < 1)
    return fail(BAIM_ERR_SHAPE, "conv_transpose2d: input and kernel sizes must be >= 1");
  if (sH < 1 || sW < 1) return fail(BAIM_ERR_SHAPE, "conv_transpose2d: stride must be >= 1");
  if (dH < 1 || dW < 1) return fail(BAIM_ERR_SHAPE, "conv_transpose2d: dilation must be >= 1");
  if (pH < 0 || pW < 0) return fail(BAIM_ERR_SHAPE, "conv_transpose2d: padding must be >= 0");
  if (H > kMaxElems || W > kMaxElems || KH > kMaxElems || KW > kMaxElems || sH > kMaxElems ||
      sW > kMaxElems || pH > kMaxElems || pW > kMaxElems || dH > kMaxElems || dW > kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE, "conv_transpose2d: size argument too large");
  if (opH < 0 || opW < 0 || opH >= (sH > dH ? sH : dH) || opW >= (sW > dW ? sW : dW))
    return fail(BAIM_ERR_SHAPE,
                "conv_transpose2d: output padding must be >= 0 and below max(stride, dilation)");
  const int64_t oh = (H - 1) * sH - 2 * pH + dH * (KH - 1) + opH + 1;
  const int64_t ow = (W - 1) * sW - 2 * pW + dW * (KW - 1) + opW + 1;
  if (oh < 1 || ow < 1)
    return fail(BAIM_ERR_SHAPE, "conv_transpose2d: empty output (%lld x %lld)", (long long)oh,
                (long long)ow);
  *OH = oh;
  *OW = ow;
  return BAIM_OK;
}

extern "C" baim_status conv_transpose2d_f32(float* out, const float* input, const float* weight,
                                            const float* bias, int64_t B, int64_t IC, int64_t H,
                                            int64_t W, int64_t OC, int64_t KH, int64_t KW,
                                            int64_t sH, int64_t sW, int64_t pH, int64_t pW,
                                            int64_t dH, int64_t dW, int64_t opH, int64_t opW,
                                            int64_t groups, void* stream) {
  g_err.clear();
  if (B < 1 || IC < 1 || OC < 1)
    return fail(BAIM_ERR_SHAPE, "conv_transpose2d: B, IC and OC must be >= 1");
  if (groups < 1 || IC % groups != 0 || OC % groups != 0)
    return fail(BAIM_ERR_SHAPE, "conv_transpose2d: groups=%lld must be >= 1 and divide IC=%lld "
                "and OC=%lld", (long long)groups, (long long)IC, (long long)OC);
  int64_t OH = 0, OW = 0;
  const baim_status hs =
      baim_conv_transpose2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, opH, opW, &OH, &OW);
  if (hs != BAIM_OK) return hs;  // message already set
  const int64_t ocg = OC / groups;
  const int64_t n_x = elems({B, IC, H, W}), n_w = elems({IC, ocg, KH, KW});
  const int64_t n_out = elems({B, OC, OH, OW}), K = elems({IC / groups, KH, KW});
  if (n_x < 0 || n_w < 0 || n_out < 0 || n_x >= kMaxElems || n_w >= kMaxElems ||
      n_out >= kMaxElems)
    return fail(BAIM_ERR_TOO_LARGE,
                "conv_transpose2d: every tensor must have fewer than 2^31 elements");
  if (n_x >= kMaxConvInput || n_w >= kMaxConvInput)
    return fail(BAIM_ERR_TOO_LARGE,
                "conv_transpose2d: input and weight must have fewer than 2^29 elements");
  if (K >= kMaxK)
    return fail(BAIM_ERR_TOO_LARGE, "conv_transpose2d: (IC/groups)*KH*KW must be below 2^21");
  if (groups > 65535) return fail(BAIM_ERR_TOO_LARGE, "conv_transpose2d: groups must be <= 65535");
  if (!out || !input || !weight)
    return fail(BAIM_ERR_NULL, "conv_transpose2d: out/input/weight is NULL");
  if (overlap(out, n_out, input, n_x) || overlap(out, n_out, weight, n_w) ||
      overlap(out, n_out, bias, OC))
    return fail(BAIM_ERR_ALIAS, "conv_transpose2d: out overlaps an input");

  baim::ConvTProblem q;
  q.out = out;
  q.x = input;
  q.w = weight;
  q.bias = bias;
  q.B = (int)B;
  q.IC = (int)IC;
  q.H = (int)H;
  q.W = (int)W;
  q.OC = (int)OC;
  q.KH = (int)KH;
  q.KW = (int)KW;
  q.sH = (int)sH;
  q.sW = (int)sW;
  q.pH = (int)pH;
  q.pW = (int)pW;
  q.dH = (int)dH;
  q.dW = (int)dW;
  q.OH = (int)OH;
  q.OW = (int)OW;
  q.groups = (int)groups;
  return launched(baim::launch_conv_transpose2d(q, (hipStream_t)stream), "conv_transpose2d_f32");
}
