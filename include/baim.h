/*
 * baim.h -- C ABI of libbaim.so: fp32 tiled GEMM with a fused epilogue on
 * AMD Instinct MI355X (gfx950), used as addmm and as groups==1 NCHW conv2d
 * through an implicit im2col.
 *
 * Common conventions
 *  - Every tensor pointer is a DEVICE pointer to caller-owned, contiguous,
 *    row-major (NCHW for images) fp32 memory.  The library never allocates,
 *    frees or retains memory; it only reads the inputs and writes `out`.
 *  - All arguments are validated on the host before anything is enqueued.
 *    A call that returns an error has launched nothing and left `out`
 *    untouched; baim_last_error() then describes the problem.
 *  - On success the work is ENQUEUED on `stream` (a hipStream_t; NULL means
 *    the default stream) and the call returns at once.  A device fault
 *    surfaces at the caller's next synchronisation, as with any HIP launch.
 *  - `out` must not overlap any input (BAIM_ERR_ALIAS).
 *  - Sizes are int64_t.  Limits (BAIM_ERR_TOO_LARGE beyond them, because
 *    in-kernel offsets are 32-bit): every tensor holds fewer than 2^31
 *    elements; K (IC*KH*KW for the conv) is below 2^21; addmm's N is below
 *    2^23; the conv input holds fewer than 2^29 elements and its padded
 *    plane (H+2pH)*(W+2pW) fewer than 2^31.
 *  - Results: any fp32 summation order is allowed (the order inside a tile,
 *    across tiles and inside the matrix cores is unspecified); the result
 *    satisfies |out - exact| <= 4e-6*sqrt(K)*(|alpha|*sum_k|a*b| + |beta*self|).
 *  - Thread safety: calls may be made from several host threads; the error
 *    text is per thread.
 */
#ifndef BAIM_H
#define BAIM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BAIM_OK = 0,
  BAIM_ERR_NULL = 1,        /* a required pointer is NULL                    */
  BAIM_ERR_SHAPE = 2,       /* a size/stride/flag is out of its domain       */
  BAIM_ERR_UNSUPPORTED = 3, /* valid call this library does not compute      */
  BAIM_ERR_TOO_LARGE = 4,   /* a tensor has 2^31 or more elements            */
  BAIM_ERR_ALIAS = 5,       /* out overlaps an input                         */
  BAIM_ERR_LAUNCH = 6       /* the HIP launch itself failed                  */
} baim_status;

/*
 * addmm_f32: out[M,N] = beta*self + alpha*(mat1[M,K] @ mat2[K,N]).
 *
 * Defined by "[ExecuTorch][WebGPU] Add optimized addmm op" (PR #20855),
 * Solution and Implementation paragraphs: mat1 [M,K] and mat2 [K,N] are
 * row-major (mat2 is read as mat2[k*N + n]); self is either the bias row
 * broadcast over rows (self_2d = 0: self[N], element self[n]) or a full
 * matrix (self_2d = 1: self[M,N], element self[m*N + n]); alpha and beta are
 * fp32 scalars (the page passes them as 32-bit floats, default 1.0).
 *
 *  out    [M,N] fp32, written in full.
 *  self   [N] or [M,N] fp32; may be NULL only when beta == 0.  When
 *         beta == 0 self is not read at all, so NaN/Inf in it do not
 *         propagate (aten's rule for addmm).
 *  mat1   [M,K], mat2 [K,N] fp32.  May be NULL only if the product is empty.
 *  M,N,K  >= 0.  M == 0 or N == 0: nothing to do, BAIM_OK.  K == 0: the
 *         product is empty and out = beta*self.
 *  stream hipStream_t or NULL.
 */
baim_status addmm_f32(float* out, const float* self, int self_2d,
                      const float* mat1, const float* mat2, int64_t M,
                      int64_t N, int64_t K, float beta, float alpha,
                      void* stream);

/*
 * linear_f32: out[M,N] = x[M,K] @ weight[N,K]^T + bias[N].
 *
 * From "[ExecuTorch][WebGPU] Add optimized addmm op", Implementation
 * paragraph: the addmm kernel shares its tiled-GEMM skeleton with
 * linear_fp32, whose weight is read transposed, as [N,K] (addmm instead
 * reads mat2 as [K,N]).  This is that linear: the same kernels and tile
 * choice as addmm_f32, with the weight's K-contiguous rows loaded directly
 * as the transposed B tile.
 *
 *  out     [M,N] fp32, written in full.
 *  x       [M,K] fp32.   weight  [N,K] fp32.   May be NULL only if K == 0.
 *  bias    [N] fp32, or NULL for no bias.
 *  M,N,K   >= 0.  M == 0 or N == 0: nothing to do, BAIM_OK.  K == 0: out is
 *          the broadcast bias (or 0).
 *  stream  hipStream_t or NULL.
 */
baim_status linear_f32(float* out, const float* x, const float* weight,
                       const float* bias, int64_t M, int64_t N, int64_t K,
                       void* stream);

/*
 * conv2d_gemm_f32: out = conv2d(input, weight, bias), NCHW, with `groups`.
 *
 * groups == 1 is computed as the GEMM  out[oc, n] = sum_kk weight[oc, kk] *
 * col[kk, n] + bias[oc], with M = OC, N = B*OH*OW, K = IC*KH*KW and col the
 * implicit im2col of the input (never materialised).
 *
 * Defined by "et_vk conv2d: route standard (groups==1) conv through an
 * im2col tiled GEMM" (PR #20873), Solution and Implementation paragraphs:
 * n decodes to (b, oh, ow) and kk to (ic, kh, kw); the input is sampled at
 * ih = oh*sH - pH + kh*dH, iw = ow*sW - pW + kw*dW, and a tap outside the
 * input reads 0 (zero padding); bias is added per output channel; the
 * output is NCHW.
 *
 * groups > 1 (the page keeps grouped and depthwise convs on its direct
 * kernels): output channel oc of group g = oc / (OC/groups) sums over the
 * input channels g*IC/groups .. (g+1)*IC/groups - 1 only.  When a group has
 * at least 32 output channels and 32 taps ((IC/groups)*KH*KW) it runs as
 * one implicit-im2col GEMM per group; otherwise (e.g. depthwise) on a
 * direct kernel, one thread per output.
 *
 *  out     [B,OC,OH,OW] fp32 NCHW, written in full; OH, OW as given by
 *          baim_conv2d_out_hw().
 *  input   [B,IC,H,W] fp32 NCHW.
 *  weight  [OC,IC/groups,KH,KW] fp32 (per group, the row-major
 *          [OC/groups, (IC/groups)*KH*KW] matrix).
 *  bias    [OC] fp32, or NULL for no bias.
 *  sizes   B, IC, H, W, OC, KH, KW >= 1; strides sH, sW >= 1;
 *          paddings pH, pW >= 0; dilations dH, dW >= 1; OH, OW >= 1.
 *  groups  >= 1 and dividing IC and OC (else BAIM_ERR_SHAPE); groups, OC
 *          and B at most 65535.
 *  stream  hipStream_t or NULL.
 */
baim_status conv2d_gemm_f32(float* out, const float* input,
                            const float* weight, const float* bias, int64_t B,
                            int64_t IC, int64_t H, int64_t W, int64_t OC,
                            int64_t KH, int64_t KW, int64_t sH, int64_t sW,
                            int64_t pH, int64_t pW, int64_t dH, int64_t dW,
                            int64_t groups, void* stream);

/*
 * conv2d_nhwc_f32: the conv of conv2d_gemm_f32 (groups == 1) on
 * channels-last tensors.
 *
 * From "et_vk conv2d: route standard (groups==1) conv through an im2col
 * tiled GEMM", Solution and Constraints paragraphs: the conv is the GEMM of
 * the weight with the implicit im2col of the input, and with NCHW the K
 * dimension is strided, so it cannot be read four at a time.  Here the
 * tensors are channels-last and K is ordered (kh, kw, ic), so each tap's
 * input channels are contiguous: out[m, oc] = sum_kk A[m, kk] * w[oc, kk]
 * + bias[oc], m = (b*OH + oh)*OW + ow, A the implicit im2col rows.  Same
 * padding, stride, dilation and output-size rules as conv2d_gemm_f32.
 *
 *  out     [B,OH,OW,OC] fp32 (NHWC), written in full.
 *  input   [B,H,W,IC] fp32 (NHWC).
 *  weight  [OC,KH,KW,IC] fp32 (OHWI: a K-contiguous [OC, KH*KW*IC] matrix).
 *  bias    [OC] fp32, or NULL for no bias.
 *  B, IC, OC >= 1; KH, KW >= 1; sH, sW, dH, dW >= 1; pH, pW >= 0
 *          (BAIM_ERR_SHAPE otherwise, or if the output would be empty).
 *  stream  hipStream_t or NULL.
 * Limits: every tensor below 2^31 elements, the input below 2^29,
 * KH*KW*IC below 2^21, OC below 2^23 (BAIM_ERR_TOO_LARGE).
 */
baim_status conv2d_nhwc_f32(float* out, const float* input,
                            const float* weight, const float* bias, int64_t B,
                            int64_t IC, int64_t H, int64_t W, int64_t OC,
                            int64_t KH, int64_t KW, int64_t sH, int64_t sW,
                            int64_t pH, int64_t pW, int64_t dH, int64_t dW,
                            void* stream);

/*
 * conv_transpose2d_f32: out = conv_transpose2d(input, weight, bias), NCHW.
 *
 * The conv page ("et_vk conv2d: route standard (groups==1) conv through an
 * im2col tiled GEMM", Solution paragraph) keeps transposed convs on their
 * own gather kernels and defines no arithmetic for them; this is the
 * standard operation (aten's conv_transpose2d, the adjoint of conv2d):
 * input element x[b, ic, ih, iw] times weight w[ic, oc, kh, kw] lands on
 * out[b, oc, ih*sH - pH + kh*dH, iw*sW - pW + kw*dW] (dropped outside the
 * output), plus bias[oc]; with groups, input channels and output channels
 * split into `groups` equal blocks that only meet each other.  Computed as
 * one dense implicit GEMM per output phase (oh % sH, ow % sW), whose taps
 * are exactly the ones that land on it.
 *
 *  out     [B,OC,OH,OW] fp32, written in full; OH, OW from
 *          baim_conv_transpose2d_out_hw().
 *  input   [B,IC,H,W] fp32.
 *  weight  [IC,OC/groups,KH,KW] fp32.
 *  bias    [OC] fp32, or NULL for no bias.
 *  opH, opW  output padding: 0 <= op < max(stride, dilation) per axis.
 *  groups  >= 1, dividing IC and OC.
 *  stream  hipStream_t or NULL.
 * Limits: every tensor below 2^31 elements, input and weight below 2^29,
 * (IC/groups)*KH*KW below 2^21, groups at most 65535 (BAIM_ERR_TOO_LARGE).
 */
baim_status conv_transpose2d_f32(float* out, const float* input,
                                 const float* weight, const float* bias,
                                 int64_t B, int64_t IC, int64_t H, int64_t W,
                                 int64_t OC, int64_t KH, int64_t KW,
                                 int64_t sH, int64_t sW, int64_t pH,
                                 int64_t pW, int64_t dH, int64_t dW,
                                 int64_t opH, int64_t opW, int64_t groups,
                                 void* stream);

/*
 * baim_conv_transpose2d_out_hw: the output size of the transposed conv,
 * OH = (H-1)*sH - 2*pH + dH*(KH-1) + opH + 1 and likewise OW (aten's
 * rule; the output padding only adds rows and columns at the far edge).
 * BAIM_ERR_SHAPE for an empty output or an output padding outside
 * [0, max(stride, dilation)).
 */
baim_status baim_conv_transpose2d_out_hw(int64_t H, int64_t W, int64_t KH,
                                         int64_t KW, int64_t sH, int64_t sW,
                                         int64_t pH, int64_t pW, int64_t dH,
                                         int64_t dW, int64_t opH, int64_t opW,
                                         int64_t* OH, int64_t* OW);

/*
 * sdpa_f32: out = softmax(q @ k^T * scale + attn_mask) @ v, non-causal.
 *
 * Defined by "[ExecuTorch][WebGPU] Add optimized SDPA op" (PR #20851),
 * Problem and Solution paragraphs: row-major [B,H,S,D] tensors with the
 * softmax along the key axis, an optional additive mask of shape
 * [B,H,Sq,Skv], Sq and Skv free to differ, scale 1/sqrt(D) when not given,
 * fp32 only, D a multiple of 4.  The leading batch and head dimensions are
 * passed flattened as BH.  Computed in one pass with a running softmax per
 * query row; no scores buffer is allocated.
 *
 *  out        [BH,Sq,D] fp32, written in full.
 *  q          [BH,Sq,D] fp32.   k, v  [BH,Skv,D] fp32.
 *             q, k and v must start on 16-byte boundaries.
 *  attn_mask  [BH,Sq,Skv] fp32 added to the scaled logits, or NULL.  -inf
 *             entries drop keys; a query row with every key dropped comes
 *             out NaN (there is no softmax over an empty set).
 *  BH,Sq,D    >= 0; any of them 0: nothing to do, BAIM_OK.
 *  Skv        >= 1 (BAIM_ERR_SHAPE otherwise, unless the output is empty).
 *  D          a multiple of 4 and at most 128 (BAIM_ERR_UNSUPPORTED).
 *  scale      host pointer to the multiplier of q.k, or NULL for
 *             1/sqrt(D) rounded to fp32.
 *  stream     hipStream_t or NULL.
 * Limits: Sq*D, Skv*D and Sq*Skv below 2^29; every tensor below 2^31
 * elements (BAIM_ERR_TOO_LARGE).
 */
baim_status sdpa_f32(float* out, const float* q, const float* k,
                     const float* v, const float* attn_mask, int64_t BH,
                     int64_t Sq, int64_t Skv, int64_t D, const float* scale,
                     void* stream);

/*
 * baim_conv2d_out_hw: the output size of the conv above,
 * OH = floor((H + 2*pH - dH*(KH-1) - 1) / sH) + 1 and likewise OW (the
 * pages print no formula; this is the standard one, which gives a 192x192
 * output for a 7x7, stride-4, pad-3 stem on a 768x768 input).
 * Writes *OH and *OW and returns BAIM_OK, or BAIM_ERR_SHAPE (with *OH, *OW
 * set to 0) if an argument is out of range or the output would be empty;
 * BAIM_ERR_NULL if OH or OW is NULL.  Host-only; touches no GPU.
 */
baim_status baim_conv2d_out_hw(int64_t H, int64_t W, int64_t KH, int64_t KW,
                               int64_t sH, int64_t sW, int64_t pH, int64_t pW,
                               int64_t dH, int64_t dW, int64_t* OH,
                               int64_t* OW);

/*
 * baim_gemm_plan: how the library computes a GEMM of size M x N x K (the
 * same choice serves both ops; for the conv M = OC, N = B*OH*OW,
 * K = IC*KH*KW).  Writes the block tile BM x BN x BK, the waves per block,
 * the number of wave groups that split each k-tile (their partial tiles
 * are summed in a fixed order), and how tiles map to blocks:
 *   splits > 1         K is cut into `splits` slices on separate blocks;
 *   stream_blocks > 0  `stream_blocks` blocks share the work evenly, so a
 *                      tile may be cut into two pieces.
 * A tile cut into exactly two pieces is combined with a fixed, order-free
 * sum (bit-reproducible).  Only with splits > 2 (grids too small to fill
 * the chip otherwise) are the slices added with atomics, and the last bits
 * may then differ from run to run.  The 256 x 256 tile (BK 16, 8 waves) is
 * addmm's alone: linear_f32 and the convs run the 128 x 128 tile where it
 * is planned.  The environment variable BAIM_TILE ("cfg", "cfg,S" or
 * "cfg,sP", cfg 0..9) overrides the choice for tuning, here and in the
 * ops.  Host-only; touches no GPU.
 */
baim_status baim_gemm_plan(int64_t M, int64_t N, int64_t K, int* bm, int* bn,
                           int* bk, int* waves, int* kgroups, int* splits,
                           int* stream_blocks);

/*
 * baim_conv2d_plan: how conv2d_gemm_f32 computes a conv of these sizes on
 * 16-byte aligned input and weight (the conv page routes groups == 1 convs
 * through its im2col tiled GEMM and the others to their own kernels: "et_vk
 * conv2d: route standard (groups==1) conv through an im2col tiled GEMM",
 * Solution paragraph).  Arguments as conv2d_gemm_f32's sizes.  Writes
 * *kernel:
 *   0  the implicit-im2col GEMM; the tile fields are baim_gemm_plan's for
 *      M = OC/groups, N = B*OH*OW, K = (IC/groups)*KH*KW;
 *   1  the LDS-window kernel for compiled small kernels (3x3 at stride 1,
 *      dilation 1 or 2, OW >= 43, W % 4 == 0, W + pW <= 60, pW <= 4,
 *      IC % 4 == 0, groups == 1): block tile BM output channels x BN
 *      output pixels of one image, BK = 16 input channels x KH*KW taps;
 *   2  the direct kernels of grouped and depthwise convs (tile fields 0,
 *      splits 1);
 *   3  the stem kernel for 3-channel 7x7 stride-4 convs (the patch-embed
 *      stem the conv page motivates itself with; dilation 1, OW >= 144,
 *      W % 4 == 0, OC % 4 == 0): one pass over all of K = 147 per block of
 *      BM = 128 output channels x BN = 144 output pixels.
 * splits and stream_blocks mean what they mean for baim_gemm_plan.  The
 * overrides BAIM_TILE (kernel 0) and BAIM_CONV_WIN ("off", "tile", "2" or
 * "sP"; kernel 1; "off" also declines kernel 3) apply here as in the op.  Returns the status
 * conv2d_gemm_f32 would return for these sizes (SHAPE, TOO_LARGE), or
 * BAIM_ERR_NULL if an output pointer is NULL.  Host-only; touches no GPU.
 */
baim_status baim_conv2d_plan(int64_t B, int64_t IC, int64_t H, int64_t W,
                             int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                             int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                             int64_t dW, int64_t groups, int* kernel, int* bm,
                             int* bn, int* bk, int* waves, int* kgroups,
                             int* splits, int* stream_blocks);

/*
 * baim_conv2d_nhwc_plan: which kernel conv2d_nhwc_f32 runs for a
 * channels-last conv of these sizes on 16-byte aligned input, weight and
 * out.  The conv page's motivating case, a 3-channel patch-embed stem ("et_vk
 * conv2d: route standard (groups==1) conv through an im2col tiled GEMM",
 * Problem paragraph), has a kernel of its own in this layout as well.
 * Arguments as conv2d_nhwc_f32's sizes.  Writes *kernel:
 *   0  the addmm kernels with an im2col A operand;
 *   3  the stem kernel for 3-channel 7x7 stride-4 convs (dilation 1,
 *      OW >= 144, W % 4 == 0, OC % 4 == 0), as baim_conv2d_plan's kernel 3.
 * BAIM_CONV_WIN="off" declines kernel 3, as in the op.  Returns the status
 * conv2d_nhwc_f32 would return for these sizes (SHAPE, TOO_LARGE), or
 * BAIM_ERR_NULL if kernel is NULL.  Host-only; touches no GPU.
 */
baim_status baim_conv2d_nhwc_plan(int64_t B, int64_t IC, int64_t H, int64_t W,
                                  int64_t OC, int64_t KH, int64_t KW,
                                  int64_t sH, int64_t sW, int64_t pH,
                                  int64_t pW, int64_t dH, int64_t dW,
                                  int* kernel);

/* Text describing the last error returned on the calling thread ("" if the
 * last call succeeded).  The pointer stays valid until the next call on the
 * same thread. */
const char* baim_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int baim_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BAIM_H */
