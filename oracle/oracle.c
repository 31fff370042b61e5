/*
 * oracle.c -- plain, slow, fp64 CPU definition of the fp32 "bias addmm",
 * linear, conv2d-as-GEMM and non-causal attention computations.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP path.
 *
 * Sources (the method's definition):
 *  - "[ExecuTorch][WebGPU] Add optimized addmm op" (pytorch/executorch PR
 *    #20855), Solution and Implementation paragraphs: the op computes
 *    out = beta*self + alpha*(mat1 @ mat2) with mat1 [M,K], mat2 [K,N]
 *    row-major (mat2 read as mat2[k*N + n]), and self either broadcast from
 *    [N] (self[c]) or a full [M,N] (self[r*N + c]).
 *  - the same page, Implementation paragraph: the addmm kernel shares its
 *    tiled-GEMM skeleton with linear_fp32, which reads a transposed [N,K]
 *    weight: linear computes out[m,n] = sum_k x[m,k] * weight[n,k] + bias[n].
 *  - grouped conv (the same conv page keeps grouped and depthwise convs on
 *    its direct kernels): with G groups, output channel oc belongs to
 *    group g = oc / (OC/G) and sums over input channels
 *    g*(IC/G) .. (g+1)*(IC/G)-1 only; the weight is [OC, IC/G, KH, KW].
 *  - "et_vk conv2d: route standard (groups==1) conv through an im2col tiled
 *    GEMM" (pytorch/executorch PR #20873), Solution and Implementation
 *    paragraphs: groups==1 conv is a GEMM with M=OC, N=B*OH*OW, K=IC*KH*KW;
 *    the B operand is the input sampled at ih = oh*sH - pH + kh*dH (and the
 *    same along W), with out-of-range taps reading 0 (this is the padding);
 *    bias is added per output channel (row) and the output is NCHW.
 *
 *  - "[ExecuTorch][WebGPU] Add optimized SDPA op" (pytorch/executorch PR
 *    #20851): non-causal attention softmax(q @ k^T * scale + mask) @ v; see
 *    the section at the end of this file.
 *
 * Arithmetic: every product and sum is done in double from the fp32 inputs
 * widened to double; the sum over k (or over the (ic,kh,kw) taps) runs in
 * increasing index order.  Next to each result the oracle also returns
 * sabs = sum |a*b| over the same terms, which scales the acceptance bound
 * |out - ref| <= 4e-6 * sqrt(K) * (|alpha|*sabs + |beta*self|).
 *
 * Readings where the pages are silent:
 *  - beta == 0: the self term is exactly 0 and self is not read (aten's rule
 *    for addmm; equal to the literal formula on finite inputs).
 *  - conv output size: OH = floor((H + 2*pH - dH*(KH-1) - 1)/sH) + 1 (same
 *    along W); zero padding symmetric per axis; iw is the W-axis analogue of
 *    the printed ih formula; a NULL bias means 0.
 *  - K == 0: the sum is empty, so ref = beta*self.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* The self term of the addmm epilogue for output (i, j). */
static double self_term(const float* self, int self_2d, float beta, int64_t i,
                        int64_t j, int64_t N) {
  if (beta == 0.0f) return 0.0;
  double s = self_2d ? (double)self[i * N + j] : (double)self[j];
  return (double)beta * s;
}

/* One addmm output element: the plain dot product over k, then the epilogue. */
static void addmm_one(int64_t i, int64_t j, int64_t N, int64_t K,
                      const float* mat1, const float* mat2, const float* self,
                      int self_2d, float beta, float alpha, double* ref,
                      double* sabs) {
  double acc = 0.0, aabs = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double p = (double)mat1[i * K + k] * (double)mat2[k * N + j];
    acc += p;
    aabs += fabs(p);
  }
  *ref = self_term(self, self_2d, beta, i, j, N) + (double)alpha * acc;
  *sabs = aabs;
}

/* Full addmm: ref and sabs are [M,N] row-major doubles. */
void oracle_addmm(int64_t M, int64_t N, int64_t K, const float* mat1,
                  const float* mat2, const float* self, int self_2d,
                  float beta, float alpha, double* ref, double* sabs) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j)
      addmm_one(i, j, N, K, mat1, mat2, self, self_2d, beta, alpha,
                &ref[i * N + j], &sabs[i * N + j]);
}

/* addmm at n sampled outputs (rows[s], cols[s]). */
void oracle_addmm_at(int64_t M, int64_t N, int64_t K, const float* mat1,
                     const float* mat2, const float* self, int self_2d,
                     float beta, float alpha, int64_t n, const int64_t* rows,
                     const int64_t* cols, double* ref, double* sabs) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n; ++s)
    addmm_one(rows[s], cols[s], N, K, mat1, mat2, self, self_2d, beta, alpha,
              &ref[s], &sabs[s]);
}

/* One linear output element: the dot product of row m of x and row n of
 * weight (both K-contiguous), plus bias[n] (NULL bias means 0). */
static void linear_one(int64_t m, int64_t n, int64_t K, const float* x,
                       const float* w, const float* bias, double* ref,
                       double* sabs) {
  double acc = 0.0, aabs = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double p = (double)x[m * K + k] * (double)w[n * K + k];
    acc += p;
    aabs += fabs(p);
  }
  *ref = (bias ? (double)bias[n] : 0.0) + acc;
  *sabs = aabs;
}

/* Full linear: ref and sabs are [M,N] row-major doubles. */
void oracle_linear(int64_t M, int64_t N, int64_t K, const float* x,
                   const float* w, const float* bias, double* ref,
                   double* sabs) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      linear_one(m, n, K, x, w, bias, &ref[m * N + n], &sabs[m * N + n]);
}

/* linear at n sampled outputs (rows[s], cols[s]). */
void oracle_linear_at(int64_t M, int64_t N, int64_t K, const float* x,
                      const float* w, const float* bias, int64_t n,
                      const int64_t* rows, const int64_t* cols, double* ref,
                      double* sabs) {
  (void)M;
  (void)N;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n; ++s)
    linear_one(rows[s], cols[s], K, x, w, bias, &ref[s], &sabs[s]);
}

/* Output spatial size of a conv along one axis; <= 0 means no valid output. */
int64_t oracle_conv_out_size(int64_t in, int64_t k, int64_t s, int64_t p,
                             int64_t d) {
  int64_t span = in + 2 * p - d * (k - 1) - 1;
  if (span < 0 || s < 1) return 0;
  return span / s + 1;
}

typedef struct {
  int64_t B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW;
} conv_shape;

static conv_shape make_shape(int64_t B, int64_t IC, int64_t H, int64_t W,
                             int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                             int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                             int64_t dW) {
  conv_shape c = {B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, 0, 0};
  c.OH = oracle_conv_out_size(H, KH, sH, pH, dH);
  c.OW = oracle_conv_out_size(W, KW, sW, pW, dW);
  return c;
}

/* One conv output element out[b, oc, oh, ow]: direct sum over (ic, kh, kw),
 * taps outside the input contribute nothing (zero padding), plus bias[oc]. */
static void conv_one(const conv_shape* c, int64_t b, int64_t oc, int64_t oh,
                     int64_t ow, const float* x, const float* w,
                     const float* bias, double* ref, double* sabs) {
  double acc = 0.0, aabs = 0.0;
  for (int64_t ic = 0; ic < c->IC; ++ic)
    for (int64_t kh = 0; kh < c->KH; ++kh)
      for (int64_t kw = 0; kw < c->KW; ++kw) {
        int64_t ih = oh * c->sH - c->pH + kh * c->dH;
        int64_t iw = ow * c->sW - c->pW + kw * c->dW;
        if (ih < 0 || ih >= c->H || iw < 0 || iw >= c->W) continue;
        double xv = (double)x[((b * c->IC + ic) * c->H + ih) * c->W + iw];
        double wv = (double)w[((oc * c->IC + ic) * c->KH + kh) * c->KW + kw];
        acc += wv * xv;
        aabs += fabs(wv * xv);
      }
  *ref = (bias ? (double)bias[oc] : 0.0) + acc;
  *sabs = aabs;
}

/* Full direct conv: ref and sabs are [B, OC, OH, OW] doubles. Returns -1 if
 * the output would be empty. */
int oracle_conv2d(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC,
                  int64_t KH, int64_t KW, int64_t sH, int64_t sW, int64_t pH,
                  int64_t pW, int64_t dH, int64_t dW, const float* x,
                  const float* w, const float* bias, double* ref,
                  double* sabs) {
  conv_shape c = make_shape(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0) return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t oc = 0; oc < OC; ++oc)
      for (int64_t oh = 0; oh < c.OH; ++oh)
        for (int64_t ow = 0; ow < c.OW; ++ow) {
          int64_t o = ((b * OC + oc) * c.OH + oh) * c.OW + ow;
          conv_one(&c, b, oc, oh, ow, x, w, bias, &ref[o], &sabs[o]);
        }
  return 0;
}

/* Direct conv at n sampled outputs, given as flat NCHW output indices. */
int oracle_conv2d_at(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC,
                     int64_t KH, int64_t KW, int64_t sH, int64_t sW,
                     int64_t pH, int64_t pW, int64_t dH, int64_t dW,
                     const float* x, const float* w, const float* bias,
                     int64_t n, const int64_t* idx, double* ref,
                     double* sabs) {
  conv_shape c = make_shape(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0) return -1;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n; ++s) {
    int64_t o = idx[s];
    int64_t ow = o % c.OW, oh = (o / c.OW) % c.OH;
    int64_t oc = (o / (c.OW * c.OH)) % OC, b = o / (c.OW * c.OH * OC);
    conv_one(&c, b, oc, oh, ow, x, w, bias, &ref[s], &sabs[s]);
  }
  return 0;
}

/* One grouped-conv output element out[b, oc, oh, ow]: the direct sum over
 * the IC/G input channels of oc's group and the (kh, kw) taps. */
static void conv_one_grouped(const conv_shape* c, int64_t G, int64_t b,
                             int64_t oc, int64_t oh, int64_t ow,
                             const float* x, const float* w,
                             const float* bias, double* ref, double* sabs) {
  const int64_t icg = c->IC / G, ocg = c->OC / G, g = oc / ocg;
  double acc = 0.0, aabs = 0.0;
  for (int64_t icl = 0; icl < icg; ++icl)
    for (int64_t kh = 0; kh < c->KH; ++kh)
      for (int64_t kw = 0; kw < c->KW; ++kw) {
        int64_t ih = oh * c->sH - c->pH + kh * c->dH;
        int64_t iw = ow * c->sW - c->pW + kw * c->dW;
        if (ih < 0 || ih >= c->H || iw < 0 || iw >= c->W) continue;
        int64_t ic = g * icg + icl;
        double xv = (double)x[((b * c->IC + ic) * c->H + ih) * c->W + iw];
        double wv = (double)w[((oc * icg + icl) * c->KH + kh) * c->KW + kw];
        acc += wv * xv;
        aabs += fabs(wv * xv);
      }
  *ref = (bias ? (double)bias[oc] : 0.0) + acc;
  *sabs = aabs;
}

/* Grouped direct conv at n sampled flat NCHW output indices.  Returns -1 if
 * the output is empty or G does not divide IC and OC. */
int oracle_conv2d_grouped_at(int64_t B, int64_t IC, int64_t H, int64_t W,
                             int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                             int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                             int64_t dW, int64_t G, const float* x,
                             const float* w, const float* bias, int64_t n,
                             const int64_t* idx, double* ref, double* sabs) {
  conv_shape c = make_shape(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0 || G < 1 || IC % G || OC % G) return -1;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t s = 0; s < n; ++s) {
    int64_t o = idx[s];
    int64_t ow = o % c.OW, oh = (o / c.OW) % c.OH;
    int64_t oc = (o / (c.OW * c.OH)) % OC, b = o / (c.OW * c.OH * OC);
    conv_one_grouped(&c, G, b, oc, oh, ow, x, w, bias, &ref[s], &sabs[s]);
  }
  return 0;
}

/* Full grouped direct conv: ref and sabs are [B, OC, OH, OW] doubles. */
int oracle_conv2d_grouped(int64_t B, int64_t IC, int64_t H, int64_t W,
                          int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                          int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                          int64_t dW, int64_t G, const float* x,
                          const float* w, const float* bias, double* ref,
                          double* sabs) {
  conv_shape c = make_shape(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0 || G < 1 || IC % G || OC % G) return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t oc = 0; oc < OC; ++oc)
      for (int64_t oh = 0; oh < c.OH; ++oh)
        for (int64_t ow = 0; ow < c.OW; ++ow) {
          int64_t o = ((b * OC + oc) * c.OH + oh) * c.OW + ow;
          conv_one_grouped(&c, G, b, oc, oh, ow, x, w, bias, &ref[o],
                           &sabs[o]);
        }
  return 0;
}

/* Explicit im2col: col is [K, B*OH*OW] (double) with row kk = (ic*KH+kh)*KW+kw
 * and column n = (b*OH+oh)*OW+ow; out-of-range taps are 0.  With this matrix
 * the conv is W[OC,K] @ col + bias (the GEMM view of the conv page). */
int oracle_im2col(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t KH,
                  int64_t KW, int64_t sH, int64_t sW, int64_t pH, int64_t pW,
                  int64_t dH, int64_t dW, const float* x, double* col) {
  conv_shape c = make_shape(B, IC, H, W, 1, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0) return -1;
  int64_t N = B * c.OH * c.OW;
  for (int64_t ic = 0; ic < IC; ++ic)
    for (int64_t kh = 0; kh < KH; ++kh)
      for (int64_t kw = 0; kw < KW; ++kw) {
        int64_t kk = (ic * KH + kh) * KW + kw;
        for (int64_t b = 0; b < B; ++b)
          for (int64_t oh = 0; oh < c.OH; ++oh)
            for (int64_t ow = 0; ow < c.OW; ++ow) {
              int64_t n = (b * c.OH + oh) * c.OW + ow;
              int64_t ih = oh * sH - pH + kh * dH, iw = ow * sW - pW + kw * dW;
              double v = 0.0;
              if (ih >= 0 && ih < H && iw >= 0 && iw < W)
                v = (double)x[((b * IC + ic) * H + ih) * W + iw];
              col[kk * N + n] = v;
            }
      }
  return 0;
}

/* ---- Scaled dot-product attention (non-causal) -------------------------
 * "[ExecuTorch][WebGPU] Add optimized SDPA op" (pytorch/executorch PR
 * #20851), Problem and Solution paragraphs: over row-major [B,H,S,D]
 * tensors, out = softmax(q @ k^T * scale + attn_mask) @ v, the softmax taken
 * along the key axis.  q is [.., Sq, D]; k and v are [.., Skv, D] (Sq may
 * differ from Skv); the optional additive mask is [.., Sq, Skv]; the scale
 * is supplied by the caller (1/sqrt(D) when the op's argument is absent).
 * The leading batch and head dimensions are flattened to BH.
 *
 * Per query row (bh, i):
 *   s_j  = scale * sum_d q[i,d] k[j,d] + mask[i,j]
 *   w_j  = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)
 *   out[i,d] = sum_j w_j v[j,d]
 * A row whose logits are all -inf has no softmax; the formula then gives NaN
 * (as the plain definition and aten do), and so does the oracle.
 *
 * Next to out the oracle returns an error scale
 *   err[i,d] = sum_j w_j (|v[j,d]| + |out[i,d]|)
 *              * (sqrt(D) a_j + |s_j - max s| + sqrt(Skv) + 1),
 *   a_j = |scale| sum_d |q[i,d] k[j,d]| + |mask[i,j]|,
 * the first-order size of an fp32 evaluation's error in units of the fp32
 * rounding unit: the logit's dot product (a_j), the exponent's argument
 * (|s_j - max|), the sums over keys (Skv) and the final division.  The
 * parity bound is |out - ref| <= 4e-6 * err. */
static void sdpa_row(int64_t bh, int64_t i, int64_t Sq, int64_t Skv, int64_t D,
                     const float* q, const float* k, const float* v,
                     const float* mask, float scale, double* s, double* a,
                     double* out, double* err) {
  const float* qi = q + (bh * Sq + i) * D;
  double m = -INFINITY;
  for (int64_t j = 0; j < Skv; ++j) {
    const float* kj = k + (bh * Skv + j) * D;
    double dot = 0.0, dabs = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      double p = (double)qi[d] * (double)kj[d];
      dot += p;
      dabs += fabs(p);
    }
    double mk = mask ? (double)mask[(bh * Sq + i) * Skv + j] : 0.0;
    s[j] = (double)scale * dot + mk;
    a[j] = fabs((double)scale) * dabs + fabs(mk);
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < Skv; ++j) l += exp(s[j] - m);
  for (int64_t d = 0; d < D; ++d) {
    double o = 0.0;
    for (int64_t j = 0; j < Skv; ++j)
      o += exp(s[j] - m) / l * (double)v[(bh * Skv + j) * D + d];
    out[d] = o;
  }
  double sd = sqrt((double)D), ss = sqrt((double)Skv);
  for (int64_t d = 0; d < D; ++d) {
    double e = 0.0;
    for (int64_t j = 0; j < Skv; ++j) {
      double w = exp(s[j] - m) / l;
      if (!(w > 0.0)) continue; /* a key with weight 0 adds no error */
      e += w * (fabs((double)v[(bh * Skv + j) * D + d]) + fabs(out[d])) *
           (sd * a[j] + fabs(s[j] - m) + ss + 1.0);
    }
    err[d] = (m == -INFINITY) ? NAN : e;
  }
}

/* Full reference: out and err are [BH, Sq, D]. */
int oracle_sdpa(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const float* q,
                const float* k, const float* v, const float* mask, float scale,
                double* out, double* err) {
  if (Skv <= 0) return -1;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * 2 * (size_t)Skv);
#pragma omp for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh)
      for (int64_t i = 0; i < Sq; ++i)
        sdpa_row(bh, i, Sq, Skv, D, q, k, v, mask, scale, s, s + Skv,
                 out + (bh * Sq + i) * D, err + (bh * Sq + i) * D);
    free(s);
  }
  return 0;
}

/* Reference at sampled query rows: rows[r] = bh*Sq + i; out and err are
 * [n, D]. */
int oracle_sdpa_rows(int64_t BH, int64_t Sq, int64_t Skv, int64_t D,
                     const float* q, const float* k, const float* v,
                     const float* mask, float scale, int64_t n,
                     const int64_t* rows, double* out, double* err) {
  if (Skv <= 0) return -1;
  (void)BH;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * 2 * (size_t)Skv);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; ++r)
      sdpa_row(rows[r] / Sq, rows[r] % Sq, Sq, Skv, D, q, k, v, mask, scale, s,
               s + Skv, out + r * D, err + r * D);
    free(s);
  }
  return 0;
}

/* ---- Channels-last conv2d (NHWC input and output, OHWI weight) ---------
 * The same convolution as oracle_conv2d (groups == 1) with the tensors laid
 * out channels-last: input x[b, ih, iw, ic] ([B,H,W,IC]), weight
 * w[oc, kh, kw, ic] ([OC,KH,KW,IC]) and output out[b, oh, ow, oc]
 * ([B,OH,OW,OC]).  "et_vk conv2d: route standard (groups==1) conv through
 * an im2col tiled GEMM", Constraints paragraph: in NCHW the channel stride
 * is not contiguous, so the GEMM's K dimension cannot be read four at a
 * time; channels-last makes the input channels, and with K ordered as
 * (kh, kw, ic) each tap's K run, contiguous.  Taps are summed in
 * (kh, kw, ic) order; out-of-range taps read 0; bias per output channel. */
static void conv_one_nhwc(const conv_shape* c, int64_t b, int64_t oh,
                          int64_t ow, int64_t oc, const float* x,
                          const float* w, const float* bias, double* ref,
                          double* sabs) {
  double acc = 0.0, aabs = 0.0;
  for (int64_t kh = 0; kh < c->KH; ++kh) {
    int64_t ih = oh * c->sH - c->pH + kh * c->dH;
    if (ih < 0 || ih >= c->H) continue;
    for (int64_t kw = 0; kw < c->KW; ++kw) {
      int64_t iw = ow * c->sW - c->pW + kw * c->dW;
      if (iw < 0 || iw >= c->W) continue;
      for (int64_t ic = 0; ic < c->IC; ++ic) {
        double p = (double)x[((b * c->H + ih) * c->W + iw) * c->IC + ic] *
                   (double)w[((oc * c->KH + kh) * c->KW + kw) * c->IC + ic];
        acc += p;
        aabs += fabs(p);
      }
    }
  }
  *ref = (bias ? (double)bias[oc] : 0.0) + acc;
  *sabs = aabs;
}

int oracle_conv2d_nhwc(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC,
                       int64_t KH, int64_t KW, int64_t sH, int64_t sW,
                       int64_t pH, int64_t pW, int64_t dH, int64_t dW,
                       const float* x, const float* w, const float* bias,
                       double* ref, double* sabs) {
  conv_shape c = make_shape(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0) return -1;
#pragma omp parallel for collapse(3) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t oh = 0; oh < c.OH; ++oh)
      for (int64_t ow = 0; ow < c.OW; ++ow)
        for (int64_t oc = 0; oc < OC; ++oc) {
          int64_t o = ((b * c.OH + oh) * c.OW + ow) * OC + oc;
          conv_one_nhwc(&c, b, oh, ow, oc, x, w, bias, &ref[o], &sabs[o]);
        }
  return 0;
}

/* Sampled channels-last conv at flat NHWC output indices idx[s]. */
int oracle_conv2d_nhwc_at(int64_t B, int64_t IC, int64_t H, int64_t W,
                          int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                          int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                          int64_t dW, const float* x, const float* w,
                          const float* bias, int64_t n, const int64_t* idx,
                          double* ref, double* sabs) {
  conv_shape c = make_shape(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW);
  if (c.OH <= 0 || c.OW <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < n; ++s) {
    int64_t o = idx[s];
    int64_t oc = o % OC, ow = (o / OC) % c.OW, oh = (o / (OC * c.OW)) % c.OH;
    int64_t b = o / (OC * c.OW * c.OH);
    conv_one_nhwc(&c, b, oh, ow, oc, x, w, bias, &ref[s], &sabs[s]);
  }
  return 0;
}

/* ---- Transposed conv2d (NCHW) -------------------------------------------
 * The conv page routes transposed convs to their own gather kernels
 * ("et_vk conv2d: route standard (groups==1) conv through an im2col tiled
 * GEMM", Solution paragraph) and defines no arithmetic for them, so the
 * oracle takes the standard definition (the adjoint of conv2d, as aten's
 * conv_transpose2d): input x [B,IC,H,W], weight w [IC,OC/G,KH,KW] for G
 * groups, and every input element scatters into
 *   out[b, oc, ih*sH - pH + kh*dH, iw*sW - pW + kw*dW] += x[b,ic,ih,iw] * w[ic,ocl,kh,kw]
 * (positions outside the output are dropped), plus bias[oc].  With groups,
 * input channel ic only reaches the output channels of its own group
 * g = ic / (IC/G): oc = g*(OC/G) + ocl.  Output size
 * OH = (H-1)*sH - 2*pH + dH*(KH-1) + opH + 1 (opH, the output padding,
 * only adds rows at the far edge) and likewise OW. */
int64_t oracle_convt_out_size(int64_t in, int64_t k, int64_t s, int64_t p,
                              int64_t d, int64_t op) {
  return (in - 1) * s - 2 * p + d * (k - 1) + op + 1;
}

/* Full reference in the scatter form above; ref/sabs are [B,OC,OH,OW]. */
int oracle_conv_transpose2d(int64_t B, int64_t IC, int64_t H, int64_t W,
                            int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                            int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                            int64_t dW, int64_t opH, int64_t opW, int64_t G,
                            const float* x, const float* w, const float* bias,
                            double* ref, double* sabs) {
  int64_t OH = oracle_convt_out_size(H, KH, sH, pH, dH, opH);
  int64_t OW = oracle_convt_out_size(W, KW, sW, pW, dW, opW);
  if (OH <= 0 || OW <= 0 || G < 1 || IC % G || OC % G) return -1;
  int64_t icg = IC / G, ocg = OC / G;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t oc = 0; oc < OC; ++oc) {
      double* r = ref + (b * OC + oc) * OH * OW;
      double* a = sabs + (b * OC + oc) * OH * OW;
      for (int64_t o = 0; o < OH * OW; ++o) {
        r[o] = 0.0;
        a[o] = 0.0;
      }
      int64_t g = oc / ocg, ocl = oc % ocg;
      for (int64_t ic = g * icg; ic < (g + 1) * icg; ++ic)
        for (int64_t ih = 0; ih < H; ++ih)
          for (int64_t iw = 0; iw < W; ++iw) {
            double xv = (double)x[((b * IC + ic) * H + ih) * W + iw];
            for (int64_t kh = 0; kh < KH; ++kh) {
              int64_t oh = ih * sH - pH + kh * dH;
              if (oh < 0 || oh >= OH) continue;
              for (int64_t kw = 0; kw < KW; ++kw) {
                int64_t ow = iw * sW - pW + kw * dW;
                if (ow < 0 || ow >= OW) continue;
                double p = xv * (double)w[((ic * ocg + ocl) * KH + kh) * KW + kw];
                r[oh * OW + ow] += p;
                a[oh * OW + ow] += fabs(p);
              }
            }
          }
      if (bias)
        for (int64_t o = 0; o < OH * OW; ++o) r[o] += (double)bias[oc];
    }
  return 0;
}

/* Sampled reference at flat NCHW output indices, in the gather form: the
 * taps of output (oh, ow) are the (ic, kh, kw) with oh + pH - kh*dH a
 * multiple of sH whose quotient ih lies in the input (and likewise along
 * W). */
int oracle_conv_transpose2d_at(int64_t B, int64_t IC, int64_t H, int64_t W,
                               int64_t OC, int64_t KH, int64_t KW, int64_t sH,
                               int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                               int64_t dW, int64_t opH, int64_t opW, int64_t G,
                               const float* x, const float* w,
                               const float* bias, int64_t n,
                               const int64_t* idx, double* ref, double* sabs) {
  int64_t OH = oracle_convt_out_size(H, KH, sH, pH, dH, opH);
  int64_t OW = oracle_convt_out_size(W, KW, sW, pW, dW, opW);
  if (OH <= 0 || OW <= 0 || B <= 0 || G < 1 || IC % G || OC % G) return -1;
  int64_t icg = IC / G, ocg = OC / G;
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < n; ++s) {
    int64_t o = idx[s];
    int64_t ow = o % OW, oh = (o / OW) % OH, oc = (o / (OW * OH)) % OC;
    int64_t b = o / (OW * OH * OC);
    int64_t g = oc / ocg, ocl = oc % ocg;
    double acc = 0.0, aabs = 0.0;
    for (int64_t ic = g * icg; ic < (g + 1) * icg; ++ic)
      for (int64_t kh = 0; kh < KH; ++kh) {
        int64_t th = oh + pH - kh * dH;
        if (th < 0 || th % sH != 0 || th / sH >= H) continue;
        for (int64_t kw = 0; kw < KW; ++kw) {
          int64_t tw = ow + pW - kw * dW;
          if (tw < 0 || tw % sW != 0 || tw / sW >= W) continue;
          double p = (double)x[((b * IC + ic) * H + th / sH) * W + tw / sW] *
                     (double)w[((ic * ocg + ocl) * KH + kh) * KW + kw];
          acc += p;
          aabs += fabs(p);
        }
      }
    ref[s] = (bias ? (double)bias[oc] : 0.0) + acc;
    sabs[s] = aabs;
  }
  return 0;
}
