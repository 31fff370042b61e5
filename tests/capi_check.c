/*
 * capi_check.c -- libbaim.so driven from plain C: no Python, no torch.
 *
 * Device memory comes from the HIP runtime; the expected values come from
 * the fp64 oracle (liboracle.so, test infrastructure).  Each entry point of
 * include/baim.h runs once on seeded inputs and is compared element by
 * element with the oracle within the bounds the Python parity tests use:
 * |out - ref| <= 4e-6*sqrt(K)*(|alpha|*sabs + |beta*self|) for the GEMM
 * ops, |out - ref| <= 4e-6*err for attention.  A few invalid calls check
 * that the status codes and baim_last_error() reach a C caller.  Prints
 * "capi_check OK" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "baim.h"

/* the oracle's C entry points (oracle/oracle.c) */
void oracle_addmm(int64_t M, int64_t N, int64_t K, const float* mat1, const float* mat2,
                  const float* self, int self_2d, float beta, float alpha, double* ref,
                  double* sabs);
void oracle_linear(int64_t M, int64_t N, int64_t K, const float* x, const float* w,
                   const float* bias, double* ref, double* sabs);
int oracle_conv2d(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC, int64_t KH,
                  int64_t KW, int64_t sH, int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                  int64_t dW, const float* x, const float* w, const float* bias, double* ref,
                  double* sabs);
int oracle_conv2d_nhwc(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC, int64_t KH,
                       int64_t KW, int64_t sH, int64_t sW, int64_t pH, int64_t pW, int64_t dH,
                       int64_t dW, const float* x, const float* w, const float* bias,
                       double* ref, double* sabs);
int oracle_conv_transpose2d(int64_t B, int64_t IC, int64_t H, int64_t W, int64_t OC,
                            int64_t KH, int64_t KW, int64_t sH, int64_t sW, int64_t pH,
                            int64_t pW, int64_t dH, int64_t dW, int64_t opH, int64_t opW,
                            int64_t groups, const float* x, const float* w, const float* bias,
                            double* ref, double* sabs);
int oracle_sdpa(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const float* q, const float* k,
                const float* v, const float* mask, float scale, double* out, double* err);

static int failures = 0;

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(2);                                                             \
    }                                                                      \
  } while (0)

/* seeded uniform(-1, 1) values (a 64-bit linear congruential generator) */
static uint64_t lcg_state;
static float* host_rand(size_t n, uint64_t seed) {
  float* p = (float*)malloc(n * sizeof(float) + 1);
  lcg_state = seed * 6364136223846793005ull + 1442695040888963407ull;
  for (size_t i = 0; i < n; ++i) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    p[i] = (float)((double)(lcg_state >> 40) / (double)(1ull << 24) * 2.0 - 1.0);
  }
  return p;
}

static float* to_device(const float* h, size_t n) {
  float* d = NULL;
  HIP_OK(hipMalloc((void**)&d, n * sizeof(float) + 16));
  HIP_OK(hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice));
  return d;
}

static float* from_device(const float* d, size_t n) {
  float* h = (float*)malloc(n * sizeof(float) + 1);
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h, d, n * sizeof(float), hipMemcpyDeviceToHost));
  return h;
}

/* |out - ref| <= c * scale elementwise */
static void compare(const char* what, const float* out, const double* ref, const double* scale,
                    const double* extra, double c, size_t n) {
  size_t bad = 0;
  double worst = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double tol = c * (scale[i] + (extra ? extra[i] : 0.0));
    const double err = fabs((double)out[i] - ref[i]);
    if (!(err <= tol)) ++bad;
    if (tol > 0 && err / tol > worst) worst = err / tol;
  }
  printf("%-28s %8zu outputs, max err/tol %.3g%s\n", what, n, worst, bad ? "  FAILED" : "");
  if (bad) ++failures;
}

static void check_status(const char* what, baim_status got, baim_status want) {
  const char* msg = baim_last_error();
  const int ok = got == want && (want == BAIM_OK || (msg && msg[0]));
  printf("%-28s status %d (want %d) \"%s\"%s\n", what, (int)got, (int)want, msg ? msg : "",
         ok ? "" : "  FAILED");
  if (!ok) ++failures;
}

static void test_addmm(void) {
  const int64_t M = 130, K = 300, N = 257;
  float* a = host_rand(M * K, 1);
  float* b = host_rand(K * N, 2);
  float* s = host_rand(M * N, 3);
  float *da = to_device(a, M * K), *db = to_device(b, K * N), *ds = to_device(s, M * N);
  float* dout = to_device(s, M * N);
  double* ref = (double*)malloc(M * N * sizeof(double));
  double* sabs = (double*)malloc(M * N * sizeof(double));
  double* selfabs = (double*)malloc(M * N * sizeof(double));
  for (int self_2d = 0; self_2d <= 1; ++self_2d) {
    const float beta = 0.5f, alpha = 2.0f;
    check_status("addmm_f32 launch", addmm_f32(dout, ds, self_2d, da, db, M, N, K, beta, alpha, NULL),
                 BAIM_OK);
    float* out = from_device(dout, M * N);
    oracle_addmm(M, N, K, a, b, s, self_2d, beta, alpha, ref, sabs);
    for (int64_t i = 0; i < M; ++i)
      for (int64_t j = 0; j < N; ++j) {
        sabs[i * N + j] *= fabs(alpha);
        selfabs[i * N + j] = fabs(beta * (double)(self_2d ? s[i * N + j] : s[j]));
      }
    compare(self_2d ? "addmm_f32 self [M,N]" : "addmm_f32 self [N]", out, ref, sabs, selfabs,
            4e-6 * sqrt((double)K), (size_t)(M * N));
    free(out);
  }
  /* linear: x [M,K] @ w[N,K]^T + bias, reusing a as x and the first N*K of b as w */
  check_status("linear_f32 launch", linear_f32(dout, da, db, ds, M, N, K, NULL), BAIM_OK);
  float* out = from_device(dout, M * N);
  oracle_linear(M, N, K, a, b, s, ref, sabs);
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) selfabs[i * N + j] = fabs((double)s[j]);
  compare("linear_f32", out, ref, sabs, selfabs, 4e-6 * sqrt((double)K), (size_t)(M * N));
  free(out);
  /* invalid calls reach C callers as statuses */
  check_status("addmm_f32 K < 0", addmm_f32(dout, ds, 0, da, db, M, N, -1, 1.0f, 1.0f, NULL),
               BAIM_ERR_SHAPE);
  check_status("addmm_f32 out aliases mat1",
               addmm_f32(da, ds, 0, da, db, M, N, K, 1.0f, 1.0f, NULL), BAIM_ERR_ALIAS);
  hipFree(da), hipFree(db), hipFree(ds), hipFree(dout);
  free(a), free(b), free(s), free(ref), free(sabs), free(selfabs);
}

static void test_convs(void) {
  const int64_t B = 2, IC = 16, H = 19, W = 17, OC = 40, KH = 3, KW = 3;
  const int64_t sH = 2, sW = 1, pH = 1, pW = 2, dH = 1, dW = 2;
  int64_t OH = 0, OW = 0;
  check_status("baim_conv2d_out_hw", baim_conv2d_out_hw(H, W, KH, KW, sH, sW, pH, pW, dH, dW, &OH, &OW),
               BAIM_OK);
  const int64_t nx = B * IC * H * W, nw = OC * IC * KH * KW, no = B * OC * OH * OW;
  float *x = host_rand(nx, 4), *w = host_rand(nw, 5), *bias = host_rand(OC, 6);
  float *dx = to_device(x, nx), *dw = to_device(w, nw), *dbias = to_device(bias, OC);
  float* dout = NULL;
  HIP_OK(hipMalloc((void**)&dout, (no > 4096 ? no : 4096) * sizeof(float) * 4));
  double* ref = (double*)calloc(4 * no, sizeof(double));
  double* sabs = (double*)calloc(4 * no, sizeof(double));
  double* babs = (double*)calloc(4 * no, sizeof(double));
  /* NCHW */
  check_status("conv2d_gemm_f32 launch",
               conv2d_gemm_f32(dout, dx, dw, dbias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH,
                               dW, 1, NULL), BAIM_OK);
  float* out = from_device(dout, no);
  oracle_conv2d(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, x, w, bias, ref, sabs);
  for (int64_t i = 0; i < no; ++i) babs[i] = fabs((double)bias[(i / (OH * OW)) % OC]);
  compare("conv2d_gemm_f32", out, ref, sabs, babs, 4e-6 * sqrt((double)(IC * KH * KW)), no);
  free(out);
  /* channels-last, on the same numbers read as [B,H,W,IC] and [OC,KH,KW,IC] */
  check_status("conv2d_nhwc_f32 launch",
               conv2d_nhwc_f32(dout, dx, dw, dbias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH,
                               dW, NULL), BAIM_OK);
  out = from_device(dout, no);
  oracle_conv2d_nhwc(B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, x, w, bias, ref, sabs);
  for (int64_t i = 0; i < no; ++i) babs[i] = fabs((double)bias[i % OC]);
  compare("conv2d_nhwc_f32", out, ref, sabs, babs, 4e-6 * sqrt((double)(IC * KH * KW)), no);
  free(out);
  /* transposed: weight [IC, OC, KH, KW] (the same numbers), stride 2, output padding 1 */
  int64_t TH = 0, TW = 0;
  check_status("baim_conv_transpose2d_out_hw",
               baim_conv_transpose2d_out_hw(H, W, KH, KW, 2, 2, 1, 1, 1, 1, 1, 1, &TH, &TW), BAIM_OK);
  const int64_t nt = B * OC * TH * TW;
  float* dtout = NULL;
  HIP_OK(hipMalloc((void**)&dtout, nt * sizeof(float)));
  double* tref = (double*)malloc(nt * sizeof(double));
  double* tsabs = (double*)malloc(nt * sizeof(double));
  double* tbabs = (double*)malloc(nt * sizeof(double));
  check_status("conv_transpose2d_f32 launch",
               conv_transpose2d_f32(dtout, dx, dw, dbias, B, IC, H, W, OC, KH, KW, 2, 2, 1, 1, 1,
                                    1, 1, 1, 1, NULL), BAIM_OK);
  out = from_device(dtout, nt);
  oracle_conv_transpose2d(B, IC, H, W, OC, KH, KW, 2, 2, 1, 1, 1, 1, 1, 1, 1, x, w, bias, tref,
                          tsabs);
  for (int64_t i = 0; i < nt; ++i) tbabs[i] = fabs((double)bias[(i / (TH * TW)) % OC]);
  compare("conv_transpose2d_f32", out, tref, tsabs, tbabs, 4e-6 * sqrt((double)(IC * KH * KW)), nt);
  free(out);
  check_status("conv2d_gemm_f32 groups=3",
               conv2d_gemm_f32(dout, dx, dw, dbias, B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH,
                               dW, 3, NULL), BAIM_ERR_SHAPE);
  hipFree(dx), hipFree(dw), hipFree(dbias), hipFree(dout), hipFree(dtout);
  free(x), free(w), free(bias), free(ref), free(sabs), free(babs), free(tref), free(tsabs),
      free(tbabs);
}

static void test_sdpa(void) {
  const int64_t BH = 6, Sq = 70, Skv = 133, D = 64;
  float *q = host_rand(BH * Sq * D, 7), *k = host_rand(BH * Skv * D, 8), *v = host_rand(BH * Skv * D, 9);
  float* mask = host_rand(BH * Sq * Skv, 10);
  float *dq = to_device(q, BH * Sq * D), *dk = to_device(k, BH * Skv * D), *dv = to_device(v, BH * Skv * D);
  float* dm = to_device(mask, BH * Sq * Skv);
  float* dout = NULL;
  HIP_OK(hipMalloc((void**)&dout, BH * Sq * D * sizeof(float)));
  double* ref = (double*)malloc(BH * Sq * D * sizeof(double));
  double* err = (double*)malloc(BH * Sq * D * sizeof(double));
  check_status("sdpa_f32 launch", sdpa_f32(dout, dq, dk, dv, dm, BH, Sq, Skv, D, NULL, NULL), BAIM_OK);
  float* out = from_device(dout, BH * Sq * D);
  oracle_sdpa(BH, Sq, Skv, D, q, k, v, mask, (float)(1.0 / sqrt((double)D)), ref, err);
  compare("sdpa_f32", out, ref, err, NULL, 4e-6, (size_t)(BH * Sq * D));
  free(out);
  check_status("sdpa_f32 D=6", sdpa_f32(dout, dq, dk, dv, dm, BH, Sq, Skv, 6, NULL, NULL),
               BAIM_ERR_UNSUPPORTED);
  hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dm), hipFree(dout);
  free(q), free(k), free(v), free(mask), free(ref), free(err);
}

/* The host-only plan queries: the stem shape takes the stem kernel in both
 * layouts, a NULL output pointer is refused. */
static void test_plans(void) {
  int bm = 0, bn = 0, bk = 0, waves = 0, kg = 0, splits = 0, sb = 0, kernel = -1;
  check_status("baim_gemm_plan",
               baim_gemm_plan(4096, 1024, 4096, &bm, &bn, &bk, &waves, &kg, &splits, &sb),
               BAIM_OK);
  if (bm < 32 || bn < 32 || waves < 4) {
    printf("FAIL baim_gemm_plan: %d x %d, %d waves\n", bm, bn, waves);
    ++failures;
  }
  check_status("baim_conv2d_plan",
               baim_conv2d_plan(1, 3, 768, 768, 128, 7, 7, 4, 4, 3, 3, 1, 1, 1, &kernel, &bm, &bn,
                                &bk, &waves, &kg, &splits, &sb),
               BAIM_OK);
  if (kernel != 3) {
    printf("FAIL baim_conv2d_plan: stem shape planned on kernel %d\n", kernel);
    ++failures;
  }
  kernel = -1;
  check_status("baim_conv2d_nhwc_plan",
               baim_conv2d_nhwc_plan(1, 3, 768, 768, 128, 7, 7, 4, 4, 3, 3, 1, 1, &kernel), BAIM_OK);
  if (kernel != 3) {
    printf("FAIL baim_conv2d_nhwc_plan: stem shape planned on kernel %d\n", kernel);
    ++failures;
  }
  check_status("baim_conv2d_nhwc_plan NULL",
               baim_conv2d_nhwc_plan(1, 3, 768, 768, 128, 7, 7, 4, 4, 3, 3, 1, 1, NULL),
               BAIM_ERR_NULL);
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    printf("capi_check: no GPU\n");
    return 3;
  }
  printf("libbaim version %d\n", baim_version());
  test_addmm();
  test_convs();
  test_sdpa();
  test_plans();
  if (failures) {
    printf("capi_check: %d FAILED\n", failures);
    return 1;
  }
  printf("capi_check OK\n");
  return 0;
}
