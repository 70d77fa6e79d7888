/* Host sanitizer driver for the CPU oracle (built with gcc
 * -fsanitize=address,undefined together with oracle/wgrad_ref.c by
 * tests/test_host_sanitizers.py): small random problems through the weight
 * gradient, bias gradient, forward and data-gradient oracles with per-axis
 * geometry, groups and chunked images; every buffer is sized exactly, so any
 * out-of-bounds access or undefined behaviour aborts the run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t oracle_out_size(int64_t in, int64_t k, int64_t pad, int64_t stride, int64_t dil);
int oracle_wgrad2_accumulate(int64_t nc, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
                             int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
                             int64_t dil_w, int64_t groups, const float* x, const float* dy, double* dw,
                             double* absacc, int nthreads);
int oracle_bgrad_accumulate(int64_t nc, int64_t Ho, int64_t Wo, int64_t K, const float* dy, double* db,
                            double* absacc);
int oracle_fwd(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S, int64_t pad_h,
               int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h, int64_t dil_w, int64_t groups,
               const float* x, const float* w, double* y, double* absacc, int nthreads);
int oracle_dgrad(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S, int64_t pad_h,
                 int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h, int64_t dil_w, int64_t groups,
                 const float* dy, const float* w, double* dx, double* absacc, int nthreads);

static uint64_t state = 12345;
static int64_t rnd(int64_t lo, int64_t hi) { /* inclusive */
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return lo + (int64_t)((state >> 33) % (uint64_t)(hi - lo + 1));
}
static float* randf(int64_t n) {
  float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
  for (int64_t i = 0; i < n; ++i) p[i] = (float)rnd(-8, 8);
  return p;
}

int main(void) {
  int runs = 0;
  for (int it = 0; it < 300; ++it) {
    const int64_t groups = rnd(1, 3), Cg = rnd(1, 4), Kg = rnd(1, 4);
    const int64_t C = groups * Cg, K = groups * Kg, N = rnd(1, 3), H = rnd(1, 7), W = rnd(1, 7);
    const int64_t R = rnd(1, 3), S = rnd(1, 3), ph = rnd(0, 2), pw = rnd(0, 2), sh = rnd(1, 3), sw = rnd(1, 3);
    const int64_t dh = rnd(1, 2), dw = rnd(1, 2);
    const int64_t Ho = oracle_out_size(H, R, ph, sh, dh), Wo = oracle_out_size(W, S, pw, sw, dw);
    if (Ho < 1 || Wo < 1) continue;
    float* x = randf(N * H * W * C);
    float* dy = randf(N * Ho * Wo * K);
    float* w = randf(K * R * S * Cg);
    const int64_t E = K * R * S * Cg;
    double* dwv = (double*)calloc((size_t)E, sizeof(double));
    double* a = (double*)calloc((size_t)E, sizeof(double));
    /* images in two chunks */
    const int64_t n1 = N / 2;
    if (oracle_wgrad2_accumulate(n1, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, x, dy, dwv, a, 2) ||
        oracle_wgrad2_accumulate(N - n1, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, x + n1 * H * W * C,
                                 dy + n1 * Ho * Wo * K, dwv, a, 3))
      return fprintf(stderr, "wgrad oracle rejected a valid problem\n"), 1;
    double* db = (double*)calloc((size_t)K, sizeof(double));
    double* dba = (double*)calloc((size_t)K, sizeof(double));
    if (oracle_bgrad_accumulate(N, Ho, Wo, K, dy, db, dba)) return 1;
    double* y = (double*)malloc((size_t)(N * Ho * Wo * K) * sizeof(double));
    double* ya = (double*)malloc((size_t)(N * Ho * Wo * K) * sizeof(double));
    if (oracle_fwd(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, x, w, y, ya, 2)) return 1;
    double* dx = (double*)malloc((size_t)(N * H * W * C) * sizeof(double));
    double* dxa = (double*)malloc((size_t)(N * H * W * C) * sizeof(double));
    if (oracle_dgrad(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, dy, w, dx, dxa, 2)) return 1;
    /* <dY, Y> == <dX, X> == <dW, W> exactly on integer data */
    double s1 = 0, s2 = 0, s3 = 0;
    for (int64_t i = 0; i < N * Ho * Wo * K; ++i) s1 += y[i] * dy[i];
    for (int64_t i = 0; i < N * H * W * C; ++i) s2 += dx[i] * x[i];
    for (int64_t i = 0; i < E; ++i) s3 += dwv[i] * w[i];
    if (s1 != s2 || s2 != s3) return fprintf(stderr, "adjoint identity broken: %g %g %g\n", s1, s2, s3), 1;
    free(x); free(dy); free(w); free(dwv); free(a); free(db); free(dba); free(y); free(ya); free(dx); free(dxa);
    ++runs;
  }
  /* invalid arguments are rejected, not read */
  if (oracle_fwd(1, 3, 4, 4, 2, 1, 1, 0, 0, 1, 1, 1, 1, 2, NULL, NULL, NULL, NULL, 1) != -1) return 1;
  if (oracle_dgrad(1, 4, 2, 2, 4, 5, 5, 0, 0, 1, 1, 1, 1, 1, NULL, NULL, NULL, NULL, 1) != -1) return 1;
  printf("oracle_asan: %d problems\n", runs);
  return 0;
}
