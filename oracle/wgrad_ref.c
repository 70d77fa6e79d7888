/*
 * Convolution weight-gradient oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU library never links or calls it,
 * and it shares no source, header or table with the GPU library.
 *
 * What it computes: the weight gradient of a 2-D convolution ("weight.grad"
 * of nn.Conv2d, as in rocm-libraries PR #11188, "fix silent zero wgrad",
 * section Motivation) over NHWC tensors with groups:
 *
 *   dW[k, r, s, c] = sum over n, ho, wo of
 *       dY[n, ho, wo, k] * Xpad[n, ho*stride + r*dil - pad,
 *                                  wo*stride + s*dil - pad, g(k)*Cg + c]
 *
 *   Cg = C / groups, Kg = K / groups, g(k) = k / Kg,
 *   Xpad = X inside [0,H) x [0,W) and 0 outside (zero padding, same pad on
 *   all four sides),
 *   Ho = (H + 2*pad - dil*(R-1) - 1) / stride + 1, Wo likewise.
 *
 * Every product of two fp32 (or bf16/fp16 widened to fp32) values is exact in
 * fp64, and the sum is accumulated in fp64.  Alongside dW the oracle
 * accumulates A[k,r,s,c] = sum |dY| * |Xpad| over the same terms; the
 * largest A is the denominator of the normalised error metric.
 *
 * This is the plain definition written out as loops: no blocking, no
 * reordering beyond splitting the (n, ho) rows over threads.  Each thread
 * owns a private fp64 copy of dW and A; the copies are added in thread-index
 * order, so the result is deterministic for a given thread count.
 *
 * The "accumulate" form adds the contribution of a chunk of images to dW and
 * A, so very large batches can be streamed through bounded host memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Output extent of one spatial axis (textbook floor formula). */
int64_t oracle_out_size(int64_t in, int64_t k, int64_t pad, int64_t stride, int64_t dil) {
  int64_t span = in + 2 * pad - dil * (k - 1) - 1;
  if (span < 0) return 0;
  return span / stride + 1;
}

/*
 * Add the contribution of nc images to dw and absacc (both [K][R][S][Cg],
 * fp64, row-major) for per-axis geometry: rows use (pad_h, stride_h, dil_h),
 * columns (pad_w, stride_w, dil_w), i.e.
 *
 *   dW[k, r, s, c] += dY[n, ho, wo, k]
 *                     * Xpad[n, ho*stride_h + r*dil_h - pad_h, wo*stride_w + s*dil_w - pad_w, g(k)*Cg + c]
 *
 * with Ho from (H, R, pad_h, stride_h, dil_h) and Wo from (W, S, pad_w,
 * stride_w, dil_w).  Per-axis padding is the pad_w of rocm-libraries PR
 * #14393's embedded depthwise-dgrad PR #14386 (section "Per-axis padding"),
 * where the column padding may differ from the row padding and Wo uses it.
 * x is [nc][H][W][C], dy is [nc][Ho][Wo][K], both fp32.
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_wgrad2_accumulate(int64_t nc, int64_t C, int64_t H, int64_t W, int64_t K,
                             int64_t R, int64_t S, int64_t pad_h, int64_t pad_w, int64_t stride_h,
                             int64_t stride_w, int64_t dil_h, int64_t dil_w, int64_t groups,
                             const float* x, const float* dy, double* dw, double* absacc,
                             int nthreads) {
  if (nc < 0 || C < 1 || H < 1 || W < 1 || K < 1 || R < 1 || S < 1 || pad_h < 0 || pad_w < 0 ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || groups < 1 || C % groups != 0 ||
      K % groups != 0)
    return -1;
  const int64_t Ho = oracle_out_size(H, R, pad_h, stride_h, dil_h);
  const int64_t Wo = oracle_out_size(W, S, pad_w, stride_w, dil_w);
  if (Ho < 1 || Wo < 1) return -1;
  const int64_t Cg = C / groups, Kg = K / groups;
  const int64_t E = K * R * S * Cg;
  if (nc == 0) return 0;
  if (nthreads < 1) nthreads = 1;

  const int64_t rows = nc * Ho; /* one row = one (n, ho) pair */
  double* priv = (double*)calloc((size_t)(2 * E * nthreads), sizeof(double));
  if (!priv) return -2;

#pragma omp parallel num_threads(nthreads)
  {
    int t = 0, T = 1;
#ifdef _OPENMP
    t = omp_get_thread_num();
    T = omp_get_num_threads();
#endif
    double* my_dw = priv + (int64_t)t * 2 * E;
    double* my_abs = my_dw + E;
    const int64_t row_lo = rows * t / T, row_hi = rows * (t + 1) / T;
    for (int64_t row = row_lo; row < row_hi; ++row) {
      const int64_t n = row / Ho, ho = row % Ho;
      for (int64_t wo = 0; wo < Wo; ++wo) {
        const float* dy_px = dy + ((n * Ho + ho) * Wo + wo) * K;
        for (int64_t k = 0; k < K; ++k) {
          const double g = (double)dy_px[k];
          const int64_t grp = k / Kg;
          for (int64_t r = 0; r < R; ++r) {
            const int64_t h = ho * stride_h + r * dil_h - pad_h;
            if (h < 0 || h >= H) continue; /* zero padding */
            for (int64_t s = 0; s < S; ++s) {
              const int64_t w = wo * stride_w + s * dil_w - pad_w;
              if (w < 0 || w >= W) continue; /* zero padding */
              const float* x_px = x + ((n * H + h) * W + w) * C + grp * Cg;
              double* d = my_dw + ((k * R + r) * S + s) * Cg;
              double* a = my_abs + ((k * R + r) * S + s) * Cg;
              for (int64_t c = 0; c < Cg; ++c) {
                const double v = (double)x_px[c];
                d[c] += g * v;
                a[c] += fabs(g) * fabs(v);
              }
            }
          }
        }
      }
    }
  }
  /* Fold the per-thread copies in ascending thread order. */
  for (int t = 0; t < nthreads; ++t) {
    const double* p = priv + (int64_t)t * 2 * E;
    for (int64_t e = 0; e < E; ++e) {
      dw[e] += p[e];
      absacc[e] += p[E + e];
    }
  }
  free(priv);
  return 0;
}

/* The same geometry on both axes (one pad, stride and dilation). */
int oracle_wgrad_accumulate(int64_t nc, int64_t C, int64_t H, int64_t W, int64_t K,
                            int64_t R, int64_t S, int64_t pad, int64_t stride, int64_t dil,
                            int64_t groups, const float* x, const float* dy, double* dw,
                            double* absacc, int nthreads) {
  return oracle_wgrad2_accumulate(nc, C, H, W, K, R, S, pad, pad, stride, stride, dil, dil, groups,
                                  x, dy, dw, absacc, nthreads);
}

/*
 * Bias gradient (the "bias.grad" beside weight.grad of nn.Conv2d in
 * rocm-libraries PR #11188, section Motivation): the output gradient summed
 * over every output pixel,
 *
 *   db[k] = sum over n, ho, wo of dY[n, ho, wo, k],
 *
 * added for nc images into db and, as its error denominator, the sum of
 * |dY[n, ho, wo, k]| into absacc (both [K], fp64).  dy is [nc][Ho][Wo][K]
 * fp32; the sum runs in pixel order, in fp64.  Returns 0, or -1 on invalid
 * arguments.
 */
int oracle_bgrad_accumulate(int64_t nc, int64_t Ho, int64_t Wo, int64_t K, const float* dy,
                            double* db, double* absacc) {
  if (nc < 0 || Ho < 1 || Wo < 1 || K < 1) return -1;
  const int64_t pixels = nc * Ho * Wo;
  for (int64_t l = 0; l < pixels; ++l) {
    const float* g = dy + l * K;
    for (int64_t k = 0; k < K; ++k) {
      db[k] += (double)g[k];
      absacc[k] += fabs((double)g[k]);
    }
  }
  return 0;
}

/*
 * Forward convolution (the other direction on the same implicit-GEMM and
 * split-K machinery, rocm-libraries PR #14393 "split-K forward implicit-GEMM
 * convolution on gfx1250", section Summary), per-axis geometry:
 *
 *   Y[n, ho, wo, k] = sum over r, s, c of
 *       Xpad[n, ho*stride_h + r*dil_h - pad_h, wo*stride_w + s*dil_w - pad_w, g(k)*Cg + c]
 *       * Wt[k, r, s, c]
 *
 * x is [N][H][W][C], w is [K][R][S][Cg] (fp32 values), y and absacc are
 * [N][Ho][Wo][K] fp64 (overwritten); absacc holds the same sum of |Xpad|*|Wt|,
 * whose largest element is the normalised-error denominator.  Output rows
 * (n, ho) are split over threads; every output element is one thread's own
 * fp64 sum in (r, s, c) order.  Returns 0, or -1 on invalid arguments.
 */
int oracle_fwd(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
               int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
               int64_t dil_w, int64_t groups, const float* x, const float* w, double* y,
               double* absacc, int nthreads) {
  if (N < 1 || C < 1 || H < 1 || W < 1 || K < 1 || R < 1 || S < 1 || pad_h < 0 || pad_w < 0 ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || groups < 1 || C % groups != 0 ||
      K % groups != 0)
    return -1;
  const int64_t Ho = oracle_out_size(H, R, pad_h, stride_h, dil_h);
  const int64_t Wo = oracle_out_size(W, S, pad_w, stride_w, dil_w);
  if (Ho < 1 || Wo < 1) return -1;
  const int64_t Cg = C / groups, Kg = K / groups;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t row = 0; row < N * Ho; ++row) {
    const int64_t n = row / Ho, ho = row % Ho;
    for (int64_t wo = 0; wo < Wo; ++wo) {
      for (int64_t k = 0; k < K; ++k) {
        const int64_t grp = k / Kg;
        double acc = 0.0, aacc = 0.0;
        for (int64_t r = 0; r < R; ++r) {
          const int64_t h = ho * stride_h + r * dil_h - pad_h;
          if (h < 0 || h >= H) continue; /* zero padding */
          for (int64_t s = 0; s < S; ++s) {
            const int64_t ww = wo * stride_w + s * dil_w - pad_w;
            if (ww < 0 || ww >= W) continue; /* zero padding */
            const float* xp = x + ((n * H + h) * W + ww) * C + grp * Cg;
            const float* wp = w + ((k * R + r) * S + s) * Cg;
            for (int64_t c = 0; c < Cg; ++c) {
              acc += (double)xp[c] * (double)wp[c];
              aacc += fabs((double)xp[c]) * fabs((double)wp[c]);
            }
          }
        }
        y[((n * Ho + ho) * Wo + wo) * K + k] = acc;
        absacc[((n * Ho + ho) * Wo + wo) * K + k] = aacc;
      }
    }
  }
  return 0;
}

/*
 * Data gradient (dgrad, the input gradient of the same convolution; the
 * pages' third direction beside wgrad and forward, rocm-libraries PR #14393,
 * section "Auto-deduced degree": "as it does for wgrad and dgrad"), written as
 * the scatter that transposes the forward sum: every term of
 *   Y[n, ho, wo, k] += Xpad[n, h, w, g(k)*Cg + c] * Wt[k, r, s, c]
 * (h = ho*stride_h + r*dil_h - pad_h, w = wo*stride_w + s*dil_w - pad_w, inside
 * the image) sends dY[n, ho, wo, k] * Wt[k, r, s, c] to dX[n, h, w, g(k)*Cg + c]:
 *
 *   dX[n, h, w, g*Cg + c] = sum over (k in group g, r, s, ho, wo) with
 *       ho*stride_h + r*dil_h - pad_h == h and wo*stride_w + s*dil_w - pad_w == w
 *       of dY[n, ho, wo, k] * Wt[k, r, s, c].
 *
 * dy is [N][Ho][Wo][K], w is [K][R][S][Cg] (fp32 values); dx and absacc are
 * [N][H][W][C] fp64 (overwritten; absacc is the sum of |dY|*|Wt|).  Images are
 * split over threads (each image's dX is written by one thread), and within an
 * image the terms are added in (ho, wo, k, r, s, c) order.  Returns 0, or -1
 * on invalid arguments.
 */
int oracle_dgrad(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
                 int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h,
                 int64_t dil_w, int64_t groups, const float* dy, const float* w, double* dx,
                 double* absacc, int nthreads) {
  if (N < 1 || C < 1 || H < 1 || W < 1 || K < 1 || R < 1 || S < 1 || pad_h < 0 || pad_w < 0 ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || groups < 1 || C % groups != 0 ||
      K % groups != 0)
    return -1;
  const int64_t Ho = oracle_out_size(H, R, pad_h, stride_h, dil_h);
  const int64_t Wo = oracle_out_size(W, S, pad_w, stride_w, dil_w);
  if (Ho < 1 || Wo < 1) return -1;
  const int64_t Cg = C / groups, Kg = K / groups;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double* dxn = dx + n * H * W * C;
    double* an = absacc + n * H * W * C;
    for (int64_t i = 0; i < H * W * C; ++i) {
      dxn[i] = 0.0;
      an[i] = 0.0;
    }
    for (int64_t ho = 0; ho < Ho; ++ho) {
      for (int64_t wo = 0; wo < Wo; ++wo) {
        const float* g = dy + ((n * Ho + ho) * Wo + wo) * K;
        for (int64_t k = 0; k < K; ++k) {
          const double gv = (double)g[k];
          const int64_t grp = k / Kg;
          for (int64_t r = 0; r < R; ++r) {
            const int64_t hi = ho * stride_h + r * dil_h - pad_h;
            if (hi < 0 || hi >= H) continue; /* the term multiplies a padding zero */
            for (int64_t s = 0; s < S; ++s) {
              const int64_t wi = wo * stride_w + s * dil_w - pad_w;
              if (wi < 0 || wi >= W) continue;
              const float* wq = w + ((k * R + r) * S + s) * Cg;
              double* d = dxn + (hi * W + wi) * C + grp * Cg;
              double* a = an + (hi * W + wi) * C + grp * Cg;
              for (int64_t c = 0; c < Cg; ++c) {
                d[c] += gv * (double)wq[c];
                a[c] += fabs(gv) * fabs((double)wq[c]);
              }
            }
          }
        }
      }
    }
  }
  return 0;
}

/* Number of threads the OpenMP runtime would give a parallel region. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
