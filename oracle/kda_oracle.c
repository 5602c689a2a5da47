/*
 * kda_oracle.c -- plain fp64 CPU oracle for the KDA layer forward.
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h for the sources, the readings
 * taken where the pages are silent, and the layouts).  Built with
 * -O2 -fno-fast-math -ffp-contract=off so IEEE semantics hold exactly
 * (exp(-inf) == 0, no contraction into FMAs).
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [SARNAS] "What exactly changed", KDA paragraph, and [LQNN-A] AliceAIKDA
 * paragraph.  Per head, for each token t, in the order the pages describe:
 *   1. forget: each row i of the state (key channel i) is multiplied by its
 *      own coefficient exp(g[t,i])              (per-row forgetting)
 *   2. read:   u = S^T k_t, the value the state holds for key k_t
 *   3. write:  S += k_t * (beta_t * (v_t - u))^T (only the beta-scaled
 *              correction is written)
 *   4. output: o_t = scale * S^T q_t, read from the updated state. */
static void recurrence_one_head(int64_t T, int64_t Dk, int64_t Dv,
                                int64_t tok_stride_k, int64_t tok_stride_v,
                                int64_t tok_stride_b, const double *q,
                                const double *k, const double *v,
                                const double *g, const double *beta,
                                const double *s0, double scale, double *o,
                                double *s_out, double *S, double *u) {
  if (s0)
    memcpy(S, s0, sizeof(double) * (size_t)(Dk * Dv));
  else
    memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));

  for (int64_t t = 0; t < T; ++t) {
    const double *qt = q + t * tok_stride_k;
    const double *kt = k + t * tok_stride_k;
    const double *gt = g + t * tok_stride_k;
    const double *vt = v + t * tok_stride_v;
    const double bt = beta[t * tok_stride_b];
    double *ot = o + t * tok_stride_v;

    /* 1. per-row forgetting */
    for (int64_t i = 0; i < Dk; ++i) {
      const double e = exp(gt[i]);
      double *row = S + i * Dv;
      for (int64_t j = 0; j < Dv; ++j) row[j] *= e;
    }
    /* 2. prediction u = S^T k */
    for (int64_t j = 0; j < Dv; ++j) u[j] = 0.0;
    for (int64_t i = 0; i < Dk; ++i) {
      const double ki = kt[i];
      const double *row = S + i * Dv;
      for (int64_t j = 0; j < Dv; ++j) u[j] += row[j] * ki;
    }
    /* 3. write the beta-scaled correction along k */
    for (int64_t j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - u[j]);
    for (int64_t i = 0; i < Dk; ++i) {
      const double ki = kt[i];
      double *row = S + i * Dv;
      for (int64_t j = 0; j < Dv; ++j) row[j] += ki * u[j];
    }
    /* 4. read-out with the updated state */
    for (int64_t j = 0; j < Dv; ++j) ot[j] = 0.0;
    for (int64_t i = 0; i < Dk; ++i) {
      const double qi = qt[i];
      const double *row = S + i * Dv;
      for (int64_t j = 0; j < Dv; ++j) ot[j] += row[j] * qi;
    }
    for (int64_t j = 0; j < Dv; ++j) ot[j] *= scale;
  }
  if (s_out) memcpy(s_out, S, sizeof(double) * (size_t)(Dk * Dv));
}

int kda_oracle_recurrence(int64_t B, int64_t T, int64_t H, int64_t Dk,
                          int64_t Dv, const double *q, const double *k,
                          const double *v, const double *g, const double *beta,
                          const double *s0, double scale, double *o,
                          double *s_out) {
  int nthreads = 1;
  const int64_t BH = B * H;
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    nthreads = omp_get_num_threads();
#endif
    double *S = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
    double *u = (double *)malloc(sizeof(double) * (size_t)Dv);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
      const int64_t b = bh / H, h = bh % H;
      /* token t of (b, h) sits at ((b*T + t)*H + h) */
      const int64_t base = b * T * H + h;
      recurrence_one_head(T, Dk, Dv, H * Dk, H * Dv, H, q + base * Dk,
                          k + base * Dk, v + base * Dv, g + base * Dk,
                          beta + base, s0 ? s0 + bh * Dk * Dv : NULL, scale,
                          o + base * Dv, s_out ? s_out + bh * Dk * Dv : NULL,
                          S, u);
    }
    free(S);
    free(u);
  }
  return nthreads;
}

/* [LQNN-A] AliceAIKDA paragraph: q, k and v each pass a kernel-size-4 causal
 * conv whose cache is updated incrementally.  Depthwise (one filter per
 * channel), cross-correlation orientation: tap W-1 multiplies the newest
 * input; inputs before t = 0 come from the history (zeros if none). */
void kda_oracle_causal_conv(int64_t B, int64_t T, int64_t Cn, int64_t W,
                            const double *x, const double *w,
                            const double *hist, double *y, double *hist_out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t c = 0; c < Cn; ++c) {
      for (int64_t t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int64_t j = 0; j < W; ++j) {
          const int64_t tau = t - (W - 1) + j; /* time of this tap's input */
          double xv;
          if (tau >= 0)
            xv = x[(b * T + tau) * Cn + c];
          else
            xv = hist ? hist[(b * Cn + c) * (W - 1) + (W - 1) + tau] : 0.0;
          acc += w[c * W + j] * xv;
        }
        y[(b * T + t) * Cn + c] = acc;
      }
      if (hist_out) {
        /* last W-1 entries of [history ; x] */
        for (int64_t m = 0; m < W - 1; ++m) {
          const int64_t tau = T - (W - 1) + m;
          double xv;
          if (tau >= 0)
            xv = x[(b * T + tau) * Cn + c];
          else
            xv = hist ? hist[(b * Cn + c) * (W - 1) + (W - 1) + tau] : 0.0;
          hist_out[(b * Cn + c) * (W - 1) + m] = xv;
        }
      }
    }
  }
}

/* [SARNAS] "Rejected decisions": the KDA layers keep a QK normalisation.
 * Reading: L2 over each head's channels, x / sqrt(sum x^2 + eps). */
void kda_oracle_l2norm(int64_t R, int64_t H, int64_t D, double eps,
                       double *x) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t h = 0; h < H; ++h) {
      double *p = x + (r * H + h) * D;
      double ss = 0.0;
      for (int64_t i = 0; i < D; ++i) ss += p[i] * p[i];
      const double inv = 1.0 / sqrt(ss + eps);
      for (int64_t i = 0; i < D; ++i) p[i] *= inv;
    }
  }
}
