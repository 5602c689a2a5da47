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

/* Gradient of the token loop above (reverse-mode, written out by hand from
 * the four steps; the training use of the layer is [SARNAS]'s KDA-vs-Gated-
 * DeltaNet pretraining comparison).  Per head, with S_{t-1} the state before
 * token t, S'_t = diag(e_t) S_{t-1}, u_t = S'_t^T k_t, delta_t = beta_t (v_t -
 * u_t), S_t = S'_t + k_t delta_t^T, o_t = scale S_t^T q_t, and dS the
 * gradient with respect to S_t (starting from dS_T), for t = T-1 .. 0:
 *   dS      += scale q_t do_t^T                  (o_t reads S_t)
 *   dq_t     = scale S_t do_t
 *   ddelta   = dS^T k_t,   dk_t = dS delta_t      (S_t = S'_t + k delta^T)
 *   dv_t     = beta_t ddelta,  dbeta_t = ddelta . (v_t - u_t)
 *   du       = -beta_t ddelta
 *   dS'      = dS + k_t du^T,  dk_t += S'_t du    (u = S'^T k)
 *   dg_t[i]  = sum_j dS'[i,j] S'_t[i,j]           (S' = exp(g) S, row i)
 *   dS       = diag(e_t) dS'                      (gradient w.r.t. S_{t-1})
 * and dS0 = dS at the end.  States are recomputed forward from checkpoints
 * taken every BWD_BLOCK tokens, one block at a time. */
#define BWD_BLOCK 64

/* one token of the rule, S_next = diag(e) S_prev + k (beta (v - S'^T k))^T
 * (S_next may equal S_prev); pred is Dv scratch */
static void bwd_token_state(const double *S_prev, double *S_next,
                            const double *kt, const double *gt,
                            const double *vt, double bt, int64_t Dk,
                            int64_t Dv, double *pred) {
  for (int64_t i = 0; i < Dk; ++i) {
    const double f = exp(gt[i]);
    for (int64_t j = 0; j < Dv; ++j)
      S_next[i * Dv + j] = S_prev[i * Dv + j] * f;
  }
  for (int64_t j = 0; j < Dv; ++j) pred[j] = 0.0;
  for (int64_t i = 0; i < Dk; ++i)
    for (int64_t j = 0; j < Dv; ++j) pred[j] += S_next[i * Dv + j] * kt[i];
  for (int64_t j = 0; j < Dv; ++j) pred[j] = bt * (vt[j] - pred[j]);
  for (int64_t i = 0; i < Dk; ++i)
    for (int64_t j = 0; j < Dv; ++j) S_next[i * Dv + j] += kt[i] * pred[j];
}

static void backward_one_head(int64_t T, int64_t Dk, int64_t Dv, int64_t sk,
                              int64_t sv, int64_t sb, const double *q,
                              const double *k, const double *v,
                              const double *g, const double *beta,
                              const double *s0, double scale,
                              const double *dO, const double *dsT, double *dq,
                              double *dk, double *dv, double *dg,
                              double *dbeta, double *ds0, double *ckpt,
                              double *prev, double *dS, double *Sp,
                              double *vec) {
  const int64_t D2 = Dk * Dv;
  const int64_t nblk = (T + BWD_BLOCK - 1) / BWD_BLOCK;
  double *u = vec, *del = vec + Dv, *ddel = vec + 2 * Dv, *du = vec + 3 * Dv;
  double *S = Sp; /* forward scratch while checkpointing */
  if (s0)
    memcpy(S, s0, sizeof(double) * (size_t)D2);
  else
    memset(S, 0, sizeof(double) * (size_t)D2);
  /* forward: checkpoint the state before every block */
  for (int64_t t = 0; t < T; ++t) {
    if (t % BWD_BLOCK == 0)
      memcpy(ckpt + (t / BWD_BLOCK) * D2, S, sizeof(double) * (size_t)D2);
    bwd_token_state(S, S, k + t * sk, g + t * sk, v + t * sv, beta[t * sb],
                    Dk, Dv, u);
  }
  if (dsT)
    memcpy(dS, dsT, sizeof(double) * (size_t)D2);
  else
    memset(dS, 0, sizeof(double) * (size_t)D2);

  for (int64_t blk = nblk - 1; blk >= 0; --blk) {
    const int64_t t0 = blk * BWD_BLOCK;
    const int64_t t1 = (t0 + BWD_BLOCK < T) ? t0 + BWD_BLOCK : T;
    /* states before each token of the block */
    memcpy(prev, ckpt + blk * D2, sizeof(double) * (size_t)D2);
    for (int64_t t = t0; t + 1 < t1; ++t)
      bwd_token_state(prev + (t - t0) * D2, prev + (t - t0 + 1) * D2,
                      k + t * sk, g + t * sk, v + t * sv, beta[t * sb], Dk,
                      Dv, u);
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const double *P = prev + (t - t0) * D2; /* S_{t-1} */
      const double *qt = q + t * sk, *kt = k + t * sk, *gt = g + t * sk;
      const double *vt = v + t * sv, *dot = dO + t * sv;
      const double bt = beta[t * sb];
      double *dqt = dq + t * sk, *dkt = dk + t * sk, *dgt = dg + t * sk;
      double *dvt = dv + t * sv;
      /* recompute this token's forward quantities */
      for (int64_t i = 0; i < Dk; ++i) {
        const double ei = exp(gt[i]);
        for (int64_t j = 0; j < Dv; ++j) Sp[i * Dv + j] = P[i * Dv + j] * ei;
      }
      for (int64_t j = 0; j < Dv; ++j) {
        double a = 0.0;
        for (int64_t i = 0; i < Dk; ++i) a += Sp[i * Dv + j] * kt[i];
        u[j] = a;
        del[j] = bt * (vt[j] - a);
      }
      /* o_t = scale S_t^T q_t */
      for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j)
          dS[i * Dv + j] += scale * qt[i] * dot[j];
      for (int64_t i = 0; i < Dk; ++i) {
        double a = 0.0;
        for (int64_t j = 0; j < Dv; ++j)
          a += (Sp[i * Dv + j] + kt[i] * del[j]) * dot[j];
        dqt[i] = scale * a;
      }
      /* S_t = S'_t + k delta^T */
      for (int64_t j = 0; j < Dv; ++j) ddel[j] = 0.0;
      for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j) ddel[j] += dS[i * Dv + j] * kt[i];
      for (int64_t i = 0; i < Dk; ++i) {
        double a = 0.0;
        for (int64_t j = 0; j < Dv; ++j) a += dS[i * Dv + j] * del[j];
        dkt[i] = a;
      }
      /* delta = beta (v - u) */
      double db = 0.0;
      for (int64_t j = 0; j < Dv; ++j) {
        dvt[j] = bt * ddel[j];
        db += ddel[j] * (vt[j] - u[j]);
        du[j] = -bt * ddel[j];
      }
      dbeta[t * sb] = db;
      /* u = S'^T k */
      for (int64_t i = 0; i < Dk; ++i) {
        double a = 0.0;
        for (int64_t j = 0; j < Dv; ++j) {
          dS[i * Dv + j] += kt[i] * du[j];
          a += Sp[i * Dv + j] * du[j];
        }
        dkt[i] += a;
      }
      /* S' = diag(exp g) S_{t-1} */
      for (int64_t i = 0; i < Dk; ++i) {
        const double e = exp(gt[i]);
        double a = 0.0;
        for (int64_t j = 0; j < Dv; ++j) {
          a += dS[i * Dv + j] * Sp[i * Dv + j];
          dS[i * Dv + j] *= e;
        }
        dgt[i] = a;
      }
    }
  }
  if (ds0) memcpy(ds0, dS, sizeof(double) * (size_t)D2);
}

int kda_oracle_backward(int64_t B, int64_t T, int64_t H, int64_t Dk,
                        int64_t Dv, const double *q, const double *k,
                        const double *v, const double *g, const double *beta,
                        const double *s0, double scale, const double *dO,
                        const double *dsT, double *dq, double *dk, double *dv,
                        double *dg, double *dbeta, double *ds0) {
  int nthreads = 1;
  const int64_t BH = B * H, D2 = Dk * Dv;
  const int64_t nblk = (T + BWD_BLOCK - 1) / BWD_BLOCK;
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    nthreads = omp_get_num_threads();
#endif
    double *ckpt = (double *)malloc(sizeof(double) * (size_t)(nblk * D2));
    double *prev = (double *)malloc(sizeof(double) * (size_t)(BWD_BLOCK * D2));
    double *dS = (double *)malloc(sizeof(double) * (size_t)D2);
    double *Sp = (double *)malloc(sizeof(double) * (size_t)D2);
    double *vec = (double *)malloc(sizeof(double) * (size_t)(4 * Dv));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
      const int64_t b = bh / H, h = bh % H;
      const int64_t base = b * T * H + h;
      backward_one_head(T, Dk, Dv, H * Dk, H * Dv, H, q + base * Dk,
                        k + base * Dk, v + base * Dv, g + base * Dk,
                        beta + base, s0 ? s0 + bh * D2 : NULL, scale,
                        dO + base * Dv, dsT ? dsT + bh * D2 : NULL,
                        dq + base * Dk, dk + base * Dk, dv + base * Dv,
                        dg + base * Dk, dbeta + base,
                        ds0 ? ds0 + bh * D2 : NULL, ckpt, prev, dS, Sp, vec);
    }
    free(ckpt);
    free(prev);
    free(dS);
    free(Sp);
    free(vec);
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
