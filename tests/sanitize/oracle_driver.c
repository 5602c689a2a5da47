/* Runs every entry point of the fp64 oracle (oracle/kda_oracle.c) on small
 * drawn inputs, including -inf gates, one-token sequences, beta up to 2,
 * d_k != d_v and sequences longer than the backward's recompute blocks.
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py; any out-of-bounds access, leak or undefined
 * operation aborts the run.  Exit status 0 = clean and all results finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "kda_oracle.h"

static uint64_t rs = 88172645463325252ull;
static double unif(void) { /* xorshift64, uniform in (0, 1) */
  rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
  return ((rs >> 11) + 0.5) / 9007199254740992.0;
}
static double normal(void) {
  return sqrt(-2.0 * log(unif())) * cos(6.283185307179586 * unif());
}
static double *draw(size_t n, double sc) {
  double *p = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = sc * normal();
  return p;
}
static int finite_all(const double *p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
               int forget, double bmax, int with_s0) {
  const size_t nk = (size_t)B * T * H * Dk, nv = (size_t)B * T * H * Dv,
               nb = (size_t)B * T * H, ns = (size_t)B * H * Dk * Dv;
  double *q = draw(nk, 0.3), *k = draw(nk, 0.3), *v = draw(nv, 1.0),
         *g = draw(nk, 1.0), *beta = draw(nb, 1.0), *s0 = draw(ns, 0.1),
         *dO = draw(nv, 1.0), *dsT = draw(ns, 1.0);
  for (size_t i = 0; i < nk; ++i) g[i] = -log1p(exp(g[i]));
  for (size_t i = 0; i < nb; ++i) beta[i] = bmax / (1.0 + exp(-beta[i]));
  if (forget && T > 2) {
    for (int64_t i = 0; i < Dk; ++i) g[(size_t)(T / 2) * H * Dk + i] = -INFINITY;
    g[(size_t)(T - 1) * H * Dk] = -INFINITY;
  }
  double *o = malloc(nv * sizeof(double)), *sT = malloc(ns * sizeof(double));
  kda_oracle_recurrence(B, T, H, Dk, Dv, q, k, v, g, beta, with_s0 ? s0 : NULL,
                        0.9, o, sT);
  int ok = finite_all(o, nv) && finite_all(sT, ns);
  double *dq = malloc(nk * sizeof(double)), *dk = malloc(nk * sizeof(double)),
         *dv = malloc(nv * sizeof(double)), *dg = malloc(nk * sizeof(double)),
         *db = malloc(nb * sizeof(double)), *ds0 = malloc(ns * sizeof(double));
  kda_oracle_backward(B, T, H, Dk, Dv, q, k, v, g, beta, with_s0 ? s0 : NULL,
                      0.9, dO, dsT, dq, dk, dv, dg, db, ds0);
  ok = ok && finite_all(dq, nk) && finite_all(dk, nk) && finite_all(dv, nv) &&
       finite_all(db, nb) && finite_all(ds0, ns);
  /* conv over H*Dk channels with and without a history, and the L2 norm */
  const int64_t Cn = H * Dk, W = 4;
  double *x = draw((size_t)B * T * Cn, 1.0), *w = draw((size_t)Cn * W, 0.5),
         *hist = draw((size_t)B * Cn * (W - 1), 1.0);
  double *y = malloc((size_t)B * T * Cn * sizeof(double)),
         *ho = malloc((size_t)B * Cn * (W - 1) * sizeof(double));
  kda_oracle_causal_conv(B, T, Cn, W, x, w, NULL, y, ho);
  kda_oracle_causal_conv(B, T, Cn, W, x, w, hist, y, ho);
  kda_oracle_l2norm(B * T, H, Dk, 1e-6, y);
  ok = ok && finite_all(y, (size_t)B * T * Cn) &&
       finite_all(ho, (size_t)B * Cn * (W - 1));
  free(q); free(k); free(v); free(g); free(beta); free(s0); free(dO);
  free(dsT); free(o); free(sT); free(dq); free(dk); free(dv); free(dg);
  free(db); free(ds0); free(x); free(w); free(hist); free(y); free(ho);
  return ok;
}

int main(void) {
  int ok = 1;
  ok &= run(1, 1, 1, 3, 2, 0, 1.0, 0);
  ok &= run(2, 9, 3, 4, 5, 1, 2.0, 1);
  ok &= run(1, 150, 2, 8, 6, 1, 1.0, 1);
  ok &= run(2, 65, 1, 16, 16, 0, 2.0, 0);
  printf("oracle under sanitizers: %s\n", ok ? "clean" : "non-finite output");
  return ok ? 0 : 1;
}
