/*
 * kda_oracle.h -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * layer forward.  TEST INFRASTRUCTURE ONLY: it exists so that tests, the
 * smoke check and the benchmark's CPU-baseline leg can check and time the HIP
 * library against an obviously correct, slow definition.  Nothing in the
 * product path (gated_delta_rule_74_amd/) includes, links or calls this code,
 * and this code includes nothing from there.
 *
 * Sources (web pages; cited by title and section):
 *  [SARNAS]  sarnas.ru blog, "Yandex opened the weights of
 *            AliceAI-Foundation-80B-A3B-Base: an MoE model trained from
 *            scratch" (Russian) -- section "What exactly changed", the KDA
 *            paragraph: a fixed-size state; reading the value stored for the
 *            new key, comparing it with the new value and writing only the
 *            difference; a separate forgetting coefficient for each row of
 *            the state matrix.  Section "Rejected decisions": QK
 *            normalisation exists in the KDA layers.
 *  [LQNN-A]  m.lqnn.cn news 205170, "two deep teardowns in two days ... who
 *            cracked the technical code of Yandex's new model first"
 *            (Chinese) -- the paragraph walking through the AliceAIKDA
 *            module: kernel-4 causal conv on q/k/v with an incrementally
 *            updated cache, the delta-rule loop that multiplies the state by
 *            exp(gate) and adds the delta, delta = prediction residual times
 *            sigmoid(beta); beta limited to (0,1) when negative eigenvalues
 *            are not allowed; conv kernel dim validated >= 2.
 *  [LQNN-B]  m.lqnn.cn news 255115, "80B parameters for 3B of compute ...
 *            check these three places before fine-tuning" (Chinese) -- the
 *            config-validation list: conv kernel >= 2, chunk size positive.
 *
 * Readings where the pages are silent:
 *  - the prediction is read from the already-decayed state;
 *  - the output is read from the updated state, o_t = scale * S_t^T q_t;
 *  - "row" of the state = key channel, so g_t in R^{Dk} scales rows;
 *  - conv tap width-1 multiplies the newest input, no bias, no activation;
 *  - L2 norm is x / sqrt(sum x^2 + eps), per head, on q and k only.
 *
 * Layouts (all contiguous, row-major, fp64):
 *   q, k, g : [B, T, H, Dk]      v, o : [B, T, H, Dv]      beta : [B, T, H]
 *   state   : [B, H, Dk, Dv]  (row i = key channel i)
 *   conv x  : [B, T, Cn]   taps w : [Cn, W]   conv state : [B, Cn, W-1]
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * against closed forms, invariants, library routines and a dense unrolled
 * form; none is "parity unpinned".
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Token-by-token KDA recurrence.  s0 may be NULL (zero initial state); s_out
 * may be NULL (final state not wanted).  Returns the number of OpenMP threads
 * that ran it. */
int kda_oracle_recurrence(int64_t B, int64_t T, int64_t H, int64_t Dk,
                          int64_t Dv, const double *q, const double *k,
                          const double *v, const double *g, const double *beta,
                          const double *s0, double scale, double *o,
                          double *s_out);

/* Gradient of kda_oracle_recurrence (reverse-mode through the token loop)
 * for the loss sum(o * dO) + sum(S_T * dsT): dq, dk, dg [B,T,H,Dk], dv
 * [B,T,H,Dv], dbeta [B,T,H], ds0 [B,H,Dk,Dv] (may be NULL).  s0 and dsT may
 * be NULL (zeros).  Returns the number of OpenMP threads that ran it. */
int kda_oracle_backward(int64_t B, int64_t T, int64_t H, int64_t Dk,
                        int64_t Dv, const double *q, const double *k,
                        const double *v, const double *g, const double *beta,
                        const double *s0, double scale, const double *dO,
                        const double *dsT, double *dq, double *dk, double *dv,
                        double *dg, double *dbeta, double *ds0);

/* Causal depthwise conv along time: y[b,t,c] = sum_j w[c,j] x[b,t-W+1+j,c]
 * where x at negative times comes from hist[b,c,W-1+tau] (hist may be NULL:
 * zeros).  If hist_out is not NULL it receives the last W-1 inputs of the
 * concatenated history+x sequence. */
void kda_oracle_causal_conv(int64_t B, int64_t T, int64_t Cn, int64_t W,
                            const double *x, const double *w,
                            const double *hist, double *y, double *hist_out);

/* In-place per-head L2 normalisation: x[r, h, :] /= sqrt(sum x^2 + eps) for
 * rows r in [0, R) and heads h in [0, H), each head D wide. */
void kda_oracle_l2norm(int64_t R, int64_t H, int64_t D, double eps, double *x);

#ifdef __cplusplus
}
#endif
#endif
