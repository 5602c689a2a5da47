/*
 * kda.h -- C ABI of libkda.so: the Kimi Delta Attention (KDA) layer forward
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Per head, with a d_k x d_v state S (row i = key channel
 * i), for each token t:
 *     S'  = diag(exp(g_t)) S              per-row forgetting, g_t <= 0
 *     S_t = S' + k_t (beta_t (v_t - S'^T k_t))^T
 *     o_t = scale * S_t^T q_t
 * Sources (web pages, cited by title and section):
 *   [SARNAS] sarnas.ru, "Yandex opened the weights of
 *     AliceAI-Foundation-80B-A3B-Base: an MoE model trained from scratch",
 *     section "What exactly changed", KDA paragraph: fixed-size state; the
 *     value stored for the key is read, compared with the new value, and only
 *     the difference is written; one forgetting coefficient per row of the
 *     state matrix.  Section "Rejected decisions": KDA layers keep a QK norm.
 *   [LQNN-A] m.lqnn.cn news 205170 ("two deep teardowns in two days ..."),
 *     the AliceAIKDA walk-through: kernel-4 causal conv on q/k/v with an
 *     incrementally updated cache; the state is multiplied by exp(gate) and
 *     the delta added; delta = prediction residual times sigmoid beta; on GPU
 *     a chunked prefill kernel and a fused recurrent (decode) kernel; beta is
 *     kept in (0,1) when negative eigenvalues are disallowed; the conv kernel
 *     dimension is validated to be at least 2.
 *   [LQNN-B] m.lqnn.cn news 255115 ("80B parameters for 3B of compute ..."),
 *     config-validation list: conv kernel >= 2, chunk size positive.
 *   [AREX] arex-research.com, "Yandex open-sources
 *     AliceAI-Foundation-80B-A3B-Base ...", deployment paragraph: vLLM
 *     serving with multi-token-prediction speculative decoding, one guessed
 *     token per step.
 *
 * Conventions shared by every entry point.
 *  - All pointers are DEVICE pointers owned by the caller; the library
 *    never allocates device memory (the prefill workspace is passed in) and
 *    keeps no global mutable state, with two exceptions: the fixed scratch
 *    array of kda_prefill_noalloc (below), and one extra stream and two
 *    events per GPU that kda_prefill creates on first use when it runs its
 *    two phases concurrently (below) and keeps until the process ends.
 *    Calls are thread-safe.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronises.
 *  - Tensors are dense, contiguous, row-major.  Pointers must be 16-byte
 *    aligned.  q, k, g: [B,T,H,Dk]; v, o: [B,T,H,Dv]; beta: [B,T,H];
 *    states: [B,H,Dk,Dv] fp32 with row i = key channel i.
 *  - Supported: Dk, Dv in {16,32,64,128}; chunk in {16,32,64}; conv width in
 *    [2,4]; dtype pairs (q/k/v, g/beta) in {(F32,F32), (BF16,F32),
 *    (BF16,BF16)}.  fp32 q/k/v with Dk = 128 and chunk 64 run as 32-token
 *    chunks (the chunked form is exact for any chunk length, so only the
 *    rounding differs; a 64-token fp32 chunk at Dk = 128 does not fit one
 *    CU's LDS), and the workspace sizes follow.  Outputs o have the q/k/v
 *    dtype; states are always fp32.
 *  - Element values are not checked: g > 0 or beta outside (0,2) are the
 *    caller's responsibility (the pages keep beta in (0,1), or (0,2) with
 *    negative eigenvalues allowed); g = -inf is supported and forgets
 *    exactly.
 *  - gate_dtype may carry the KDA_GATE_HEAD flag (one log-decay per token
 *    and head); a q/k/v dtype with the flag is KDA_EINVAL.
 *  - Errors: arguments are validated before anything is launched.
 *    KDA_EINVAL: a NULL required pointer, a size <= 0, chunk <= 0, conv
 *    width < 2, a misaligned pointer, a workspace that is too small.
 *    KDA_EUNSUPPORTED: a valid request outside the supported set above.
 *    KDA_EHIP: a HIP launch error (the HIP error is cleared and reported
 *    through this code only).  Nothing is written on an error return that
 *    happens before a launch.  No C++ exception crosses this boundary.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_OK = 0,
  KDA_EINVAL = 1,
  KDA_EUNSUPPORTED = 2,
  KDA_EHIP = 3,
  /* kda_prefill_noalloc only: the request needs more workspace than its
   * fixed scratch array holds (KDA_NOALLOC_SCRATCH_BYTES) */
  KDA_ENOSPACE = 4
} kda_status;

typedef enum kda_dtype {
  KDA_F32 = 0,
  KDA_BF16 = 1,
  /* Flag for a gate_dtype argument only (OR it into KDA_F32 or KDA_BF16):
   * g then holds ONE log-decay per token and head, [B,T,H] (decode:
   * [N,H] / [N,L,H]), shared by every key channel -- the single forgetting
   * coefficient of Gated DeltaNet, which [SARNAS] (KDA paragraph) names as
   * what KDA refines into one coefficient per state row.  The result is
   * exactly that of the per-channel gate with g repeated over d_k; only g's
   * traffic shrinks (d_k-fold). */
  KDA_GATE_HEAD = 16
} kda_dtype;

/* beta ([LQNN-A] configuration checks): the model keeps beta in (0,1) so
 * the update contracts; with "negative eigenvalues" allowed it may reach
 * (0,2) (the transition I - beta k k^T then has an eigenvalue in (-1,0) for
 * a unit k).  No entry point clamps or checks beta's values. */

/* Optional fused conv prologue for kda_prefill ([LQNN-A] conv paragraph;
 * [SARNAS] "Rejected decisions" QK norm).  For each channel c of the
 * projections x* = [B,T,H*D] (q/k/v dtype):
 *     y[t,c] = sum_{j<width} w[c*width + j] * x[t-width+1+j, c]
 * with zeros before t = 0 (tap width-1 multiplies the newest input; no bias,
 * no activation).  If l2norm_qk, q and k are then divided per head by
 * sqrt(sum y^2 + eps); v is not normalised. */
typedef struct kda_conv_desc {
  const void *xq, *xk, *xv;   /* [B,T,H*Dk], [B,T,H*Dk], [B,T,H*Dv]      */
  const float *wq, *wk, *wv;  /* [H*Dk,width], [H*Dk,width], [H*Dv,width] */
  int width;                  /* 2..4 */
  int l2norm_qk;              /* 0 or 1 */
  float eps;                  /* e.g. 1e-6 */
} kda_conv_desc;

/* ABI version of this header (bumped on any incompatible change). */
#define KDA_ABI_VERSION 6
int kda_abi_version(void);

/* Static text for a status code (never NULL). */
const char *kda_status_string(kda_status s);

/* Bytes of device workspace kda_prefill needs for these sizes (0 if the
 * sizes are invalid or unsupported).  The workspace holds the chunk-local
 * factors of every (batch, head, chunk), then a small int array (a counter
 * and one flag per (batch, head, chunk), 256-byte aligned) that the
 * concurrent mode of kda_prefill uses; contents need no initialisation. */
size_t kda_prefill_workspace_size(int B, int T, int H, int Dk, int Dv,
                                  int chunk, kda_dtype qkv_dtype);

/* Chunked prefill ([LQNN-A]: the chunked GPU prefill path; chunk size a
 * positive config value per [LQNN-B]).
 *   q,k,v     inputs (ignored, may be NULL, when conv != NULL)
 *   g, beta   log-decay per key channel [B,T,H,Dk] (or per head [B,T,H]
 *             with KDA_GATE_HEAD in gate_dtype) and write strength
 *             [B,T,H], in gate_dtype
 *   s0        initial state [B,H,Dk,Dv] fp32, or NULL for zeros
 *   s_out     final state [B,H,Dk,Dv] fp32, or NULL; may equal s0
 *   o         output [B,T,H,Dv] in qkv_dtype; must not alias an input
 *   chunk     tokens per chunk (16, 32 or 64); T need not be a multiple
 *   scale     output scale (1.0 reproduces o_t = S_t^T q_t)
 *   conv      NULL, or the fused conv prologue above
 *   workspace device buffer of at least kda_prefill_workspace_size() bytes
 *             (a buffer that holds only the factor blocks, as
 *             kda_prefill_chunk_prep requires, is accepted and runs the
 *             two phases one after the other)
 * Runs kda_prefill_chunk_prep then kda_prefill_state_pass on `stream`.
 * Concurrent mode: for bf16 q/k/v, Dk = Dv = 128, chunk 64, a gate per key
 * channel, no conv, B*H*8 <= the GPU's compute units, and at least 1024
 * chunks per sequence, the two phases run at the same time on the same
 * compute units instead: the chunk prep on `stream` publishes each chunk's
 * factors with a ready flag in the workspace, and the state pass, on a
 * second stream of the library's that waits for `stream` and that `stream`
 * then waits for, consumes them in order.  Results are bit for bit those of
 * the two phases run in turn, and work queued on `stream` after the call
 * still sees them.  The mode is not used while `stream` is being captured
 * into a graph.  KDA_CONCURRENT in the environment (read at every call)
 * overrides the choice: "0" never, "1" for every shape above whatever the
 * sequence length. */
kda_status kda_prefill(const void *q, const void *k, const void *v,
                       kda_dtype qkv_dtype, const void *g, const void *beta,
                       kda_dtype gate_dtype, const float *s0, float *s_out,
                       void *o, int B, int T, int H, int Dk, int Dv,
                       int chunk, float scale, const kda_conv_desc *conv,
                       void *workspace, size_t workspace_bytes, void *stream);

/* kda_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, arithmetic, results (bit for bit) and errors as
 * kda_prefill, without the workspace arguments: the workspace is a static
 * device array of KDA_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library,
 * one per GPU, held until the process ends.  Its device address is looked
 * up once per GPU, on the first call made with that GPU current (the
 * caller's current device must be the one `stream` belongs to).  Requests
 * whose kda_prefill_workspace_size() exceeds the array return KDA_ENOSPACE
 * before anything is launched (64 MiB holds 903 chunk-heads at
 * Dk = Dv = 128, chunk 64, bf16: B*H*ceil(T/64) <= 903, e.g. T <= 1792 at
 * B = 1, H = 32).  It always runs the two phases one after the other.  The call allocates nothing, host or device.  Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (on different streams, or from several threads) race and corrupt
 * each other's results; serialise them (one stream, or events).  The
 * array needs no initialisation and keeps the last call's contents. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v,
                               kda_dtype qkv_dtype, const void *g,
                               const void *beta, kda_dtype gate_dtype,
                               const float *s0, float *s_out, void *o,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               float scale, const kda_conv_desc *conv,
                               void *stream);

/* First phase of kda_prefill alone: every (batch, head, chunk) is reduced
 * to its state-independent factors (the UT-transform of the chunk's
 * triangular system, decay-weighted keys and queries, and the intra-chunk
 * query-key matrix), written to `workspace`.  Fully parallel over chunks. */
kda_status kda_prefill_chunk_prep(const void *q, const void *k, const void *v,
                                  kda_dtype qkv_dtype, const void *g,
                                  const void *beta, kda_dtype gate_dtype,
                                  int B, int T, int H, int Dk, int Dv,
                                  int chunk, float scale,
                                  const kda_conv_desc *conv, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Second phase of kda_prefill alone: the sequential pass over chunks that
 * carries the state and writes o and s_out, reading the factors that
 * kda_prefill_chunk_prep left in `workspace` (same sizes and dtypes). */
kda_status kda_prefill_state_pass(kda_dtype qkv_dtype, const float *s0,
                                  float *s_out, void *o, int B, int T, int H,
                                  int Dk, int Dv, int chunk,
                                  const void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Bytes of device workspace kda_prefill_backward needs (0 if the sizes are
 * invalid or unsupported): the forward's factors, the state at every chunk
 * start and the gradient at every chunk end (fp32, Dk*Dv per chunk-head),
 * and per-chunk intermediates; about 2.6x the forward's input bytes plus
 * 8*Dk*Dv bytes per chunk-head. */
size_t kda_prefill_backward_workspace_size(int B, int T, int H, int Dk,
                                           int Dv, int chunk,
                                           kda_dtype qkv_dtype);

/* Gradient of kda_prefill (without the conv prologue) for training: the
 * layer is trained end to end ([SARNAS] "What exactly changed", the
 * pretraining comparison of KDA against Gated DeltaNet).  Reverse mode of
 * the token rule, evaluated in chunks: the forward is recomputed (chunk
 * prep, then the state pass keeping the state at every chunk start), the
 * gradient of the state is carried back over the chunks, and every chunk's
 * inputs get their gradients in parallel.  Loss-gradient inputs:
 *   dO    [B,T,H,Dv] in qkv_dtype (gradient of o)
 *   dsT   [B,H,Dk,Dv] fp32 gradient of the final state, or NULL (zero)
 * Outputs (each written in full; none may alias an input or each other):
 *   dq, dk [B,T,H,Dk] and dv [B,T,H,Dv] in qkv_dtype
 *   dg     [B,T,H,Dk] in gate_dtype ([B,T,H] with KDA_GATE_HEAD: the sum
 *          over the key channels the gate multiplies)
 *   dbeta  [B,T,H] in gate_dtype
 *   ds0    [B,H,Dk,Dv] fp32 gradient of s0, or NULL
 * Other arguments, sizes and errors as for kda_prefill (q, k, v must be
 * given; s0 may be NULL for zeros).  workspace: at least
 * kda_prefill_backward_workspace_size() bytes. */
kda_status kda_prefill_backward(
    const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
    const void *g, const void *beta, kda_dtype gate_dtype, const float *s0,
    const void *dO, const float *dsT, void *dq, void *dk, void *dv, void *dg,
    void *dbeta, float *ds0, int B, int T, int H, int Dk, int Dv, int chunk,
    float scale, void *workspace, size_t workspace_bytes, void *stream);

/* One recurrent decode step for N independent sequences ([LQNN-A]: the
 * fused recurrent GPU kernel used for generation).
 *   q,k,g [N,H,Dk]; v [N,H,Dv]; beta [N,H]   (qkv_dtype / gate_dtype;
 *   g is [N,H] with KDA_GATE_HEAD)
 *   state [N,H,Dk,Dv] fp32, read and updated IN PLACE
 *   o     [N,H,Dv] in qkv_dtype; must not alias an input */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           kda_dtype qkv_dtype, const void *g,
                           const void *beta, kda_dtype gate_dtype,
                           float *state, void *o, int N, int H, int Dk,
                           int Dv, float scale, void *stream);

/* L tokens of the recurrent rule per sequence in one call: the verify step
 * of speculative decoding with the multi-token-prediction head ([AREX]
 * deployment paragraph and [LQNN-A] serving notes: speculative decoding
 * through the model's MTP module, one guessed token per step, so L = 2),
 * or a short prompt extension.  Equal, up to rounding, to L successive
 * kda_decode_step calls; the state is read once, carried through the L
 * tokens and written once.
 *   q,k,g [N,L,H,Dk]; v [N,L,H,Dv]; beta [N,L,H]   (qkv_dtype / gate_dtype;
 *   g is [N,L,H] with KDA_GATE_HEAD)
 *   state_in      [N,H,Dk,Dv] fp32, the state before the first token
 *   state_out     [N,H,Dk,Dv] fp32, the state after the last token; may
 *                 equal state_in (in place)
 *   token_states  [N,L,H,Dk,Dv] fp32 or NULL: the state after each token,
 *                 so a caller that accepts only the first a tokens of a
 *                 sequence continues from token_states[n][a-1]; must not
 *                 alias state_in or state_out
 *   o             [N,L,H,Dv] in qkv_dtype; must not alias an input
 *   conv          NULL, or a fused conv prologue ([LQNN-A]: the kernel-4
 *                 conv whose cache is updated incrementally with the
 *                 state): q,k,v are then made from the raw projections
 *                 conv->x* [N,L,H*D] (q, k, v may be NULL), with the
 *                 taps, width and L2 norm of kda_conv_desc
 *   conv_state    with conv: NULL (zeros before the first token), or the
 *                 fp32 history [N,3,H*D_max,width-1] of kda_conv_prologue,
 *                 read as the inputs before the first token and then, when
 *                 conv_state_out is NULL or equal to it, rolled forward in
 *                 place to end with the L new raw inputs (a second, small
 *                 kernel on the same stream)
 *   conv_state_out  NULL, or a second history buffer of the same layout
 *                 that receives the rolled history instead (conv_state is
 *                 then only read and may be NULL); written by the decode
 *                 kernel itself, so a caller that alternates two buffers
 *                 saves the in-place roll.  Must not alias o, the states or
 *                 the raw inputs.
 *                 (conv_state and conv_state_out must be NULL without conv)
 * With conv and L = 1 this is the generation step with its conv cache.
 * Errors as for kda_decode_step; L <= 0 is KDA_EINVAL. */
kda_status kda_decode_tokens(const void *q, const void *k, const void *v,
                             kda_dtype qkv_dtype, const void *g,
                             const void *beta, kda_dtype gate_dtype,
                             const float *state_in, float *state_out,
                             float *token_states, void *o, int N, int L,
                             int H, int Dk, int Dv, float scale,
                             const kda_conv_desc *conv, float *conv_state,
                             float *conv_state_out, void *stream);

/* Standalone conv prologue ([LQNN-A]: kernel-4 causal conv with a cache
 * updated incrementally).  Same arithmetic as kda_conv_desc; outputs
 * q,k [B,T,H,Dk] and v [B,T,H,Dv] in `dtype` (the raw inputs' dtype).
 *   conv_state  NULL (zeros before t = 0), or fp32 [B,3,H*D_max,width-1]
 *               laid out as [b][stream q,k,v][channel][tap], D_max =
 *               max(Dk,Dv): read as the inputs before t = 0, then
 *               overwritten with the last width-1 inputs of history+x. */
kda_status kda_conv_prologue(const void *xq, const void *xk, const void *xv,
                             kda_dtype dtype, const float *wq,
                             const float *wk, const float *wv, int width,
                             float *conv_state, void *q, void *k, void *v,
                             int B, int T, int H, int Dk, int Dv,
                             int l2norm_qk, float eps, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
