// kda_internal.h -- launcher interface between the C ABI (kda_api.cpp) and
// the HIP kernels.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

struct PrefillParams {
  const void *q, *k, *v;      // [B,T,H,D] (unused when use_conv)
  const void *g, *beta;       // gates
  int gate_bf16;              // 1: g/beta are bf16, 0: fp32
  int gate_head;              // 1: g is [B,T,H], one value per head
  const float *s0;            // [B,H,Dk,Dv] or null
  float *s_out;               // [B,H,Dk,Dv] or null
  void *o;                    // [B,T,H,Dv]
  int B, T, H, Dk, Dv, C, NC; // NC = ceil(T / C)
  float scale;
  int use_conv, cw, l2;       // fused conv prologue
  float eps;
  const void *xq, *xk, *xv;
  const float *wq, *wk, *wv;
  char *ws;                   // workspace base
  size_t wsb;                 // bytes per (bh, chunk) block
  float *ckpt;                // state pass: if set, the state at the start
                              // of every chunk, [B,H,NC,Dk,Dv] fp32
  float *train_at;            // chunk prep: if set, per (bh, chunk) the
                              // matrix A then T^T, C x C fp32 each
  int *sync;                  // concurrent prefill only (else null): task
                              // counter, wait-timeout flag, then one ready
                              // flag per chunk task (see SYNC_* below)
};

// The concurrent prefill (chunk prep and state pass running at the same
// time on the same CUs, bf16 q/k/v, d_k = d_v = 128, chunk 64, per-channel
// gate, no conv): layout of its int array `sync`, cleared before each call.
//   sync[SYNC_NEXT]    next chunk task to claim (chunk-major: task
//                      t = n * B*H + bh)
//   sync[SYNC_TIMEOUT] set to 1 if a state-pass wave gave up waiting
//   sync[SYNC_FLAGS + bh * NC + n]  1 once the factors of chunk n of
//                      batch*head bh are in memory (a head's flags are
//                      contiguous: one vector load reads 64 of them)
constexpr int SYNC_NEXT = 0, SYNC_TIMEOUT = 1, SYNC_FLAGS = 64;
inline size_t sync_bytes(int B, int H, int NC) {
  return (((size_t)SYNC_FLAGS + (size_t)B * H * NC) * 4 + 255) & ~(size_t)255;
}

// gradient of the chunked prefill (kda_backward.hip)
struct BwdParams {
  PrefillParams f;       // forward sizes, inputs and its workspace (ws, wsb)
  const void *dO;        // [B,T,H,Dv] in the q/k/v dtype
  const float *dsT;      // [B,H,Dk,Dv] or null
  float *ds0;            // [B,H,Dk,Dv] or null
  float *dD;             // dDelta, [B,T,H,Dv] in the q/k/v dtype (scratch
                         // sized for fp32)
  float *dSc;            // gradient at the end of every chunk [B,H,NC,Dk,Dv]
  const float *Sc;       // forward state at the start of every chunk
  float *gs;             // per-chunk intermediates (second kernel -> third)
  void *dq, *dk, *dv, *dg, *dbeta;
};


struct DecodeParams {
  const void *q, *k, *v, *g, *beta;  // [N,L,H,*], beta [N,L,H]
  int gate_bf16;
  int gate_head;          // 1: g is [N,L,H], one value per head
  const float *state_in;  // [N,H,Dk,Dv]
  float *state_out;       // [N,H,Dk,Dv], may equal state_in
  float *tstates;         // [N,L,H,Dk,Dv] or null
  void *o;                // [N,L,H,Dv]
  int N, L, H, Dk, Dv;
  float scale;
  // optional fused conv prologue (xq != null): raw inputs [N,L,H*D], taps
  // [H*D,cw], history [N,3,H*Dmax,cw-1] (null: zeros); cstate_out (or
  // null) receives the history rolled forward by the L inputs and must not
  // alias cstate
  const void *xq, *xk, *xv;
  const float *wq, *wk, *wv;
  int cw, l2, Dmax;
  float eps;
  const float *cstate;
  float *cstate_out;
};

struct ConvParams {
  const void *x[3];
  const float *w[3];
  void *y[3];
  int D[3];
  int B, T, H, W, l2, io_bf16;
  float eps;
  float *state;  // [B,3,H*Dmax,W-1] or null
  int Dmax;
};

hipError_t launch_prefill_prep(const PrefillParams &p, int io_bf16,
                               hipStream_t s);
// per dtype pair (q/k/v, g/beta); launch_prefill_prep picks one
hipError_t launch_prefill_prep_f32(const PrefillParams &p, hipStream_t s);
hipError_t launch_prefill_prep_bf16_f32(const PrefillParams &p, hipStream_t s);
hipError_t launch_prefill_prep_bf16_bf16(const PrefillParams &p,
                                         hipStream_t s);
// the chunk prep for one gate per token-head (bf16 q/k/v, d_k = 128,
// chunk 64, no conv, no backward outputs): whether it serves p, and its
// launcher
bool prep_gdn_applies(const PrefillParams &p, int io_bf16);
hipError_t launch_prefill_prep_gdn(const PrefillParams &p, hipStream_t s);
// the chunk prep for one gate per key channel at bf16 q/k/v,
// d_k = d_v = 128, chunk 64, no conv (eight waves per task)
bool prep_d128_applies(const PrefillParams &p, int io_bf16);
hipError_t launch_prefill_prep_d128(const PrefillParams &p, hipStream_t s);
hipError_t launch_state_pass(const PrefillParams &p, int io_bf16,
                             hipStream_t s);
// the concurrent prefill: whether p (with p.sync set) qualifies, the
// clearing of p.sync, and its state pass (the prep is the d128 launcher's,
// which takes the concurrent path when p.sync is set)
bool prefill_concurrent_applies(const PrefillParams &p, int io_bf16);
hipError_t launch_sync_clear(const PrefillParams &p, hipStream_t s);
hipError_t launch_state_pass_concurrent(const PrefillParams &p, hipStream_t s);
hipError_t launch_decode(const DecodeParams &p, int io_bf16, hipStream_t s);
// the three backward kernels (the forward's prep and state pass, with state
// checkpoints, must have filled bp.f.ws and bp.Sc first)
hipError_t launch_backward(const BwdParams &bp, int io_bf16, hipStream_t s);
// whether the backward kernels' LDS fits for these sizes
bool backward_fits(int io_bf16, int Dk, int C);
// floats of per-chunk backward intermediates
size_t backward_chunk_floats(int C, int Dk, int Dv);
hipError_t launch_conv(const ConvParams &p, hipStream_t s);
// the history update alone (after a consumer of the old history has run)
hipError_t launch_conv_cache(const ConvParams &p, hipStream_t s);

}  // namespace kda
