// kda_api.hip -- the extern "C" boundary of libkda.so: argument validation
// and dispatch to the launchers.  Every check happens before any launch, so
// an error return leaves every output untouched.  See include/kda.h.
#include "../../include/kda.h"

#include <math.h>
#include <stdlib.h>

#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
bool dtype_valid(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16; }
// a gate dtype: KDA_F32 or KDA_BF16, optionally with KDA_GATE_HEAD
bool gate_valid(kda_dtype d) {
  return dtype_valid((kda_dtype)(d & ~KDA_GATE_HEAD));
}
kda_dtype gate_base(kda_dtype d) { return (kda_dtype)(d & ~KDA_GATE_HEAD); }
int gate_head(kda_dtype d) { return (d & KDA_GATE_HEAD) ? 1 : 0; }
bool pair_ok(kda_dtype io, kda_dtype gt) {
  gt = gate_base(gt);
  return (io == KDA_F32 && gt == KDA_F32) ||
         (io == KDA_BF16 && (gt == KDA_F32 || gt == KDA_BF16));
}
// Chunk length the kernels run for a requested chunk.  The chunked form is
// exact algebra for any chunk length, so this changes only rounding: fp32
// q/k/v with d_k = 128 runs a requested 64-token chunk as two 32-token
// chunks, because the chunk prep's LDS for a 64-token fp32 chunk at
// d_k = 128 exceeds the 160 KiB of one CU.
int run_chunk(kda_dtype io, int Dk, int chunk) {
  return (io == KDA_F32 && Dk == 128 && chunk == 64) ? 32 : chunk;
}

kda_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  (void)hipGetLastError();
  return KDA_EHIP;
}

// shared validation of the prefill family; fills p (without workspace)
kda_status prefill_check(const void *q, const void *k, const void *v,
                         kda_dtype io, const void *g, const void *beta,
                         kda_dtype gt, int B, int T, int H, int Dk, int Dv,
                         int chunk, float scale, const kda_conv_desc *conv,
                         bool need_inputs, kda::PrefillParams &p) {
  if (B <= 0 || T <= 0 || H <= 0 || Dk <= 0 || Dv <= 0 || chunk <= 0)
    return KDA_EINVAL;
  if (!dtype_valid(io) || !gate_valid(gt)) return KDA_EINVAL;
  if (!isfinite(scale)) return KDA_EINVAL;
  if (need_inputs) {
    if (!g || !beta) return KDA_EINVAL;
    if (!aligned16(g) || !aligned16(beta)) return KDA_EINVAL;
    if (conv) {
      if (!conv->xq || !conv->xk || !conv->xv || !conv->wq || !conv->wk ||
          !conv->wv)
        return KDA_EINVAL;
      if (!aligned16(conv->xq) || !aligned16(conv->xk) ||
          !aligned16(conv->xv) || !aligned16(conv->wq) ||
          !aligned16(conv->wk) || !aligned16(conv->wv))
        return KDA_EINVAL;
      if (conv->width < 2) return KDA_EINVAL;
      if (conv->l2norm_qk != 0 && conv->l2norm_qk != 1) return KDA_EINVAL;
      if (!(conv->eps >= 0.f) || !isfinite(conv->eps)) return KDA_EINVAL;
    } else {
      if (!q || !k || !v) return KDA_EINVAL;
      if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return KDA_EINVAL;
    }
  }
  if (!dim_ok(Dk) || !dim_ok(Dv) || !chunk_ok(chunk)) return KDA_EUNSUPPORTED;
  if (!pair_ok(io, gt)) return KDA_EUNSUPPORTED;
  if (need_inputs && conv && conv->width > 4) return KDA_EUNSUPPORTED;
  chunk = run_chunk(io, Dk, chunk);
  const long long nc = ((long long)T + chunk - 1) / chunk;
  if ((long long)B * H * nc > 0x7fffffffLL) return KDA_EUNSUPPORTED;
  if ((long long)B * H * (Dv / 16) > 0x7fffffffLL) return KDA_EUNSUPPORTED;
  p = kda::PrefillParams{};
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
  p.gate_bf16 = gate_base(gt) == KDA_BF16;
  p.gate_head = gate_head(gt);
  p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.C = chunk;
  p.NC = (int)nc;
  p.scale = scale;
  if (need_inputs && conv) {
    p.use_conv = 1; p.cw = conv->width; p.l2 = conv->l2norm_qk;
    p.eps = conv->eps;
    p.xq = conv->xq; p.xk = conv->xk; p.xv = conv->xv;
    p.wq = conv->wq; p.wk = conv->wk; p.wv = conv->wv;
  }
  return KDA_OK;
}

size_t ws_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                kda_dtype io) {
  chunk = run_chunk(io, Dk, chunk);
  const size_t nc = ((size_t)T + chunk - 1) / chunk;
  const kda::WsLayout L = kda::ws_layout(Dk, Dv, chunk, io == KDA_BF16 ? 2 : 4);
  return (size_t)B * H * nc * L.bytes;
}

// kda_prefill's workspace: the factor blocks, then the int array of the
// concurrent mode (task counter and per-chunk-task ready flags)
size_t prefill_ws_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                        kda_dtype io) {
  const int c = run_chunk(io, Dk, chunk);
  const int nc = (int)(((long long)T + c - 1) / c);
  return ws_bytes(B, T, H, Dk, Dv, chunk, io) + kda::sync_bytes(B, H, nc);
}

// backward workspace: [forward factors | state at every chunk start |
// gradient at every chunk end | dDelta | per-chunk intermediates | A and
// T^T of every chunk | the forward's output o, which the backward does not
// use]
struct BwdWs {
  size_t sc, dsc, dd, gs, at, o, total;
};
BwdWs bwd_ws(int B, int T, int H, int Dk, int Dv, int chunk, kda_dtype io) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const int requested = chunk;
  chunk = run_chunk(io, Dk, chunk);
  const size_t nc = ((size_t)T + chunk - 1) / chunk, BH = (size_t)B * H;
  BwdWs w;
  size_t off = al(ws_bytes(B, T, H, Dk, Dv, requested, io));
  w.sc = off;
  off = al(off + BH * nc * Dk * Dv * 4);
  w.dsc = off;
  off = al(off + BH * nc * Dk * Dv * 4);
  w.dd = off;
  off = al(off + (size_t)B * T * H * Dv * 4);
  w.gs = off;
  off = al(off + BH * nc * kda::backward_chunk_floats(chunk, Dk, Dv) * 4);
  w.at = off;
  off = al(off + BH * nc * 2 * (size_t)chunk * chunk * 4);
  w.o = off;
  off = al(off + (size_t)B * T * H * Dv * (io == KDA_BF16 ? 2 : 4));
  w.total = off;
  return w;
}

// validation shared by kda_prefill and kda_prefill_noalloc (everything but
// the workspace); fills p without it
kda_status prefill_args(const void *q, const void *k, const void *v,
                        kda_dtype io, const void *g, const void *beta,
                        kda_dtype gt, const float *s0, float *s_out, void *o,
                        int B, int T, int H, int Dk, int Dv, int chunk,
                        float scale, const kda_conv_desc *conv,
                        kda::PrefillParams &p) {
  kda_status st = prefill_check(q, k, v, io, g, beta, gt, B, T, H, Dk, Dv,
                                chunk, scale, conv, true, p);
  if (st != KDA_OK) return st;
  if (!o) return KDA_EINVAL;
  if (!aligned16(o) || (s0 && !aligned16(s0)) || (s_out && !aligned16(s_out)))
    return KDA_EINVAL;
  if (o == q || o == k || o == v || o == g || o == beta) return KDA_EINVAL;
  p.s0 = s0; p.s_out = s_out; p.o = o;
  return KDA_OK;
}

// ---------------------------------------------------------------------------
// The fixed workspace of kda_prefill_noalloc.  In host code the name
// `scratch` is only a host-side stand-in: kernels get the device address
// that hipGetSymbolAddress reports for the current GPU (each GPU holds its
// own copy of the array at its own address), looked up once per GPU and
// kept.  It needs no initialisation: the chunk prep writes every byte of
// the workspace that the state pass reads.
__device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::once_flag scratch_once[SCRATCH_MAX_DEVICES];
void *scratch_ptr[SCRATCH_MAX_DEVICES];
hipError_t scratch_err[SCRATCH_MAX_DEVICES];

kda_status scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hip_status(hipErrorNoDevice);
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return KDA_EUNSUPPORTED;
  std::call_once(scratch_once[dev], [dev]() {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    scratch_err[dev] = e;
    scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev])
    return hip_status(scratch_err[dev] != hipSuccess ? scratch_err[dev]
                                                     : hipErrorInvalidSymbol);
  *out = scratch_ptr[dev];
  return KDA_OK;
}

// ---------------------------------------------------------------------------
// The concurrent prefill.  The chunk prep runs on the caller's stream and
// the state pass on a second stream of the library's (one per GPU, created
// on first use, default priority, never destroyed), joined by two events so
// that the call still starts after earlier work on the caller's stream and
// later work waits for both kernels.  The event pair of a GPU is reused, so
// the record/wait sequence of one call is kept whole under a per-GPU lock.
//
// Both kernels lean on the same per-CU path from the L2 into the vector
// registers, so running them together gains only where the steady state
// dominates: measured on the long-context workload (4096 chunks per head)
// the call is 8 % faster, on the 8192-token one (128 chunks) 3 % slower.
// The mode is therefore used for sequences of at least CO_MIN_CHUNKS chunks.
// KDA_CONCURRENT in the environment, read at every call, overrides that:
// "0" never, "1" for every shape the mode covers.
constexpr int CO_MAX_DEVICES = 64;
struct CoStreams {
  std::once_flag once;
  hipError_t err = hipSuccess;
  hipStream_t side = nullptr;
  hipEvent_t start = nullptr, done = nullptr;
  std::mutex mu;
};
CoStreams co_streams[CO_MAX_DEVICES];

constexpr int CO_MIN_CHUNKS = 1024;
bool concurrent_wanted(int NC) {
  const char *e = getenv("KDA_CONCURRENT");
  if (e && e[0] == '0') return false;
  if (e && e[0] == '1') return true;
  return NC >= CO_MIN_CHUNKS;
}

CoStreams *co_streams_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= CO_MAX_DEVICES)
    return nullptr;
  CoStreams &c = co_streams[dev];
  std::call_once(c.once, [&c]() {
    hipError_t e = hipStreamCreateWithFlags(&c.side, hipStreamNonBlocking);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&c.start, hipEventDisableTiming);
    if (e == hipSuccess)
      e = hipEventCreateWithFlags(&c.done, hipEventDisableTiming);
    c.err = e;
  });
  return c.err == hipSuccess ? &c : nullptr;
}

// whether a call on `stream` is being captured into a graph (the concurrent
// mode is then not used: the capture keeps the plain two-kernel sequence)
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return true;
  return st != hipStreamCaptureStatusNone;
}

// clear the sync array, then the prep on `stream` beside the state pass on
// the side stream; returns hipErrorNotSupported (nothing launched) when the
// side stream is unavailable
hipError_t launch_prefill_concurrent(kda::PrefillParams &p,
                                     hipStream_t stream) {
  CoStreams *c = co_streams_for_current_device();
  if (!c) return hipErrorNotSupported;
  std::lock_guard<std::mutex> lock(c->mu);
  hipError_t e = kda::launch_sync_clear(p, stream);
  if (e == hipSuccess) e = hipEventRecord(c->start, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(c->side, c->start, 0);
  if (e == hipSuccess) e = kda::launch_prefill_prep(p, 1, stream);
  if (e == hipSuccess) e = kda::launch_state_pass_concurrent(p, c->side);
  if (e == hipSuccess) e = hipEventRecord(c->done, c->side);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, c->done, 0);
  return e;
}

}  // namespace

namespace kda {
hipError_t launch_prefill_prep(const PrefillParams &p, int io_bf16,
                               hipStream_t s) {
  if (prep_gdn_applies(p, io_bf16)) return launch_prefill_prep_gdn(p, s);
  if (prep_d128_applies(p, io_bf16)) return launch_prefill_prep_d128(p, s);
  if (!io_bf16) return launch_prefill_prep_f32(p, s);
  return p.gate_bf16 ? launch_prefill_prep_bf16_bf16(p, s)
                     : launch_prefill_prep_bf16_f32(p, s);
}
}  // namespace kda

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_EINVAL: return "KDA_EINVAL: invalid argument";
    case KDA_EUNSUPPORTED: return "KDA_EUNSUPPORTED: valid but unsupported";
    case KDA_EHIP: return "KDA_EHIP: HIP launch error";
    case KDA_ENOSPACE:
      return "KDA_ENOSPACE: larger than the fixed scratch of "
             "kda_prefill_noalloc";
  }
  return "KDA: unknown status";
}

size_t kda_prefill_workspace_size(int B, int T, int H, int Dk, int Dv,
                                  int chunk, kda_dtype qkv_dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || !dim_ok(Dk) || !dim_ok(Dv) ||
      !chunk_ok(chunk) || !dtype_valid(qkv_dtype))
    return 0;
  return prefill_ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype);
}

kda_status kda_prefill_chunk_prep(const void *q, const void *k, const void *v,
                                  kda_dtype qkv_dtype, const void *g,
                                  const void *beta, kda_dtype gate_dtype,
                                  int B, int T, int H, int Dk, int Dv,
                                  int chunk, float scale,
                                  const kda_conv_desc *conv, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  kda::PrefillParams p;
  kda_status st = prefill_check(q, k, v, qkv_dtype, g, beta, gate_dtype, B, T,
                                H, Dk, Dv, chunk, scale, conv, true, p);
  if (st != KDA_OK) return st;
  if (!workspace || !aligned16(workspace)) return KDA_EINVAL;
  if (workspace_bytes < ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype))
    return KDA_EINVAL;
  p.ws = (char *)workspace;
  p.wsb = kda::ws_layout(Dk, Dv, p.C, qkv_dtype == KDA_BF16 ? 2 : 4).bytes;
  return hip_status(kda::launch_prefill_prep(p, qkv_dtype == KDA_BF16,
                                             (hipStream_t)stream));
}

kda_status kda_prefill_state_pass(kda_dtype qkv_dtype, const float *s0,
                                  float *s_out, void *o, int B, int T, int H,
                                  int Dk, int Dv, int chunk,
                                  const void *workspace,
                                  size_t workspace_bytes, void *stream) {
  kda::PrefillParams p;
  kda_status st = prefill_check(nullptr, nullptr, nullptr, qkv_dtype, nullptr,
                                nullptr, qkv_dtype, B, T, H, Dk, Dv, chunk,
                                1.0f, nullptr, false, p);
  if (st != KDA_OK) return st;
  if (!o || !workspace) return KDA_EINVAL;
  if (!aligned16(o) || !aligned16(workspace) || (s0 && !aligned16(s0)) ||
      (s_out && !aligned16(s_out)))
    return KDA_EINVAL;
  if (workspace_bytes < ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype))
    return KDA_EINVAL;
  p.s0 = s0; p.s_out = s_out; p.o = o;
  p.ws = (char *)workspace;
  p.wsb = kda::ws_layout(Dk, Dv, p.C, qkv_dtype == KDA_BF16 ? 2 : 4).bytes;
  return hip_status(kda::launch_state_pass(p, qkv_dtype == KDA_BF16,
                                           (hipStream_t)stream));
}

kda_status kda_prefill(const void *q, const void *k, const void *v,
                       kda_dtype qkv_dtype, const void *g, const void *beta,
                       kda_dtype gate_dtype, const float *s0, float *s_out,
                       void *o, int B, int T, int H, int Dk, int Dv,
                       int chunk, float scale, const kda_conv_desc *conv,
                       void *workspace, size_t workspace_bytes,
                       void *stream) {
  kda::PrefillParams p;
  kda_status st = prefill_args(q, k, v, qkv_dtype, g, beta, gate_dtype, s0,
                               s_out, o, B, T, H, Dk, Dv, chunk, scale, conv,
                               p);
  if (st != KDA_OK) return st;
  if (!workspace || !aligned16(workspace)) return KDA_EINVAL;
  if (workspace_bytes < ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype))
    return KDA_EINVAL;
  p.ws = (char *)workspace;
  p.wsb = kda::ws_layout(Dk, Dv, p.C, qkv_dtype == KDA_BF16 ? 2 : 4).bytes;
  const int bf = qkv_dtype == KDA_BF16;
  hipStream_t s = (hipStream_t)stream;
  // the concurrent mode needs the sync array after the factor blocks
  const size_t fb = ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype);
  if (workspace_bytes >= prefill_ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype) &&
      concurrent_wanted(p.NC) && kda::prefill_concurrent_applies(p, bf) &&
      !capturing(s)) {
    p.sync = (int *)((char *)workspace + fb);
    const hipError_t e = launch_prefill_concurrent(p, s);
    if (e != hipErrorNotSupported) return hip_status(e);
    p.sync = nullptr;
  }
  hipError_t e = kda::launch_prefill_prep(p, bf, s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(kda::launch_state_pass(p, bf, s));
}

kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v,
                               kda_dtype qkv_dtype, const void *g,
                               const void *beta, kda_dtype gate_dtype,
                               const float *s0, float *s_out, void *o,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               float scale, const kda_conv_desc *conv,
                               void *stream) {
  kda::PrefillParams p;
  kda_status st = prefill_args(q, k, v, qkv_dtype, g, beta, gate_dtype, s0,
                               s_out, o, B, T, H, Dk, Dv, chunk, scale, conv,
                               p);
  if (st != KDA_OK) return st;
  if (prefill_ws_bytes(B, T, H, Dk, Dv, chunk, qkv_dtype) >
      KDA_NOALLOC_SCRATCH_BYTES)
    return KDA_ENOSPACE;
  void *ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != KDA_OK) return st;
  p.ws = (char *)ws;
  p.wsb = kda::ws_layout(Dk, Dv, p.C, qkv_dtype == KDA_BF16 ? 2 : 4).bytes;
  const int bf = qkv_dtype == KDA_BF16;
  hipError_t e = kda::launch_prefill_prep(p, bf, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(kda::launch_state_pass(p, bf, (hipStream_t)stream));
}

size_t kda_prefill_backward_workspace_size(int B, int T, int H, int Dk,
                                           int Dv, int chunk,
                                           kda_dtype qkv_dtype) {
  if (kda_prefill_workspace_size(B, T, H, Dk, Dv, chunk, qkv_dtype) == 0)
    return 0;
  return bwd_ws(B, T, H, Dk, Dv, chunk, qkv_dtype).total;
}

kda_status kda_prefill_backward(
    const void *q, const void *k, const void *v, kda_dtype qkv_dtype,
    const void *g, const void *beta, kda_dtype gate_dtype, const float *s0,
    const void *dO, const float *dsT, void *dq, void *dk, void *dv, void *dg,
    void *dbeta, float *ds0, int B, int T, int H, int Dk, int Dv, int chunk,
    float scale, void *workspace, size_t workspace_bytes, void *stream) {
  kda::PrefillParams p;
  kda_status st = prefill_check(q, k, v, qkv_dtype, g, beta, gate_dtype, B, T,
                                H, Dk, Dv, chunk, scale, nullptr, true, p);
  if (st != KDA_OK) return st;
  const void *outs[] = {dq, dk, dv, dg, dbeta};
  for (const void *o : outs)
    if (!o || !aligned16(o)) return KDA_EINVAL;
  if (!dO || !workspace || !aligned16(dO) || !aligned16(workspace))
    return KDA_EINVAL;
  const void *opt[] = {s0, dsT, ds0};
  for (const void *o : opt)
    if (o && !aligned16(o)) return KDA_EINVAL;
  // no output may alias an input or another output
  const void *ins[] = {q, k, v, g, beta, s0, dO, dsT};
  const void *all_out[] = {dq, dk, dv, dg, dbeta, ds0};
  for (int i = 0; i < 6; ++i) {
    if (!all_out[i]) continue;
    for (const void *x : ins)
      if (x && x == all_out[i]) return KDA_EINVAL;
    for (int j = i + 1; j < 6; ++j)
      if (all_out[j] == all_out[i]) return KDA_EINVAL;
  }
  if (!kda::backward_fits(qkv_dtype == KDA_BF16, Dk, p.C))
    return KDA_EUNSUPPORTED;
  const BwdWs L = bwd_ws(B, T, H, Dk, Dv, chunk, qkv_dtype);
  if (workspace_bytes < L.total) return KDA_EINVAL;
  char *wsb = (char *)workspace;
  const int bf = qkv_dtype == KDA_BF16;
  hipStream_t s = (hipStream_t)stream;
  // recompute the forward, keeping the state at every chunk start
  p.s0 = s0;
  p.s_out = nullptr;
  p.o = wsb + L.o;
  p.ws = wsb;
  p.wsb = kda::ws_layout(Dk, Dv, p.C, bf ? 2 : 4).bytes;
  p.ckpt = (float *)(wsb + L.sc);
  p.train_at = (float *)(wsb + L.at);
  hipError_t e = kda::launch_prefill_prep(p, bf, s);
  if (e == hipSuccess) e = kda::launch_state_pass(p, bf, s);
  if (e != hipSuccess) return hip_status(e);
  kda::BwdParams bp{};
  bp.f = p;
  bp.f.ckpt = nullptr;
  bp.dO = dO;
  bp.dsT = dsT;
  bp.ds0 = ds0;
  bp.dD = (float *)(wsb + L.dd);
  bp.dSc = (float *)(wsb + L.dsc);
  bp.Sc = (const float *)(wsb + L.sc);
  bp.gs = (float *)(wsb + L.gs);
  bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dg; bp.dbeta = dbeta;
  return hip_status(kda::launch_backward(bp, bf, s));
}

kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           kda_dtype qkv_dtype, const void *g,
                           const void *beta, kda_dtype gate_dtype,
                           float *state, void *o, int N, int H, int Dk,
                           int Dv, float scale, void *stream) {
  if (N <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_EINVAL;
  if (!q || !k || !v || !g || !beta || !state || !o) return KDA_EINVAL;
  if (!dtype_valid(qkv_dtype) || !gate_valid(gate_dtype)) return KDA_EINVAL;
  if (!isfinite(scale)) return KDA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
      !aligned16(beta) || !aligned16(state) || !aligned16(o))
    return KDA_EINVAL;
  if (o == q || o == k || o == v || o == g || o == beta || o == state)
    return KDA_EINVAL;
  if (!dim_ok(Dk) || !dim_ok(Dv)) return KDA_EUNSUPPORTED;
  if (!pair_ok(qkv_dtype, gate_dtype)) return KDA_EUNSUPPORTED;
  if ((long long)N * H > 0x7fffffffLL) return KDA_EUNSUPPORTED;
  kda::DecodeParams p{};
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
  p.gate_bf16 = gate_base(gate_dtype) == KDA_BF16;
  p.gate_head = gate_head(gate_dtype);
  p.state_in = state; p.state_out = state; p.tstates = nullptr; p.o = o;
  p.N = N; p.L = 1; p.H = H; p.Dk = Dk; p.Dv = Dv; p.scale = scale;
  return hip_status(kda::launch_decode(p, qkv_dtype == KDA_BF16,
                                       (hipStream_t)stream));
}

kda_status kda_decode_tokens(const void *q, const void *k, const void *v,
                             kda_dtype qkv_dtype, const void *g,
                             const void *beta, kda_dtype gate_dtype,
                             const float *state_in, float *state_out,
                             float *token_states, void *o, int N, int L,
                             int H, int Dk, int Dv, float scale,
                             const kda_conv_desc *conv, float *conv_state,
                             float *conv_state_out, void *stream) {
  if (N <= 0 || L <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_EINVAL;
  if (!g || !beta || !state_in || !state_out || !o) return KDA_EINVAL;
  if (!conv && (!q || !k || !v)) return KDA_EINVAL;
  if (!conv && (conv_state || conv_state_out)) return KDA_EINVAL;
  if (conv_state_out == conv_state) conv_state_out = nullptr;  // in place
  if (conv) {
    if (!conv->xq || !conv->xk || !conv->xv || !conv->wq || !conv->wk ||
        !conv->wv)
      return KDA_EINVAL;
    if (conv->width < 2) return KDA_EINVAL;
    if (conv->l2norm_qk != 0 && conv->l2norm_qk != 1) return KDA_EINVAL;
    if (!(conv->eps >= 0.f) || !isfinite(conv->eps)) return KDA_EINVAL;
    const void *cp[] = {conv->xq, conv->xk, conv->xv, conv->wq, conv->wk,
                        conv->wv, conv_state, conv_state_out};
    for (const void *ptr : cp)
      if (ptr && !aligned16(ptr)) return KDA_EINVAL;
    if (conv->width > 4) return KDA_EUNSUPPORTED;
  }
  if (!dtype_valid(qkv_dtype) || !gate_valid(gate_dtype)) return KDA_EINVAL;
  if (!isfinite(scale)) return KDA_EINVAL;
  const void *ptrs[] = {q, k, v, g, beta, state_in, state_out, token_states, o};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_EINVAL;
  if ((q && o == q) || (k && o == k) || (v && o == v) || o == g ||
      o == beta || o == state_in || o == state_out ||
      (token_states && (token_states == state_in ||
                        token_states == state_out)))
    return KDA_EINVAL;
  if (conv && (o == conv->xq || o == conv->xk || o == conv->xv ||
               (conv_state && ((const void *)conv_state == o ||
                               conv_state == state_out)) ||
               (conv_state_out &&
                ((const void *)conv_state_out == o ||
                 conv_state_out == state_out ||
                 conv_state_out == state_in ||
                 (const void *)conv_state_out == conv->xq ||
                 (const void *)conv_state_out == conv->xk ||
                 (const void *)conv_state_out == conv->xv))))
    return KDA_EINVAL;
  if (!dim_ok(Dk) || !dim_ok(Dv)) return KDA_EUNSUPPORTED;
  if (!pair_ok(qkv_dtype, gate_dtype)) return KDA_EUNSUPPORTED;
  if ((long long)N * H > 0x7fffffffLL || (long long)N * L * H > 0x7fffffffLL)
    return KDA_EUNSUPPORTED;
  kda::DecodeParams p{};
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
  p.gate_bf16 = gate_base(gate_dtype) == KDA_BF16;
  p.gate_head = gate_head(gate_dtype);
  p.state_in = state_in; p.state_out = state_out; p.tstates = token_states;
  p.o = o;
  p.N = N; p.L = L; p.H = H; p.Dk = Dk; p.Dv = Dv; p.scale = scale;
  const int Dmax = Dk > Dv ? Dk : Dv;
  if (conv) {
    p.xq = conv->xq; p.xk = conv->xk; p.xv = conv->xv;
    p.wq = conv->wq; p.wk = conv->wk; p.wv = conv->wv;
    p.cw = conv->width; p.l2 = conv->l2norm_qk; p.eps = conv->eps;
    p.cstate = conv_state; p.cstate_out = conv_state_out; p.Dmax = Dmax;
  }
  hipError_t e = kda::launch_decode(p, qkv_dtype == KDA_BF16,
                                    (hipStream_t)stream);
  if (e != hipSuccess || !conv || !conv_state || conv_state_out)
    return hip_status(e);
  // in place: roll the conv history forward by the L raw inputs (after the
  // decode kernel has read the old history on the same stream)
  kda::ConvParams c{};
  c.x[0] = conv->xq; c.x[1] = conv->xk; c.x[2] = conv->xv;
  c.D[0] = Dk; c.D[1] = Dk; c.D[2] = Dv;
  c.B = N; c.T = L; c.H = H; c.W = conv->width;
  c.io_bf16 = qkv_dtype == KDA_BF16;
  c.state = conv_state; c.Dmax = Dmax;
  return hip_status(kda::launch_conv_cache(c, (hipStream_t)stream));
}

kda_status kda_conv_prologue(const void *xq, const void *xk, const void *xv,
                             kda_dtype dtype, const float *wq,
                             const float *wk, const float *wv, int width,
                             float *conv_state, void *q, void *k, void *v,
                             int B, int T, int H, int Dk, int Dv,
                             int l2norm_qk, float eps, void *stream) {
  if (B <= 0 || T <= 0 || H <= 0 || Dk <= 0 || Dv <= 0) return KDA_EINVAL;
  if (!xq || !xk || !xv || !wq || !wk || !wv || !q || !k || !v)
    return KDA_EINVAL;
  if (!dtype_valid(dtype)) return KDA_EINVAL;
  if (width < 2) return KDA_EINVAL;
  if (l2norm_qk != 0 && l2norm_qk != 1) return KDA_EINVAL;
  if (!(eps >= 0.f) || !isfinite(eps)) return KDA_EINVAL;
  const void *ptrs[] = {xq, xk, xv, wq, wk, wv, q, k, v, conv_state};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_EINVAL;
  if (q == xq || k == xk || v == xv) return KDA_EINVAL;
  if (width > 4 || !dim_ok(Dk) || !dim_ok(Dv)) return KDA_EUNSUPPORTED;
  if ((long long)B * 3 > 65535 || H > 65535) return KDA_EUNSUPPORTED;
  kda::ConvParams p{};
  p.x[0] = xq; p.x[1] = xk; p.x[2] = xv;
  p.w[0] = wq; p.w[1] = wk; p.w[2] = wv;
  p.y[0] = q; p.y[1] = k; p.y[2] = v;
  p.D[0] = Dk; p.D[1] = Dk; p.D[2] = Dv;
  p.B = B; p.T = T; p.H = H; p.W = width; p.l2 = l2norm_qk;
  p.io_bf16 = dtype == KDA_BF16;
  p.eps = eps;
  p.state = conv_state;
  p.Dmax = Dk > Dv ? Dk : Dv;
  return hip_status(kda::launch_conv(p, (hipStream_t)stream));
}

}  // extern "C"
