// kda_decode.hip -- recurrent KDA steps for N independent sequences: one
// token (the generation step) or L tokens at once (the verify step of
// speculative decoding).
//
// Per (sequence, head) and token, with e = exp(g) per key channel (see
// include/kda.h for the sources):
//   u = S^T (e * k)      value the decayed state predicts for k
//   y = S^T (e * q)      read-out of the decayed state
//   delta = beta (v - u)
//   S <- diag(e) S + k delta^T
//   o = scale (y + (q . k) delta)            (= scale S_new^T q)
// The state is the only large operand (Dk*Dv fp32 per head), so the kernel
// is an HBM stream: each workgroup loads its share of the state once with
// 16-byte non-temporal loads into registers, carries it through the L
// tokens there (reducing over rows through LDS), and writes it back once
// (plus once per token when the per-token states are asked for).  Every sum
// runs over rows (key channels) for a fixed value column, so a head's
// columns split over CS workgroups with no exchange between them; each
// takes 32 columns (128-byte row segments, 16 KiB at d_k = 128), which
// streams better than whole 64 KiB heads.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int DEC_THREADS = 256;

__device__ __forceinline__ float dec_gate(const void *p, size_t i, int bf) {
  return bf ? (float)((const bf16 *)p)[i] : ((const float *)p)[i];
}

// a channel's conv taps right-aligned into 4 (tap 3 multiplies the newest
// input) and its last 3 inputs before the first token (oldest first; from
// the history when given, zeros beyond it)
struct ConvLane {
  float w[4], h[3];
  __device__ void init(const float *taps, const float *hist, int W) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jj = j - (4 - W);
      w[j] = jj >= 0 ? taps[jj] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int mm = m - (3 - (W - 1));  // history entry of slot m
      h[m] = (hist && mm >= 0) ? hist[mm] : 0.f;
    }
  }
  // conv output for the next input x, then x joins the history
  __device__ float step(float x) {
    const float y = w[0] * h[0] + w[1] * h[1] + w[2] * h[2] + w[3] * x;
    h[0] = h[1];
    h[1] = h[2];
    h[2] = x;
    return y;
  }
};

template <typename IO, int DK, int DV, int CS, bool CONV>
__global__ __launch_bounds__(DEC_THREADS) void kda_decode(DecodeParams p) {
  constexpr int DVB = DV / CS;  // value columns of this workgroup
  constexpr int NQ = DVB / 4;   // column quads
  constexpr int NT = (NQ * DK < DEC_THREADS) ? NQ * DK : DEC_THREADS;
  constexpr int RG = NT / NQ;    // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  static_assert(RG * NQ == NT && RPT * RG == DK, "thread mapping");

  // per-token key-side vectors, double-buffered by token parity so the
  // next token's can be written while the state update still reads these
  __shared__ float s_ek[2][DK], s_eq[2][DK], s_e[2][DK], s_k[2][DK];
  __shared__ __attribute__((aligned(16))) float s_part[2][RG][DVB];
  __shared__ __attribute__((aligned(16))) float s_d[DVB];
  __shared__ float s_qk[DEC_THREADS / 64];
  __shared__ float s_l2[2][2][DEC_THREADS / 64];  // conv: q/k sums of squares

  const int tid = threadIdx.x;
  const int L = p.L, H = p.H;
  const size_t nh = blockIdx.x / CS;           // n * H + h
  const size_t n = nh / H, h = nh % H;
  const int c0 = (blockIdx.x % CS) * DVB;      // first value column
  const int q4 = tid % NQ, rg = tid / NQ;
  const size_t so = nh * DK * DV + c0;         // state offset of this share

  // 1. issue the state loads first: they are the whole cost
  f32x4 s[RPT];
  if (tid < NT) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RG * i;
      s[i] = __builtin_nontemporal_load(
          (const f32x4 *)(p.state_in + so + (size_t)row * DV + 4 * q4));
    }
  }
  // fused conv prologue: this thread's q/k channel (tid < DK) and value
  // column (tid < DVB) keep their taps and last inputs in registers
  ConvLane cq, ck, cv;
  if (CONV) {
    const int W = p.cw;
    const size_t hs = (size_t)H * p.Dmax * (W - 1);  // one stream's history
    const float *hist = p.cstate ? p.cstate + n * 3 * hs : nullptr;
    if (tid < DK) {
      const size_t ch = h * DK + tid;
      cq.init(p.wq + ch * W, hist ? hist + ch * (W - 1) : nullptr, W);
      ck.init(p.wk + ch * W, hist ? hist + hs + ch * (W - 1) : nullptr, W);
    }
    if (tid < DVB) {
      const size_t ch = h * DV + c0 + tid;
      cv.init(p.wv + ch * W, hist ? hist + 2 * hs + ch * (W - 1) : nullptr, W);
    }
  }
  for (int t = 0; t < L; ++t) {
    const int pb = t & 1;
    const size_t ti = (n * L + t) * H + h;     // (sequence, token, head)
    float qc = 0.f, kc = 0.f;
    if (CONV) {
      if (tid < DK) {
        qc = cq.step(to_f32(((const IO *)p.xq)[ti * DK + tid]));
        kc = ck.step(to_f32(((const IO *)p.xk)[ti * DK + tid]));
      }
      if (p.l2) {
        // per-head L2 norm of q and k
        float sq = qc * qc, sk = kc * kc;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          sq += __shfl_xor(sq, off, 64);
          sk += __shfl_xor(sk, off, 64);
        }
        if ((tid & 63) == 0) {
          s_l2[pb][0][tid >> 6] = sq;
          s_l2[pb][1][tid >> 6] = sk;
        }
        __syncthreads();
        sq = 0.f;
        sk = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_THREADS / 64; ++w) {
          sq += s_l2[pb][0][w];
          sk += s_l2[pb][1][w];
        }
        qc *= 1.f / sqrtf(sq + p.eps);
        kc *= 1.f / sqrtf(sk + p.eps);
      }
    }
    // 2. per-channel gate, decayed key and query
    float qk = 0.f;
    if (tid < DK) {
      const float e = __expf(dec_gate(p.g, ti * DK + tid, p.gate_bf16));
      const float kk = CONV ? kc : to_f32(((const IO *)p.k)[ti * DK + tid]);
      const float qq = CONV ? qc : to_f32(((const IO *)p.q)[ti * DK + tid]);
      s_e[pb][tid] = e;
      s_k[pb][tid] = kk;
      s_ek[pb][tid] = e * kk;
      s_eq[pb][tid] = e * qq;
      qk = qq * kk;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qk += __shfl_xor(qk, off, 64);
    if ((tid & 63) == 0) s_qk[tid >> 6] = qk;
    __syncthreads();

    // 3. partial column sums over this thread's rows
    if (tid < NT) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        u += s[i] * s_ek[pb][row];
        y += s[i] * s_eq[pb][row];
      }
      *(f32x4 *)&s_part[0][rg][4 * q4] = u;
      *(f32x4 *)&s_part[1][rg][4 * q4] = y;
    }
    __syncthreads();

    // 4. per column: delta and output
    if (tid < DVB) {
      float u = 0.f, y = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        u += s_part[0][r][tid];
        y += s_part[1][r][tid];
      }
      float qkt = 0.f;
#pragma unroll
      for (int w = 0; w < DEC_THREADS / 64; ++w) qkt += s_qk[w];
      const float bt = dec_gate(p.beta, ti, p.gate_bf16);
      const float vv =
          CONV ? cv.step(to_f32(((const IO *)p.xv)[ti * DV + c0 + tid]))
               : to_f32(((const IO *)p.v)[ti * DV + c0 + tid]);
      const float d = bt * (vv - u);
      s_d[tid] = d;
      ((IO *)p.o)[ti * DV + c0 + tid] = from_f32<IO>(p.scale * (y + qkt * d));
    }
    __syncthreads();

    // 5. S <- diag(e) S + k delta^T, in registers; optionally stored
    if (tid < NT) {
      const f32x4 d = *(const f32x4 *)&s_d[4 * q4];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        s[i] = s[i] * s_e[pb][row] + d * s_k[pb][row];
      }
      if (p.tstates) {
        float *ts = p.tstates + ti * DK * DV + c0;
#pragma unroll
        for (int i = 0; i < RPT; ++i)
          __builtin_nontemporal_store(
              s[i], (f32x4 *)(ts + (size_t)(rg + RG * i) * DV + 4 * q4));
      }
    }
  }
  // 6. the state after the last token
  if (tid < NT) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(
          s[i], (f32x4 *)(p.state_out + so + (size_t)(rg + RG * i) * DV +
                          4 * q4));
  }
}

template <typename IO, int DK, int DV>
static hipError_t dec_one(const DecodeParams &p, hipStream_t s) {
  // column split: 32 value columns (128-byte row segments) per workgroup
  // once a head's state exceeds 16 KiB
  constexpr int CS = (DK * DV * 4 > 16384 && DV >= 64) ? DV / 32 : 1;
  const dim3 grid((unsigned)(p.N * p.H) * CS);
  if (p.xq)
    hipLaunchKernelGGL((kda_decode<IO, DK, DV, CS, true>), grid,
                       dim3(DEC_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL((kda_decode<IO, DK, DV, CS, false>), grid,
                       dim3(DEC_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DK>
static hipError_t dec_dv(const DecodeParams &p, hipStream_t s) {
  switch (p.Dv) {
    case 16: return dec_one<IO, DK, 16>(p, s);
    case 32: return dec_one<IO, DK, 32>(p, s);
    case 64: return dec_one<IO, DK, 64>(p, s);
    case 128: return dec_one<IO, DK, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
static hipError_t dec_dk(const DecodeParams &p, hipStream_t s) {
  switch (p.Dk) {
    case 16: return dec_dv<IO, 16>(p, s);
    case 32: return dec_dv<IO, 32>(p, s);
    case 64: return dec_dv<IO, 64>(p, s);
    case 128: return dec_dv<IO, 128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams &p, int io_bf16, hipStream_t s) {
  return io_bf16 ? dec_dk<bf16>(p, s) : dec_dk<float>(p, s);
}

}  // namespace kda
