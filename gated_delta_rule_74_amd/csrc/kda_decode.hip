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
// tokens there (reducing over rows with lane shuffles, then over waves
// through LDS), and writes it back once
// (plus once per token when the per-token states are asked for).  Every sum
// runs over rows (key channels) for a fixed value column, so a head's
// columns split over CS workgroups with no exchange between them; each
// takes 32 columns (128-byte row segments, 16 KiB at d_k = 128), which
// streams better than whole 64 KiB heads.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int DEC_THREADS = 256;

// a gate or beta element as loaded (fp32 bits, or bf16 bits in the low
// half); converted only where it is used so a prefetch does not wait
__device__ __forceinline__ unsigned dec_raw(const void *p, size_t i, int bf) {
  return bf ? (unsigned)((const unsigned short *)p)[i]
            : ((const unsigned *)p)[i];
}
__device__ __forceinline__ float dec_val(unsigned raw, int bf) {
  return __uint_as_float(bf ? raw << 16 : raw);
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

// one token's inputs for this thread, as loaded: key channel tid's gate,
// query and key (tid < d_k), value column tid (tid < value columns), and
// the head's beta (raw projections in place of q, k, v with the conv)
template <typename IO>
struct TokIn {
  unsigned g, b;
  IO q, k, v;
};

template <typename IO, int DK, bool CONV>
__device__ __forceinline__ void load_tok(TokIn<IO> &r, const DecodeParams &p,
                                         size_t ti, int tid, int dvb,
                                         size_t vcol) {
  if (tid < DK) {
    r.g = dec_raw(p.g, p.gate_head ? ti : ti * DK + tid, p.gate_bf16);
    r.q = ((const IO *)(CONV ? p.xq : p.q))[ti * DK + tid];
    r.k = ((const IO *)(CONV ? p.xk : p.k))[ti * DK + tid];
  }
  if (tid < dvb) r.v = ((const IO *)(CONV ? p.xv : p.v))[vcol];
  r.b = dec_raw(p.beta, ti, p.gate_bf16);
}

template <typename IO, int DK, int DV, int CS, bool CONV>
__global__ __launch_bounds__(DEC_THREADS) void kda_decode(DecodeParams p) {
  constexpr int DVB = DV / CS;  // value columns of this workgroup
  constexpr int NQ = DVB / 4;   // column quads
  constexpr int NT = (NQ * DK < DEC_THREADS) ? NQ * DK : DEC_THREADS;
  constexpr int RG = NT / NQ;    // row groups
  constexpr int RPT = DK / RG;   // rows per thread
  constexpr int NW = NT / 64;    // waves holding state
  constexpr int WK = DK > 64 ? DK / 64 : 1;  // waves holding key channels
  static_assert(RG * NQ == NT && RPT * RG == DK && NW * 64 == NT &&
                    NQ < 64,
                "thread mapping");

  // per-token vectors, double-buffered by token parity: token t+1 writes
  // one set while the last readers of token t may still read the other
  __shared__ float s_e[2][DK], s_k[2][DK], s_ek[2][DK], s_eq[2][DK];
  __shared__ float s_v[2][DVB];
  __shared__ float s_red[2][3][WK];        // per wave: q.k, |q|^2, |k|^2
  __shared__ f32x4 s_part[2][2][NW][NQ];   // per wave: column sums u, y

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int L = p.L, H = p.H;
  // consecutive workgroups go to the 8 XCDs in turn; renumber so that the
  // CS column shares of a head run on one XCD one after another, which
  // keeps the head's DRAM pages and L2 lines on one die
  const unsigned G = gridDim.x, G8 = G & ~7u, b = blockIdx.x;
  const unsigned wid = b < G8 ? (b & 7) * (G8 >> 3) + (b >> 3) : b;
  const size_t nh = wid / CS;                  // n * H + h
  const size_t n = nh / H, h = nh % H;
  const int c0 = (wid % CS) * DVB;             // first value column
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
  // token inputs: token 0 now, then each next token one step ahead
  auto tok_index = [&](int t) { return (n * L + t) * H + h; };
  TokIn<IO> cur, nxt;
  load_tok<IO, DK, CONV>(cur, p, tok_index(0), tid, DVB,
                         tok_index(0) * DV + c0 + tid);
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
  const bool l2 = CONV && p.l2;

  for (int t = 0; t < L; ++t) {
    const int pb = t & 1;
    const size_t ti = tok_index(t);
    if (t + 1 < L)
      load_tok<IO, DK, CONV>(nxt, p, tok_index(t + 1), tid, DVB,
                             tok_index(t + 1) * DV + c0 + tid);

    // 2. per key channel: gate, key, decayed key and query (unnormalised
    //    with the conv: the per-head L2 factors come out of every sum)
    float qq = 0.f, kk = 0.f;
    if (tid < DK) {
      const float e = __expf(dec_val(cur.g, p.gate_bf16));
      kk = CONV ? ck.step(to_f32(cur.k)) : to_f32(cur.k);
      qq = CONV ? cq.step(to_f32(cur.q)) : to_f32(cur.q);
      s_e[pb][tid] = e;
      s_k[pb][tid] = kk;
      s_ek[pb][tid] = e * kk;
      s_eq[pb][tid] = e * qq;
    }
    if (tid < DVB)
      s_v[pb][tid] = CONV ? cv.step(to_f32(cur.v)) : to_f32(cur.v);
    if (wv < WK) {
      float a = qq * kk, b = qq * qq, c = kk * kk;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        a += __shfl_xor(a, off, 64);
        if (l2) {
          b += __shfl_xor(b, off, 64);
          c += __shfl_xor(c, off, 64);
        }
      }
      if (lane == 0) {
        s_red[pb][0][wv] = a;
        s_red[pb][1][wv] = b;
        s_red[pb][2][wv] = c;
      }
    }
    __syncthreads();

    // 3. column sums over this thread's rows, then over the wave's rows
    if (tid < NT) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int row = rg + RG * i;
        u += s[i] * s_ek[pb][row];
        y += s[i] * s_eq[pb][row];
      }
#pragma unroll
      for (int off = NQ; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u[c] += __shfl_xor(u[c], off, 64);
          y[c] += __shfl_xor(y[c], off, 64);
        }
      }
      if (lane < NQ) {
        s_part[pb][0][wv][lane] = u;
        s_part[pb][1][wv][lane] = y;
      }
    }
    __syncthreads();

    // 4. every thread finishes its own four columns: delta, the output
    //    (row group 0), and S <- diag(e) S + k delta^T in registers
    if (tid < NT) {
      f32x4 u = s_part[pb][0][0][q4], y = s_part[pb][1][0][q4];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        u += s_part[pb][0][w][q4];
        y += s_part[pb][1][w][q4];
      }
      float qk = s_red[pb][0][0], q2 = s_red[pb][1][0], k2 = s_red[pb][2][0];
#pragma unroll
      for (int w = 1; w < WK; ++w) {
        qk += s_red[pb][0][w];
        q2 += s_red[pb][1][w];
        k2 += s_red[pb][2][w];
      }
      float rq = 1.f, rk = 1.f;
      if (l2) {
        rq = l2_inv_norm(q2 + p.eps);
        rk = l2_inv_norm(k2 + p.eps);
      }
      const f32x4 vv = *(const f32x4 *)&s_v[pb][4 * q4];
      const float bt = dec_val(cur.b, p.gate_bf16);
      f32x4 d = bt * (vv - rk * u);
      if (rg == 0) {
        const f32x4 o = p.scale * (rq * y + (rq * rk * qk) * d);
        IO *dst = (IO *)p.o + ti * DV + c0 + 4 * q4;
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = from_f32<IO>(o[c]);
      }
      d *= rk;
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
    cur = nxt;
  }
  // 5. the state after the last token
  if (tid < NT) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(
          s[i], (f32x4 *)(p.state_out + so + (size_t)(rg + RG * i) * DV +
                          4 * q4));
  }
  // 6. the conv history rolled forward, into a buffer other than the one
  //    read: every column share of the head holds the whole q/k history, so
  //    share cg writes q/k channels [cg DK/CS, (cg+1) DK/CS) and each share
  //    its own value columns
  if (CONV && p.cstate_out) {
    const int W = p.cw;
    const size_t hs = (size_t)H * p.Dmax * (W - 1);
    float *out = p.cstate_out + n * 3 * hs;
    // slot m of the 3 kept inputs is history entry m - (4 - W); constant
    // slot indices keep the inputs in registers
    if (tid < DK && tid / (DK / CS) == (int)(wid % CS)) {
      const size_t base = (h * DK + tid) * (W - 1);
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= 4 - W) {
          const size_t e = base + (m - (4 - W));
          out[e] = cq.h[m];
          out[hs + e] = ck.h[m];
        }
    }
    if (tid < DVB) {
      const size_t base = 2 * hs + (h * DV + c0 + tid) * (W - 1);
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= 4 - W) out[base + (m - (4 - W))] = cv.h[m];
    }
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
