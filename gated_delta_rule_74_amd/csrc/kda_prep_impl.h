// kda_prep_impl.h -- chunk-local factors of the chunked KDA prefill (gfx950),
// instantiated per dtype pair by the kda_prep_*.hip files.
//
// Method (per head; see include/kda.h for the sources).  The token rule
//   S' = diag(e_t) S,  e_t = exp(g_t);  S_t = S' + k_t (beta_t (v_t - S'^T k_t))^T;
//   o_t = scale S_t^T q_t
// is evaluated over chunks of C tokens in its WY / UT-transform form.  With
// Gam_r the within-chunk running product of e and S0 the chunk's start state:
//   A[r,s] = beta_r sum_i k_ri k_si Gam_ri/Gam_si  (s<r),  T = (I + A)^-1
//   P[r,s] = scale sum_i q_ri k_si Gam_ri/Gam_si   (s<=r)
//   W = T diag(beta)(K*Gam),  U = T diag(beta) V
//   Delta = U - W S0,  O = scale (Q*Gam) S0 + P Delta,
//   S_C = diag(Gam_C) S0 + (K*Gam_C/Gam)^T Delta.
// This kernel computes every state-independent factor (-W, U, P,
// Qtil = scale Q*Gam, Ktil^T = (K*Gam_C/Gam)^T, Gam_C) of every
// (batch*head, chunk) and writes them to the workspace in matrix-core
// fragment order; kda_state_pass then runs the sequential part.
//
// Decay ratios are never formed as Gam_r / Gam_s.  Within a chunk they are
// products of e over (s, r], split at 16-token sub-chunk boundaries so every
// factor is a product of values <= 1 (no overflow; g = -inf gives an exact
// 0).  Only the 16x16 diagonal sub-blocks use a ratio (rho_r / rho_s against
// the sub-chunk start), and only when every such rho of the chunk is at
// least 2^-64; otherwise those blocks are summed directly with running
// products (exact and slow; reached only by extreme forgetting).
//
// Which kernel runs: bf16 q/k/v at d_k = d_v = 128 with 64-token chunks is
// served by kda_prep_d128.hip (per-channel gate, with or without the conv;
// eight waves per task) or kda_prep_gdn.hip (one gate per token-head); this
// generic kernel serves every other shape and dtype.
//
// Execution: a persistent grid (one workgroup of 256 threads per CU) walks
// the (batch*head, chunk) tasks, last chunk first: the state pass reads the
// chunks in order right afterwards, so its early chunks are the most
// recently written ones and tend to still sit in the memory-side cache.
// Thread t owns 4 consecutive key channels x 8 consecutive tokens of a task;
// its raw inputs are fetched with 8/16-byte vector loads into registers one
// task ahead, so the fetch of task i+1 overlaps the matrix-core phases of
// task i.  The chunk's betas (and, with the conv, the head's taps) are
// fetched the same way by a few lanes and handed to every thread through
// LDS.  Inputs (read once) and the workspace (written once) use streaming
// accesses, which keeps the L2 free of dirty lines for the state pass.
#pragma once
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int PREP_THREADS = 256;
constexpr int DVMAX = 128;
constexpr float SAFE_MIN = 5.42101086242752217e-20f;  // 2^-64

template <typename IO> struct Vec4;  // 4 IO values as raw bits
template <> struct Vec4<bf16> {
  typedef uint2 raw;
  __device__ static __forceinline__ void get(raw r, float *f) {
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xffff0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xffff0000u);
  }
  __device__ static __forceinline__ raw put(const float *f) {
    bf16x4 v = {(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3]};
    return __builtin_bit_cast(raw, v);
  }
};
template <> struct Vec4<float> {
  typedef uint4 raw;
  __device__ static __forceinline__ void get(raw r, float *f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
  __device__ static __forceinline__ raw put(const float *f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

template <typename IO, int DK, int C, bool CONV = false>
struct PL {  // prep LDS layout
  static constexpr int NB = C / 16, NKT = DK / 16, TPU = Mma<IO>::TPU;
  static constexpr int NKU = (NKT + TPU - 1) / TPU;
  static constexpr int NTU = (NB + TPU - 1) / TPU;
  static constexpr int KU = 16 * TPU;
  static constexpr int PE = 16 / (int)sizeof(IO);
  static constexpr int LDK = DK + PE;  // token-major rows [C][LDK]
  static constexpr int LDC = C + PE;   // channel-major rows [*][LDC]
  static constexpr int LDA = C + 4;    // fp32 rows
  static constexpr int NP2 = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 0;
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t TOK = al((size_t)C * LDK * sizeof(IO));
  // region A (tasks' phase E -> AP): row/column operands of A and P
  static constexpr size_t oKR = 0, oQR = TOK, oKS = 2 * TOK, oKIR = 3 * TOK;
  static constexpr size_t endA = 4 * TOK;
  // region D overlays A (phases T -> WU)
  static constexpr size_t oTt = 0;
  static constexpr size_t oTaa = al(oTt + (size_t)C * LDA * 4);
  static constexpr size_t oTb = al(oTaa + (size_t)NB * 256 * 4);
  static constexpr size_t oKG = al(oTb + (size_t)C * LDC * sizeof(IO));
  static constexpr size_t oVT = al(oKG + (size_t)DK * LDC * sizeof(IO));
  static constexpr size_t endD = al(oVT + (size_t)DVMAX * LDC * sizeof(IO));
  // A (fp32); during phase E of a fallback task it holds the raw q rows
  static constexpr size_t oAf = endA > endD ? endA : endD;
  static constexpr size_t AFB = al((size_t)C * LDA * 4) > TOK
                                    ? al((size_t)C * LDA * 4) : TOK;
  // raw k rows (the exact diagonal path reads them)
  static constexpr size_t oKraw = oAf + AFB;
  static constexpr size_t oF = al(oKraw + TOK);
  static constexpr size_t oM = al(oF + (size_t)NB * DK * 4);
  static constexpr size_t oFb = al(oM + (size_t)(NP2 ? NP2 : 1) * DK * 4);
  static constexpr size_t oVote = al(oFb + (size_t)2 * NB * 256 * 4);
  // channel-major copy of the k*sigma operand (bf16 only: the Ktil^T units
  // are assembled from it 16 bytes per lane)
  static constexpr size_t oKST = al(oVote + 64);
  // beta of the chunk's tokens (fp32), written at the end of the previous
  // task from one coalesced load
  static constexpr size_t oBeta =
      al(oKST + (TPU == 2 ? (size_t)DK * LDC * sizeof(IO) : 0));
  // conv taps of the chunk's head, right-aligned, one float4 per channel:
  // q channels, then k, then v (conv only); written like the betas
  static constexpr size_t oTap = al(oBeta + 64 * 4);
  static constexpr size_t total =
      oTap + (CONV ? (size_t)(2 * DK + DVMAX) * 16 : 0);
  __device__ static int p2(int a, int b) { return (a - 2) * (a - 1) / 2 + b; }
};

template <typename IO, bool CONV> struct Stage {
  static constexpr int XR = CONV ? 11 : 8;  // rows of q/k/v (conv: +3 halo)
  typename Vec4<IO>::raw xq[XR], xk[XR], xv[XR];
  uint4 g[8];
  uint32_t beta;  // wave 0: beta of token lane of the chunk (raw bits)
  f32x4 tap[CONV ? 2 : 1];  // conv: taps of channel items tid, tid + 256
};

// PART selects what to fetch: 1 = g and beta, 2 = q, 4 = k, 8 = v; the parts
// are issued in different phases of the previous task so the vector memory
// queue drains between them.  beta is one coalesced load by wave 0 (token =
// lane), later written to LDS for both the K and the V side.
template <int PART, typename IO, typename GT, int DK, int C, bool CONV>
__device__ __forceinline__ void prep_load(const PrefillParams &p, int task,
                                          Stage<IO, CONV> &st, int tid) {
  constexpr int NQ = DK / 4, NTG = C / 8;
  constexpr bool GB = sizeof(GT) == 2;  // bf16 gates
  typedef typename Vec4<IO>::raw R;
  const int BH = p.B * p.H;
  const int bh = task % BH, n = p.NC - 1 - task / BH;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T, H = p.H, Dv = p.Dv;
  const int t0 = n * C;
  const int tlast = T - 1;
  const size_t tok0 = (size_t)b * T;  // first token row of batch b
  // 64-bit bases of (batch b, head h) and 64-bit row offsets (a batch
  // may hold more than 2^32 elements)
  const size_t kb = (tok0 * H + h) * DK;
  const size_t rowK = (size_t)H * DK;
  if ((PART & 1) && tid < 64) {
    const size_t bi = (tok0 + (unsigned)min(t0 + tid, tlast)) * H + h;
    st.beta = GB ? (uint32_t)((const unsigned short *)p.beta)[bi]
                 : ((const unsigned *)p.beta)[bi];
  }
  if constexpr (CONV) {
    // the head's taps: item = q channel, DK + k channel, 2 DK + v channel
    // (fetched with the last part: they are live only until the task ends)
    if (PART & 8) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int it = tid + PREP_THREADS * r;
        if (it >= 2 * DK + Dv) break;
        const float *w = it < DK ? p.wq + ((size_t)h * DK + it) * p.cw
                       : it < 2 * DK ? p.wk + ((size_t)h * DK + it - DK) * p.cw
                                     : p.wv + ((size_t)h * Dv + it - 2 * DK) * p.cw;
        if (p.cw == 4) {
          st.tap[r] = *(const f32x4 *)w;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jj = i - (4 - p.cw);
            st.tap[r][i] = (jj >= 0) ? w[jj] : 0.f;
          }
        }
      }
    }
  }
  if (tid < NQ * NTG) {
    const int cq = tid % NQ, tg = tid / NQ;
    const float *gf = (const float *)p.g + kb + 4 * cq;
    const bf16 *gh = (const bf16 *)p.g + kb + 4 * cq;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!(PART & 1)) break;
      const unsigned t = (unsigned)min(t0 + 8 * tg + i, tlast);
      if (p.gate_head) {
        // one gate per (token, head): kept as loaded in .x, widened in E1
        const size_t gi = (tok0 + t) * H + h;
        st.g[i].x = GB ? (unsigned)((const unsigned short *)p.g)[gi]
                       : ((const unsigned *)p.g)[gi];
      } else if (GB) {
        const uint2 v = ld_stream<uint2>(gh + (size_t)t * rowK);
        st.g[i] = make_uint4(v.x, v.y, 0u, 0u);
      } else {
        st.g[i] = ld_stream<uint4>(gf + (size_t)t * rowK);
      }
    }
    const IO *xq = (const IO *)(CONV ? p.xq : p.q) + kb + 4 * cq;
    const IO *xk = (const IO *)(CONV ? p.xk : p.k) + kb + 4 * cq;
#pragma unroll
    for (int i = 0; i < Stage<IO, CONV>::XR; ++i) {
      const unsigned t =
          (unsigned)min(max(t0 + 8 * tg + i - (CONV ? 3 : 0), 0), tlast);
      if (PART & 2) st.xq[i] = ld_stream<R>(xq + (size_t)t * rowK);
      if (PART & 4) st.xk[i] = ld_stream<R>(xk + (size_t)t * rowK);
    }
  }
  const int NQV = Dv / 4;
  if ((PART & 8) && tid < NQV * NTG) {
    const int cv = tid % NQV, tg = tid / NQV;
    const size_t rowV = (size_t)H * Dv;
    const IO *xv = (const IO *)(CONV ? p.xv : p.v) + (tok0 * H + h) * Dv +
                   4 * cv;
#pragma unroll
    for (int i = 0; i < Stage<IO, CONV>::XR; ++i) {
      const unsigned t =
          (unsigned)min(max(t0 + 8 * tg + i - (CONV ? 3 : 0), 0), tlast);
      st.xv[i] = ld_stream<R>(xv + (size_t)t * rowV);
    }
  }
}

// Channel-major operand rows ([channel][token], LDC elements per row): the
// 4-element blocks of row r are stored XOR-swizzled by r / 4.  The
// transposed writes of phases E1 and T0 (a wave's lanes write the same block
// of rows 4 apart) then spread over the LDS banks instead of piling onto a
// few, and the k-contiguous unit reads stay conflict-free.
template <int C>
__device__ __forceinline__ int cm_off(int row, int col) {
  constexpr int M = C / 4 - 1;  // blocks per row - 1, a power of two
  return (((col >> 2) ^ ((row >> 2) & M)) << 2) | (col & 3);
}
// operand unit (k = k0 ...) from swizzled channel-major row `row`
template <typename IO, int C>
__device__ __forceinline__ typename Mma<IO>::frag load_k_cm(const IO *rowp,
                                                            int row, int k0,
                                                            int g,
                                                            bool full) {
  if constexpr (sizeof(IO) == 2) {
    const bf16x4 lo = *(const bf16x4 *)(rowp + cm_off<C>(row, k0 + 4 * g));
    const bf16x4 hi =
        full ? *(const bf16x4 *)(rowp + cm_off<C>(row, k0 + 16 + 4 * g))
             : bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  } else {
    return *(const f32x4 *)(rowp + cm_off<C>(row, k0 + 4 * g));
  }
}

// block j of the A/P sub-block list: (aa, bb), bb <= aa.  With four
// sub-chunks the order spreads the four costly blocks (the three that need
// mid products, and the last row) over the four waves.
template <int NB>
__device__ __forceinline__ void ap_block(int j, int &aa, int &bb) {
  if constexpr (NB == 4) {
    switch (j) {
      case 0: aa = 0; bb = 0; break;
      case 1: aa = 1; bb = 0; break;
      case 2: aa = 2; bb = 0; break;
      case 3: aa = 3; bb = 0; break;
      case 4: aa = 3; bb = 3; break;
      case 5: aa = 1; bb = 1; break;
      case 6: aa = 2; bb = 1; break;
      case 7: aa = 3; bb = 1; break;
      case 8: aa = 3; bb = 2; break;
      default: aa = 2; bb = 2; break;
    }
  } else {
    aa = 0;
    while (j > aa) {
      j -= aa + 1;
      ++aa;
    }
    bb = j;
  }
}


template <typename IO, typename GT, int DK, int C, bool CONV>
__global__ __launch_bounds__(PREP_THREADS, 1) void kda_chunk_prep(
    PrefillParams p) {
  using L = PL<IO, DK, C, CONV>;
  using M = Mma<IO>;
  using V4 = Vec4<IO>;
  typedef typename M::frag frag;
  constexpr int NB = L::NB, NKT = L::NKT, TPU = L::TPU, NKU = L::NKU,
                NTU = L::NTU, KU = L::KU, LDK = L::LDK, LDC = L::LDC,
                LDA = L::LDA;
  constexpr int NQ = DK / 4, NTG = C / 8, XR = Stage<IO, CONV>::XR;
  constexpr int XO = CONV ? 3 : 0;  // first own row inside the x window
  constexpr bool GB = sizeof(GT) == 2;  // bf16 gates

  __shared__ __attribute__((aligned(16))) char sm[L::total];
  IO *Xkr = (IO *)(sm + L::oKR), *Xqr = (IO *)(sm + L::oQR);
  IO *Xks = (IO *)(sm + L::oKS), *Xkir = (IO *)(sm + L::oKIR);
  float *Tt = (float *)(sm + L::oTt), *Taa = (float *)(sm + L::oTaa);
  IO *Tb = (IO *)(sm + L::oTb), *XkgT = (IO *)(sm + L::oKG);
  IO *XvT = (IO *)(sm + L::oVT);
  float *Af = (float *)(sm + L::oAf);
  IO *Aq = (IO *)(sm + L::oAf);  // raw q rows until phase AP
  IO *Kraw = (IO *)(sm + L::oKraw);
  float *Fs = (float *)(sm + L::oF), *Mid = (float *)(sm + L::oM);
  float *FbA = (float *)(sm + L::oFb), *FbP = FbA + NB * 256;
  int *votes = (int *)(sm + L::oVote);
  IO *XksT = (IO *)(sm + L::oKST);  // [DK][LDC], bf16 only
  float *betas = (float *)(sm + L::oBeta);  // [64], token of the chunk
  f32x4 *taps = (f32x4 *)(sm + (CONV ? L::oTap : 0));  // conv only

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, m16 = lane & 15;
  const int BH = p.B * p.H, T = p.T, H = p.H, Dv = p.Dv, nvt = Dv / 16;
  const int ntask = BH * p.NC;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  const bool kthr = tid < NQ * NTG;
  const int cq = tid % NQ, tg = tid / NQ;
  const int c0 = 4 * cq, r0 = 8 * tg;
  const int a = r0 / 16, half = (r0 / 8) & 1;
  const int NQV = Dv / 4;
  const bool vthr = tid < NQV * NTG;
  const int cv = tid % NQV, tgv = tid / NQV;

  Stage<IO, CONV> st;
  int task = blockIdx.x;
  if (task < ntask) prep_load<15, IO, GT, DK, C, CONV>(p, task, st, tid);
  // wave 0 moves the staged betas of a task into LDS
  auto put_beta = [&]() {
    if (wave == 0)
      betas[lane] = GB ? __uint_as_float(st.beta << 16)
                       : __uint_as_float(st.beta);
    if constexpr (CONV) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (tid + PREP_THREADS * r < 2 * DK + Dv)
          taps[tid + PREP_THREADS * r] = st.tap[r];
    }
  };
  if (task < ntask) put_beta();
  __syncthreads();

  for (; task < ntask; task += gridDim.x) {
    const int bh = task % BH, n = p.NC - 1 - task / BH;
    const int b = bh / H, h = bh % H;
    const int t0 = n * C;
    char *blk = p.ws + ((size_t)bh * p.NC + n) * p.wsb;

    // ---- E1: decay, running products within the sub-chunk, conv + L2 -----
    // Writes the A/P operands (region A), raw k/q rows and F_a; rho and
    // sigma are running products written out as they are formed.
    int vote = 0;
    float F[4] = {1.f, 1.f, 1.f, 1.f};
    // raw k and q rows (packed as stored): only the exact fallback reads
    // them, so they go to LDS after B1 and only when the vote asks for it
    typename V4::raw kraw[8], qraw[8];
    if (kthr) {
      float e[8][4], kk[8][4], qq[8][4], bt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = t0 + r0 + i < T;
        float gv[4];
        if (GB)
          Vec4<bf16>::get(make_uint2(st.g[i].x, st.g[i].y), gv);
        else
          Vec4<float>::get(st.g[i], gv);
        bt[i] = ok ? betas[r0 + i] : 0.f;
        if (p.gate_head) {
          // the head's one gate, shared by the 4 channels: one exp
          const float e0 =
              ok ? __expf(__uint_as_float(GB ? st.g[i].x << 16 : st.g[i].x))
                 : 1.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) e[i][j] = e0;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) e[i][j] = ok ? __expf(gv[j]) : 1.f;
        }
      }
      if (CONV) {
        f32x4 tq[4], tk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tq[j] = taps[c0 + j];
          tk[j] = taps[DK + c0 + j];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float sq = 0.f, sk = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) { qq[i][j] = 0.f; kk[i][j] = 0.f; }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = t0 + r0 + i + u - XO;
            const bool ok = t >= 0 && t < T;
            float xq[4], xk[4];
            V4::get(st.xq[i + u], xq);
            V4::get(st.xk[i + u], xk);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              qq[i][j] += ok ? tq[j][u] * xq[j] : 0.f;
              kk[i][j] += ok ? tk[j][u] * xk[j] : 0.f;
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sq += qq[i][j] * qq[i][j];
            sk += kk[i][j] * kk[i][j];
          }
          if (p.l2) {
            // per-token sum over the head: the NQ lanes sharing this token
            sq = group_sum<NQ>(sq);
            sk = group_sum<NQ>(sk);
            const float iq = l2_inv_norm(sq + p.eps);
            const float ik = l2_inv_norm(sk + p.eps);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              qq[i][j] *= iq;
              kk[i][j] *= ik;
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          V4::get(st.xq[i], qq[i]);
          V4::get(st.xk[i], kk[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = r0 + i;
        if (t0 + r >= T)
#pragma unroll
          for (int j = 0; j < 4; ++j) qq[i][j] = kk[i][j] = 0.f;
        if constexpr (CONV) {
          kraw[i] = V4::put(kk[i]);
          qraw[i] = V4::put(qq[i]);
        }
      }
      // this thread's 8-token product, then the other half of the 16-token
      // sub-chunk (lane ^ NQ) for the cross terms
      float ltp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lt = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) lt *= e[i][j];
        ltp[j] = __shfl_xor(lt, NQ, 64);
        F[j] = lt * ltp[j];
      }
      // forward: rho = inclusive prefix within the sub-chunk
      {
        float pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[j] = half ? ltp[j] : 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = r0 + i;
          float xkr[4], xqr[4], xki[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pr[j] *= e[i][j];
            if (!(pr[j] >= SAFE_MIN)) vote = 1;
            xkr[j] = bt[i] * kk[i][j] * pr[j];
            xqr[j] = p.scale * qq[i][j] * pr[j];
            xki[j] = kk[i][j] * __builtin_amdgcn_rcpf(pr[j]);
          }
          *(typename V4::raw *)(Xkr + r * LDK + c0) = V4::put(xkr);
          *(typename V4::raw *)(Xqr + r * LDK + c0) = V4::put(xqr);
          *(typename V4::raw *)(Xkir + r * LDK + c0) = V4::put(xki);
        }
      }
      // backward: sigma = exclusive suffix within the sub-chunk
      {
        float sf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sf[j] = half ? 1.f : ltp[j];
        float xkc[4][8];  // the same values by channel
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          const int r = r0 + i;
          float xks[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xks[j] = kk[i][j] * sf[j];
            xkc[j][i] = xks[j];
            sf[j] *= e[i][j];
          }
          *(typename V4::raw *)(Xks + r * LDK + c0) = V4::put(xks);
        }
        if constexpr (TPU == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(typename V4::raw *)(XksT + (c0 + j) * LDC +
                                  cm_off<C>(c0 + j, r0)) =
                V4::put(&xkc[j][0]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(typename V4::raw *)(XksT + (c0 + j) * LDC +
                                  cm_off<C>(c0 + j, r0 + 4)) =
                V4::put(&xkc[j][4]);
        }
      }
      if (!half) *(f32x4 *)(Fs + a * DK + c0) = f32x4{F[0], F[1], F[2], F[3]};
    }
    // beta * V for the W/U phase (V side)
    float bv[8][4];
    if (vthr) {
      float bvt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = t0 + 8 * tgv + i < T;
        bvt[i] = ok ? betas[8 * tgv + i] : 0.f;
      }
      if (CONV) {
        f32x4 tv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) tv[j] = taps[2 * DK + 4 * cv + j];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[i][j] = 0.f;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = t0 + 8 * tgv + i + u - XO;
            const bool ok = t >= 0 && t < T;
            float xv[4];
            V4::get(st.xv[i + u], xv);
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[i][j] += ok ? tv[j][u] * xv[j] : 0.f;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[i][j] *= bvt[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float vv[4];
          V4::get(st.xv[i], vv);
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[i][j] = bvt[i] * vv[j];
        }
      }
    }
    {
      const unsigned long long bal = __ballot(vote);
      if (lane == 0) votes[wave] = bal != 0ull;
    }
    __syncthreads();  // B1: region A, Fs, votes

    // ---- E2: Qtil and Ktil^T units, gamma_C, beta K Gam for W ------------
    // the next task's g and beta (this task's were last read in E1) go out
    // first, ahead of this phase's workspace stores
    const bool more = task + (int)gridDim.x < ntask;
    if (more) prep_load<1, IO, GT, DK, C, CONV>(p, task + gridDim.x, st, tid);
    const bool fallback =
        (votes[0] | votes[1] | votes[2] | votes[3]) != 0;
    if (fallback) {  // read after B2 by the exact diagonal sums
      for (int i = tid; i < 2 * NB * 64; i += PREP_THREADS)
        ((f32x4 *)FbA)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (CONV && kthr) {  // without the conv they are read from q and k
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          *(typename V4::raw *)(Kraw + (r0 + i) * LDK + c0) = kraw[i];
          *(typename V4::raw *)(Aq + (r0 + i) * LDK + c0) = qraw[i];
        }
      }
    }
    float kgb[8][4];
    if (kthr) {
      float fpre[4], fsuf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) { fpre[j] = 1.f; fsuf[j] = 1.f; }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const f32x4 f = *(const f32x4 *)(Fs + bb * DK + c0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (bb < a) fpre[j] *= f[j];
          if (bb > a) fsuf[j] *= f[j];
        }
      }
      typename V4::raw rkr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rkr[i] = *(const typename V4::raw *)(Xkr + (r0 + i) * LDK + c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float xkr[4];
        V4::get(rkr[i], xkr);
#pragma unroll
        for (int j = 0; j < 4; ++j) kgb[i][j] = xkr[j] * fpre[j];
      }
      if constexpr (TPU == 1) {
        // fp32 units: a lane's 16-byte slot is 4 consecutive k, which this
        // thread holds, so it stores its own Qtil and Ktil^T values
        const int ct = c0 / 16;
        float kt[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = r0 + i;
          float xqr[4], xks[4], qt[4];
          V4::get(*(const typename V4::raw *)(Xqr + r * LDK + c0), xqr);
          V4::get(*(const typename V4::raw *)(Xks + r * LDK + c0), xks);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            qt[j] = xqr[j] * fpre[j];
            kt[i][j] = xks[j] * fsuf[j];
          }
          const int u = c0 / KU, gq = (c0 % KU) / 4;
          const int ln = (r & 15) + 16 * gq;
          st_stream(blk + W.off_qt + ((size_t)(a * NKU + u) * 64 + ln) * 16,
                    V4::put(qt));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = c0 + j;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int rr = r0 + 4 * hh;  // first token of the run
            const int u = rr / KU, gq = (rr % KU) / 4;
            const int ln = (c & 15) + 16 * gq;
            float v4[4] = {kt[4 * hh + 0][j], kt[4 * hh + 1][j],
                           kt[4 * hh + 2][j], kt[4 * hh + 3][j]};
            st_stream(blk + W.off_ktt + ((size_t)(ct * NTU + u) * 64 + ln) * 16,
                      V4::put(v4));
          }
        }
      }
      if (a == NB - 1 && half == 1) {
        *(f32x4 *)((float *)(blk + W.off_gam) + c0) =
            f32x4{fpre[0] * F[0], fpre[1] * F[1], fpre[2] * F[2],
                  fpre[3] * F[3]};
      }
    }
    if constexpr (TPU == 2) {
      // bf16 units: a lane's 16-byte slot holds k = 4g..4g+3 and
      // 16+4g..16+4g+3 of its unit, which two different threads produced in
      // E1, so the slots are assembled here from LDS and written whole (one
      // coalesced 1 KiB store per unit).  Values beyond d_k or the chunk
      // (an odd number of 16-wide tiles) are zero.
      constexpr int NW4 = PREP_THREADS / 64;
      constexpr bool QHI = DK > 16;  // the unit's upper 16 channels exist
      constexpr bool KHI = C > 16;   // the unit's upper 16 tokens exist
      // every load below is unconditional (all addresses lie inside the
      // arrays) so the compiler can batch them ahead of the arithmetic
#pragma unroll
      for (int it = 0; it < (NB * NKU + NW4 - 1) / NW4; ++it) {
        // Qtil = scale Q*Gam: row tile aa (sub-chunk aa), channel unit u
        const int w = wave + NW4 * it;
        if constexpr ((NB * NKU) % NW4 != 0) {
          if (w >= NB * NKU) break;
        }
        const int aa = w / NKU, u = w % NKU;
        const int tok = 16 * aa + m16;
        const int ch0 = KU * u + 4 * g4, ch1 = QHI ? ch0 + 16 : ch0;
        f32x4 f0 = {1.f, 1.f, 1.f, 1.f}, f1 = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int bb = 0; bb < NB - 1; ++bb) {
          const f32x4 l0 = *(const f32x4 *)(Fs + bb * DK + ch0);
          const f32x4 l1 = *(const f32x4 *)(Fs + bb * DK + ch1);
          if (bb < aa) {
            f0 *= l0;
            f1 *= l1;
          }
        }
        float x0[4], x1[4], y0[4], y1[4];
        V4::get(*(const typename V4::raw *)(Xqr + tok * LDK + ch0), x0);
        V4::get(*(const typename V4::raw *)(Xqr + tok * LDK + ch1), x1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y0[j] = x0[j] * f0[j];
          y1[j] = QHI ? x1[j] * f1[j] : 0.f;
        }
        const typename V4::raw lo = V4::put(y0), up = V4::put(y1);
        st_stream(blk + W.off_qt + ((size_t)(aa * NKU + u) * 64 + lane) * 16,
                  make_uint4(lo.x, lo.y, up.x, up.y));
      }
#pragma unroll
      for (int it = 0; it < (NKT * NTU + NW4 - 1) / NW4; ++it) {
        // Ktil^T = (K*Gam_C/Gam)^T: channel tile ct, token unit u
        const int w = wave + NW4 * it;
        if constexpr ((NKT * NTU) % NW4 != 0) {
          if (w >= NKT * NTU) break;
        }
        const int ct = w / NTU, u = w % NTU;
        const int ch = 16 * ct + m16;
        const int tk0 = KU * u + 4 * g4, tk1 = KHI ? tk0 + 16 : tk0;
        const int a0 = 2 * u;  // sub-chunk of tk0; tk1 lies in a0 + 1
        float fl[NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) fl[bb] = Fs[bb * DK + ch];
        float s0 = 1.f, s1 = 1.f;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          if (bb > a0) s0 *= fl[bb];
          if (bb > a0 + 1) s1 *= fl[bb];
        }
        float x0[4], x1[4], y0[4], y1[4];
        V4::get(*(const typename V4::raw *)(XksT + ch * LDC +
                                            cm_off<C>(ch, tk0)), x0);
        V4::get(*(const typename V4::raw *)(XksT + ch * LDC +
                                            cm_off<C>(ch, tk1)), x1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y0[j] = x0[j] * s0;
          y1[j] = KHI ? x1[j] * s1 : 0.f;
        }
        const typename V4::raw lo = V4::put(y0), up = V4::put(y1);
        st_stream(blk + W.off_ktt + ((size_t)(ct * NTU + u) * 64 + lane) * 16,
                  make_uint4(lo.x, lo.y, up.x, up.y));
      }
    }
    // mid products M_{b->a} = prod_{b<d<a} F_d for sub-chunk pairs a-b >= 2
    if (L::NP2 > 0) {
      for (int i = tid; i < L::NP2 * DK; i += PREP_THREADS) {
        const int c = i % DK, pi = i / DK;
        int aa = 2, bb = pi;
        while (bb >= aa - 1) { bb -= aa - 1; ++aa; }
        float mp = 1.f;
        for (int d = bb + 1; d < aa; ++d) mp *= Fs[d * DK + c];
        Mid[pi * DK + c] = mp;
      }
    }
    __syncthreads();  // B2: region A complete

    // the next task's q, k and v follow while this one runs on the matrix
    // cores, a part per phase (one phase later with the conv, whose staged
    // rows hold three more tokens and so more registers)
    if constexpr (!CONV)
      if (more) prep_load<2, IO, GT, DK, C, CONV>(p, task + gridDim.x, st, tid);

    if (fallback) {
      // exact diagonal-block sums: task (sub-chunk a, column s, 16 channels)
      const size_t tokb = (size_t)b * T;
      for (int w = tid; w < NB * 16 * (DK / 16); w += PREP_THREADS) {
        const int cg = w % (DK / 16), s = (w / (DK / 16)) % 16,
                  aa = w / (16 * (DK / 16));
        float pr[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) pr[c] = 1.f;
        for (int r = s; r < 16; ++r) {
          const int tr = t0 + 16 * aa + r;
          const int trc = min(tr, T - 1);
          float sa = 0.f, sp = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const int ch = cg * 16 + c;
            if (r > s) {
              const size_t gi = p.gate_head ? (tokb + trc) * H + h
                                            : ((tokb + trc) * H + h) * DK + ch;
              const float gv = GB ? (float)((const bf16 *)p.g)[gi]
                                           : ((const float *)p.g)[gi];
              pr[c] *= (tr < T) ? __expf(gv) : 1.f;
            }
            float ks, kr, qr;
            if constexpr (CONV) {
              ks = to_f32(Kraw[(16 * aa + s) * LDK + ch]);
              kr = to_f32(Kraw[(16 * aa + r) * LDK + ch]);
              qr = to_f32(Aq[(16 * aa + r) * LDK + ch]);
            } else {  // raw k, q of the input rows, zero beyond the sequence
              const int ts = t0 + 16 * aa + s;
              const size_t ob = ((tokb + min(ts, T - 1)) * H + h) * DK + ch;
              const size_t orr = ((tokb + trc) * H + h) * DK + ch;
              ks = ts < T ? to_f32(((const IO *)p.k)[ob]) : 0.f;
              kr = tr < T ? to_f32(((const IO *)p.k)[orr]) : 0.f;
              qr = tr < T ? to_f32(((const IO *)p.q)[orr]) : 0.f;
            }
            sa += kr * ks * pr[c];
            sp += qr * ks * pr[c];
          }
          const float br = (tr < T)
              ? (GB ? (float)((const bf16 *)p.beta)[(tokb + trc) * H + h]
                             : ((const float *)p.beta)[(tokb + trc) * H + h])
              : 0.f;
          if (r > s) atomicAdd(&FbA[(aa * 16 + r) * 16 + s], br * sa);
          atomicAdd(&FbP[(aa * 16 + r) * 16 + s], p.scale * sp);
        }
      }
      __syncthreads();
    }

    // ---- AP: A^T and P^T sub-blocks on the matrix cores --------------------
    // the NB(NB+1)/2 blocks (aa, bb <= aa) are dealt to the waves in an
    // order that evens out their cost (blocks two or more sub-chunks apart
    // also scale an operand by the mid products)
    // consecutive blocks of a wave often share their row sub-chunk: its
    // k and q operands are then kept rather than read again (not with the
    // conv, whose build has no registers to spare for them)
    frag kf[NKU], qf[NKU];
    int row_aa = -1;
    for (int j = wave; j < NB * (NB + 1) / 2; j += PREP_THREADS / 64) {
      int aa, bb;
      ap_block<NB>(j, aa, bb);
      if (CONV || aa != row_aa) {
        row_aa = aa;
        const IO *kb = Xkr + (16 * aa + m16) * LDK;
        const IO *qb = Xqr + (16 * aa + m16) * LDK;
#pragma unroll
        for (int u = 0; u < NKU; ++u) {
          const bool full = (TPU == 1) || (TPU * u + 1 < NKT);
          kf[u] = M::load_k(kb + KU * u, g4, full);
          qf[u] = M::load_k(qb + KU * u, g4, full);
        }
      }
      {
        const bool diag = (aa == bb);
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
        if (diag && fallback) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            accA[j] = FbA[(aa * 16 + m16) * 16 + 4 * g4 + j];
            accP[j] = FbP[(aa * 16 + m16) * 16 + 4 * g4 + j];
          }
        } else {
          const IO *cb = (diag ? Xkir : Xks) + (16 * bb + m16) * LDK;
          const float *mid =
              (aa - bb >= 2) ? Mid + L::p2(aa, bb) * DK : nullptr;
          frag cf[NKU];
#pragma unroll
          for (int u = 0; u < NKU; ++u) {
            const bool full = (TPU == 1) || (TPU * u + 1 < NKT);
            cf[u] = M::load_k(cb + KU * u, g4, full);
          }
#pragma unroll
          for (int u = 0; u < NKU; ++u) {
            if (mid) {
#pragma unroll
              for (int ee = 0; ee < M::NE; ++ee) {
                const int kx = KU * u + M::koff(g4, ee);
                if (kx < DK) M::set(cf[u], ee, M::elem(cf[u], ee) * mid[kx]);
              }
            }
            accA = M::mma(cf[u], kf[u], accA);
            accP = M::mma(cf[u], qf[u], accP);
          }
        }
        // lane (n = m16, g4): element j is row 16aa + m16, col 16bb + 4g4 + j
        if (diag) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int sc = 4 * g4 + j;
            if (!(sc < m16)) accA[j] = 0.f;
            if (!(sc <= m16)) accP[j] = 0.f;
          }
        }
        *(f32x4 *)(Af + (16 * aa + m16) * LDA + 16 * bb + 4 * g4) = accA;
        {
          const int u = bb / TPU, hf = bb % TPU;
          char *dst = blk + W.off_p + ((size_t)(aa * NTU + u) * 64 + lane) * 16 +
                      hf * 4 * sizeof(IO);
          const float a4[4] = {accP[0], accP[1], accP[2], accP[3]};
          st_stream(dst, V4::put(a4));
          if (TPU == 2 && diag && (aa % 2) == 0) {
            const float z[4] = {0.f, 0.f, 0.f, 0.f};
            *(typename V4::raw *)(dst + 4 * sizeof(IO)) = V4::put(z);
          }
        }
      }
    }
    __syncthreads();  // B3: region A no longer read
    if (more) {
      if constexpr (CONV)
        prep_load<2, IO, GT, DK, C, CONV>(p, task + gridDim.x, st, tid);
      else
        prep_load<4, IO, GT, DK, C, CONV>(p, task + gridDim.x, st, tid);
    }

    // ---- T0: W/U inputs into the freed region, T zero-filled --------------
    // W/U read T in whole token units: with 32-token (bf16) units the upper
    // block (r, r+1) of every even token tile r is read and must be zero;
    // every other block they read is written by T1/T2
    if constexpr (TPU == 2) {
      static_assert((LDC * sizeof(IO)) % 16 == 0, "Tb rows");
      for (int i = tid; i < (NB / 2) * 32; i += PREP_THREADS) {
        const int rt = 2 * (i / 32), row = (i % 32) / 2, hv = i % 2;
        *(uint4 *)(Tb + (16 * rt + row) * LDC + 16 * (rt + 1) + 8 * hv) =
            make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (kthr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo[4] = {kgb[0][j], kgb[1][j], kgb[2][j], kgb[3][j]};
        float hi[4] = {kgb[4][j], kgb[5][j], kgb[6][j], kgb[7][j]};
        IO *row = XkgT + (c0 + j) * LDC;
        *(typename V4::raw *)(row + cm_off<C>(c0 + j, r0)) = V4::put(lo);
        *(typename V4::raw *)(row + cm_off<C>(c0 + j, r0 + 4)) = V4::put(hi);
      }
    }
    if (vthr) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo[4] = {bv[0][j], bv[1][j], bv[2][j], bv[3][j]};
        float hi[4] = {bv[4][j], bv[5][j], bv[6][j], bv[7][j]};
        IO *row = XvT + (4 * cv + j) * LDC;
        *(typename V4::raw *)(row + cm_off<C>(4 * cv + j, 8 * tgv)) =
            V4::put(lo);
        *(typename V4::raw *)(row + cm_off<C>(4 * cv + j, 8 * tgv + 4)) =
            V4::put(hi);
      }
    }
    __syncthreads();  // B4
    if constexpr (CONV)
      if (more) prep_load<4, IO, GT, DK, C, CONV>(p, task + gridDim.x, st, tid);

    // ---- T1: inverse of each unit-lower 16x16 diagonal block (fp32) ------
    // With L the strictly lower block (L^16 = 0),
    //   (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8),
    // all polynomials in L, so they commute: T = (I + L^8)((I + L^4)((I + L^2)
    // (I - L))).  One wave per block on the fp32 matrix cores.  A product of
    // two matrices given in operand form yields the second-operand form of
    // the result; the first-operand form of X equals the second-operand form
    // of X^T, so both forms of L^2 and L^4 come from products of L and L^T.
    f32x4 Tcol[NB];  // Tcol[j] = T_{w+j, w} of this wave's column w (B form)
    if (wave < NB) {
      const int aa = wave;
      const float *ab = Af + (16 * aa) * LDA + 16 * aa;
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      const f32x4 LA = *(const f32x4 *)(ab + m16 * LDA + 4 * g4);
      f32x4 LB, Y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        LB[j] = ab[(4 * g4 + j) * LDA + m16];
        Y[j] = ((4 * g4 + j) == m16 ? 1.f : 0.f) - LB[j];  // I - L
      }
      const f32x4 L2B = mma16_f32(LA, LB, z4);   // L^2
      const f32x4 L2A = mma16_f32(LB, LA, z4);   // (L^2)^T: first form of L^2
      const f32x4 L4B = mma16_f32(L2A, L2B, z4);
      const f32x4 L4A = mma16_f32(L2B, L2A, z4);
      const f32x4 L8A = mma16_f32(L4B, L4A, z4);
      Y = mma16_f32(L2A, Y, Y);
      Y = mma16_f32(L4A, Y, Y);
      Y = mma16_f32(L8A, Y, Y);
      // lane (g4, m16) holds T_aa[4 g4 + j][m16]
      Tcol[0] = Y;
      *(f32x4 *)(Tt + (16 * aa + m16) * LDA + 16 * aa + 4 * g4) = Y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Taa[(aa * 16 + 4 * g4 + j) * 16 + m16] = Y[j];
        Tb[(16 * aa + 4 * g4 + j) * LDC + 16 * aa + m16] = from_f32<IO>(Y[j]);
      }
    }
    __syncthreads();
    // ---- T2: off-diagonal blocks, one block column per wave ---------------
    //   T_ab = -T_aa * sum_{c=b}^{a-1} A_ac T_cb   (fp32 matrix cores)
    // Column b needs only its own earlier blocks T_cb, which the wave keeps
    // in registers (a product's result is the next product's B operand),
    // and the diagonal inverses of T1: one barrier for the whole phase.
    if (wave < NB) {
      const int bb = wave;
#pragma unroll
      for (int k = 1; k < NB; ++k) {
        if (bb + k >= NB) break;
        const int aa = bb + k;
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < k; ++j) {
          const f32x4 af = *(const f32x4 *)(Af + (16 * aa + m16) * LDA +
                                            16 * (bb + j) + 4 * g4);
          X = mma16_f32(af, Tcol[j], X);
        }
        const f32x4 ta = *(const f32x4 *)(Taa + (aa * 16 + m16) * 16 + 4 * g4);
        const f32x4 Tn = -mma16_f32(ta, X, f32x4{0.f, 0.f, 0.f, 0.f});
        Tcol[k] = Tn;
        // lane (n = m16, g4) holds T_ab[4g4 + j][m16]
        *(f32x4 *)(Tt + (16 * bb + m16) * LDA + 16 * aa + 4 * g4) = Tn;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Tb[(16 * aa + 4 * g4 + j) * LDC + 16 * bb + m16] = from_f32<IO>(Tn[j]);
      }
    }
    __syncthreads();

    if (more) prep_load<8, IO, GT, DK, C, CONV>(p, task + gridDim.x, st, tid);
    if (p.train_at) {
      // for the backward pass: A = diag(beta) M and T^T, fp32
      float *dst = p.train_at + ((size_t)bh * p.NC + n) * 2 * C * C;
      for (int i = tid; i < C * C; i += PREP_THREADS) {
        const int r = i / C, c = i % C;
        dst[i] = Af[r * LDA + c];
        dst[C * C + i] = Tt[r * LDA + c];
      }
    }
    // ---- WU: -W (A-operand units) and U (accumulator tiles) ----------------
    // wave rt takes token tile rt: its rows of T are read once and serve
    // every key unit of W and its value slabs of U
    auto load_t = [&](int rt, frag *tb) {
      const int umax = (16 * rt + 15) / KU;  // last token unit T row rt uses
#pragma unroll
      for (int uu = 0; uu < NTU; ++uu) {
        const bool fullT = (TPU == 1) || (TPU * uu + 1 < NB);
        tb[uu] = M::load_k(Tb + (16 * rt + m16) * LDC + KU * min(uu, umax), g4,
                           fullT);
      }
    };
    auto u_tiles = [&](int rt, const frag *tb, int v0, int v1) {
      const int umax = (16 * rt + 15) / KU;
      for (int vt = v0; vt < v1; ++vt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        frag vb[NTU];
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu) {
          const bool fullT = (TPU == 1) || (TPU * uu + 1 < NB);
          vb[uu] = load_k_cm<IO, C>(XvT + (16 * vt + m16) * LDC, 16 * vt + m16,
                                    KU * uu, g4, fullT);
        }
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          if (uu <= umax) acc = M::mma(tb[uu], vb[uu], acc);
        IO *dst = (IO *)(blk + W.off_u) +
                  ((size_t)(vt * NB + rt) * 64 + lane) * 4;
        float a4[4] = {acc[0], acc[1], acc[2], acc[3]};
        st_stream(dst, V4::put(a4));
      }
    };
    for (int rt = wave; rt < NB; rt += PREP_THREADS / 64) {
      const int umax = (16 * rt + 15) / KU;  // last token unit T row rt uses
      frag tb[NTU];
      load_t(rt, tb);
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        frag xa[NTU][TPU];
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu) {
          const bool fullT = (TPU == 1) || (TPU * uu + 1 < NB);
#pragma unroll
          for (int hh = 0; hh < TPU; ++hh) {
            const int ct = (TPU * u + hh) % NKT;
            xa[uu][hh] = load_k_cm<IO, C>(XkgT + (16 * ct + m16) * LDC,
                                          16 * ct + m16, KU * uu, g4, fullT);
          }
        }
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          if (uu <= umax)
#pragma unroll
            for (int hh = 0; hh < TPU; ++hh)
              if (TPU * u + hh < NKT) acc[hh] = M::mma(xa[uu][hh], tb[uu], acc[hh]);
        const frag out = M::pack(-acc[0], -acc[1]);
        st_stream(blk + W.off_negw + ((size_t)(rt * NKU + u) * 64 + lane) * 16,
                  out);
      }
      if constexpr (TPU == 2 && NB == 4) {
        // token tiles 2 and 3 use two units of T against one for tiles 0
        // and 1, so waves 0 and 1 also take the first half of tiles 2 and
        // 3's value slabs: every wave then does the same number of products
        if (rt < 2) {
          u_tiles(rt, tb, 0, nvt);
          frag tb2[NTU];
          load_t(rt + 2, tb2);
          u_tiles(rt + 2, tb2, 0, nvt / 2);
        } else {
          u_tiles(rt, tb, nvt / 2, nvt);
        }
      } else {
        u_tiles(rt, tb, 0, nvt);
      }
    }
    if (more) put_beta();  // the current task's betas were last read in E1
    __syncthreads();  // B5: LDS free for the next task
  }
}

// ---------------------------------------------------------------------------
template <typename IO, int DK, int C>
struct Fits {
  static constexpr bool value = PL<IO, DK, C, true>::total <= 160 * 1024;
};

static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n <= 0)
    return 256;
  return n;
}

template <typename IO, typename GT, int DK, int C>
static hipError_t prep_one(const PrefillParams &p, hipStream_t s) {
  if constexpr (!Fits<IO, DK, C>::value) {
    return hipErrorInvalidValue;
  } else {
    const long long ntask = (long long)p.B * p.H * p.NC;
    const unsigned grid = (unsigned)std::min<long long>(ntask, cu_count());
    if (p.use_conv)
      hipLaunchKernelGGL((kda_chunk_prep<IO, GT, DK, C, true>), dim3(grid),
                         dim3(PREP_THREADS), 0, s, p);
    else
      hipLaunchKernelGGL((kda_chunk_prep<IO, GT, DK, C, false>), dim3(grid),
                         dim3(PREP_THREADS), 0, s, p);
    return hipGetLastError();
  }
}

template <typename IO, typename GT>
static hipError_t prep_dk(const PrefillParams &p, hipStream_t s) {
  switch (p.Dk * 1000 + p.C) {
    case 16016: return prep_one<IO, GT, 16, 16>(p, s);
    case 16032: return prep_one<IO, GT, 16, 32>(p, s);
    case 16064: return prep_one<IO, GT, 16, 64>(p, s);
    case 32016: return prep_one<IO, GT, 32, 16>(p, s);
    case 32032: return prep_one<IO, GT, 32, 32>(p, s);
    case 32064: return prep_one<IO, GT, 32, 64>(p, s);
    case 64016: return prep_one<IO, GT, 64, 16>(p, s);
    case 64032: return prep_one<IO, GT, 64, 32>(p, s);
    case 64064: return prep_one<IO, GT, 64, 64>(p, s);
    case 128016: return prep_one<IO, GT, 128, 16>(p, s);
    case 128032: return prep_one<IO, GT, 128, 32>(p, s);
    case 128064: return prep_one<IO, GT, 128, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
