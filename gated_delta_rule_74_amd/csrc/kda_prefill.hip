// kda_prefill.hip -- chunked KDA prefill on gfx950.
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
// Two kernels:
//   kda_chunk_prep  -- one workgroup per (head, chunk), all in parallel:
//                      decay products, A and P on the matrix cores, the
//                      triangular inverse T, then W and U; writes the
//                      state-independent factors to the workspace in
//                      matrix-core fragment order.
//   kda_state_pass  -- one wave per (head, 16 value columns): the sequential
//                      chunk loop; the state lives in registers as
//                      accumulator tiles and every product is one MFMA chain.
// Decay ratios are never formed as Gam_r / Gam_s.  Within a chunk they are
// products of e over (s, r], split at 16-token sub-chunk boundaries so that
// every factor is a product of values <= 1 (no overflow; g = -inf gives an
// exact 0).  Only the 16x16 diagonal sub-blocks use a ratio (rho_r / rho_s
// against the sub-chunk start), and only when every rho in the chunk is at
// least 2^-64; otherwise those blocks are summed directly with running
// products (an exact, slow path for extreme forgetting).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int PREP_THREADS = 256;
constexpr int DVMAX = 128;
constexpr float SAFE_MIN = 5.42101086242752217e-20f;  // 2^-64

__device__ __forceinline__ float ld_gate(const void *p, size_t i, int bf) {
  return bf ? (float)((const bf16 *)p)[i] : ((const float *)p)[i];
}

template <typename IO, int DK, int C> struct PL {  // prep LDS layout
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
  // region A: phase E -> AP
  static constexpr size_t oKR = 0, oQR = TOK, oKS = 2 * TOK, oKIR = 3 * TOK;
  static constexpr size_t endA = 4 * TOK;
  // region D overlays A: phases T -> WU
  static constexpr size_t oTt = 0;
  static constexpr size_t oTaa = al(oTt + (size_t)C * LDA * 4);
  static constexpr size_t oTb = al(oTaa + (size_t)NB * 256 * 4);
  static constexpr size_t oKG = al(oTb + (size_t)C * LDC * sizeof(IO));
  static constexpr size_t oVT = al(oKG + (size_t)DK * LDC * sizeof(IO));
  static constexpr size_t endD = al(oVT + (size_t)DVMAX * LDC * sizeof(IO));
  static constexpr size_t oAf = endA > endD ? endA : endD;
  static constexpr size_t oF = al(oAf + (size_t)C * LDA * 4);
  static constexpr size_t oFp = al(oF + (size_t)NB * DK * 4);
  static constexpr size_t oM = al(oFp + (size_t)NB * DK * 4);
  static constexpr size_t oFb = al(oM + (size_t)(NP2 ? NP2 : 1) * DK * 4);
  static constexpr size_t oL2 = al(oFb + (size_t)2 * NB * 256 * 4);
  static constexpr size_t oFlag = al(oL2 + (size_t)2 * NB * 2 * 16 * 4);
  static constexpr size_t total = oFlag + 16;
  // index of sub-chunk pair (a, b), a - b >= 2, into the mid-product table
  __device__ static int p2(int a, int b) { return (a - 2) * (a - 1) / 2 + b; }
};

// window conv for 16 consecutive tokens of one channel: x points at the
// channel in token 0, tokens are `ts` elements apart.
template <typename IO>
__device__ __forceinline__ void conv16(const IO *x, size_t ts, int tf, int T,
                                       const float *w, int W, float *y) {
  float win[19];
#pragma unroll
  for (int i = 0; i < 19; ++i) {
    const int t = tf - 3 + i;
    win[i] = (t >= 0 && t < T) ? to_f32(x[(size_t)t * ts]) : 0.f;
  }
  float w4[4];  // taps right-aligned so w4[3] multiplies the newest input
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = i - (4 - W);
    w4[i] = (j >= 0) ? w[j] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    y[i] = w4[0] * win[i] + w4[1] * win[i + 1] + w4[2] * win[i + 2] +
           w4[3] * win[i + 3];
}

template <typename IO, int DK, int C>
__global__ __launch_bounds__(PREP_THREADS) void kda_chunk_prep(
    PrefillParams p) {
  using L = PL<IO, DK, C>;
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int NB = L::NB, NKT = L::NKT, TPU = L::TPU, NKU = L::NKU,
                NTU = L::NTU, KU = L::KU, LDK = L::LDK, LDC = L::LDC,
                LDA = L::LDA;
  constexpr int NIT = (DK * NB + PREP_THREADS - 1) / PREP_THREADS;
  constexpr int NVIT = (DVMAX * NB + PREP_THREADS - 1) / PREP_THREADS;

  __shared__ __attribute__((aligned(16))) char sm[L::total];
  IO *Xkr = (IO *)(sm + L::oKR), *Xqr = (IO *)(sm + L::oQR);
  IO *Xks = (IO *)(sm + L::oKS), *Xkir = (IO *)(sm + L::oKIR);
  float *Tt = (float *)(sm + L::oTt), *Taa = (float *)(sm + L::oTaa);
  IO *Tb = (IO *)(sm + L::oTb), *XkgT = (IO *)(sm + L::oKG);
  IO *XvT = (IO *)(sm + L::oVT);
  float *Af = (float *)(sm + L::oAf), *Fs = (float *)(sm + L::oF);
  float *Fp = (float *)(sm + L::oFp), *Mid = (float *)(sm + L::oM);
  float *FbA = (float *)(sm + L::oFb), *FbP = FbA + NB * 256;
  float *L2s = (float *)(sm + L::oL2);
  int *flag = (int *)(sm + L::oFlag);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, m16 = lane & 15;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH, n = blockIdx.x / BH;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T, H = p.H, Dv = p.Dv, nvt = Dv / 16;
  const int t0 = n * C;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  char *blk = p.ws + ((size_t)bh * p.NC + n) * p.wsb;
  const size_t rowK = (size_t)H * DK, rowV = (size_t)H * Dv;
  const size_t tokbase = (size_t)b * T;  // token index base of batch b

  if (tid == 0) flag[0] = 0;
  for (int i = tid; i < 2 * NB * 256; i += PREP_THREADS) FbA[i] = 0.f;

  // ---- phase E, pass 1: gates, decay, (conv + L2 partials) ---------------
  float e[NIT][16], kv[NIT][16], qv[NIT][16], bt[NIT][16];
  int vote = 0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int item = tid + it * PREP_THREADS;
    if (item >= DK * NB) break;
    const int c = item % DK, a = item / DK;
    const int tf = t0 + 16 * a;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = tf + i;
      const bool ok = t < T;
      const size_t ik = ((tokbase + t) * H + h) * DK + c;
      const float gv = ok ? ld_gate(p.g, ik, p.gate_bf16) : 0.f;
      e[it][i] = __expf(gv);
      bt[it][i] = ok ? ld_gate(p.beta, (tokbase + t) * H + h, p.gate_bf16)
                     : 0.f;
      if (!p.use_conv) {
        kv[it][i] = ok ? to_f32(((const IO *)p.k)[ik]) : 0.f;
        qv[it][i] = ok ? to_f32(((const IO *)p.q)[ik]) : 0.f;
      }
    }
    float pr = 1.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pr *= e[it][i];
      if (i < 15 && !(pr >= SAFE_MIN)) vote = 1;
    }
    Fs[a * DK + c] = pr;
    if (p.use_conv) {
      const size_t xo = tokbase * rowK + (size_t)h * DK + c;
      conv16((const IO *)p.xq + xo, rowK, tf, T,
             p.wq + ((size_t)h * DK + c) * p.cw, p.cw, qv[it]);
      conv16((const IO *)p.xk + xo, rowK, tf, T,
             p.wk + ((size_t)h * DK + c) * p.cw, p.cw, kv[it]);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (tf + i >= T) qv[it][i] = kv[it][i] = 0.f;
      if (p.l2) {
        // sums of squares over the head's channels: butterfly within groups
        // of min(DK,64) lanes (one sub-chunk, consecutive channels), then
        // up to two partials per token through LDS
        constexpr int GS = DK < 64 ? DK : 64;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float sq = qv[it][i] * qv[it][i], sk = kv[it][i] * kv[it][i];
#pragma unroll
          for (int off = GS / 2; off >= 1; off >>= 1) {
            sq += __shfl_xor(sq, off, 64);
            sk += __shfl_xor(sk, off, 64);
          }
          if ((c % GS) == 0) {
            const int part = c / 64;
            L2s[((0 * NB + a) * 2 + part) * 16 + i] = sq;
            L2s[((1 * NB + a) * 2 + part) * 16 + i] = sk;
          }
        }
      }
    }
  }
  if (vote) flag[0] = 1;
  __syncthreads();
  const bool fallback = flag[0] != 0;

  // ---- phase E, pass 2: operands for A/P, K~^T, gamma, W/U inputs ---------
  float kgb[NIT][16];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int item = tid + it * PREP_THREADS;
    if (item >= DK * NB) break;
    const int c = item % DK, a = item / DK;
    if (p.use_conv && p.l2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sq = L2s[((0 * NB + a) * 2 + 0) * 16 + i];
        float sk = L2s[((1 * NB + a) * 2 + 0) * 16 + i];
        if (DK > 64) {
          sq += L2s[((0 * NB + a) * 2 + 1) * 16 + i];
          sk += L2s[((1 * NB + a) * 2 + 1) * 16 + i];
        }
        qv[it][i] *= 1.f / sqrtf(sq + p.eps);
        kv[it][i] *= 1.f / sqrtf(sk + p.eps);
      }
    }
    float fpre = 1.f, fsuf = 1.f;
    for (int bb = 0; bb < a; ++bb) fpre *= Fs[bb * DK + c];
    for (int bb = a + 1; bb < NB; ++bb) fsuf *= Fs[bb * DK + c];
    Fp[a * DK + c] = fpre;
    float rho[16], sig[16];
    {
      float pr = 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) { pr *= e[it][i]; rho[i] = pr; }
      float sf = 1.f;
#pragma unroll
      for (int i = 15; i >= 0; --i) { sig[i] = sf; sf *= e[it][i]; }
    }
    float kt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * a + i;
      const float kk = kv[it][i], qq = qv[it][i], bb = bt[it][i];
      Xkr[r * LDK + c] = from_f32<IO>(bb * kk * rho[i]);
      Xqr[r * LDK + c] = from_f32<IO>(p.scale * qq * rho[i]);
      Xks[r * LDK + c] = from_f32<IO>(kk * sig[i]);
      if (!fallback) Xkir[r * LDK + c] = from_f32<IO>(kk / rho[i]);
      kt[i] = kk * sig[i] * fsuf;
      kgb[it][i] = bb * kk * rho[i] * fpre;
    }
    // K~^T as A-operand units (rows = channels, k = tokens)
    {
      const int ct = c / 16, u = a / TPU, half = a % TPU;
      char *base = blk + W.off_ktt + ((size_t)(ct * NTU + u) * 64) * 16;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ln = (c % 16) + 16 * gq;
        IO *dst = (IO *)(base + ln * 16) + half * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = from_f32<IO>(kt[4 * gq + j]);
        if (TPU == 2 && a == NB - 1 && (a % 2) == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[4 + j] = from_f32<IO>(0.f);
        }
      }
    }
    if (a == 0) ((float *)(blk + W.off_gam))[c] = rho[15] * fsuf;
    if (fallback) {
      // exact diagonal-block sums with running products
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        float pr = 1.f;
        const float ks = kv[it][s];
#pragma unroll
        for (int r = s; r < 16; ++r) {
          if (r > s) pr *= e[it][r];
          const float w = ks * pr;
          if (r > s) atomicAdd(&FbA[(a * 16 + r) * 16 + s],
                               bt[it][r] * kv[it][r] * w);
          atomicAdd(&FbP[(a * 16 + r) * 16 + s], p.scale * qv[it][r] * w);
        }
      }
    }
  }
  // mid products M_{b->a} = prod_{b<d<a} F_d for sub-chunk pairs a-b >= 2
  if (L::NP2 > 0) {
    for (int i = tid; i < L::NP2 * DK; i += PREP_THREADS) {
      const int c = i % DK, pi = i / DK;
      int a = 2, bb = pi;
      while (bb >= a - 1) { bb -= a - 1; ++a; }
      float mp = 1.f;
      for (int d = bb + 1; d < a; ++d) mp *= Fs[d * DK + c];
      Mid[pi * DK + c] = mp;
    }
  }
  // beta * V items (conv: v = conv(xv))
  float bv[NVIT][16];
#pragma unroll
  for (int it = 0; it < NVIT; ++it) {
    const int item = tid + it * PREP_THREADS;
    if (item >= Dv * NB) break;
    const int c = item % Dv, a = item / Dv;
    const int tf = t0 + 16 * a;
    float vv[16];
    if (p.use_conv) {
      conv16((const IO *)p.xv + tokbase * rowV + (size_t)h * Dv + c, rowV,
             tf, T, p.wv + ((size_t)h * Dv + c) * p.cw, p.cw, vv);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = tf + i;
        vv[i] = (t < T) ? to_f32(((const IO *)p.v)[((tokbase + t) * H + h) *
                                                       Dv + c])
                        : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = tf + i;
      const float bb =
          (t < T) ? ld_gate(p.beta, (tokbase + t) * H + h, p.gate_bf16) : 0.f;
      bv[it][i] = bb * vv[i];
    }
  }
  __syncthreads();

  // ---- phase E-out: Q~ = scale Q*Gam as A-operand units -------------------
  for (int task = tid; task < NB * NKU * 64; task += PREP_THREADS) {
    const int l = task & 63, ru = task >> 6;
    const int rt = ru / NKU, u = ru % NKU;
    const int m = l & 15, g = l >> 4;
    const bool full = (TPU == 1) || (TPU * u + 1 < NKT);
    frag f = M::load_k(Xqr + (16 * rt + m) * LDK + KU * u, g, full);
    if (rt > 0) {
#pragma unroll
      for (int ee = 0; ee < M::NE; ++ee) {
        const int kk = KU * u + M::koff(g, ee);
        if (kk < DK) M::set(f, ee, M::elem(f, ee) * Fp[rt * DK + kk]);
      }
    }
    *(frag *)(blk + W.off_qt + ((size_t)(rt * NKU + u) * 64 + l) * 16) = f;
  }

  // ---- phase AP: A^T and P^T sub-blocks on the matrix cores ---------------
  for (int task = wave; task < NB * (NB + 1) / 2; task += PREP_THREADS / 64) {
    int a = 0, bb = task;
    while (bb > a) { bb -= a + 1; ++a; }
    const bool diag = (a == bb);
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
    if (diag && fallback) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        accA[j] = FbA[(a * 16 + m16) * 16 + 4 * g4 + j];
        accP[j] = FbP[(a * 16 + m16) * 16 + 4 * g4 + j];
      }
    } else {
      const IO *cb = (diag ? Xkir : Xks) + (16 * bb + m16) * LDK;
      const IO *kb = Xkr + (16 * a + m16) * LDK;
      const IO *qb = Xqr + (16 * a + m16) * LDK;
      const float *mid = (a - bb >= 2) ? Mid + L::p2(a, bb) * DK : nullptr;
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        const bool full = (TPU == 1) || (TPU * u + 1 < NKT);
        frag cf = M::load_k(cb + KU * u, g4, full);
        if (mid) {
#pragma unroll
          for (int ee = 0; ee < M::NE; ++ee) {
            const int kk = KU * u + M::koff(g4, ee);
            if (kk < DK) M::set(cf, ee, M::elem(cf, ee) * mid[kk]);
          }
        }
        accA = M::mma(cf, M::load_k(kb + KU * u, g4, full), accA);
        accP = M::mma(cf, M::load_k(qb + KU * u, g4, full), accP);
      }
    }
    // lane (n = m16, g4): element j holds row r = 16a + m16, col s = 16bb+4g4+j
    if (diag) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 4 * g4 + j;
        if (!(s < m16)) accA[j] = 0.f;
        if (!(s <= m16)) accP[j] = 0.f;
      }
    }
    *(f32x4 *)(Af + (16 * a + m16) * LDA + 16 * bb + 4 * g4) = accA;
    {
      const int u = bb / TPU, half = bb % TPU;
      IO *dst = (IO *)(blk + W.off_p + ((size_t)(a * NTU + u) * 64 + lane) *
                                           16) + half * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = from_f32<IO>(accP[j]);
      if (TPU == 2 && diag && (a % 2) == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[4 + j] = from_f32<IO>(0.f);
      }
    }
  }
  __syncthreads();

  // ---- phase T0: W/U inputs into the freed region, T zero-filled ----------
  for (int i = tid; i < C * LDC; i += PREP_THREADS) Tb[i] = from_f32<IO>(0.f);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int item = tid + it * PREP_THREADS;
    if (item >= DK * NB) break;
    const int c = item % DK, a = item / DK;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      XkgT[c * LDC + 16 * a + i] = from_f32<IO>(kgb[it][i]);
  }
#pragma unroll
  for (int it = 0; it < NVIT; ++it) {
    const int item = tid + it * PREP_THREADS;
    if (item >= Dv * NB) break;
    const int c = item % Dv, a = item / Dv;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      XvT[c * LDC + 16 * a + i] = from_f32<IO>(bv[it][i]);
  }
  __syncthreads();

  // ---- phase T1: inverse of each unit-lower 16x16 diagonal block (fp32) --
  if (tid < 16 * NB) {
    const int a = tid / 16, s = tid % 16;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
      const float *arow = Af + (16 * a + r) * LDA + 16 * a;
#pragma unroll
      for (int cc = 0; cc < r; ++cc) acc += arow[cc] * col[cc];
      col[r] = (r == s) ? 1.f : ((r < s) ? 0.f : -acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      Tt[(16 * a + s) * LDA + 16 * a + r] = col[r];
      Taa[(a * 16 + r) * 16 + s] = col[r];
      Tb[(16 * a + r) * LDC + 16 * a + s] = from_f32<IO>(col[r]);
    }
  }
  __syncthreads();
  // ---- phase T2: off-diagonal blocks, one block-diagonal at a time ---------
  //   T_ab = -T_aa * sum_{c=b}^{a-1} A_ac T_cb   (fp32 matrix cores)
  for (int d = 1; d < NB; ++d) {
    for (int task = wave; task < NB - d; task += PREP_THREADS / 64) {
      const int a = d + task, bb = task;
      f32x4 X = {0.f, 0.f, 0.f, 0.f};
      for (int cc = bb; cc < a; ++cc) {
        const f32x4 af = *(const f32x4 *)(Af + (16 * a + m16) * LDA + 16 * cc +
                                          4 * g4);
        const f32x4 tf = *(const f32x4 *)(Tt + (16 * bb + m16) * LDA +
                                          16 * cc + 4 * g4);
        X = mma16_f32(af, tf, X);
      }
      const f32x4 ta = *(const f32x4 *)(Taa + (a * 16 + m16) * 16 + 4 * g4);
      f32x4 R = mma16_f32(ta, X, f32x4{0.f, 0.f, 0.f, 0.f});
      // lane (n = m16, g4) holds T_ab[4g4 + j][m16]
      f32x4 Tn = -R;
      *(f32x4 *)(Tt + (16 * bb + m16) * LDA + 16 * a + 4 * g4) = Tn;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Tb[(16 * a + 4 * g4 + j) * LDC + 16 * bb + m16] = from_f32<IO>(Tn[j]);
    }
    __syncthreads();
  }

  // ---- phase WU: -W (A-operand units) and U (accumulator tiles) ------------
  const int nW = NB * NKU, nU = NB * nvt;
  for (int task = wave; task < nW + nU; task += PREP_THREADS / 64) {
    if (task < nW) {
      const int rt = task / NKU, u = task % NKU;
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      const int umax = (16 * rt + 15) / KU;
      for (int uu = 0; uu <= umax; ++uu) {
        const bool fullT = (TPU == 1) || (TPU * uu + 1 < NB);
        const frag tb = M::load_k(Tb + (16 * rt + m16) * LDC + KU * uu, g4,
                                  fullT);
#pragma unroll
        for (int hh = 0; hh < TPU; ++hh) {
          const int ct = TPU * u + hh;
          if (ct < NKT) {
            const frag xa = M::load_k(XkgT + (16 * ct + m16) * LDC + KU * uu,
                                      g4, fullT);
            acc[hh] = M::mma(xa, tb, acc[hh]);
          }
        }
      }
      const frag out = M::pack(-acc[0], -acc[1]);
      *(frag *)(blk + W.off_negw + ((size_t)(rt * NKU + u) * 64 + lane) *
                                       16) = out;
    } else {
      const int t2 = task - nW, rt = t2 / nvt, vt = t2 % nvt;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int umax = (16 * rt + 15) / KU;
      for (int uu = 0; uu <= umax; ++uu) {
        const bool fullT = (TPU == 1) || (TPU * uu + 1 < NB);
        const frag ta = M::load_k(Tb + (16 * rt + m16) * LDC + KU * uu, g4,
                                  fullT);
        const frag vb = M::load_k(XvT + (16 * vt + m16) * LDC + KU * uu, g4,
                                  fullT);
        acc = M::mma(ta, vb, acc);
      }
      IO *dst = (IO *)(blk + W.off_u) + ((size_t)(rt * nvt + vt) * 64 + lane) *
                                            4;
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = from_f32<IO>(acc[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// Sequential state pass: one wave per (batch*head, 16 value columns).
template <typename IO, int DK, int C>
__global__ __launch_bounds__(64) void kda_state_pass(PrefillParams p) {
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int NB = C / 16, NKT = DK / 16, TPU = M::TPU;
  constexpr int NKU = (NKT + TPU - 1) / TPU, NTU = (NB + TPU - 1) / TPU;
  const int lane = threadIdx.x, m16 = lane & 15, g4 = lane >> 4;
  const int Dv = p.Dv, nvt = Dv / 16, H = p.H, T = p.T;
  const int bh = blockIdx.x / nvt, vt = blockIdx.x % nvt;
  const int b = bh / H, h = bh % H;
  const int col = 16 * vt + m16;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  // state tile t: lane (n = m16, g4) holds S[16t + 4g4 + j][col]
  f32x4 S[NKT];
#pragma unroll
  for (int t = 0; t < NKT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[t][j] = p.s0 ? p.s0[((size_t)bh * DK + 16 * t + 4 * g4 + j) * Dv + col]
                     : 0.f;

  for (int n = 0; n < p.NC; ++n) {
    const char *blk = p.ws + ((size_t)bh * p.NC + n) * p.wsb;
    frag Sb[NKU];
#pragma unroll
    for (int u = 0; u < NKU; ++u)
      Sb[u] = M::pack(S[TPU * u], (TPU == 2 && TPU * u + 1 < NKT)
                                      ? S[(TPU * u + 1) % NKT]
                                      : zero);
    // Delta = U - W S0
    f32x4 D[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      const IO *up = (const IO *)(blk + W.off_u) +
                     ((size_t)(rt * nvt + vt) * 64 + lane) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) D[rt][j] = to_f32(up[j]);
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        const frag w = *(const frag *)(blk + W.off_negw +
                                       ((size_t)(rt * NKU + u) * 64 + lane) *
                                           16);
        D[rt] = M::mma(w, Sb[u], D[rt]);
      }
    }
    frag Db[NTU];
#pragma unroll
    for (int u = 0; u < NTU; ++u)
      Db[u] = M::pack(D[TPU * u], (TPU == 2 && TPU * u + 1 < NB)
                                      ? D[(TPU * u + 1) % NB]
                                      : zero);
    // O = Q~ S0 + P Delta
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      f32x4 O = zero;
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        const frag qf = *(const frag *)(blk + W.off_qt +
                                        ((size_t)(rt * NKU + u) * 64 + lane) *
                                            16);
        O = M::mma(qf, Sb[u], O);
      }
#pragma unroll
      for (int u = 0; u < NTU; ++u) {
        if (u <= rt / TPU) {
          const frag pf = *(const frag *)(blk + W.off_p +
                                          ((size_t)(rt * NTU + u) * 64 +
                                           lane) * 16);
          O = M::mma(pf, Db[u], O);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = n * C + 16 * rt + 4 * g4 + j;
        if (t < T)
          ((IO *)p.o)[(((size_t)b * T + t) * H + h) * Dv + col] =
              from_f32<IO>(O[j]);
      }
    }
    // S_C = diag(gamma_C) S0 + K~^T Delta
    const float *gam = (const float *)(blk + W.off_gam);
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const f32x4 gm = *(const f32x4 *)(gam + 16 * t + 4 * g4);
      S[t] *= gm;
#pragma unroll
      for (int u = 0; u < NTU; ++u) {
        const frag kf = *(const frag *)(blk + W.off_ktt +
                                        ((size_t)(t * NTU + u) * 64 + lane) *
                                            16);
        S[t] = M::mma(kf, Db[u], S[t]);
      }
    }
  }
  if (p.s_out) {
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p.s_out[((size_t)bh * DK + 16 * t + 4 * g4 + j) * Dv + col] = S[t][j];
  }
}

// ---------------------------------------------------------------------------
template <typename IO, int DK, int C>
static hipError_t prep_one(const PrefillParams &p, hipStream_t s) {
  const unsigned nblk = (unsigned)(p.B * p.H) * (unsigned)p.NC;
  hipLaunchKernelGGL((kda_chunk_prep<IO, DK, C>), dim3(nblk),
                     dim3(PREP_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DK, int C>
static hipError_t state_one(const PrefillParams &p, hipStream_t s) {
  const unsigned nblk = (unsigned)(p.B * p.H) * (unsigned)(p.Dv / 16);
  hipLaunchKernelGGL((kda_state_pass<IO, DK, C>), dim3(nblk), dim3(64), 0, s,
                     p);
  return hipGetLastError();
}

// fp32 q/k/v with Dk = 128 and chunk = 64 would need more than the 160 KiB
// of LDS a workgroup may use; the C ABI reports it as unsupported.
template <typename IO, int DK, int C>
struct Fits {
  static constexpr bool value = PL<IO, DK, C>::total <= 160 * 1024;
};

#define KDA_DISPATCH(FN)                                                    \
  template <typename IO>                                                    \
  static hipError_t FN##_dk(const PrefillParams &p, hipStream_t s) {        \
    switch (p.Dk * 1000 + p.C) {                                            \
      case 16016: return FN<IO, 16, 16>(p, s);                              \
      case 16032: return FN<IO, 16, 32>(p, s);                              \
      case 16064: return FN<IO, 16, 64>(p, s);                              \
      case 32016: return FN<IO, 32, 16>(p, s);                              \
      case 32032: return FN<IO, 32, 32>(p, s);                              \
      case 32064: return FN<IO, 32, 64>(p, s);                              \
      case 64016: return FN<IO, 64, 16>(p, s);                              \
      case 64032: return FN<IO, 64, 32>(p, s);                              \
      case 64064: return FN<IO, 64, 64>(p, s);                              \
      case 128016: return FN<IO, 128, 16>(p, s);                            \
      case 128032: return FN<IO, 128, 32>(p, s);                            \
      case 128064:                                                          \
        if constexpr (Fits<IO, 128, 64>::value)                             \
          return FN<IO, 128, 64>(p, s);                                     \
        break;                                                              \
    }                                                                       \
    return hipErrorInvalidValue;                                            \
  }

KDA_DISPATCH(prep_one)
KDA_DISPATCH(state_one)

hipError_t launch_prefill_prep(const PrefillParams &p, int io_bf16,
                               hipStream_t s) {
  return io_bf16 ? prep_one_dk<bf16>(p, s) : prep_one_dk<float>(p, s);
}

hipError_t launch_state_pass(const PrefillParams &p, int io_bf16,
                             hipStream_t s) {
  return io_bf16 ? state_one_dk<bf16>(p, s) : state_one_dk<float>(p, s);
}

}  // namespace kda
