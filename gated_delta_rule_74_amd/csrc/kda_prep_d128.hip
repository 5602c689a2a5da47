// kda_prep_d128.hip -- chunk prep of the chunked KDA prefill for one gate per
// key channel at bf16 q/k/v, d_k = d_v = 128 and 64-token chunks (gfx950),
// without the fused conv.
//
// It computes exactly the factors of kda_prep_impl.h (see there for the
// method, the decay-ratio splitting and the exact diagonal fallback) and
// writes them in the same workspace layout, so kda_state_pass consumes
// either.  What differs is the execution shape:
//
//  * Eight waves (512 threads, two waves per SIMD) work on one task instead
//    of four.  Every phase of a task is a short dependent chain (LDS reads,
//    matrix-core products, a barrier); with two waves per SIMD one wave's
//    waits overlap the other's issue.  The register budget that allows it
//    (at most 256 per lane) comes from giving each thread half the data.
//  * Wave w holds sub-chunk w / 2 (16 tokens) and key channels
//    64 (w % 2) .. 64 (w % 2) + 63; lane 32 h + c holds channels
//    64 (w % 2) + 2c, +1 of tokens 8h .. 8h + 7 of the sub-chunk.  The two
//    8-token halves of a sub-chunk sit in lanes l and l ^ 32 of one wave, so
//    the running decay products need no exchange through LDS.
//  * (beta V)^T and (beta K Gam)^T, the channel-major inputs of W and U,
//    have their own LDS and are written as soon as they are formed (phase
//    E1 and E2) instead of in a separate phase after the A/P products.
//  * A and P blocks are dealt out as 20 half-blocks (A or P of one 16x16
//    block), three or two per wave, so each SIMD does the same share; the W
//    and U products follow a fixed table that gives every wave 12 of the 96
//    matrix-core steps.
#include "kda_prep_impl.h"

namespace kda {
namespace pc {

constexpr int NT = 512, NW = NT / 64;
constexpr int DK = 128, DV = 128, C = 64;
constexpr int NB = 4, NKT = 8, NKU = 4, NTU = 2, NVT = 8, KU = 32;
constexpr int LDK = DK + 8;  // token-major bf16 rows [C][LDK]
constexpr int LDC = C + 8;   // channel-major bf16 rows [*][LDC]
constexpr int LDA = C + 4;   // fp32 rows [C][LDA]

// LDS layout (bytes).  Region A (E1 -> the P products) holds the row and
// column operands of A and P; region D (T1 -> WU: the diagonal inverses and
// T in bf16) overlays the rows of beta K rho, which only the A products
// read, so P and the Qtil / Ktil^T units can still run beside T1 and T2.
constexpr size_t TOK = (size_t)C * LDK * 2;
constexpr size_t oKR = 0, oKIR = TOK, oQR = 2 * TOK, oKS = 3 * TOK;
constexpr size_t oTaa = 0;                                 // diagonal T^T
constexpr size_t oTb = oTaa + (size_t)NB * 256 * 4;        // T bf16
static_assert(oTb + (size_t)C * LDC * 2 <= TOK, "region D inside beta K rho");
constexpr size_t oAf = 4 * TOK;                            // A fp32
constexpr size_t oFb = oAf + (size_t)C * LDA * 4;          // exact diagonals
constexpr size_t oKST = oFb + (size_t)2 * NB * 256 * 4;    // (K sigma)^T
constexpr size_t oKG = oKST + (size_t)DK * LDC * 2;        // (beta K Gam)^T
constexpr size_t oVT = oKG + (size_t)DK * LDC * 2;         // (beta V)^T
constexpr size_t oF = oVT + (size_t)DV * LDC * 2;          // F per sub-chunk
constexpr size_t oM = oF + (size_t)NB * DK * 4;            // mid products
constexpr size_t oVote = oM + (size_t)3 * DK * 4;
constexpr size_t oBeta = oVote + 64;
constexpr size_t LDS = oBeta + 64 * 4;
constexpr size_t oClaim = LDS;           // concurrent mode: the next task
constexpr size_t LDS_CO = oClaim + 16;
// with the fused conv: the head's taps (one f32x4 per q, k and v channel),
// per-token L2 scales of q and k (for the exact diagonal path), and the
// two channel halves' partial sums of squares
constexpr size_t oTap = LDS;
constexpr size_t oNrm = oTap + (size_t)(2 * DK + DV) * 16;
constexpr size_t oL2p = oNrm + (size_t)C * 2 * 4;
constexpr size_t LDS_CONV = oL2p + (size_t)NW * 16 * 2 * 4;
static_assert(LDS_CONV <= 160 * 1024, "one workgroup per CU");

// two bf16 values as raw bits
__device__ __forceinline__ void get2(uint32_t r, float &a, float &b) {
  a = __uint_as_float(r << 16);
  b = __uint_as_float(r & 0xffff0000u);
}
__device__ __forceinline__ uint32_t put2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t ld4_stream(const void *p) {
  return __builtin_nontemporal_load((const uint32_t *)p);
}

template <typename GT> struct GRaw;  // two gates as loaded
template <> struct GRaw<float> {
  typedef uint2 raw;
  __device__ static __forceinline__ raw load(const float *p) {
    return ld_stream<uint2>(p);
  }
  __device__ static __forceinline__ void get(raw r, float &a, float &b) {
    a = __uint_as_float(r.x);
    b = __uint_as_float(r.y);
  }
};
template <> struct GRaw<bf16> {
  typedef uint32_t raw;
  __device__ static __forceinline__ raw load(const bf16 *p) {
    return ld4_stream(p);
  }
  __device__ static __forceinline__ void get(raw r, float &a, float &b) {
    get2(r, a, b);
  }
};

// the next task's inputs, one task ahead in registers: 2 channels x 8 tokens
// of q, k, v and g per thread (with the conv: the raw projections and three
// earlier rows), and (wave 0) the chunk's betas, token = lane; with the
// conv, thread t < 384 also holds tap set t of the head
template <typename GT, bool CONV> struct Stage {
  static constexpr int XR = CONV ? 11 : 8;
  uint32_t q[XR], k[XR], v[XR];
  typename GRaw<GT>::raw g[8];
  uint32_t beta;
  f32x4 tap;
};

// task -> (batch*head, chunk): last chunk first (the state pass launched
// after the prep then finds its first chunks in the memory-side cache), or
// with CO first chunk first (the concurrent state pass consumes them in
// that order)
template <bool CO>
__device__ __forceinline__ int task_chunk(int task, int BH, int NC) {
  return CO ? task / BH : NC - 1 - task / BH;
}

// PART: 1 = g and beta, 2 = q, 4 = k, 8 = v (and the conv taps)
template <int PART, typename GT, bool CONV, bool CO>
__device__ __forceinline__ void load_task(const PrefillParams &p, int task,
                                          Stage<GT, CONV> &st, int tid, int c0,
                                          int r0) {
  constexpr int XR = Stage<GT, CONV>::XR, XO = CONV ? 3 : 0;
  const int BH = p.B * p.H;
  const int bh = task % BH, n = task_chunk<CO>(task, BH, p.NC);
  const int b = bh / p.H, h = bh % p.H, T = p.T, H = p.H;
  const int t0 = n * C, tlast = T - 1;
  const size_t tok0 = (size_t)b * T;
  const size_t kb = (tok0 * H + h) * DK + c0, rowK = (size_t)H * DK;
  if ((PART & 1) && tid < 64) {
    const size_t bi = (tok0 + (unsigned)min(t0 + tid, tlast)) * H + h;
    st.beta = sizeof(GT) == 2 ? (uint32_t)((const unsigned short *)p.beta)[bi]
                              : ((const unsigned *)p.beta)[bi];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const size_t t = (size_t)min(t0 + r0 + i, tlast);
    if (PART & 1) st.g[i] = GRaw<GT>::load((const GT *)p.g + kb + t * rowK);
  }
  const bf16 *xq = (const bf16 *)(CONV ? p.xq : p.q);
  const bf16 *xk = (const bf16 *)(CONV ? p.xk : p.k);
  const bf16 *xv = (const bf16 *)(CONV ? p.xv : p.v);
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const size_t t = (size_t)min(max(t0 + r0 + i - XO, 0), tlast);
    if (PART & 2) st.q[i] = ld4_stream(xq + kb + t * rowK);
    if (PART & 4) st.k[i] = ld4_stream(xk + kb + t * rowK);
    if (PART & 8)
      st.v[i] = ld4_stream(xv + (tok0 * H + h) * DV + c0 + t * (size_t)H * DV);
  }
  if constexpr (CONV) {
    // tap set `tid`: q channel, DK + k channel, 2 DK + v channel, right-
    // aligned (tap u multiplies the row u - 3 tokens back)
    if ((PART & 8) && tid < 2 * DK + DV) {
      const float *w = tid < DK ? p.wq + ((size_t)h * DK + tid) * p.cw
                     : tid < 2 * DK ? p.wk + ((size_t)h * DK + tid - DK) * p.cw
                                    : p.wv + ((size_t)h * DV + tid - 2 * DK) * p.cw;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = u - (4 - p.cw);
        st.tap[u] = jj >= 0 ? w[jj] : 0.f;
      }
    }
  }
}

// CO: the concurrent mode (no conv, no backward outputs).  Tasks are claimed
// one at a time from p.sync[SYNC_NEXT] in chunk order, so a workgroup that
// is not yet resident holds up nothing; the workspace is written with
// device-coherent stores; and once every wave has waited for its stores of
// a task (just before the next task's first barrier), thread 0 sets the
// task's ready flag for the state pass running beside the prep.
template <typename GT, bool CONV, bool CO>
__global__ __launch_bounds__(NT, 1) void kda_chunk_prep_d128(PrefillParams p) {
  static_assert(!(CO && CONV), "the concurrent mode has no conv");
  using M = Mma<bf16>;
  typedef M::frag frag;
  typedef Vec4<bf16>::raw R4;
  constexpr int XO = CONV ? 3 : 0;  // first own row inside the staged rows

  __shared__ __attribute__((aligned(16))) char sm[CONV ? LDS_CONV
                                                  : CO ? LDS_CO : LDS];
  int *claim = (int *)(sm + oClaim);  // CO only
  f32x4 *taps = (f32x4 *)(sm + oTap);  // conv only
  float *nrm = (float *)(sm + oNrm), *l2p = (float *)(sm + oL2p);
  bf16 *Xkr = (bf16 *)(sm + oKR), *Xqr = (bf16 *)(sm + oQR);
  bf16 *Xks = (bf16 *)(sm + oKS), *Xkir = (bf16 *)(sm + oKIR);
  float *Taa = (float *)(sm + oTaa);
  bf16 *Tb = (bf16 *)(sm + oTb);
  float *Af = (float *)(sm + oAf);
  float *FbA = (float *)(sm + oFb), *FbP = FbA + NB * 256;
  bf16 *XksT = (bf16 *)(sm + oKST), *XkgT = (bf16 *)(sm + oKG);
  bf16 *XvT = (bf16 *)(sm + oVT);
  float *Fs = (float *)(sm + oF), *Mid = (float *)(sm + oM);
  int *votes = (int *)(sm + oVote);
  float *betas = (float *)(sm + oBeta);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave0 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave0;
  const int g4 = lane >> 4, m16 = lane & 15;
  const int BH = p.B * p.H, T = p.T, H = p.H;
  const int ntask = BH * p.NC;
  constexpr WsLayout W = ws_layout(DK, DV, C, 2);  // offsets as immediates
  // this thread's share of a task: sub-chunk a, token half hh, 2 channels
  const int a = wave >> 1, hh = lane >> 5;
  const int c0 = 64 * (wave & 1) + 2 * (lane & 31);
  const int r0 = 16 * a + 8 * hh;
  constexpr bool GB = sizeof(GT) == 2;

  Stage<GT, CONV> st;
  int task = blockIdx.x;
  if constexpr (CO) {
    if (tid == 0)
      claim[0] = __hip_atomic_fetch_add(p.sync + SYNC_NEXT, 1,
                                        __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    task = claim[0];
  }
  int done = -1;  // CO, thread 0: flag index of the finished task not yet
                  // published
  if (task < ntask) load_task<15, GT, CONV, CO>(p, task, st, tid, c0, r0);
  auto put_beta = [&]() {
    if (wave == 0)
      betas[lane] = GB ? __uint_as_float(st.beta << 16)
                       : __uint_as_float(st.beta);
    if constexpr (CONV)
      if (tid < 2 * DK + DV) taps[tid] = st.tap;
  };
  if (task < ntask) put_beta();
  __syncthreads();

  while (task < ntask) {
    // per-lane indices are rebuilt from an opaque copy every task: the
    // compiler would otherwise keep dozens of addresses derived from them
    // live across the whole loop, past the 256 registers a lane may hold
    int lid = tid;
    asm volatile("" : "+v"(lid));
    // the same for the wave index: values derived from it would otherwise
    // be hoisted too and spill out of the scalar registers
    int wave = wave0;
    asm volatile("" : "+s"(wave));
    const int lane = lid & 63, g4 = lane >> 4, m16 = lane & 15;
    const int hh = lane >> 5;
    const int c0 = 64 * (wave & 1) + 2 * (lane & 31);
    const int r0 = 16 * a + 8 * hh;
    const int bh = task % BH, n = task_chunk<CO>(task, BH, p.NC);
    const int b = bh / H, h = bh % H;
    const int t0 = n * C;
    char *blk = p.ws + ((size_t)bh * p.NC + n) * p.wsb;
    if constexpr (CO) {
      // the task after this one (read back after B1)
      if (tid == 0)
        claim[0] = __hip_atomic_fetch_add(p.sync + SYNC_NEXT, 1,
                                          __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- E1: decay, running products, A/P operands, (beta V)^T -----------
    float F[2], xkr[8][2];
    int vote;
    {
      float e[8][2], kk[8][2], qq[8][2], bt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = t0 + r0 + i < T;
        float g0, g1;
        GRaw<GT>::get(st.g[i], g0, g1);
        bt[i] = ok ? betas[r0 + i] : 0.f;
        e[i][0] = ok ? __expf(g0) : 1.f;
        e[i][1] = ok ? __expf(g1) : 1.f;
        if constexpr (!CONV) {
          get2(st.k[i], kk[i][0], kk[i][1]);
          get2(st.q[i], qq[i][0], qq[i][1]);
        }
      }
      if constexpr (CONV) {
        // causal conv over the staged rows (row i + u holds token
        // t0 + r0 + i + u - 3; rows before the sequence start or past its
        // end, loaded clamped, count as zero: cleared once per row here)
#pragma unroll
        for (int j = 0; j < Stage<GT, CONV>::XR; ++j) {
          const int t = t0 + r0 + j - XO;
          if (!(t >= 0 && t < T)) st.q[j] = st.k[j] = st.v[j] = 0u;
        }
        f32x4 tq[2], tk[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          tq[j] = taps[c0 + j];
          tk[j] = taps[DK + c0 + j];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          qq[i][0] = qq[i][1] = kk[i][0] = kk[i][1] = 0.f;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float x0, x1, y0, y1;
            get2(st.q[i + u], x0, x1);
            get2(st.k[i + u], y0, y1);
            qq[i][0] += tq[0][u] * x0;
            qq[i][1] += tq[1][u] * x1;
            kk[i][0] += tk[0][u] * y0;
            kk[i][1] += tk[1][u] * y1;
          }
        }
        // L2 over the head's 128 channels per token: 64 of them in this
        // wave's 32 lanes of the token half, 64 in the partner wave (w ^ 1)
        float sq[8], sk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sq[i] = group_sum<32>(qq[i][0] * qq[i][0] + qq[i][1] * qq[i][1]);
          sk[i] = group_sum<32>(kk[i][0] * kk[i][0] + kk[i][1] * kk[i][1]);
        }
        if ((lane & 31) == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            *(float2 *)(l2p + ((wave * 16 + 8 * hh + i) * 2)) =
                make_float2(sq[i], sk[i]);
        }
        __syncthreads();  // conv: partial sums of squares of both halves
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float2 o = *(const float2 *)(l2p + (((wave ^ 1) * 16 + 8 * hh + i) * 2));
          const float iq = p.l2 ? l2_inv_norm(sq[i] + o.x + p.eps) : 1.f;
          const float ik = p.l2 ? l2_inv_norm(sk[i] + o.y + p.eps) : 1.f;
          qq[i][0] *= iq;
          qq[i][1] *= iq;
          kk[i][0] *= ik;
          kk[i][1] *= ik;
          if ((wave & 1) == 0 && (lane & 31) == 0)
            *(float2 *)(nrm + 2 * (r0 + i)) = make_float2(iq, ik);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (!(t0 + r0 + i < T)) kk[i][0] = kk[i][1] = qq[i][0] = qq[i][1] = 0.f;
      // this half's 8-token product, then the other half's (lane ^ 32)
      float ltp[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float lt = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) lt *= e[i][j];
        ltp[j] = __shfl_xor(lt, 32, 64);
        F[j] = lt * ltp[j];
      }
      // rho is non-increasing within the sub-chunk: its least value is F
      vote = !(F[0] >= SAFE_MIN) || !(F[1] >= SAFE_MIN);
      // forward: rho = inclusive prefix within the sub-chunk
      {
        float pr0 = hh ? ltp[0] : 1.f, pr1 = hh ? ltp[1] : 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = r0 + i;
          pr0 *= e[i][0];
          pr1 *= e[i][1];
          xkr[i][0] = bt[i] * kk[i][0] * pr0;
          xkr[i][1] = bt[i] * kk[i][1] * pr1;
          *(uint32_t *)(Xkr + r * LDK + c0) = put2(xkr[i][0], xkr[i][1]);
          *(uint32_t *)(Xqr + r * LDK + c0) =
              put2(p.scale * qq[i][0] * pr0, p.scale * qq[i][1] * pr1);
        }
      }
      // backward: sigma = exclusive suffix within the sub-chunk; k / rho,
      // the diagonal blocks' column operand, as k sigma / F (rho sigma = F):
      // one reciprocal per channel instead of one per token.  It is read
      // only when every F of the task is at least 2^-64 (else the exact
      // diagonal sums replace those blocks), so 1 / F stays finite there.
      {
        float sf0 = hh ? 1.f : ltp[0], sf1 = hh ? 1.f : ltp[1];
        const float iF0 = __builtin_amdgcn_rcpf(F[0]);
        const float iF1 = __builtin_amdgcn_rcpf(F[1]);
        float xc0[8], xc1[8];  // the same values by channel
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          xc0[i] = kk[i][0] * sf0;
          xc1[i] = kk[i][1] * sf1;
          sf0 *= e[i][0];
          sf1 *= e[i][1];
          *(uint32_t *)(Xks + (r0 + i) * LDK + c0) = put2(xc0[i], xc1[i]);
          *(uint32_t *)(Xkir + (r0 + i) * LDK + c0) =
              put2(xc0[i] * iF0, xc1[i] * iF1);
        }
        bf16 *row0 = XksT + c0 * LDC, *row1 = row0 + LDC;
        *(R4 *)(row0 + cm_off<C>(c0, r0)) = Vec4<bf16>::put(&xc0[0]);
        *(R4 *)(row0 + cm_off<C>(c0, r0 + 4)) = Vec4<bf16>::put(&xc0[4]);
        *(R4 *)(row1 + cm_off<C>(c0 + 1, r0)) = Vec4<bf16>::put(&xc1[0]);
        *(R4 *)(row1 + cm_off<C>(c0 + 1, r0 + 4)) = Vec4<bf16>::put(&xc1[4]);
      }
      if (!hh) *(float2 *)(Fs + a * DK + c0) = make_float2(F[0], F[1]);
      // (beta V)^T for U: value channels c0, c0 + 1 (beta is 0 past T)
      {
        float bv0[8], bv1[8];
        if constexpr (CONV) {
          const f32x4 tv0 = taps[2 * DK + c0], tv1 = taps[2 * DK + c0 + 1];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float v0, v1;
              get2(st.v[i + u], v0, v1);
              a0 += tv0[u] * v0;
              a1 += tv1[u] * v1;
            }
            bv0[i] = bt[i] * a0;
            bv1[i] = bt[i] * a1;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float v0, v1;
            get2(st.v[i], v0, v1);
            bv0[i] = bt[i] * v0;
            bv1[i] = bt[i] * v1;
          }
        }
        bf16 *row0 = XvT + c0 * LDC, *row1 = row0 + LDC;
        *(R4 *)(row0 + cm_off<C>(c0, r0)) = Vec4<bf16>::put(&bv0[0]);
        *(R4 *)(row0 + cm_off<C>(c0, r0 + 4)) = Vec4<bf16>::put(&bv0[4]);
        *(R4 *)(row1 + cm_off<C>(c0 + 1, r0)) = Vec4<bf16>::put(&bv1[0]);
        *(R4 *)(row1 + cm_off<C>(c0 + 1, r0 + 4)) = Vec4<bf16>::put(&bv1[4]);
      }
    }
    {
      const unsigned long long bal = __ballot(vote);
      if (lane == 0) votes[wave] = bal != 0ull;
    }
    // CO: the previous task's workspace stores complete (nothing else is in
    // flight here: this task's inputs were consumed above)
    if constexpr (CO) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // B1: region A, (K sigma)^T, (beta V)^T, Fs, votes
    if constexpr (CO) {
      if (tid == 0 && done >= 0)
        __hip_atomic_store(p.sync + SYNC_FLAGS + done, 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      done = bh * p.NC + n;  // the flag of this task
    }

    // ---- E2: Qtil and Ktil^T units, gamma_C, (beta K Gam)^T, mid products -
    const int next = CO ? claim[0] : task + (int)gridDim.x;
    const bool more = next < ntask;
    if (more) load_task<1, GT, CONV, CO>(p, next, st, tid, c0, r0);
    int anyv = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) anyv |= votes[w];
    const bool fallback = anyv != 0;
    if (fallback)  // accumulated by the exact diagonal sums after B2
      ((f32x4 *)FbA)[tid] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      // Gam at the sub-chunk start: product of the earlier sub-chunks' F
      float fp0 = 1.f, fp1 = 1.f;
#pragma unroll
      for (int bb = 0; bb < NB - 1; ++bb) {
        const float2 f = *(const float2 *)(Fs + bb * DK + c0);
        if (bb < a) { fp0 *= f.x; fp1 *= f.y; }
      }
      float k0[8], k1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        k0[i] = xkr[i][0] * fp0;
        k1[i] = xkr[i][1] * fp1;
      }
      bf16 *row0 = XkgT + c0 * LDC, *row1 = row0 + LDC;
      *(R4 *)(row0 + cm_off<C>(c0, r0)) = Vec4<bf16>::put(&k0[0]);
      *(R4 *)(row0 + cm_off<C>(c0, r0 + 4)) = Vec4<bf16>::put(&k0[4]);
      *(R4 *)(row1 + cm_off<C>(c0 + 1, r0)) = Vec4<bf16>::put(&k1[0]);
      *(R4 *)(row1 + cm_off<C>(c0 + 1, r0 + 4)) = Vec4<bf16>::put(&k1[4]);
      if (a == NB - 1 && hh == 1)
        st_ws<CO>((float *)(blk + W.off_gam) + c0,
                  make_float2(fp0 * F[0], fp1 * F[1]));
    }
    // mid products M_{b->a} = prod_{b<d<a} F_d for sub-chunk pairs a-b >= 2:
    // pairs (2,0), (3,0), (3,1) at index 0, 1, 2
    if (tid < 3 * DK) {
      const int c = tid % DK, pi = tid / DK;
      const int aa = pi == 0 ? 2 : 3, bb = pi == 2 ? 1 : 0;
      float mp = 1.f;
#pragma unroll
      for (int d = 1; d < 3; ++d)
        if (d > bb && d < aa) mp *= Fs[d * DK + c];
      Mid[pi * DK + c] = mp;
    }
    __syncthreads();  // B2

    if (more) load_task<2, GT, CONV, CO>(p, next, st, tid, c0, r0);

    if (fallback) {
      // exact diagonal-block sums: item (sub-chunk aa, column s, 16
      // channels), one per thread; raw k and q of the input rows
      const size_t tokb = (size_t)b * T;
      const int cg = tid % 8, s = (tid / 8) % 16, aa = tid / 128;
      float pr[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) pr[c] = 1.f;
      const int ts = t0 + 16 * aa + s;
      for (int r = s; r < 16; ++r) {
        const int tr = t0 + 16 * aa + r;
        const int trc = min(tr, T - 1);
        float sa = 0.f, sp = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const int ch = cg * 16 + c;
          if (r > s) {
            const size_t gi = ((tokb + trc) * H + h) * DK + ch;
            const float gv = GB ? (float)((const bf16 *)p.g)[gi]
                                : ((const float *)p.g)[gi];
            pr[c] *= (tr < T) ? __expf(gv) : 1.f;
          }
          float ks, kr, qr;
          if constexpr (CONV) {
            // the conv and L2 of the input rows, recomputed (exact path only)
            auto cv = [&](const void *x, int item, int t) -> float {
              const f32x4 tp = taps[item];
              float acc = 0.f;
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int tt = t + u - 3;
                if (tt >= 0 && tt < T)
                  acc += tp[u] * (float)((const bf16 *)x)
                                     [((tokb + tt) * H + h) * DK + ch];
              }
              return acc;
            };
            ks = ts < T ? cv(p.xk, DK + ch, ts) * nrm[2 * (ts - t0) + 1] : 0.f;
            kr = tr < T ? cv(p.xk, DK + ch, tr) * nrm[2 * (tr - t0) + 1] : 0.f;
            qr = tr < T ? cv(p.xq, ch, tr) * nrm[2 * (tr - t0)] : 0.f;
          } else {
            const size_t ob = ((tokb + min(ts, T - 1)) * H + h) * DK + ch;
            const size_t orr = ((tokb + trc) * H + h) * DK + ch;
            ks = ts < T ? (float)((const bf16 *)p.k)[ob] : 0.f;
            kr = tr < T ? (float)((const bf16 *)p.k)[orr] : 0.f;
            qr = tr < T ? (float)((const bf16 *)p.q)[orr] : 0.f;
          }
          sa += kr * ks * pr[c];
          sp += qr * ks * pr[c];
        }
        const float br =
            (tr < T) ? (GB ? (float)((const bf16 *)p.beta)[(tokb + trc) * H + h]
                           : ((const float *)p.beta)[(tokb + trc) * H + h])
                     : 0.f;
        if (r > s) atomicAdd(&FbA[(aa * 16 + r) * 16 + s], br * sa);
        atomicAdd(&FbP[(aa * 16 + r) * 16 + s], p.scale * sp);
      }
      __syncthreads();
    }

    // Qtil = scale Q*Gam, unit w (row tile w / 4, channel unit w % 4): a
    // lane's 16-byte slot holds channels 32u + 4g4 .. +3 and 32u + 16 + 4g4
    // .. +3 of token 16aa + m16
    auto q_unit = [&](int w) {
      const int aa = w / NKU, u = w % NKU;
      const int tok = 16 * aa + m16;
      const int ch0 = KU * u + 4 * g4, ch1 = ch0 + 16;
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
      Vec4<bf16>::get(*(const R4 *)(Xqr + tok * LDK + ch0), x0);
      Vec4<bf16>::get(*(const R4 *)(Xqr + tok * LDK + ch1), x1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y0[j] = x0[j] * f0[j];
        y1[j] = x1[j] * f1[j];
      }
      const R4 lo = Vec4<bf16>::put(y0), up = Vec4<bf16>::put(y1);
      st_ws<CO>(blk + W.off_qt + ((size_t)(aa * NKU + u) * 64 + lane) * 16,
                make_uint4(lo.x, lo.y, up.x, up.y));
    };
    // Ktil^T = (K*Gam_C/Gam)^T, unit w (channel tile w / 2, token unit w % 2)
    auto k_unit = [&](int w) {
      const int ct = w / NTU, u = w % NTU;
      const int ch = 16 * ct + m16;
      const int tk0 = KU * u + 4 * g4, tk1 = tk0 + 16;
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
      Vec4<bf16>::get(*(const R4 *)(XksT + ch * LDC + cm_off<C>(ch, tk0)), x0);
      Vec4<bf16>::get(*(const R4 *)(XksT + ch * LDC + cm_off<C>(ch, tk1)), x1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y0[j] = x0[j] * s0;
        y1[j] = x1[j] * s1;
      }
      const R4 lo = Vec4<bf16>::put(y0), up = Vec4<bf16>::put(y1);
      st_ws<CO>(blk + W.off_ktt + ((size_t)(ct * NTU + u) * 64 + lane) * 16,
                make_uint4(lo.x, lo.y, up.x, up.y));
    };
    // block j (ap_block order) of A (into LDS) and/or P (into the
    // workspace); both products share the column operand
    auto ap_item = [&](int j, bool doA, bool doP) {
      int aa, bb;
      ap_block<NB>(j, aa, bb);
      const bool diag = aa == bb;
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      if (diag && fallback) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accA[i] = FbA[(aa * 16 + m16) * 16 + 4 * g4 + i];
          accP[i] = FbP[(aa * 16 + m16) * 16 + 4 * g4 + i];
        }
      } else {
        const bf16 *kb = Xkr + (16 * aa + m16) * LDK;
        const bf16 *qb = Xqr + (16 * aa + m16) * LDK;
        const bf16 *cb = (diag ? Xkir : Xks) + (16 * bb + m16) * LDK;
        frag kf[NKU], qf[NKU], cf[NKU];
#pragma unroll
        for (int u = 0; u < NKU; ++u) {
          cf[u] = M::load_k(cb + KU * u, g4);
          if (doA) kf[u] = M::load_k(kb + KU * u, g4);
          if (doP) qf[u] = M::load_k(qb + KU * u, g4);
        }
        if (aa - bb >= 2) {
          // decay across the sub-chunks strictly between bb and aa, per
          // channel, on the column operand (lane slots 32u + 4g4 + e and
          // 32u + 16 + 4g4 + e)
          const float *mid = Mid + (aa == 2 ? 0 : (bb == 0 ? 1 : 2)) * DK;
#pragma unroll
          for (int u = 0; u < NKU; ++u) {
            const f32x4 m0 = *(const f32x4 *)(mid + KU * u + 4 * g4);
            const f32x4 m1 = *(const f32x4 *)(mid + KU * u + 16 + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              cf[u][e] = (bf16)((float)cf[u][e] * m0[e]);
              cf[u][4 + e] = (bf16)((float)cf[u][4 + e] * m1[e]);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < NKU; ++u) {
          if (doA) accA = M::mma(cf[u], kf[u], accA);
          if (doP) accP = M::mma(cf[u], qf[u], accP);
        }
      }
      // lane (m16, g4): element i is row 16aa + m16, col 16bb + 4g4 + i
      if (diag) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sc = 4 * g4 + i;
          if (!(sc < m16)) accA[i] = 0.f;
          if (!(sc <= m16)) accP[i] = 0.f;
        }
      }
      if (doA)
        *(f32x4 *)(Af + (16 * aa + m16) * LDA + 16 * bb + 4 * g4) = accA;
      if (doP) {
        char *dst = blk + W.off_p +
                    ((size_t)(aa * NTU + bb / 2) * 64 + lane) * 16 +
                    (bb % 2) * 8;
        const float a4[4] = {accP[0], accP[1], accP[2], accP[3]};
        st_ws<CO>(dst, Vec4<bf16>::put(a4));
        if (diag && (aa % 2) == 0) {
          const float z[4] = {0.f, 0.f, 0.f, 0.f};
          st_ws<CO>(dst + 8, Vec4<bf16>::put(z));
        }
      }
    };
    // for the backward pass: A = diag(beta) M and T^T, fp32 (only their
    // lower and upper triangles are read)
    float *tat = p.train_at ? p.train_at + ((size_t)bh * p.NC + n) * 2 * C * C
                            : nullptr;

    // ---- AP: A and P blocks on the matrix cores --------------------------
    // eight blocks whole (A and P), blocks (0,0) and (1,1) split into their
    // A and P halves on waves 4-7: 20 products per SIMD (waves w, w + 4);
    // the three blocks with mid products go to waves 0-2
    {
      const int full = wave < 4 ? (wave == 0 ? 2 : wave == 1 ? 3 : wave == 2 ? 7 : 1)
                                : (wave == 4 ? 4 : wave == 5 ? 6 : wave == 6 ? 8 : 9);
      ap_item(full, true, true);
      if (wave >= 4) ap_item(wave < 6 ? 0 : 5, (wave & 1) == 0, (wave & 1) == 1);
    }
    __syncthreads();  // B3: A complete; beta K rho no longer read
    if (more) load_task<4, GT, CONV, CO>(p, next, st, tid, c0, r0);

    // ---- T1: diagonal inverses (waves 0-3, as in kda_prep_impl.h) beside
    // part of the Qtil / Ktil^T unit stores (waves 4-7), which no later phase
    // reads.  Waves 4-7 also zero the upper block (r, r+1) of every even
    // token tile r of the bf16 T, which the W/U products read as part of
    // whole 32-token units.
    f32x4 Tcol[NB];
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
      const f32x4 L2B = mma16_f32(LA, LB, z4);
      const f32x4 L2A = mma16_f32(LB, LA, z4);
      const f32x4 L4B = mma16_f32(L2A, L2B, z4);
      const f32x4 L4A = mma16_f32(L2B, L2A, z4);
      const f32x4 L8A = mma16_f32(L4B, L4A, z4);
      Y = mma16_f32(L2A, Y, Y);
      Y = mma16_f32(L4A, Y, Y);
      Y = mma16_f32(L8A, Y, Y);
      // lane (g4, m16) holds T_aa[4 g4 + j][m16]
      Tcol[0] = Y;
      if (tat)
        *(f32x4 *)(tat + C * C + (16 * aa + m16) * C + 16 * aa + 4 * g4) = Y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Taa[(aa * 16 + 4 * g4 + j) * 16 + m16] = Y[j];
        Tb[(16 * aa + 4 * g4 + j) * LDC + 16 * aa + m16] = (bf16)Y[j];
      }
    } else {
      if (tid - 256 < 64) {
        // rows 16 rt .. 16 rt + 15 (rt = 0, 2), 16 columns from 16 (rt + 1)
        const int i = tid - 256;
        const int rt = 2 * (i / 32), row = (i % 32) / 2, hv = i % 2;
        *(uint4 *)(Tb + (16 * rt + row) * LDC + 16 * (rt + 1) + 8 * hv) =
            make_uint4(0u, 0u, 0u, 0u);
      }
      // units 0 .. 11 of the 32 Qtil / Ktil^T units (3 per wave)
      for (int w = wave - NB; w < 12; w += NW - NB) q_unit(w);
      if (tat)
        for (int i = tid - 256; i < C * C; i += NT - 256)
          tat[i] = Af[(i / C) * LDA + i % C];
    }
    __syncthreads();
    // ---- T2: off-diagonal blocks of T, one block column per wave (waves
    // 0-2), beside the Qtil and Ktil^T units (waves 3-7)
    if (wave < NB - 1) {
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
        if (tat)
          *(f32x4 *)(tat + C * C + (16 * bb + m16) * C + 16 * aa + 4 * g4) = Tn;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Tb[(16 * aa + 4 * g4 + j) * LDC + 16 * bb + m16] = (bf16)Tn[j];
      }
    } else {
      // units 12 .. 31 (4 per wave)
      for (int w = 12 + wave - (NB - 1); w < 2 * NB * NKU; w += NW - (NB - 1)) {
        if (w < NB * NKU)
          q_unit(w);
        else
          k_unit(w - NB * NKU);
      }
    }
    __syncthreads();
    if (more) load_task<8, GT, CONV, CO>(p, next, st, tid, c0, r0);

    // ---- WU: -W (A-operand units) and U (accumulator tiles) ----------------
    // token tile rt reads T rows 16 rt .. 16 rt + 15 over token units
    // 0 .. umax(rt) = rt / 2; W costs 2 (umax + 1) steps per key unit, U
    // (umax + 1) per value tile.  Waves 0-3 make -W, waves 4-7 U, 12 steps
    // each.
    auto load_t = [&](int rt, frag *tb) {
      const int umax = rt / 2;
#pragma unroll
      for (int uu = 0; uu < NTU; ++uu)
        tb[uu] = M::load_k(Tb + (16 * rt + m16) * LDC + KU * min(uu, umax), g4);
    };
    auto w_units = [&](int rt, int u0, int u1) {
      frag tb[NTU];
      load_t(rt, tb);
      const int umax = rt / 2;
      for (int u = u0; u < u1; ++u) {
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        frag xa[NTU][2];
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int ct = 2 * u + h2;
            xa[uu][h2] = load_k_cm<bf16, C>(XkgT + (16 * ct + m16) * LDC,
                                            16 * ct + m16, KU * uu, g4, true);
          }
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          if (uu <= umax)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              acc[h2] = M::mma(xa[uu][h2], tb[uu], acc[h2]);
        st_ws<CO>(blk + W.off_negw + ((size_t)(rt * NKU + u) * 64 + lane) * 16,
                  M::pack(-acc[0], -acc[1]));
      }
    };
    auto u_tiles = [&](int rt, int v0, int v1) {
      frag tb[NTU];
      load_t(rt, tb);
      const int umax = rt / 2;
      for (int vt = v0; vt < v1; ++vt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        frag vb[NTU];
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          vb[uu] = load_k_cm<bf16, C>(XvT + (16 * vt + m16) * LDC,
                                      16 * vt + m16, KU * uu, g4, true);
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          if (uu <= umax) acc = M::mma(tb[uu], vb[uu], acc);
        bf16 *dst = (bf16 *)(blk + W.off_u) +
                    ((size_t)(vt * NB + rt) * 64 + lane) * 4;
        const float a4[4] = {acc[0], acc[1], acc[2], acc[3]};
        st_ws<CO>(dst, Vec4<bf16>::put(a4));
      }
    };
    if (wave < 4) {
      const int u0 = 2 * (wave & 1);
      w_units(2 + (wave >> 1), u0, u0 + 2);
      w_units(wave >> 1, u0, u0 + 2);
    } else if (wave == 4) {
      u_tiles(2, 0, 6);
    } else if (wave == 5) {
      u_tiles(3, 0, 6);
    } else if (wave == 6) {
      u_tiles(2, 6, 8);
      u_tiles(3, 6, 8);
      u_tiles(0, 0, 4);
    } else {
      u_tiles(0, 4, 8);
      u_tiles(1, 0, 8);
    }
    if (more) put_beta();  // the current task's betas were last read in E1
    __syncthreads();       // B5: LDS free for the next task
    task = next;
  }
  if constexpr (CO) {
    // the last task's flag, once every wave's stores have completed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0 && done >= 0)
      __hip_atomic_store(p.sync + SYNC_FLAGS + done, 1, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace pc

bool prep_d128_applies(const PrefillParams &p, int io_bf16) {
  return io_bf16 && !p.gate_head && p.Dk == pc::DK && p.Dv == pc::DV &&
         p.C == pc::C && (!p.use_conv || (p.cw >= 1 && p.cw <= 4));
}

template <typename GT>
static void launch_d128(const PrefillParams &p, unsigned grid, hipStream_t s) {
  if (p.use_conv)
    hipLaunchKernelGGL((pc::kda_chunk_prep_d128<GT, true, false>), dim3(grid),
                       dim3(pc::NT), 0, s, p);
  else if (p.sync)
    hipLaunchKernelGGL((pc::kda_chunk_prep_d128<GT, false, true>), dim3(grid),
                       dim3(pc::NT), 0, s, p);
  else
    hipLaunchKernelGGL((pc::kda_chunk_prep_d128<GT, false, false>), dim3(grid),
                       dim3(pc::NT), 0, s, p);
}

hipError_t launch_prefill_prep_d128(const PrefillParams &p, hipStream_t s) {
  const long long ntask = (long long)p.B * p.H * p.NC;
  const unsigned grid = (unsigned)std::min<long long>(ntask, cu_count());
  if (p.gate_bf16)
    launch_d128<bf16>(p, grid, s);
  else
    launch_d128<float>(p, grid, s);
  return hipGetLastError();
}

}  // namespace kda
