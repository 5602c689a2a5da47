// kda_prep_gdn.hip -- chunk prep for one log-decay per token-head (the gate
// of Gated DeltaNet: KDA_GATE_HEAD), bf16 q/k/v, d_k = 128, 64-token chunks.
//
// It writes the same workspace factors as kda_chunk_prep (kda_prep_impl.h:
// -W, Qtil, Ktil^T, P, gamma_C, U in the operand-unit layout of
// kda_device.h), so kda_state_pass runs unchanged.  What the scalar gate
// changes is the algebra of the chunk-local part.  With e_r = exp(g_r) one
// value per token, every decay factor is a scalar per token pair:
//   D[r][s] = prod_{u = s+1 .. r} e_u            (s <= r)
//   A[r][s] = beta_r (k_r . k_s) D[r][s]  (s < r),   P[r][s] = scale (q_r . k_s) D[r][s]
//   W = T diag(beta Gam) K,   U = T diag(beta) V,   T = (I + A)^-1
//   Qtil = scale diag(Gam) Q,  Ktil^T = (diag(Gam_C / Gam) K)^T
// so the Gram products run on the raw keys and queries and the decay is
// applied to the 64 x 64 results (and to T's columns, and to rows of Q and
// K) instead of to every key and query element.  There are no per-channel
// exponentials, running products or scaled operand copies, and no ratio of
// running products: the diagonal 16 x 16 blocks take D as a direct product
// of at most 15 gates, so g = -inf is exact without any fallback path.
//
// Decay factors, all products of values <= 1 (no overflow, -inf exact):
// within each 16-token sub-chunk a the prefix rho (inclusive) and suffix
// sigma (exclusive) of e, the whole-sub-chunk products F_a, Gam_r (prefix
// over the chunk) and Gam_C / Gam_r (suffix); for s in an earlier
// sub-chunk than r, D[r][s] = rho_r * (F of the sub-chunks between) *
// sigma_s.
//
// Execution follows kda_prep_d128.hip: a persistent grid of one 512-thread
// workgroup (eight waves, two per SIMD) per CU walks the (batch*head, chunk)
// tasks last chunk first.  Each thread fetches 2 channels x 8 tokens of the
// next task's q, k and v into registers in parts spread over the current
// task's phases; wave 0 fetches the chunk's 64 gates and betas, one per
// lane, and forms the decay factors with DPP scans over the 16-lane rows
// (one row per sub-chunk).  A and P blocks are dealt out so that every SIMD
// runs the same number of products, the Qtil / Ktil^T unit stores run on the
// waves that the two T phases leave idle, and W and U follow a fixed table
// of 12 matrix-core steps per wave.
#include "kda_prep_impl.h"

namespace kda {
namespace gdn {

constexpr int NT = 512, NW = NT / 64;
constexpr int DK = 128, C = 64, NB = 4, NKU = 4, NTU = 2, NKT = 8;
constexpr int LDK = DK + 8;  // token-major bf16 rows
constexpr int LDC = C + 8;   // channel-major bf16 rows (blocks swizzled)
constexpr int LDA = C + 4;   // fp32 rows of A
constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
// LDS, at most 80 KiB so that two workgroups share a CU.  The raw key and
// query rows live from the staging to the A/P products (barrier B2); after
// B2 their region holds V^T, the diagonal inverses and T in bf16.
constexpr size_t oXk = 0;                                     // [C][LDK]
constexpr size_t oXq = al(oXk + (size_t)C * LDK * 2);         // [C][LDK]
constexpr size_t oVT = 0;                                     // [128][LDC]
constexpr size_t oTaa = al(oVT + (size_t)128 * LDC * 2);      // [NB][256]
constexpr size_t oTb = al(oTaa + (size_t)NB * 256 * 4);       // [C][LDC]
static_assert(oTb + (size_t)C * LDC * 2 <= oXq + (size_t)C * LDK * 2,
              "V^T and T inside the raw rows");
constexpr size_t oKT = al(oXq + (size_t)C * LDK * 2);         // [DK][LDC]
constexpr size_t oAf = al(oKT + (size_t)DK * LDC * 2);        // [C][LDA]
// per-token scalars of the chunk: e, rho, sigma, beta, Gam, Gam_C/Gam,
// beta * Gam, then F[4]
constexpr size_t oSc = al(oAf + (size_t)C * LDA * 4);
constexpr size_t LDS_BYTES = oSc + (7 * 64 + 4) * 4;
static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");

// v lanes without a source in the DPP row read 1 (the product identity)
template <int CTRL>
__device__ __forceinline__ float dpp_or_one(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(1.0f), __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ uint32_t ld4_stream(const void *p) {
  return __builtin_nontemporal_load((const uint32_t *)p);
}

// a task's raw inputs for one thread (2 channels x 8 tokens of q, k and v;
// wave 0: the gate and beta of token `lane`)
struct Raw {
  uint32_t q[8], k[8], v[8];
  unsigned g, beta;
};

// PART: 1 = gate and beta, 2 = q, 4 = k, 8 = v (issued in different phases
// of the previous task, so the memory queues drain between them)
template <int PART, typename GT>
__device__ __forceinline__ void load_raw(const PrefillParams &p, int task,
                                         Raw &x, int tid, int c0, int r0) {
  constexpr bool GB = sizeof(GT) == 2;
  const int BH = p.B * p.H;
  const int bh = task % BH, n = p.NC - 1 - task / BH;
  const int b = bh / p.H, h = bh % p.H;
  const int t0 = n * C, tlast = p.T - 1;
  const size_t tok0 = (size_t)b * p.T;
  if ((PART & 1) && tid < 64) {
    const size_t gi = (tok0 + min(t0 + tid, tlast)) * p.H + h;
    x.g = GB ? (unsigned)((const unsigned short *)p.g)[gi]
             : ((const unsigned *)p.g)[gi];
    x.beta = GB ? (unsigned)((const unsigned short *)p.beta)[gi]
                : ((const unsigned *)p.beta)[gi];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const size_t t = (size_t)min(t0 + r0 + i, tlast);
    const size_t kb = ((tok0 + t) * p.H + h) * DK + c0;
    if (PART & 2) x.q[i] = ld4_stream((const bf16 *)p.q + kb);
    if (PART & 4) x.k[i] = ld4_stream((const bf16 *)p.k + kb);
    if ((PART & 8) && c0 < p.Dv)
      x.v[i] = ld4_stream((const bf16 *)p.v + ((tok0 + t) * p.H + h) * p.Dv +
                          c0);
  }
}

// four bf16 (as raw 16-bit values) packed into 8 bytes
__device__ __forceinline__ uint2 bf_pack(unsigned a, unsigned b, unsigned c,
                                         unsigned d) {
  return make_uint2((a & 0xffffu) | (b << 16), (c & 0xffffu) | (d << 16));
}

template <typename GT>
__global__ __launch_bounds__(NT, 2) void kda_chunk_prep_gdn(PrefillParams p) {
  using M = Mma<bf16>;
  typedef M::frag frag;
  constexpr bool GB = sizeof(GT) == 2;
  __shared__ __attribute__((aligned(16))) char sm[LDS_BYTES];
  bf16 *Xk = (bf16 *)(sm + oXk), *Xq = (bf16 *)(sm + oXq);
  bf16 *KT = (bf16 *)(sm + oKT), *VT = (bf16 *)(sm + oVT);
  float *Af = (float *)(sm + oAf), *Taa = (float *)(sm + oTaa);
  bf16 *Tb = (bf16 *)(sm + oTb);
  float *s_e = (float *)(sm + oSc), *s_rho = s_e + 64, *s_sig = s_e + 128,
        *s_beta = s_e + 192, *s_gam = s_e + 256, *s_sfx = s_e + 320,
        *s_bg = s_e + 384, *s_F = s_e + 448;

  const int tid = threadIdx.x;
  const int wave0 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wave0;
  const int BH = p.B * p.H, T = p.T, Dv = p.Dv, nvt = Dv / 16;
  const int ntask = BH * p.NC;
  // the section offsets do not depend on d_v: immediates
  constexpr WsLayout W = ws_layout(DK, 128, C, 2);
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  // this thread's staging share: sub-chunk wave / 2, channels
  // 64 (wave % 2) + 2 (lane % 32), +1 of tokens 8 (lane / 32) .. +7
  const int c0i = 64 * (wave & 1) + 2 * (tid & 31);
  const int r0i = 16 * (wave >> 1) + 8 * ((tid >> 5) & 1);

  Raw x;
  int task = blockIdx.x;
  if (task < ntask) load_raw<15, GT>(p, task, x, tid, c0i, r0i);

  for (; task < ntask; task += gridDim.x) {
    // per-lane indices from an opaque copy every task, so that addresses
    // derived from them are not kept live across the loop
    int lid = tid;
    asm volatile("" : "+v"(lid));
    // the same for the wave index: values derived from it would otherwise
    // be hoisted too and spill out of the scalar registers
    int wave = wave0;
    asm volatile("" : "+s"(wave));
    const int lane = lid & 63, g4 = lane >> 4, m16 = lane & 15;
    const int c0 = 64 * (wave & 1) + 2 * (lane & 31);
    const int r0 = 16 * (wave >> 1) + 8 * (lane >> 5);
    const int bh = task % BH, n = p.NC - 1 - task / BH;
    const int t0 = n * C;
    char *blk = p.ws + ((size_t)bh * p.NC + n) * p.wsb;
    const bool more = task + (int)gridDim.x < ntask;

    // ---- stage: raw rows (token-major), K^T (channel-major), and the
    //      chunk's decay scalars; V stays in registers until B2 ---------------
    uint32_t vz[8];
    {
      uint32_t kz[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = t0 + r0 + i < T;  // rows past the end are zero
        kz[i] = ok ? x.k[i] : 0u;
        vz[i] = ok ? x.v[i] : 0u;
        *(uint32_t *)(Xk + (r0 + i) * LDK + c0) = kz[i];
        *(uint32_t *)(Xq + (r0 + i) * LDK + c0) = ok ? x.q[i] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int sh = 16 * j;
        bf16 *kr = KT + (c0 + j) * LDC;
        *(uint2 *)(kr + cm_off<C>(c0 + j, r0)) =
            bf_pack(kz[0] >> sh, kz[1] >> sh, kz[2] >> sh, kz[3] >> sh);
        *(uint2 *)(kr + cm_off<C>(c0 + j, r0 + 4)) =
            bf_pack(kz[4] >> sh, kz[5] >> sh, kz[6] >> sh, kz[7] >> sh);
      }
      if (wave == 0) {
        // lane = token of the chunk; DPP rows of 16 lanes = sub-chunks
        const bool ok = t0 + lane < T;
        const float gv = __uint_as_float(GB ? x.g << 16 : x.g);
        const float bv = __uint_as_float(GB ? x.beta << 16 : x.beta);
        const float e = ok ? __expf(gv) : 1.f;
        const float beta = ok ? bv : 0.f;
        float rho = e;
        rho *= dpp_or_one<0x111>(rho);  // row_shr:1
        rho *= dpp_or_one<0x112>(rho);  // row_shr:2
        rho *= dpp_or_one<0x114>(rho);  // row_shr:4
        rho *= dpp_or_one<0x118>(rho);  // row_shr:8
        float sig = e;
        sig *= dpp_or_one<0x101>(sig);  // row_shl:1
        sig *= dpp_or_one<0x102>(sig);  // row_shl:2
        sig *= dpp_or_one<0x104>(sig);  // row_shl:4
        sig *= dpp_or_one<0x108>(sig);  // row_shl:8
        sig = dpp_or_one<0x101>(sig);   // exclusive
        // whole-sub-chunk products: rho at the last lane of each row
        float F[NB];
        F[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rho), 15));
        F[1] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rho), 31));
        F[2] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rho), 47));
        F[3] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rho), 63));
        const int a = g4;  // sub-chunk of this token
        float pre = 1.f, suf = 1.f;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          if (bb < a) pre *= F[bb];
          if (bb > a) suf *= F[bb];
        }
        const float gam = rho * pre;
        s_e[lane] = e;
        s_rho[lane] = rho;
        s_sig[lane] = sig;
        s_beta[lane] = beta;
        s_gam[lane] = gam;
        s_sfx[lane] = sig * suf;
        s_bg[lane] = beta * gam;
        if (lane < NB)
          s_F[lane] = lane == 0 ? F[0] : lane == 1 ? F[1] : lane == 2 ? F[2] : F[3];
      }
    }
    __syncthreads();  // B1

    // the next task's gates, betas, q and v (all staged into LDS above)
    if (more) load_raw<1 | 2 | 8, GT>(p, task + gridDim.x, x, tid, c0, r0);

    // ---- Qtil = scale diag(Gam) Q and Ktil^T = (diag(Gam_C/Gam) K)^T ------
    // units: the 16 Qtil units beside the A/P products (the raw query rows
    // are overwritten after B2), the 16 Ktil^T units on the waves that the
    // two T phases leave idle
    auto qk_unit = [&](int it) {
      if (it < NB * NKU) {
        const int rt = it / NKU, u = it % NKU;
        const int r = 16 * rt + m16;
        frag f = M::load_k(Xq + r * LDK + 32 * u, g4, true);
        const float sc = p.scale * s_gam[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)((float)f[e] * sc);
        st_stream(blk + W.off_qt + ((size_t)(rt * NKU + u) * 64 + lane) * 16, f);
      } else {
        const int i2 = it - NB * NKU, ct = i2 / NTU, uu = i2 % NTU;
        const int ch = 16 * ct + m16;
        frag f = load_k_cm<bf16, C>(KT + ch * LDC, ch, 32 * uu, g4, true);
        // scale of token k = 32 uu + koff(g, e): two runs of 4 tokens
        const f32x4 lo = *(const f32x4 *)(s_sfx + 32 * uu + 4 * g4);
        const f32x4 hi = *(const f32x4 *)(s_sfx + 32 * uu + 16 + 4 * g4);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          f[e] = (bf16)((float)f[e] * (e < 4 ? lo[e] : hi[e - 4]));
        st_stream(blk + W.off_ktt + ((size_t)(ct * NTU + uu) * 64 + lane) * 16,
                  f);
      }
    };

    // ---- A and P blocks on the raw keys and queries, times the decay ------
    // block j (ap_block order): A and/or P, sharing the column operand.
    // D = mma(column operand: tokens s of bb, row operand: tokens r of aa):
    // lane (g, n) holds G[r = 16 aa + n][s = 16 bb + 4 g + j]
    auto ap_item = [&](int jb, bool doA, bool doP) {
      int aa, bb;
      ap_block<NB>(jb, aa, bb);
      f32x4 accA = z4, accP = z4;
      {
        const bf16 *kb = Xk + (16 * aa + m16) * LDK;
        const bf16 *qb = Xq + (16 * aa + m16) * LDK;
        const bf16 *cb = Xk + (16 * bb + m16) * LDK;
        frag cf[NKU], rf[NKU], qf[NKU];
#pragma unroll
        for (int u = 0; u < NKU; ++u) {
          cf[u] = M::load_k(cb + 32 * u, g4, true);
          if (doA) rf[u] = M::load_k(kb + 32 * u, g4, true);
          if (doP) qf[u] = M::load_k(qb + 32 * u, g4, true);
        }
#pragma unroll
        for (int u = 0; u < NKU; ++u) {
          if (doA) accA = M::mma(cf[u], rf[u], accA);
          if (doP) accP = M::mma(cf[u], qf[u], accP);
        }
      }
      const int r = 16 * aa + m16;
      const float br = s_beta[r];
      float dv[4];
      if (aa > bb) {
        float mid = 1.f;
        for (int d = bb + 1; d < aa; ++d) mid *= s_F[d];
        const float rm = s_rho[r] * mid;
        const f32x4 sg = *(const f32x4 *)(s_sig + 16 * bb + 4 * g4);
#pragma unroll
        for (int j = 0; j < 4; ++j) dv[j] = rm * sg[j];
      } else {
        // D[r][s] = prod_{u = s+1 .. r} e_u within the sub-chunk, directly:
        // the sub-chunk's 16 gates in registers, the product over
        // u in [4g + 4, m] (positions in the sub-chunk), then one more gate
        // per element going down from s = 4g + 3 to 4g
        float ev[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 e4 = *(const f32x4 *)(s_e + 16 * bb + 4 * q4);
#pragma unroll
          for (int j = 0; j < 4; ++j) ev[4 * q4 + j] = e4[j];
        }
        float pr = 1.f;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          pr *= (u >= 4 * g4 + 4 && u <= m16) ? ev[u] : 1.f;
        const f32x4 eg = *(const f32x4 *)(s_e + 16 * bb + 4 * g4);
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          dv[j] = pr;
          if (4 * g4 + j <= m16) pr *= eg[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 16 * bb + 4 * g4 + j;
        accA[j] = (s < r) ? br * accA[j] * dv[j] : 0.f;
        accP[j] = (s <= r) ? p.scale * accP[j] * dv[j] : 0.f;
      }
      if (doA) *(f32x4 *)(Af + r * LDA + 16 * bb + 4 * g4) = accA;
      if (doP) {
        char *dst = blk + W.off_p +
                    ((size_t)(aa * NTU + bb / 2) * 64 + lane) * 16 + (bb & 1) * 8;
        const float a4[4] = {accP[0], accP[1], accP[2], accP[3]};
        st_stream(dst, Vec4<bf16>::put(a4));
        if (aa == bb && (aa & 1) == 0) st_stream(dst + 8, make_uint2(0u, 0u));
      }
    };
    // eight blocks whole, blocks (0,0) and (1,1) split into their A and P
    // halves on waves 4-7: 20 products per SIMD (waves w, w + 4)
    {
      const int full = wave < 4 ? (wave == 0 ? 2 : wave == 1 ? 3 : wave == 2 ? 7 : 1)
                                : (wave == 4 ? 4 : wave == 5 ? 6 : wave == 6 ? 8 : 9);
      ap_item(full, true, true);
      if (wave >= 4) ap_item(wave < 6 ? 0 : 5, (wave & 1) == 0, (wave & 1) == 1);
      qk_unit(wave);
      qk_unit(wave + NW);
    }
    if (wave == 1 && lane < 32) {
      const float gc = s_F[0] * s_F[1] * s_F[2] * s_F[3];
      *(f32x4 *)((float *)(blk + W.off_gam) + 4 * lane) = f32x4{gc, gc, gc, gc};
    }
    __syncthreads();  // B2: A complete

    // the next task's k
    if (more) load_raw<4, GT>(p, task + gridDim.x, x, tid, c0, r0);

    // V^T (channel-major) over the raw rows, for U
    if (c0 < Dv) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int sh = 16 * j;
        bf16 *vr = VT + (c0 + j) * LDC;
        *(uint2 *)(vr + cm_off<C>(c0 + j, r0)) =
            bf_pack(vz[0] >> sh, vz[1] >> sh, vz[2] >> sh, vz[3] >> sh);
        *(uint2 *)(vr + cm_off<C>(c0 + j, r0 + 4)) =
            bf_pack(vz[4] >> sh, vz[5] >> sh, vz[6] >> sh, vz[7] >> sh);
      }
    }

    // ---- T = (I + A)^-1 (as in kda_prep_impl.h) ---------------------------
    // T1 on waves 0-3; waves 4-7 zero the upper block (rt, rt + 1) of every
    // even token tile rt of the bf16 T (W/U read T in whole 32-token units)
    // and store Ktil^T units 0 .. 7
    f32x4 Tcol[NB];
    if (wave < NB) {
      const int aa = wave;
      const float *ab = Af + (16 * aa) * LDA + 16 * aa;
      const f32x4 LA = *(const f32x4 *)(ab + m16 * LDA + 4 * g4);
      f32x4 LB, Y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        LB[j] = ab[(4 * g4 + j) * LDA + m16];
        Y[j] = ((4 * g4 + j) == m16 ? 1.f : 0.f) - LB[j];
      }
      const f32x4 L2B = mma16_f32(LA, LB, z4);
      const f32x4 L2A = mma16_f32(LB, LA, z4);
      const f32x4 L4B = mma16_f32(L2A, L2B, z4);
      const f32x4 L4A = mma16_f32(L2B, L2A, z4);
      const f32x4 L8A = mma16_f32(L4B, L4A, z4);
      Y = mma16_f32(L2A, Y, Y);
      Y = mma16_f32(L4A, Y, Y);
      Y = mma16_f32(L8A, Y, Y);
      Tcol[0] = Y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Taa[(aa * 16 + 4 * g4 + j) * 16 + m16] = Y[j];
        Tb[(16 * aa + 4 * g4 + j) * LDC + 16 * aa + m16] = (bf16)Y[j];
      }
    } else {
      if (tid - 256 < 64) {
        const int i = tid - 256;
        const int rt = 2 * (i / 32), rw = (i % 32) / 2, hv = i % 2;
        *(uint4 *)(Tb + (16 * rt + rw) * LDC + 16 * (rt + 1) + 8 * hv) =
            make_uint4(0u, 0u, 0u, 0u);
      }
      for (int it = wave - NB; it < 8; it += NW - NB) qk_unit(NB * NKU + it);
    }
    __syncthreads();  // B3
    // T2 on waves 0-2 (one block column each); waves 3-7 store Ktil^T units
    // 8 .. 15
    if (wave < NB - 1) {
      const int bb = wave;
#pragma unroll
      for (int k = 1; k < NB; ++k) {
        if (bb + k >= NB) break;
        const int aa = bb + k;
        f32x4 X = z4;
#pragma unroll
        for (int j = 0; j < k; ++j) {
          const f32x4 af = *(const f32x4 *)(Af + (16 * aa + m16) * LDA +
                                            16 * (bb + j) + 4 * g4);
          X = mma16_f32(af, Tcol[j], X);
        }
        const f32x4 ta = *(const f32x4 *)(Taa + (aa * 16 + m16) * 16 + 4 * g4);
        const f32x4 Tn = -mma16_f32(ta, X, z4);
        Tcol[k] = Tn;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Tb[(16 * aa + 4 * g4 + j) * LDC + 16 * bb + m16] = (bf16)Tn[j];
      }
    } else {
      for (int it = 8 + wave - (NB - 1); it < NKT * NTU; it += NW - (NB - 1))
        qk_unit(NB * NKU + it);
    }
    __syncthreads();  // B4

    // ---- W (as -W A-operand units) and U (accumulator tiles) -------------
    // rows of T scaled by beta_s Gam_s (for W) or beta_s (for U) along s;
    // token tile rt uses token units 0 .. rt / 2.  Waves 0-3 make -W, waves
    // 4-7 U, 12 matrix-core steps each (at d_v = 128).
    auto load_t = [&](int rt, frag *tf, const float *sc) {
      const int umax = rt / 2;
#pragma unroll
      for (int uu = 0; uu < NTU; ++uu) {
        const int k0 = 32 * min(uu, umax);
        const frag t = M::load_k(Tb + (16 * rt + m16) * LDC + k0, g4, true);
        // scales of tokens k0 + koff(g, e): two runs of 4 tokens
        const f32x4 lo = *(const f32x4 *)(sc + k0 + 4 * g4);
        const f32x4 hi = *(const f32x4 *)(sc + k0 + 16 + 4 * g4);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          tf[uu][e] = (bf16)((float)t[e] * (e < 4 ? lo[e] : hi[e - 4]));
      }
    };
    auto w_units = [&](int rt, int u0, int u1) {
      frag tw[NTU];
      load_t(rt, tw, s_bg);
      const int umax = rt / 2;
      for (int u = u0; u < u1; ++u) {
        f32x4 acc[2] = {z4, z4};
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          if (uu <= umax)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int ct = 2 * u + hh;
              acc[hh] = M::mma(load_k_cm<bf16, C>(KT + (16 * ct + m16) * LDC,
                                                  16 * ct + m16, 32 * uu, g4,
                                                  true),
                               tw[uu], acc[hh]);
            }
        st_stream(blk + W.off_negw + ((size_t)(rt * NKU + u) * 64 + lane) * 16,
                  M::pack(-acc[0], -acc[1]));
      }
    };
    auto u_tiles = [&](int rt, int v0, int v1) {
      v1 = min(v1, nvt);
      if (v0 >= v1) return;
      frag tu[NTU];
      load_t(rt, tu, s_beta);
      const int umax = rt / 2;
      for (int vt = v0; vt < v1; ++vt) {
        f32x4 acc = z4;
#pragma unroll
        for (int uu = 0; uu < NTU; ++uu)
          if (uu <= umax)
            acc = M::mma(tu[uu],
                         load_k_cm<bf16, C>(VT + (16 * vt + m16) * LDC,
                                            16 * vt + m16, 32 * uu, g4, true),
                         acc);
        const float a4[4] = {acc[0], acc[1], acc[2], acc[3]};
        st_stream((bf16 *)(blk + W.off_u) + ((size_t)(vt * NB + rt) * 64 + lane) * 4,
                  Vec4<bf16>::put(a4));
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
    __syncthreads();  // B5: LDS free for the next task
  }
}

}  // namespace gdn

bool prep_gdn_applies(const PrefillParams &p, int io_bf16) {
  return io_bf16 && p.gate_head && !p.use_conv && !p.train_at &&
         p.Dk == gdn::DK && p.C == gdn::C && p.Dv % 16 == 0 && p.Dv <= 128;
}

hipError_t launch_prefill_prep_gdn(const PrefillParams &p, hipStream_t s) {
  const long long ntask = (long long)p.B * p.H * p.NC;
  // two workgroups per CU
  const unsigned grid = (unsigned)std::min<long long>(ntask, 2LL * cu_count());
  if (p.gate_bf16)
    hipLaunchKernelGGL(gdn::kda_chunk_prep_gdn<bf16>, dim3(grid),
                       dim3(gdn::NT), 0, s, p);
  else
    hipLaunchKernelGGL(gdn::kda_chunk_prep_gdn<float>, dim3(grid),
                       dim3(gdn::NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace kda
