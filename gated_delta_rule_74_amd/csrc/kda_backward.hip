// kda_backward.hip -- gradient of the chunked KDA prefill (gfx950).
//
// With the chunk factors of the forward (kda_prep_impl.h: P, Qtil = scale
// Q*Gam, Ktil = K*gam/Gam, W, U, gam per (batch*head, chunk)) and the state
// S_n at the start of every chunk (saved by the forward state pass), the
// loss gradient flows back through each chunk n as
//   dDelta = P^T dO + Ktil dS'                  (dS' = gradient at the end)
//   dS     = diag(gam) dS' + Qtil^T dO - W^T dDelta   (gradient at the start)
// which is sequential over chunks (this file's first kernel, last chunk
// first), and then, for every chunk independently, through the UT transform
// and the decayed Gram products of that chunk into dq, dk, dv, dg, dbeta
// (the second and third kernels).  The algebra is the reverse mode of the
// token rule (see include/kda.h for the sources); each step below names the
// forward product it differentiates.
#include "kda_device.h"
#include "kda_internal.h"

#include <type_traits>

namespace kda {

constexpr int BWD_THREADS = 256;
constexpr int DVMAX_BWD = 128;
// the widest contraction of the tile products below (d_k, d_v <= 128,
// chunk <= 64): they issue the reads of that many k for every tile
constexpr int TILE_KMAX = 128;

// 8 consecutive elements of a row as one 16-byte (bf16) or two 16-byte
// (fp32) accesses: raw copies between global memory and LDS, and
// conversions to and from fp32
template <typename T> struct Row8 {
  static_assert(sizeof(T) == 2 || sizeof(T) == 4, "bf16 or fp32");
  static constexpr int NQ = sizeof(T) / 2;  // 16-byte quads per 8 elements
  uint4 q[NQ];
  __device__ __forceinline__ void load(const T *p) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) q[i] = ((const uint4 *)p)[i];
  }
  __device__ __forceinline__ void store(T *p) const {
#pragma unroll
    for (int i = 0; i < NQ; ++i) ((uint4 *)p)[i] = q[i];
  }
  __device__ __forceinline__ float get(int e) const {
    const unsigned w = ((const unsigned *)q)[NQ == 1 ? e / 2 : e];
    return NQ == 1 ? __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16))
                   : __uint_as_float(w);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < NQ; ++i) q[i] = make_uint4(0u, 0u, 0u, 0u);
  }
};
// 8 floats to 8 elements of type T at p (LDS), rounding to nearest even
template <typename T>
__device__ __forceinline__ void put8(T *p, const float v[8]) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
    *(bf16x8 *)p = r;
  } else {
    *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4 *)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// ---------------------------------------------------------------------------
// helpers: fragment units <-> LDS
// ---------------------------------------------------------------------------

// Write the A-operand units of a matrix X (row tile a, k unit u at
// sec[(a * nku + u) * 64 + lane]) transposed into LDS: XT[k][16a + m].
// Units with u > a / TPU are taken as zero when `lower` (the never-written
// units above the diagonal of P).
template <typename IO>
__device__ __forceinline__ void units_to_lds_t(const char *sec, int nrt,
                                               int nku, int kmax, bool lower,
                                               IO *XT, int ldt, int tid) {
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int KU = 16 * M::TPU;
  for (int w = tid; w < nrt * nku * 64; w += BWD_THREADS) {
    const int lane = w & 63, unit = w >> 6;
    const int a = unit / nku, u = unit % nku;
    const int m = lane & 15, g = lane >> 4;
    frag f;
    if (lower && u > a / M::TPU) {
      f = frag{};
    } else {
      f = *(const frag *)(sec + (size_t)w * 16);
    }
#pragma unroll
    for (int e = 0; e < M::NE; ++e) {
      const int k = KU * u + M::koff(g, e);
      if (k < kmax) XT[k * ldt + 16 * a + m] = (IO)M::elem(f, e);
    }
  }
}

// the same, split in two steps so the global loads of the next chunk can be
// in flight while the current one is computed: each thread holds its NU
// units' raw bytes (slots w = tid + 256 j) between fetch and store
template <typename IO, int NU>
struct UnitStage {
  uint4 raw[NU];
  __device__ __forceinline__ void fetch(const char *sec, int nrt, int nku,
                                        bool lower, int tid) {
    using M = Mma<IO>;
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      // every slot loads (past the end: the last unit again), so that the
      // compiler counts the loads exactly; store_t skips or zeroes the
      // slots that carry nothing
      // (units above the diagonal of a lower-triangular factor: the
      // diagonal unit of the row again, an L1 hit)
      const int w = min(tid + BWD_THREADS * j, nrt * nku * 64 - 1);
      const int unit = w >> 6, a = unit / nku, u = unit % nku;
      const int ws = (lower && u > a / M::TPU)
                         ? ((a * nku + a / M::TPU) << 6) + (w & 63)
                         : w;
      raw[j] = *(const uint4 *)(sec + (size_t)ws * 16);
    }
  }
  __device__ __forceinline__ void store_t(int nrt, int nku, int kmax, IO *XT,
                                          int ldt, int tid,
                                          bool lower = false) const {
    using M = Mma<IO>;
    typedef typename M::frag frag;
    constexpr int KU = 16 * M::TPU;
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int w = tid + BWD_THREADS * j;
      if (w >= nrt * nku * 64) break;
      const int lane = w & 63, unit = w >> 6;
      const int a = unit / nku, u = unit % nku;
      const int m = lane & 15, g = lane >> 4;
      // units above the diagonal of a lower-triangular factor hold nothing
      // the prep wrote: zeros
      const uint4 rw = (lower && u > a / M::TPU) ? make_uint4(0u, 0u, 0u, 0u)
                                                 : raw[j];
      const frag f = __builtin_bit_cast(frag, rw);
#pragma unroll
      for (int e = 0; e < M::NE; ++e) {
        const int k = KU * u + M::koff(g, e);
        if (k < kmax) XT[k * ldt + 16 * a + m] = (IO)M::elem(f, e);
      }
    }
  }
};

// same, not transposed: X[16a + m][k]
template <typename IO>
__device__ __forceinline__ void units_to_lds(const char *sec, int nrt, int nku,
                                             int kmax, IO *X, int ld, int tid) {
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int KU = 16 * M::TPU;
  for (int w = tid; w < nrt * nku * 64; w += BWD_THREADS) {
    const int lane = w & 63, unit = w >> 6;
    const int a = unit / nku, u = unit % nku;
    const int m = lane & 15, g = lane >> 4;
    const frag f = *(const frag *)(sec + (size_t)w * 16);
#pragma unroll
    for (int e = 0; e < M::NE; ++e) {
      const int k = KU * u + M::koff(g, e);
      if (k < kmax) X[(16 * a + m) * ld + k] = (IO)M::elem(f, e);
    }
  }
}

// B-operand unit from a LDS array whose rows are the product's columns n
// and are contiguous in k (as load_k); k beyond kmax reads zero
template <typename IO>
__device__ __forceinline__ typename Mma<IO>::frag lds_unit(const IO *row,
                                                           int u, int g,
                                                           int kmax) {
  using M = Mma<IO>;
  constexpr int KU = 16 * M::TPU;
  return M::load_k(row + KU * u, g, KU * u + 16 < kmax || M::TPU == 1);
}

// ---------------------------------------------------------------------------
// kernel 1: reverse state pass
// ---------------------------------------------------------------------------

template <typename IO, int DK, int C> struct BL {  // reverse-pass LDS layout
  static constexpr int PE = 16 / (int)sizeof(IO);
  static constexpr int LDC = C + PE, LDK = DK + PE;
  static constexpr int TPU = Mma<IO>::TPU;
  static constexpr int NB = C / 16, NKT = DK / 16;
  static constexpr int NTU = (NB + TPU - 1) / TPU, NKU = (NKT + TPU - 1) / TPU;
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t oPT = 0;                                  // [C][LDC]
  static constexpr size_t oKK = al(oPT + (size_t)C * LDC * sizeof(IO));   // [C][LDK]
  static constexpr size_t oQT = al(oKK + (size_t)C * LDK * sizeof(IO));   // [DK][LDC]
  static constexpr size_t oWT = al(oQT + (size_t)DK * LDC * sizeof(IO));  // [DK][LDC]
  static constexpr size_t oOT = al(oWT + (size_t)DK * LDC * sizeof(IO));  // [16][LDC]
  static constexpr size_t oSU = al(oOT + (size_t)16 * LDC * sizeof(IO));  // dS units
  static constexpr size_t oDU = al(oSU + (size_t)NKU * 1024);             // dDelta units
  static constexpr size_t oGm = al(oDU + (size_t)NTU * 1024);             // gam [DK]
  static constexpr size_t total = oGm + DK * 4;
};

// the reverse pass's workgroup: the four working waves and one L2 warm-up
// wave
constexpr int BWD_STATE_THREADS = BWD_THREADS + 64;
constexpr int BWD_STATE_PF = 4;  // chunks between warming and use

template <typename IO, int DK, int C>
__global__ __launch_bounds__(BWD_STATE_THREADS) void kda_bwd_state(
    BwdParams bp) {
  using M = Mma<IO>;
  using L = BL<IO, DK, C>;
  typedef typename M::frag frag;
  constexpr int NB = L::NB, NKT = L::NKT, TPU = L::TPU, NTU = L::NTU,
                NKU = L::NKU, LDC = L::LDC, LDK = L::LDK;
  constexpr int KT = (NKT + 3) / 4;  // key tiles per wave
  const PrefillParams &p = bp.f;
  __shared__ __attribute__((aligned(16))) char sm[L::total];
  IO *PT = (IO *)(sm + L::oPT), *KK = (IO *)(sm + L::oKK);
  IO *QT = (IO *)(sm + L::oQT), *WT = (IO *)(sm + L::oWT);
  IO *OT = (IO *)(sm + L::oOT);
  frag *SU = (frag *)(sm + L::oSU), *DU = (frag *)(sm + L::oDU);
  float *Gm = (float *)(sm + L::oGm);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15, g4 = lane >> 4;
  const int Dv = p.Dv, H = p.H, T = p.T, NC = p.NC;
  const int nvt = Dv / 16;
  int bh, vt;
  {
    // a head's slab workgroups on one XCD (blocks go round-robin over the
    // 8 XCDs), so they read the head's factors through one L2
    const int blk = blockIdx.x, BH = p.B * H;
    if (nvt > 1 && (BH & 7) == 0) {
      const int x = blk & 7, jj = blk >> 3;
      bh = (jj / nvt) * 8 + x;
      vt = jj % nvt;
    } else {
      bh = blk / nvt;
      vt = blk % nvt;
    }
  }
  const int b = bh / H, h = bh % H;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const size_t orow = (size_t)H * Dv;  // elements between tokens

  if (wave == BWD_THREADS / 64) {
    // L2 warm-up wave: while chunk n is worked on, touches 4 bytes of every
    // 128-byte line of chunk n - PF's factor block (the head's nvt
    // workgroups split the lines) and of the chunk's dO rows of this slab,
    // as direct-to-LDS loads into a sink that nothing reads.  It takes part
    // in every barrier of the other waves (one before the loop, three per
    // chunk) without waiting for its loads.
    __shared__ __attribute__((aligned(256))) char sink[256];
    const int nline = (int)((p.wsb + 127) / 128);
    const int share = (nline + nvt - 1) / nvt;
    const char *ws0 = p.ws + (size_t)bh * NC * p.wsb;
    auto warm = [&](int n) {
      const char *blk = ws0 + (size_t)n * p.wsb;
      for (int k0 = 0; k0 < share; k0 += 64) {
        const int ln = min(vt * share + min(k0 + lane, share - 1), nline - 1);
        __builtin_amdgcn_global_load_lds(
            (const void *)(blk + (size_t)ln * 128),
            (__attribute__((address_space(3))) void *)sink, 4, 0, 0);
      }
      const int t = min(n * C + min(lane, C - 1), T - 1);
      __builtin_amdgcn_global_load_lds(
          (const void *)((const IO *)bp.dO + ((size_t)b * T + t) * orow +
                         (size_t)h * Dv + 16 * vt),
          (__attribute__((address_space(3))) void *)sink, 4, 0, 0);
    };
    for (int n = NC - 1; n >= 0 && n >= NC - BWD_STATE_PF; --n) warm(n);
    barrier_keep_vmem();
    for (int n = NC - 1; n >= 0; --n) {
      if (n - BWD_STATE_PF >= 0) warm(n - BWD_STATE_PF);
      barrier_keep_vmem();
      barrier_keep_vmem();
      barrier_keep_vmem();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // dS key tiles owned by this wave: t = wave + 4 j (accumulator layout:
  // lane 16 g + n holds column n, rows 4g..4g+3 of the tile)
  f32x4 dS[KT];
#pragma unroll
  for (int j = 0; j < KT; ++j) {
    dS[j] = zero;
    const int t = wave + 4 * j;
    if (bp.dsT && t < NKT) {
      const float *src = bp.dsT + ((size_t)bh * DK + 16 * t + 4 * g4) * Dv +
                         16 * vt + m16;
#pragma unroll
      for (int e = 0; e < 4; ++e) dS[j][e] = src[(size_t)e * Dv];
    }
  }
  auto publish_ds = [&]() {
    // B units of dS (k = key channel, n = value column)
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int t = wave + 4 * j;
      if (t < NKT) {
        frag *dst = SU + (t / TPU) * 64 + lane;
        if (TPU == 2) {
          bf16x4 v4 = {(bf16)dS[j][0], (bf16)dS[j][1], (bf16)dS[j][2],
                       (bf16)dS[j][3]};
          *(bf16x4 *)((char *)dst + 8 * (t & 1)) = v4;
        } else {
          *(f32x4 *)dst = dS[j];
        }
      }
    }
  };
  // zero the units once (an odd tile count leaves a half that is never
  // written)
  for (int i = tid; i < (NKU + NTU) * 256; i += BWD_THREADS)
    ((float *)SU)[i] = 0.f;
  __syncthreads();
  publish_ds();

  // the next chunk's factors, dO slab and gam wait in registers
  constexpr int NUP = (NB * NTU * 64 + BWD_THREADS - 1) / BWD_THREADS;
  constexpr int NUK = (NKT * NTU * 64 + BWD_THREADS - 1) / BWD_THREADS;
  constexpr int NUQ = (NB * NKU * 64 + BWD_THREADS - 1) / BWD_THREADS;
  static_assert(2 * C <= BWD_THREADS, "two lanes per token of the chunk");
  UnitStage<IO, NUP> stP;
  UnitStage<IO, NUK> stK;
  UnitStage<IO, NUQ> stQ, stW;
  Row8<IO> ov;  // lanes 2r, 2r + 1: token r, value columns 8 (tid & 1) + 0..7
  bool ovz = false;  // the token lies past the sequence: ov counts as zero
  float gv = 0.f;
  auto blk_of = [&](int n) { return p.ws + ((size_t)bh * NC + n) * p.wsb; };
  auto fetch_ov = [&](int n) {
    const char *blk = blk_of(n);
    if (tid < 2 * C) {
      const int r = tid >> 1, t = min(n * C + r, T - 1);
      ov.load((const IO *)bp.dO + ((size_t)b * T + t) * orow + (size_t)h * Dv +
              16 * vt + 8 * (tid & 1));
      // zeroed where it is used: writing the registers of a load in flight
      // would make the wave wait here for every load just issued
      ovz = n * C + r >= T;
    }
    if (tid < DK) gv = ((const float *)(blk + W.off_gam))[tid];
  };
  {
    const char *blk = blk_of(NC - 1);
    stP.fetch(blk + W.off_p, NB, NTU, true, tid);
    stK.fetch(blk + W.off_ktt, NKT, NTU, false, tid);
    stQ.fetch(blk + W.off_qt, NB, NKU, false, tid);
    stW.fetch(blk + W.off_negw, NB, NKU, false, tid);
    fetch_ov(NC - 1);
  }

  for (int n = NC - 1; n >= 0; --n) {
    const int t0 = n * C;
    // ---- stage the chunk's factors, transposed where the products need it;
    // each part's registers take the next chunk's loads as soon as they are
    // staged (chunk 0 loads itself again), so the waves' waits at issue for
    // the texture units overlap the LDS writes of the other parts
    const char *nblk = blk_of(max(n - 1, 0));
    stP.store_t(NB, NTU, C, PT, LDC, tid, true);
    stP.fetch(nblk + W.off_p, NB, NTU, true, tid);
    stK.store_t(NKT, NTU, C, KK, LDK, tid);
    stK.fetch(nblk + W.off_ktt, NKT, NTU, false, tid);
    stQ.store_t(NB, NKU, DK, QT, LDC, tid);
    stQ.fetch(nblk + W.off_qt, NB, NKU, false, tid);
    stW.store_t(NB, NKU, DK, WT, LDC, tid);
    stW.fetch(nblk + W.off_negw, NB, NKU, false, tid);
    if (tid < 2 * C) {
      // dO slab transposed: OT[value column][token]
      const int r = tid >> 1, c0 = 8 * (tid & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        OT[(c0 + e) * LDC + r] = from_f32<IO>(ovz ? 0.f : ov.get(e));
    }
    if (tid < DK) Gm[tid] = gv;
    fetch_ov(max(n - 1, 0));
    __syncthreads();

    // ---- the gradient at this chunk's end, for the per-chunk kernels
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int t = wave + 4 * j;
      if (t < NKT) {
        float *dst = bp.dSc + (((size_t)bh * NC + n) * DK + 16 * t + 4 * g4) * Dv +
                     16 * vt + m16;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)e * Dv] = dS[j][e];
      }
    }

    // ---- dDelta = P^T dO + Ktil dS'   (token tile rt = wave)
    if (wave < NB) {
      const int rt = wave;
      f32x4 acc = zero;
#pragma unroll
      for (int u = 0; u < NTU; ++u)
        acc = M::mma(lds_unit<IO>(PT + (16 * rt + m16) * LDC, u, g4, C),
                     lds_unit<IO>(OT + m16 * LDC, u, g4, C), acc);
#pragma unroll
      for (int u = 0; u < NKU; ++u)
        acc = M::mma(lds_unit<IO>(KK + (16 * rt + m16) * LDK, u, g4, DK),
                     SU[u * 64 + lane], acc);
      // lane holds dDelta[16 rt + 4 g4 + e][16 vt + m16]
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + 16 * rt + 4 * g4 + e;
        // stored in the q/k/v dtype: every reader rounds it to that type
        // as an operand anyway, so the results are the same bit for bit
        if (t < T)
          ((IO *)bp.dD)[((size_t)b * T + t) * orow + (size_t)h * Dv + 16 * vt +
                        m16] = from_f32<IO>(acc[e]);
      }
      frag *dst = DU + (rt / TPU) * 64 + lane;
      if (TPU == 2) {
        bf16x4 v4 = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
        *(bf16x4 *)((char *)dst + 8 * (rt & 1)) = v4;
      } else {
        *(f32x4 *)dst = acc;
      }
    }
    __syncthreads();

    // ---- dS <- diag(gam) dS' + Qtil^T dO + (-W)^T dDelta
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int t = wave + 4 * j;
      if (t < NKT) {
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = dS[j][e] * Gm[16 * t + 4 * g4 + e];
#pragma unroll
        for (int u = 0; u < NTU; ++u) {
          acc = M::mma(lds_unit<IO>(QT + (16 * t + m16) * LDC, u, g4, C),
                       lds_unit<IO>(OT + m16 * LDC, u, g4, C), acc);
          acc = M::mma(lds_unit<IO>(WT + (16 * t + m16) * LDC, u, g4, C),
                       DU[u * 64 + lane], acc);
        }
        dS[j] = acc;
      }
    }
    __syncthreads();  // every read of this chunk's LDS is done
    publish_ds();
  }
  if (bp.ds0) {
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int t = wave + 4 * j;
      if (t < NKT) {
        float *dst = bp.ds0 + ((size_t)bh * DK + 16 * t + 4 * g4) * Dv +
                     16 * vt + m16;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)e * Dv] = dS[j][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// one 16x16 tile of op(A) op(B) on the matrix cores, operands gathered from
// LDS (element types TA / TB, fp32 or the q/k/v dtype) and rounded to the
// product's operand type:
//   op(A)[m][k] = AT ? A[k * lda + m] : A[m * lda + k]
//   op(B)[k][n] = BT ? B[n * ldb + k] : B[k * ldb + n]
// acc is in the accumulator layout: lane 16 g + n holds column n0 + n and
// rows m0 + 4g .. m0 + 4g + 3.
// ---------------------------------------------------------------------------
template <typename IO, bool AT, bool BT, typename TA, typename TB>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const TA *A, int lda,
                                          const TB *B, int ldb, int m0, int n0,
                                          int K, int lane) {
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int KU = 16 * M::TPU;
  constexpr int NU = TILE_KMAX / KU;
  const int m = lane & 15, g = lane >> 4;
  const int ulast = (K - 1) / KU;
  // every unit's operands first, then the products: the reads overlap
  // instead of each product waiting for its own
  frag fa[NU], fb[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int uu = min(u, ulast);  // units past K re-read the last one
    if constexpr (!AT && sizeof(TA) == 4) {
      // fp32 rows of A: a lane's k values come in runs of 4 (k = 4g + e and,
      // for 32-wide units, 16 + 4g + e), one 16-byte read each; K is a
      // multiple of 16, so a run is wholly inside or outside it
#pragma unroll
      for (int h = 0; h < M::NE / 4; ++h) {
        const int k = KU * uu + 16 * h + 4 * g;
        const f32x4 a4 = k < K ? *(const f32x4 *)(A + (m0 + m) * lda + k)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) M::set(fa[u], 4 * h + e, a4[e]);
      }
#pragma unroll
      for (int e = 0; e < M::NE; ++e) {
        const int k = KU * uu + M::koff(g, e);
        M::set(fb[u], e,
               k < K ? to_f32(BT ? B[(n0 + m) * ldb + k] : B[k * ldb + n0 + m])
                     : 0.f);
      }
    } else {
#pragma unroll
      for (int e = 0; e < M::NE; ++e) {
        const int k = KU * uu + M::koff(g, e);
        float av = 0.f, bv = 0.f;
        if (k < K) {
          av = to_f32(AT ? A[k * lda + m0 + m] : A[(m0 + m) * lda + k]);
          bv = to_f32(BT ? B[(n0 + m) * ldb + k] : B[k * ldb + n0 + m]);
        }
        M::set(fa[u], e, av);
        M::set(fb[u], e, bv);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (u <= ulast) acc = M::mma(fa[u], fb[u], acc);
  return acc;
}

// the same for A and B both given as k-contiguous rows of the q/k/v dtype
// (op(A) = A, op(B) = B^T): whole fragment units per load, no gathers
template <typename IO>
__device__ __forceinline__ f32x4 tile_mma_rows(f32x4 acc, const IO *A, int lda,
                                               const IO *B, int ldb, int m0,
                                               int n0, int K, int lane) {
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int KU = 16 * M::TPU;
  constexpr int NU = TILE_KMAX / KU;
  const int m = lane & 15, g = lane >> 4;
  const int ulast = (K - 1) / KU;
  frag fa[NU], fb[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int uu = min(u, ulast);
    const bool full = KU * uu + 16 < K || M::TPU == 1;
    fa[u] = M::load_k(A + (m0 + m) * lda + KU * uu, g, full);
    fb[u] = M::load_k(B + (n0 + m) * ldb + KU * uu, g, full);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (u <= ulast) acc = M::mma(fa[u], fb[u], acc);
  return acc;
}

// A as fp32 rows (k contiguous, 16-byte reads, rounded to the product's
// operand type) and B given by the k-contiguous rows of B^T in the q/k/v
// dtype (op(B) = B^T rows, whole fragment units per load)
template <typename IO>
__device__ __forceinline__ f32x4 tile_mma_f32a(f32x4 acc, const float *A,
                                               int lda, const IO *Bt, int ldb,
                                               int m0, int n0, int K,
                                               int lane) {
  using M = Mma<IO>;
  typedef typename M::frag frag;
  constexpr int KU = 16 * M::TPU;
  constexpr int NU = TILE_KMAX / KU;
  const int m = lane & 15, g = lane >> 4;
  const int ulast = (K - 1) / KU;
  frag fa[NU], fb[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int uu = min(u, ulast);
#pragma unroll
    for (int h = 0; h < M::NE / 4; ++h) {
      const int k = KU * uu + 16 * h + 4 * g;
      const f32x4 a4 = k < K ? *(const f32x4 *)(A + (m0 + m) * lda + k)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) M::set(fa[u], 4 * h + e, a4[e]);
    }
    const bool full = KU * uu + 16 < K || M::TPU == 1;
    fb[u] = M::load_k(Bt + (n0 + m) * ldb + KU * uu, g, full);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (u <= ulast) acc = M::mma(fa[u], fb[u], acc);
  return acc;
}

// per-chunk intermediates: the second kernel writes
// [Delta C x Dv | dQtil C x Dk | dKtil C x Dk | dW C x Dk | dgam Dk], the
// third adds [Kd = K*Gam | dKd] (C x Dk each) for its own later phases;
// fp32 slots, Delta and dW stored in the q/k/v dtype (their readers only
// use them as operands of that type)
// dQtil, dKtil and dKd (C x Dk each) are kept tile by tile in the
// accumulator layout: tile (rt, it) is 64 lanes x 4 floats, lane 16 g + n
// holding rows 16 rt + 4 g .. + 3 of column 16 it + n, so the lane that
// produces a tile and the lane that later consumes it move 16 bytes at once
__host__ __device__ inline size_t bwd_tile_off(int rt, int it, int nkt,
                                               int lane) {
  return (((size_t)rt * nkt + it) * 64 + lane) * 4;
}
__host__ __device__ inline size_t bwd_gs_floats(int C, int Dk, int Dv) {
  return (size_t)C * (Dv + 5 * Dk) + Dk;
}

// ---------------------------------------------------------------------------
// kernel 2: per chunk, the products with the chunk's start state S and the
// gradient at its end dS' (recomputed Delta = U - W S; dQtil = dO S^T;
// dW = -dDelta S^T; dKtil = Delta dS'^T; dgam = rowsum(dS' * S)), 32 value
// columns at a time
// ---------------------------------------------------------------------------
template <typename IO, int DK, int C> struct G1L {
  static constexpr int SV = 32;  // value columns per slab
  static constexpr int PE = 16 / (int)sizeof(IO);  // row padding
  static constexpr int LK = DK + PE, LS = SV + PE;
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  // every array in the q/k/v dtype, rows contiguous in the contracted index
  static constexpr size_t oW = 0;                                    // -W [C][LK]
  static constexpr size_t oST = al(oW + (size_t)C * LK * sizeof(IO));  // S^T [SV][LK]
  static constexpr size_t oS = al(oST + (size_t)SV * LK * sizeof(IO)); // S [DK][LS]
  static constexpr size_t odS = al(oS + (size_t)DK * LS * sizeof(IO)); // dS' [DK][LS]
  static constexpr size_t oO = al(odS + (size_t)DK * LS * sizeof(IO)); // dO [C][LS]
  static constexpr size_t odD = al(oO + (size_t)C * LS * sizeof(IO));  // dDelta
  static constexpr size_t oD = al(odD + (size_t)C * LS * sizeof(IO));  // Delta
  static constexpr size_t oG = al(oD + (size_t)C * LS * sizeof(IO));   // dgam [DK]
  static constexpr size_t total = oG + DK * 4;
};

template <typename IO, int DK, int C>
__global__ __launch_bounds__(BWD_THREADS, 2) void kda_bwd_chunk_state(
    BwdParams bp) {
  using L = G1L<IO, DK, C>;
  constexpr int SV = L::SV, NB = C / 16, NKT = DK / 16, LK = L::LK, LS = L::LS;
  constexpr int NTL = NB * NKT;          // C x DK output tiles
  constexpr int TW = (NTL + 3) / 4;      // of them per wave
  constexpr int NKU = (NKT + Mma<IO>::TPU - 1) / Mma<IO>::TPU;
  const PrefillParams &p = bp.f;
  __shared__ __attribute__((aligned(16))) char sm[L::total];
  IO *nW = (IO *)(sm + L::oW), *STs = (IO *)(sm + L::oST);
  IO *Ss = (IO *)(sm + L::oS), *dSs = (IO *)(sm + L::odS);
  IO *Os = (IO *)(sm + L::oO), *dDs = (IO *)(sm + L::odD);
  IO *Ds = (IO *)(sm + L::oD);
  float *dgs = (float *)(sm + L::oG);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15, g4 = lane >> 4;
  const int Dv = p.Dv, H = p.H, T = p.T, NC = p.NC;
  const int bh = blockIdx.x / NC, n = blockIdx.x % NC;
  const int b = bh / H, h = bh % H, t0 = n * C;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  const char *blk = p.ws + ((size_t)bh * NC + n) * p.wsb;
  const float *S = bp.Sc + ((size_t)bh * NC + n) * DK * Dv;
  const float *dS = bp.dSc + ((size_t)bh * NC + n) * DK * Dv;
  float *gs = bp.gs + ((size_t)bh * NC + n) * bwd_gs_floats(C, DK, Dv);
  const size_t orow = (size_t)H * Dv;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

  constexpr int NGA = (DK * SV / 8 + BWD_THREADS - 1) / BWD_THREADS;
  // a slab's global loads (clamped addresses, branch-free): rows of S and
  // dS', 8 columns of a row per lane (sv is a multiple of 16), rows of dO
  // and dDelta, and this wave's U tiles (accumulator layout, 4 elements per
  // lane).  The next slab's are issued as soon as this slab's have gone to
  // LDS, so they arrive while this slab's products run.
  constexpr int NO8 = (C * SV / 8 + BWD_THREADS - 1) / BWD_THREADS;
  constexpr int NUT = (NB * (SV / 16) + 3) / 4;
  typedef std::conditional_t<sizeof(IO) == 2, uint2, uint4> U4;
  Row8<float> la[NGA], lb[NGA];
  Row8<IO> lo[NO8], ld[NO8];
  U4 ur[NUT];
  auto issue = [&](int c0) {
    const int sv = min(SV, Dv - c0);
#pragma unroll
    for (int j = 0; j < NGA; ++j) {
      const int i = min(8 * (tid + BWD_THREADS * j), DK * SV - 8);
      const int r = i / SV, c = min(i % SV, sv - 8);
      la[j].load(S + (size_t)r * Dv + c0 + c);
      lb[j].load(dS + (size_t)r * Dv + c0 + c);
    }
#pragma unroll
    for (int j = 0; j < NO8; ++j) {
      const int i = min(8 * (tid + BWD_THREADS * j), C * SV - 8);
      const int r = i / SV, c = min(i % SV, sv - 8), t = min(t0 + r, T - 1);
      const size_t gi = ((size_t)b * T + t) * orow + (size_t)h * Dv + c0 + c;
      lo[j].load((const IO *)bp.dO + gi);
      ld[j].load((const IO *)bp.dD + gi);
    }
#pragma unroll
    for (int j = 0; j < NUT; ++j) {
      const int tl = min(wave + 4 * j, NB * (SV / 16) - 1);
      const int rt = tl % NB, vt = min((c0 >> 4) + tl / NB, Dv / 16 - 1);
      ur[j] = *((const U4 *)(blk + W.off_u) + (size_t)(vt * NB + rt) * 64 + lane);
    }
  };

  units_to_lds<IO>(blk + W.off_negw, NB, NKU, DK, nW, LK, tid);  // -W[r][i]
  for (int i = tid; i < DK; i += BWD_THREADS) dgs[i] = 0.f;
  __syncthreads();
  // (issued before the -W staging instead, the first slab's loads slow it)
  issue(0);

  f32x4 aQ[TW], aK[TW], aW[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) aQ[j] = aK[j] = aW[j] = zero;
  // dgam = rowsum(dS' * S): this thread's 8 columns of key row
  // 8 (tid + 256 j) / SV, summed over the value slabs here and over the SV / 8
  // lanes of a row at the end
  float dga[NGA];
#pragma unroll
  for (int j = 0; j < NGA; ++j) dga[j] = 0.f;

  for (int c0 = 0; c0 < Dv; c0 += SV) {
    const int sv = min(SV, Dv - c0);
#pragma unroll
    for (int j = 0; j < NGA; ++j) {
      const int i = 8 * (tid + BWD_THREADS * j), r = i / SV, c = i % SV;
      if (i < DK * SV) {
        const bool ok = c < sv;
        float s8[8], d8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s8[e] = ok ? la[j].get(e) : 0.f;
          d8[e] = ok ? lb[j].get(e) : 0.f;
          dga[j] += s8[e] * d8[e];
          STs[(c + e) * LK + r] = (IO)s8[e];
        }
        put8(Ss + r * LS + c, s8);
        put8(dSs + r * LS + c, d8);
      }
    }
#pragma unroll
    for (int j = 0; j < NO8; ++j) {
      const int i = 8 * (tid + BWD_THREADS * j), r = i / SV, c = i % SV;
      if (i < C * SV) {
        const bool ok = c < sv && t0 + r < T;
        float o8[8], d8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o8[e] = ok ? lo[j].get(e) : 0.f;
          d8[e] = ok ? ld[j].get(e) : 0.f;
        }
        put8(Os + r * LS + c, o8);
        put8(dDs + r * LS + c, d8);
      }
    }
    U4 uc[NUT];
#pragma unroll
    for (int j = 0; j < NUT; ++j) uc[j] = ur[j];
    if (c0 + SV < Dv) issue(c0 + SV);
    __syncthreads();
    // Delta = U - W S on this slab (U in accumulator tiles [vt][rt])
#pragma unroll
    for (int j = 0; j < NUT; ++j) {
      const int tl = wave + 4 * j;
      if (tl >= NB * (SV / 16)) break;
      const int rt = tl % NB, ct = tl / NB;
      f32x4 acc = zero;
      if (16 * ct < sv) {
        const IO *us = (const IO *)&uc[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = to_f32(us[e]);
        acc = tile_mma_rows<IO>(acc, nW, LK, STs, LK, 16 * rt, 16 * ct, DK,
                                lane);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * g4 + e;
        Ds[r * LS + 16 * ct + m16] = (IO)acc[e];
        if (16 * ct < sv)
          ((IO *)gs)[(size_t)r * Dv + c0 + 16 * ct + m16] =
              from_f32<IO>(t0 + r < T ? acc[e] : 0.f);
      }
    }
    __syncthreads();
    // dQtil += dO S^T, dW += -dDelta S^T, dKtil += Delta dS'^T
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int tl = wave + 4 * j;
      if (tl < NTL) {
        const int rt = tl % NB, it = tl / NB;
        aQ[j] = tile_mma_rows<IO>(aQ[j], Os, LS, Ss, LS, 16 * rt, 16 * it, SV,
                                  lane);
        aW[j] = tile_mma_rows<IO>(aW[j], dDs, LS, Ss, LS, 16 * rt, 16 * it, SV,
                                  lane);
        aK[j] = tile_mma_rows<IO>(aK[j], Ds, LS, dSs, LS, 16 * rt, 16 * it, SV,
                                  lane);
      }
    }
    __syncthreads();
  }
  static_assert(SV % 8 == 0 && SV / 8 <= 32 && 64 % (SV / 8) == 0,
                "a key row's lanes form a group");
#pragma unroll
  for (int j = 0; j < NGA; ++j) {
    const float x = group_sum<SV / 8>(dga[j]);
    const int i = 8 * (tid + BWD_THREADS * j);
    if (lane % (SV / 8) == 0 && i < DK * SV) atomicAdd(&dgs[i / SV], x);
  }
  __syncthreads();
  float *gQ = gs + (size_t)C * Dv, *gK = gQ + (size_t)C * DK;
  float *gW = gK + (size_t)C * DK, *gG = gW + (size_t)C * DK;
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int tl = wave + 4 * j;
    if (tl < NTL) {
      const int rt = tl % NB, it = tl / NB;
      const size_t ot = bwd_tile_off(rt, it, NKT, lane);
      *(f32x4 *)(gQ + ot) = aQ[j];
      *(f32x4 *)(gK + ot) = aK[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const size_t o = (size_t)(16 * rt + 4 * g4 + e) * DK + 16 * it + m16;
        ((IO *)gW)[o] = from_f32<IO>(-aW[j][e]);
      }
    }
  }
  if (tid < DK) gG[tid] = dgs[tid];
}

// rows r0 .. r0+3 (lane group g of an accumulator tile) += the sums of x[e]
// over the 16 columns of the tile: reduced across the tile's 16 lanes first,
// then one LDS atomic per row instead of one per element
__device__ __forceinline__ void add_rows(float *dst, int r0, const float x[4],
                                         int m16) {
  float sum[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sum[e] = group_sum<16>(x[e]);
  if (m16 == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(&dst[r0 + e], sum[e]);
  }
}

// ---------------------------------------------------------------------------
// kernel 3: per chunk, everything else.  The UT transform T = (I + A)^-1
// and A = diag(beta) M, M[r,s] = sum_i k_ri k_si D_rsi (D_rs = Gam_r/Gam_s,
// a product of e over (s, r]) come from the forward's chunk prep, which
// saves them when it runs for the backward; the gradients are
//   dT = dDelta (beta V)^T + dW (beta Kd)^T,  dv = beta T^T dDelta,
//   dKd = beta T^T dW,  dA = -T^T dT T^T (strictly lower),  dM = beta dA,
//   dP = tril(dO Delta^T),  dbeta = rowsum(V*T^T dDelta + Kd*T^T dW + dA*M)
// then, per key channel i and token r (one owner thread per pair), the
// decayed products
//   rowK_r = sum_{s<r} dM_rs k_s D_rs,    rowQ_r = sum_{s<=r} dPm_rs k_s D_rs
//   colK_r = sum_{s>r} dM_sr k_s D_sr,    colQ_r = sum_{s>=r} dPm_sr q_s D_sr
// (dPm = scale dP) and the elementwise terms of Kd = K*Gam, Qtil = scale
// Q*Gam, Ktil = K*gam/Gam, gam:
//   dk = rowK + colK + colQ + dKd*Gam + dKtil*gam/Gam
//   dq = rowQ + scale dQtil*Gam
//   dG = k rowK + q rowQ - k (colK + colQ) + dKd*Kd + dQtil*Qtil - dKtil*Ktil
//   dG_last += sum_r dKtil*Ktil + dgam*gam,   dg_u = sum_{r>=u} dG_r
// ---------------------------------------------------------------------------
template <typename IO, int DK, int C> struct G2L {
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  // C x C fp32 arrays with rows padded to C + 4: the 16 rows a lane group
  // reads at once then fall in different banks, and rows stay 16-byte
  // aligned for f32x4 accesses
  static constexpr int LCC = C + 4;
  static constexpr size_t CC = (size_t)C * LCC * 4;
  static constexpr size_t oM = 0, oT = CC, odP = 2 * CC, odM = 3 * CC;
  static constexpr size_t oSm = 4 * CC;  // small arrays
  static constexpr int RG = BWD_THREADS / DK;  // row groups of owner threads
  static constexpr size_t oBeta = oSm, odB = oBeta + C * 4,
                          odGl = odB + C * 4, oTail = odGl + DK * 4,
                          odgh = oTail + (size_t)RG * DK * 4,
                          oVote = odgh + C * 4;
  static constexpr size_t oR = al(oVote + 16);  // phase region
  // largest phase: k, q, sigma (q/k/v dtype) and e / rho (fp32); two C x Dv
  // arrays; or the C x C product of phase 5
  static constexpr size_t RK = (size_t)C * DK * (3 * sizeof(IO) + 4);
  // bf16: phases 3 and 4 also keep dDelta^T / dW^T (rows padded to C + 8)
  // as the k-contiguous operand of T^T dDelta and T^T dW
  static constexpr bool TRB = sizeof(IO) == 2;
  static constexpr int LT = C + 8;
  // the C x Dv and C x DK operand arrays of phases 3, 4 and 6 have rows
  // padded by 16 bytes: unpadded, a row is a whole number of bank rows, so
  // the 16 rows that a fragment read takes at once would all hit the same
  // banks
  static constexpr int PE = 16 / (int)sizeof(IO);
  static constexpr int LKP = DK + PE;
  static constexpr size_t RV = 2 * (size_t)C * (DVMAX_BWD + PE) * sizeof(IO) +
                               (TRB ? (size_t)DVMAX_BWD * LT * 2 : 0);
  static constexpr size_t RW =
      TRB ? 2 * (size_t)C * LKP * 2 + (size_t)DK * LT * 2
          : 2 * (size_t)C * LKP * sizeof(IO);
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t RR = mx(mx(RK, RV), mx(RW, CC));
  static constexpr size_t total = oR + RR;
};
template <typename IO, int DK, int C> struct BwdFits {
  static constexpr bool value = G2L<IO, DK, C>::total <= 160 * 1024 &&
                                BL<IO, DK, C>::total <= 160 * 1024 &&
                                G1L<IO, DK, C>::total <= 160 * 1024;
};

template <typename IO, typename GT, int DK, int C>
__global__ __launch_bounds__(BWD_THREADS) void kda_bwd_chunk_grad(
    BwdParams bp) {
  using L = G2L<IO, DK, C>;
  constexpr int NB = C / 16, NKT = DK / 16;
  constexpr int RG = L::RG, RP = C / RG;  // owner rows per thread
  constexpr int LCC = L::LCC;             // row stride of the C x C arrays
  static_assert(RG * DK == BWD_THREADS && RP * RG == C, "owner mapping");
  constexpr bool GB = sizeof(GT) == 2;
  const PrefillParams &p = bp.f;
  __shared__ __attribute__((aligned(16))) char sm[L::total];
  float *Mm = (float *)(sm + L::oM), *TTm = (float *)(sm + L::oT);  // M, T^T
  float *dPm = (float *)(sm + L::odP), *dMm = (float *)(sm + L::odM);
  int *vote = (int *)(sm + L::oVote);
  float *bet = (float *)(sm + L::oBeta), *dB = (float *)(sm + L::odB);
  float *dGl = (float *)(sm + L::odGl), *tail = (float *)(sm + L::oTail);
  float *dgh = (float *)(sm + L::odgh);
  char *R = sm + L::oR;
  float *Xm = (float *)R;  // phase 5 only

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15, g4 = lane >> 4;
  const int Dv = p.Dv, H = p.H, T = p.T, NC = p.NC, nvt = Dv / 16;
  const int bh = blockIdx.x / NC, n = blockIdx.x % NC;
  const int b = bh / H, h = bh % H, t0 = n * C;
  const float scale = p.scale;
  float *gs = bp.gs + ((size_t)bh * NC + n) * bwd_gs_floats(C, DK, Dv);
  float *gD = gs, *gQ = gs + (size_t)C * Dv, *gK = gQ + (size_t)C * DK;
  float *gW = gK + (size_t)C * DK, *gG = gW + (size_t)C * DK;
  float *gKd = gG + DK, *gdKd = gKd + (size_t)C * DK;
  const size_t krow = (size_t)H * DK, vrow = (size_t)H * Dv;
  const size_t kb = ((size_t)b * T * H + h) * DK;  // token 0 of (b, h), q/k/g
  const size_t vb = ((size_t)b * T * H + h) * Dv;  // token 0, v / dO / dv
  const size_t bb0 = (size_t)b * T * H + h;        // token 0, beta
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const int oi = tid % DK, orh = tid / DK;  // owner: channel, row group
  // a wave's output tiles (tl = wave, wave + 4, ...) in groups of four: the
  // four products first, then their epilogues, so the operand reads and
  // matrix-core steps of one tile overlap another's instead of every tile
  // waiting out its own chain
  auto tiles = [&](int ntile, auto prod, auto epi) {
    constexpr int NBAT = 4;
    for (int tb = wave; tb < ntile; tb += 4 * NBAT) {
      f32x4 acc[NBAT];
#pragma unroll
      for (int b = 0; b < NBAT; ++b) {
        const int tl = tb + 4 * b;
        acc[b] = tl < ntile ? prod(tl) : zero;
      }
#pragma unroll
      for (int b = 0; b < NBAT; ++b) {
        const int tl = tb + 4 * b;
        if (tl < ntile) epi(tl, acc[b]);
      }
    }
  };

  auto gate_at = [&](int t, int i) -> float {
    const size_t gi = p.gate_head ? bb0 + (size_t)t * H
                                  : kb + (size_t)t * krow + i;
    return GB ? (float)((const bf16 *)p.g)[gi] : ((const float *)p.g)[gi];
  };
  // e for rows beyond the sequence is 1 (as in the forward)
  // k, q and e = exp(g) of the chunk as [C][DK] rows, 8 channels per lane
  auto load_ke = [&](IO *ks, IO *qs, float *es) {
    constexpr int N8 = (C * DK / 8 + BWD_THREADS - 1) / BWD_THREADS;
    Row8<IO> lk[N8], lq[N8];
    Row8<GT> lg[N8];
#pragma unroll
    for (int j = 0; j < N8; ++j) {
      const int x = min(8 * (tid + BWD_THREADS * j), C * DK - 8);
      const int r = x / DK, i = x % DK, t = min(t0 + r, T - 1);
      lk[j].load((const IO *)p.k + kb + (size_t)t * krow + i);
      if (qs) lq[j].load((const IO *)p.q + kb + (size_t)t * krow + i);
      if (p.gate_head) {
        // one gate per token: element 0 carries it
        lg[j].zero();
        ((GT *)lg[j].q)[0] = ((const GT *)p.g)[bb0 + (size_t)t * H];
      } else {
        lg[j].load((const GT *)p.g + kb + (size_t)t * krow + i);
      }
    }
#pragma unroll
    for (int j = 0; j < N8; ++j) {
      const int x = 8 * (tid + BWD_THREADS * j);
      if (x < C * DK) {
        const bool ok = t0 + x / DK < T;
        if (!ok) {
          lk[j].zero();
          lq[j].zero();
        }
        lk[j].store(ks + x);
        if (qs) lq[j].store(qs + x);
        float ev[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          ev[e] = ok ? __expf(lg[j].get(p.gate_head ? 0 : e)) : 1.f;
        put8(es + x, ev);
      }
    }
  };

  // ---- phase 1: beta, accumulators, M and T from the forward, Kd -----------
  static_assert(C <= 64, "one wave holds the chunk's betas");
  if (tid < 64) {
    const int x = tid, t = t0 + x;
    float bv = 0.f;
    if (x < C) {
      bv = t < T ? (GB ? (float)((const bf16 *)p.beta)[bb0 + (size_t)t * H]
                       : ((const float *)p.beta)[bb0 + (size_t)t * H])
                 : 0.f;
      bet[x] = bv;
      dB[x] = 0.f;
      dgh[x] = 0.f;
    }
    // any row inside the sequence with beta = 0 (its M is rebuilt below)
    const unsigned long long bz = __ballot(x < C && t < T && bv == 0.f);
    if (x == 0) vote[1] = bz != 0ull;
  }
  for (int x = tid; x < DK; x += BWD_THREADS) dGl[x] = 0.f;
  IO *ks = (IO *)R;
  float *es = (float *)(R + (size_t)C * DK * sizeof(IO));
  load_ke(ks, nullptr, es);
  __syncthreads();
  {
    // A = diag(beta) M and T^T as the forward's chunk prep left them (only
    // the lower triangles are meaningful)
    const float *at = p.train_at + ((size_t)bh * NC + n) * 2 * C * C;
    constexpr int N4 = (C * C / 4 + BWD_THREADS - 1) / BWD_THREADS;
    // Kd = K*Gam needs each owner thread's prefix product of e over the rows
    // before its own: every thread multiplies its own RP rows here, and the
    // products of the earlier row groups are read back after a barrier
    {
      float lp = 1.f;
#pragma unroll
      for (int j = 0; j < RP; ++j) lp *= es[(orh * RP + j) * DK + oi];
      tail[orh * DK + oi] = lp;
    }
    f32x4 la[N4], lt[N4];
#pragma unroll
    for (int j = 0; j < N4; ++j) {
      const int x = min(4 * (tid + BWD_THREADS * j), C * C - 4);
      la[j] = *(const f32x4 *)(at + x);
      lt[j] = *(const f32x4 *)(at + C * C + x);
    }
#pragma unroll
    for (int j = 0; j < N4; ++j) {
      const int x4 = 4 * (tid + BWD_THREADS * j);
      if (x4 < C * C) {
        // four consecutive columns of one row (C is a multiple of 4)
        const int r = x4 / C, c0 = x4 % C;
        const float br = bet[r];
        const float ib = br != 0.f ? 1.f / br : 0.f;
        f32x4 mv, tv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = c0 + e;
          mv[e] = c < r ? la[j][e] * ib : 0.f;
          tv[e] = r <= c ? lt[j][e] : 0.f;  // T^T: upper triangle
        }
        *(f32x4 *)(Mm + r * LCC + c0) = mv;
        *(f32x4 *)(TTm + r * LCC + c0) = tv;
      }
    }
    // rows with beta = 0 (A carries no M there): M directly, with running
    // products of e over (s, r] -- exact, and rare
    for (int r = 1; r < C && vote[1]; ++r) {
      if (bet[r] != 0.f || t0 + r >= T) continue;
      for (int s2 = tid; s2 < r; s2 += BWD_THREADS) {
        float m = 0.f;
        for (int i = 0; i < DK; ++i) {
          float D = 1.f;
          for (int u = s2 + 1; u <= r; ++u) D *= es[u * DK + i];
          m += to_f32(ks[r * DK + i]) * to_f32(ks[s2 * DK + i]) * D;
        }
        Mm[r * LCC + s2] = m;
      }
    }
  }
  __syncthreads();
  {
    // Kd = K*Gam for the later phases (owner threads: prefix products)
    float G = 1.f;
#pragma unroll
    for (int rg = 0; rg < RG - 1; ++rg)
      if (rg < orh) G *= tail[rg * DK + oi];
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const int r = orh * RP + j;
      G *= es[r * DK + oi];
      gKd[(size_t)r * DK + oi] = to_f32(ks[r * DK + oi]) * G;
    }
  }
  __syncthreads();

  // ---- phase 3: value side: dT = dDelta (beta V)^T, dv = beta T^T dDelta --
  {
    const int LV = Dv + L::PE;  // padded row stride of dDs and vS
    IO *dDs = (IO *)R, *vS = dDs + C * LV;
    IO *dDT = vS + C * LV;  // bf16 only: dDelta^T [Dv][LT]
    constexpr int N8 = (C * DVMAX_BWD / 8 + BWD_THREADS - 1) / BWD_THREADS;
    Row8<IO> lv[N8];
#pragma unroll
    for (int jj = 0; jj < N8; ++jj) {
      const int x = min(8 * (tid + BWD_THREADS * jj), C * Dv - 8);
      const int r = x / Dv, j = x % Dv, t = min(t0 + r, T - 1);
      lv[jj].load((const IO *)p.v + vb + (size_t)t * vrow + j);
    }
    if constexpr (L::TRB) {
      // dDelta by columns: thread = (column j, 8 consecutive rows), so it
      // writes the rows of dDelta element by element and the row of
      // dDelta^T as one 16-byte store; lanes take consecutive columns
      float dd[N8][8];
#pragma unroll
      for (int jj = 0; jj < N8; ++jj) {
        const int q = min(tid + BWD_THREADS * jj, C * Dv / 8 - 1);
        const int j = q % Dv, r0 = 8 * (q / Dv);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dd[jj][e] = to_f32(
              ((const IO *)bp.dD)[vb + (size_t)min(t0 + r0 + e, T - 1) * vrow + j]);
      }
#pragma unroll
      for (int jj = 0; jj < N8; ++jj) {
        const int q = tid + BWD_THREADS * jj;
        if (q < C * Dv / 8) {
          const int j = q % Dv, r0 = 8 * (q / Dv);
          float d8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            d8[e] = t0 + r0 + e < T ? dd[jj][e] : 0.f;
            dDs[(r0 + e) * LV + j] = (IO)d8[e];
          }
          put8(dDT + j * L::LT + r0, d8);
        }
      }
    } else {
      Row8<IO> ld[N8];
#pragma unroll
      for (int jj = 0; jj < N8; ++jj) {
        const int x = min(8 * (tid + BWD_THREADS * jj), C * Dv - 8);
        const int r = x / Dv, j = x % Dv, t = min(t0 + r, T - 1);
        ld[jj].load((const IO *)bp.dD + vb + (size_t)t * vrow + j);
      }
#pragma unroll
      for (int jj = 0; jj < N8; ++jj) {
        const int x = 8 * (tid + BWD_THREADS * jj);
        if (x < C * Dv) {
          float d8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            d8[e] = t0 + x / Dv < T ? ld[jj].get(e) : 0.f;
          put8(dDs + (x / Dv) * LV + x % Dv, d8);
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < N8; ++jj) {
      const int x = 8 * (tid + BWD_THREADS * jj);
      if (x < C * Dv) {
        if (t0 + x / Dv >= T) lv[jj].zero();
        lv[jj].store(vS + (x / Dv) * LV + x % Dv);
      }
    }
    __syncthreads();
    tiles(
        NB * NB,
        [&](int tl) {
          return tile_mma_rows<IO>(zero, dDs, LV, vS, LV, 16 * (tl % NB),
                                   16 * (tl / NB), Dv, lane);
        },
        [&](int tl, f32x4 acc) {
          const int rt = tl % NB, st = tl / NB;
          const float bs = bet[16 * st + m16];  // (beta V)^T: beta of column s
#pragma unroll
          for (int e = 0; e < 4; ++e)  // dT
            dMm[(16 * rt + 4 * g4 + e) * LCC + 16 * st + m16] = bs * acc[e];
        });
    tiles(
        NB * nvt,
        [&](int tl) {
          const int rt = tl % NB, ct = tl / NB;
          if constexpr (L::TRB)
            return tile_mma_f32a<IO>(zero, TTm, LCC, dDT, L::LT, 16 * rt,
                                     16 * ct, C, lane);
          else
            return tile_mma<IO, false, false>(zero, TTm, LCC, dDs, LV, 16 * rt,
                                              16 * ct, C, lane);
        },
        [&](int tl, f32x4 acc) {
          const int rt = tl % NB, ct = tl / NB;
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * g4 + e, j = 16 * ct + m16, t = t0 + r;
            if (t < T)
              ((IO *)bp.dv)[vb + (size_t)t * vrow + j] =
                  from_f32<IO>(bet[r] * acc[e]);
            x[e] = to_f32(vS[r * LV + j]) * acc[e];
          }
          add_rows(dB, 16 * rt + 4 * g4, x, m16);
        });
    __syncthreads();
  }

  // ---- phase 4: key side: dT += dW (beta Kd)^T, dKd = beta T^T dW ---------
  {
    constexpr int LKP = L::LKP;  // padded row stride of dWs and KdS
    IO *dWs = (IO *)R, *KdS = dWs + C * LKP;
    IO *dWT = KdS + C * LKP;  // bf16 only: dW^T [DK][LT]
    constexpr int N8 = (C * DK / 8 + BWD_THREADS - 1) / BWD_THREADS;
    Row8<float> lk[N8];
#pragma unroll
    for (int j = 0; j < N8; ++j) {
      const int x = min(8 * (tid + BWD_THREADS * j), C * DK - 8);
      lk[j].load(gKd + x);
    }
    if constexpr (L::TRB) {
      // dW by columns, as dDelta in phase 3
      float dw[N8][8];
#pragma unroll
      for (int jj = 0; jj < N8; ++jj) {
        const int q = min(tid + BWD_THREADS * jj, C * DK / 8 - 1);
        const int i = q % DK, r0 = 8 * (q / DK);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          dw[jj][e] = to_f32(((const IO *)gW)[(r0 + e) * DK + i]);
      }
#pragma unroll
      for (int jj = 0; jj < N8; ++jj) {
        const int q = tid + BWD_THREADS * jj;
        if (q < C * DK / 8) {
          const int i = q % DK, r0 = 8 * (q / DK);
#pragma unroll
          for (int e = 0; e < 8; ++e) dWs[(r0 + e) * LKP + i] = (IO)dw[jj][e];
          put8(dWT + i * L::LT + r0, dw[jj]);
        }
      }
    } else {
      Row8<IO> lw[N8];
#pragma unroll
      for (int j = 0; j < N8; ++j) {
        const int x = min(8 * (tid + BWD_THREADS * j), C * DK - 8);
        lw[j].load((const IO *)gW + x);
      }
#pragma unroll
      for (int j = 0; j < N8; ++j) {
        const int x = 8 * (tid + BWD_THREADS * j);
        if (x < C * DK) {
          float w8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) w8[e] = lw[j].get(e);
          put8(dWs + (x / DK) * LKP + x % DK, w8);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < N8; ++j) {
      const int x = 8 * (tid + BWD_THREADS * j);
      if (x < C * DK) {
        float k8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) k8[e] = lk[j].get(e);
        put8(KdS + (x / DK) * LKP + x % DK, k8);
      }
    }
    __syncthreads();
    tiles(
        NB * NB,
        [&](int tl) {
          return tile_mma_rows<IO>(zero, dWs, LKP, KdS, LKP, 16 * (tl % NB),
                                   16 * (tl / NB), DK, lane);
        },
        [&](int tl, f32x4 acc) {
          const int rt = tl % NB, st = tl / NB;
          const float bs = bet[16 * st + m16];  // (beta Kd)^T: beta of column s
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dMm[(16 * rt + 4 * g4 + e) * LCC + 16 * st + m16] += bs * acc[e];
        });
    tiles(
        NB * NKT,
        [&](int tl) {
          const int rt = tl % NB, it = tl / NB;
          if constexpr (L::TRB)
            return tile_mma_f32a<IO>(zero, TTm, LCC, dWT, L::LT, 16 * rt,
                                     16 * it, C, lane);
          else
            return tile_mma<IO, false, false>(zero, TTm, LCC, dWs, LKP, 16 * rt,
                                              16 * it, C, lane);
        },
        [&](int tl, f32x4 acc) {
          const int rt = tl % NB, it = tl / NB;
          float x[4];
          f32x4 dk4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * g4 + e, i = 16 * it + m16;
            dk4[e] = bet[r] * acc[e];
            x[e] = to_f32(KdS[r * LKP + i]) * acc[e];
          }
          *(f32x4 *)(gdKd + bwd_tile_off(rt, it, NKT, lane)) = dk4;
          add_rows(dB, 16 * rt + 4 * g4, x, m16);
        });
    __syncthreads();
  }

  // ---- phase 5: dA = -T^T dT T^T (strictly lower); dM = beta dA ------------
  tiles(
      NB * NB,
      [&](int tl) {
        return tile_mma<float, false, false>(zero, dMm, LCC, TTm, LCC,
                                             16 * (tl % NB), 16 * (tl / NB), C,
                                             lane);
      },
      [&](int tl, f32x4 acc) {
        const int rt = tl % NB, st = tl / NB;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Xm[(16 * rt + 4 * g4 + e) * LCC + 16 * st + m16] = acc[e];
      });
  __syncthreads();
  tiles(
      NB * NB,
      [&](int tl) {
        return tile_mma<float, false, false>(zero, TTm, LCC, Xm, LCC,
                                             16 * (tl % NB), 16 * (tl / NB), C,
                                             lane);
      },
      [&](int tl, f32x4 acc) {
        const int rt = tl % NB, st = tl / NB;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g4 + e, s = 16 * st + m16;
          const float dA = s < r ? -acc[e] : 0.f;
          x[e] = dA * Mm[r * LCC + s];
          dMm[r * LCC + s] = bet[r] * dA;  // read only after the next barrier
        }
        add_rows(dB, 16 * rt + 4 * g4, x, m16);
      });
  __syncthreads();

  // ---- phase 6: dPm = scale tril(dO Delta^T) --------------------------------
  {
    const int LV = Dv + L::PE;  // padded row stride of Os and Ds
    IO *Os = (IO *)R, *Ds = Os + C * LV;
    constexpr int N8 = (C * DVMAX_BWD / 8 + BWD_THREADS - 1) / BWD_THREADS;
    Row8<IO> lo[N8];
    Row8<IO> ld[N8];
#pragma unroll
    for (int jj = 0; jj < N8; ++jj) {
      const int x = min(8 * (tid + BWD_THREADS * jj), C * Dv - 8);
      const int r = x / Dv, j = x % Dv, t = min(t0 + r, T - 1);
      lo[jj].load((const IO *)bp.dO + vb + (size_t)t * vrow + j);
      ld[jj].load((const IO *)gD + x);
    }
#pragma unroll
    for (int jj = 0; jj < N8; ++jj) {
      const int x = 8 * (tid + BWD_THREADS * jj);
      if (x < C * Dv) {
        if (t0 + x / Dv >= T) lo[jj].zero();
        lo[jj].store(Os + (x / Dv) * LV + x % Dv);
        float d8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) d8[e] = ld[jj].get(e);
        put8(Ds + (x / Dv) * LV + x % Dv, d8);
      }
    }
    __syncthreads();
    tiles(
        NB * NB,
        [&](int tl) {
          return tile_mma_rows<IO>(zero, Os, LV, Ds, LV, 16 * (tl % NB),
                                   16 * (tl / NB), Dv, lane);
        },
        [&](int tl, f32x4 acc) {
          const int rt = tl % NB, st = tl / NB;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * g4 + e, s = 16 * st + m16;
            dPm[r * LCC + s] = s <= r ? scale * acc[e] : 0.f;
          }
        });
    __syncthreads();
  }

  // ---- phase 7: elementwise terms, then the decayed products -------------
  IO *qs = ks + C * DK;
  es = (float *)(R + (size_t)2 * C * DK * sizeof(IO));  // e, later rho
  IO *sg = (IO *)(R + (size_t)2 * C * DK * sizeof(IO) + (size_t)C * DK * 4);
  load_ke(ks, qs, es);
  if (tid == 0) *vote = 0;
  __syncthreads();
  // per 16-token sub-chunk and channel: sigma (exclusive suffix product),
  // rho (inclusive prefix, over e in place) and the sub-chunk product F;
  // a vote records any rho below 2^-64 (diagonal ratios then unsafe)
  float *Fs = Mm, *Mid = TTm;  // [NB][DK], [pairs a-b >= 2][DK]
  for (int w = tid; w < NB * DK; w += BWD_THREADS) {
    const int a = w / DK, i = w % DK;
    float P = 1.f;
    for (int j = 15; j >= 0; --j) {
      const int r = 16 * a + j;
      sg[r * DK + i] = (IO)P;
      P *= es[r * DK + i];
    }
    P = 1.f;
    int bad = 0;
    for (int j = 0; j < 16; ++j) {
      const int r = 16 * a + j;
      P *= es[r * DK + i];
      es[r * DK + i] = P;
      if (!(P >= 5.42101086242752217e-20f)) bad = 1;
    }
    Fs[a * DK + i] = P;
    if (bad) *vote = 1;
  }
  __syncthreads();
  constexpr int NP2 = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 0;
  for (int w = tid; w < NP2 * DK; w += BWD_THREADS) {
    const int pi = w / DK, i = w % DK;
    int aa = 2, bb = pi;
    while (bb >= aa - 1) { bb -= aa - 1; ++aa; }
    float mp = 1.f;
    for (int d = bb + 1; d < aa; ++d) mp *= Fs[d * DK + i];
    Mid[pi * DK + i] = mp;
  }
  __syncthreads();
  // One wave per 16-channel tile; each lane owns, in the accumulator
  // layout, rows 16a + 4g + e of every sub-chunk a for channel 16 it + m16
  // and keeps dk, dq, dG of those (r, i) in registers.  D_rs = rho_r Mid_ba
  // sigma_s for s in sub-chunk b < a (r in a), rho_r / rho_s inside one.
  constexpr int JT = (NKT + 3) / 4;
  // dG of the lane's (r, i) stays in registers for the reverse sum after
  // the barrier; dk and dq are final at the end of a channel tile and go
  // out straight from registers
  f32x4 aG_[JT][NB];
  {
    using MM = Mma<IO>;
    typedef typename MM::frag frag;
    const bool dok = *vote == 0;
    const float *rho = es;
    auto mid = [&](int a, int b, int i) -> float {
      return a - b >= 2 ? Mid[((a - 2) * (a - 1) / 2 + b) * DK + i] : 1.f;
    };
    // exact diagonal-block sums with running products (vote fallback)
    auto diag_exact = [&](int r, int i, bool row, const IO *xv, const float *cm,
                          bool strict) -> float {
      const int lo = r & ~15, hi = lo + 15;
      float acc = 0.f, D = 1.f;
      if (row) {  // sum_{s<=r in the sub-chunk} c[r][s] x_s prod_{s<u<=r} e_u
        for (int s2 = r; s2 >= lo; --s2) {
          if (s2 < r) {
            const int tu = t0 + s2 + 1;
            D *= tu < T ? __expf(gate_at(tu, i)) : 1.f;
          }
          if (!(strict && s2 == r))
            acc += cm[r * LCC + s2] * to_f32(xv[s2 * DK + i]) * D;
        }
      } else {    // sum_{r2>=r in the sub-chunk} c[r2][r] x_r2 prod_{r<u<=r2} e_u
        for (int r2 = r; r2 <= hi; ++r2) {
          if (r2 > r) D *= t0 + r2 < T ? __expf(gate_at(t0 + r2, i)) : 1.f;
          if (!(strict && r2 == r))
            acc += cm[r2 * LCC + r] * to_f32(xv[r2 * DK + i]) * D;
        }
      }
      return acc;
    };
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) {
      const int it = wave + 4 * jt;
      if (it >= NKT) continue;
      const int ib = 16 * it + m16;  // B-operand / output column (channel)
      f32x4 aK_[NB], aQ_[NB];
      // ---- elementwise terms of Kd = K*Gam, Qtil, Ktil = K*gam/Gam, gam
      float Fb[NB];
#pragma unroll
      for (int a = 0; a < NB; ++a) Fb[a] = Fs[a * DK + ib];
      float kil = 0.f;
      // this lane's dKd, dQtil, dKtil of every sub-chunk: 16-byte loads
      // issued together, before any of them is used
      f32x4 vdkd[NB], vdq[NB], vdk[NB];
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const size_t ot = bwd_tile_off(a, it, NKT, lane);
        vdkd[a] = *(const f32x4 *)(gdKd + ot);
        vdq[a] = *(const f32x4 *)(gQ + ot);
        vdk[a] = *(const f32x4 *)(gK + ot);
      }
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        float pre = 1.f, post = 1.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < a) pre *= Fb[b];
          if (b > a) post *= Fb[b];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * a + 4 * g4 + e;
          const float G = rho[r * DK + ib] * pre;              // Gam_r
          const float sf = to_f32(sg[r * DK + ib]) * post;      // gam / Gam_r
          const float kr = to_f32(ks[r * DK + ib]), qr = to_f32(qs[r * DK + ib]);
          const float dkd = vdkd[a][e], dqd = vdq[a][e], dki = vdk[a][e];
          aK_[a][e] = dkd * G + dki * sf;
          aQ_[a][e] = scale * dqd * G;
          float dg = dkd * kr * G + dqd * scale * qr * G - dki * kr * sf;
          if (r == C - 1) dg += gG[ib] * G;  // dgam * gam (G = gam here)
          aG_[jt][a][e] = dg;
          kil += dki * kr * sf;
        }
      }
      atomicAdd(&dGl[ib], kil);
      // the 4 tokens 16 b + 4 g4 + e of every sub-chunk b at this lane's
      // channel ib, as the products' per-token factors need them
      float kx[NB][4], xr[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sb = 16 * b + 4 * g4 + e;
          kx[b][e] = to_f32(ks[sb * DK + ib]);
          xr[b][e] = rho[sb * DK + ib];
        }
      // ---- row role: rowK, rowQ of sub-chunk a
      {
        // column operand values: k sigma (times mid) off the diagonal,
        // k / rho on it
        float ksg[NB][4], kir[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int sb = 16 * b + 4 * g4 + e;
            ksg[b][e] = kx[b][e] * to_f32(sg[sb * DK + ib]);
            kir[b][e] = kx[b][e] * __builtin_amdgcn_rcpf(xr[b][e]);
          }
#pragma unroll
        for (int a = 0; a < NB; ++a) {
          f32x4 zk = zero, zq = zero;
#pragma unroll
          for (int b = 0; b <= a; ++b) {
            if (b == a && !dok) continue;
            // lane (g4, m16): row 16a + m16, k = 16 b + 4 g4 + e (e < 4)
            const f32x4 mk = *(const f32x4 *)(dMm + (16 * a + m16) * LCC + 16 * b +
                                              4 * g4);
            const f32x4 mq = *(const f32x4 *)(dPm + (16 * a + m16) * LCC + 16 * b +
                                              4 * g4);
            const float md = mid(a, b, ib);
            frag fk, fq, fb;
#pragma unroll
            for (int e = 0; e < MM::NE; ++e) {
              const bool lo = e < 4;
              MM::set(fk, e, lo ? mk[e & 3] : 0.f);
              MM::set(fq, e, lo ? mq[e & 3] : 0.f);
              MM::set(fb, e, lo ? (b < a ? ksg[b][e & 3] * md : kir[b][e & 3])
                                : 0.f);
            }
            zk = MM::mma(fk, fb, zk);
            zq = MM::mma(fq, fb, zq);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * a + 4 * g4 + e;
            const float rr = xr[a][e];
            float rK = rr * zk[e], rQ = rr * zq[e];
            if (!dok) {
              rK += diag_exact(r, ib, true, ks, dMm, true);
              rQ += diag_exact(r, ib, true, ks, dPm, false);
            }
            aK_[a][e] += rK;
            aQ_[a][e] += rQ;
            aG_[jt][a][e] += kx[a][e] * rK + to_f32(qs[r * DK + ib]) * rQ;
          }
        }
      }
      // ---- column role: colK, colQ of sub-chunk b
      {
        // row-side values k rho and q rho of the 4 tokens of every sub-chunk
        float kr4[NB][4], qr4[NB][4];
#pragma unroll
        for (int a = 0; a < NB; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ra = 16 * a + 4 * g4 + e;
            kr4[a][e] = kx[a][e] * xr[a][e];
            qr4[a][e] = to_f32(qs[ra * DK + ib]) * xr[a][e];
          }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4 ok_ = zero, oq = zero, dk2 = zero, dq2 = zero;
#pragma unroll
          for (int a = b; a < NB; ++a) {
            if (a == b && !dok) continue;
            const float md = a > b ? mid(a, b, ib) : 1.f;
            frag fk, fq, bk, bq;
#pragma unroll
            for (int e = 0; e < MM::NE; ++e) {
              const bool lo = e < 4;
              // dM^T: row 16 b + m16, k = 16 a + 4 g4 + e
              const int ra = 16 * a + 4 * g4 + (e & 3), sb = 16 * b + m16;
              MM::set(fk, e, lo ? dMm[ra * LCC + sb] : 0.f);
              MM::set(fq, e, lo ? dPm[ra * LCC + sb] : 0.f);
              MM::set(bk, e, lo ? kr4[a][e & 3] * md : 0.f);
              MM::set(bq, e, lo ? qr4[a][e & 3] * md : 0.f);
            }
            if (a > b) {
              ok_ = MM::mma(fk, bk, ok_);
              oq = MM::mma(fq, bq, oq);
            } else {
              dk2 = MM::mma(fk, bk, dk2);
              dq2 = MM::mma(fq, bq, dq2);
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s2 = 16 * b + 4 * g4 + e;
            const float sgv = to_f32(sg[s2 * DK + ib]);
            float cK = sgv * ok_[e], cQ = sgv * oq[e];
            if (dok) {
              const float ir = __builtin_amdgcn_rcpf(xr[b][e]);
              cK += dk2[e] * ir;
              cQ += dq2[e] * ir;
            } else {
              cK += diag_exact(s2, ib, false, ks, dMm, true);
              cQ += diag_exact(s2, ib, false, qs, dPm, false);
            }
            aK_[b][e] += cK + cQ;
            aG_[jt][b][e] -= kx[b][e] * (cK + cQ);
          }
        }
      }
      // dq and dk of rows 16 a + 4 g4 + e at channel ib (16 lanes write 16
      // consecutive channels of a row)
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * a + 4 * g4 + e;
          if (t0 + r < T) {
            const size_t o = kb + (size_t)(t0 + r) * krow + ib;
            ((IO *)bp.dq)[o] = from_f32<IO>(aQ_[a][e]);
            ((IO *)bp.dk)[o] = from_f32<IO>(aK_[a][e]);
          }
        }
    }
  }
  __syncthreads();  // dGl complete; rho no longer read
  // ---- phase 8: dg = reverse cumulative sum of dG ---------------------------
  float *dGs = es;  // [C][DK] fp32, in place of rho
#pragma unroll
  for (int jt = 0; jt < JT; ++jt) {
    const int it = wave + 4 * jt;
    if (it >= NKT) continue;
    const int ib = 16 * it + m16;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * a + 4 * g4 + e, t = t0 + r;
        float dgv = aG_[jt][a][e];
        if (r == C - 1) dgv += dGl[ib];  // sum_r dKtil*Ktil (d log gam)
        dGs[r * DK + ib] = dgv;
        (void)t;
      }
  }
  __syncthreads();
  constexpr int NO8 = (C * DK / 8 + BWD_THREADS - 1) / BWD_THREADS;
  {
    const int i = oi, R0 = orh * RP;
    float own = 0.f;
    for (int j = 0; j < RP; ++j) own += dGs[(R0 + j) * DK + i];
    tail[orh * DK + i] = own;
    __syncthreads();
    float acc = 0.f;
    for (int rr = orh + 1; rr < RG; ++rr) acc += tail[rr * DK + i];
    for (int j = RP - 1; j >= 0; --j) {
      const int r = R0 + j, t = t0 + r;
      acc += dGs[r * DK + i];
      dGs[r * DK + i] = acc;  // this thread's own (r, i): read just above
      if (t < T && p.gate_head) atomicAdd(&dgh[r], acc);
    }
    __syncthreads();
    if (!p.gate_head) {
      // rows of dg out, 8 channels per lane
#pragma unroll
      for (int j = 0; j < NO8; ++j) {
        const int x = 8 * (tid + BWD_THREADS * j), r = x / DK, ii = x % DK;
        if (x < C * DK && t0 + r < T) {
          float v8[8];
          *(f32x4 *)v8 = *(const f32x4 *)(dGs + x);
          *(f32x4 *)(v8 + 4) = *(const f32x4 *)(dGs + x + 4);
          GT *dst = (GT *)bp.dg + kb + (size_t)(t0 + r) * krow + ii;
          if constexpr (sizeof(GT) == 2) {
            bf16x8 h8;
#pragma unroll
            for (int e = 0; e < 8; ++e) h8[e] = (bf16)v8[e];
            *(bf16x8 *)dst = h8;
          } else {
            *(f32x4 *)dst = *(const f32x4 *)v8;
            *(f32x4 *)(dst + 4) = *(const f32x4 *)(v8 + 4);
          }
        }
      }
    }
    for (int r = tid; r < C; r += BWD_THREADS) {
      const int t = t0 + r;
      if (t < T) {
        ((GT *)bp.dbeta)[bb0 + (size_t)t * H] = (GT)dB[r];
        if (p.gate_head) ((GT *)bp.dg)[bb0 + (size_t)t * H] = (GT)dgh[r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename IO, typename GT, int DK, int C>
static hipError_t bwd_one(const BwdParams &bp, hipStream_t s) {
  if constexpr (!BwdFits<IO, DK, C>::value) {
    return hipErrorInvalidValue;
  } else {
    const PrefillParams &p = bp.f;
    const unsigned heads = (unsigned)(p.B * p.H);
    hipLaunchKernelGGL((kda_bwd_state<IO, DK, C>), dim3(heads * (p.Dv / 16)),
                       dim3(BWD_STATE_THREADS), 0, s, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kda_bwd_chunk_state<IO, DK, C>), dim3(heads * p.NC),
                       dim3(BWD_THREADS), 0, s, bp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kda_bwd_chunk_grad<IO, GT, DK, C>), dim3(heads * p.NC),
                       dim3(BWD_THREADS), 0, s, bp);
    return hipGetLastError();
  }
}

template <typename IO, typename GT>
static hipError_t bwd_dk(const BwdParams &bp, hipStream_t s) {
  switch (bp.f.Dk * 1000 + bp.f.C) {
    case 16016: return bwd_one<IO, GT, 16, 16>(bp, s);
    case 16032: return bwd_one<IO, GT, 16, 32>(bp, s);
    case 16064: return bwd_one<IO, GT, 16, 64>(bp, s);
    case 32016: return bwd_one<IO, GT, 32, 16>(bp, s);
    case 32032: return bwd_one<IO, GT, 32, 32>(bp, s);
    case 32064: return bwd_one<IO, GT, 32, 64>(bp, s);
    case 64016: return bwd_one<IO, GT, 64, 16>(bp, s);
    case 64032: return bwd_one<IO, GT, 64, 32>(bp, s);
    case 64064: return bwd_one<IO, GT, 64, 64>(bp, s);
    case 128016: return bwd_one<IO, GT, 128, 16>(bp, s);
    case 128032: return bwd_one<IO, GT, 128, 32>(bp, s);
    case 128064: return bwd_one<IO, GT, 128, 64>(bp, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_backward(const BwdParams &bp, int io_bf16, hipStream_t s) {
  if (!io_bf16) return bwd_dk<float, float>(bp, s);
  return bp.f.gate_bf16 ? bwd_dk<bf16, bf16>(bp, s) : bwd_dk<bf16, float>(bp, s);
}

template <typename IO>
static bool fits_io(int Dk, int C) {
  switch (Dk * 1000 + C) {
#define KDA_FIT(D, CC) \
  case D * 1000 + CC: return BwdFits<IO, D, CC>::value;
    KDA_FIT(16, 16) KDA_FIT(16, 32) KDA_FIT(16, 64)
    KDA_FIT(32, 16) KDA_FIT(32, 32) KDA_FIT(32, 64)
    KDA_FIT(64, 16) KDA_FIT(64, 32) KDA_FIT(64, 64)
    KDA_FIT(128, 16) KDA_FIT(128, 32) KDA_FIT(128, 64)
#undef KDA_FIT
  }
  return false;
}

bool backward_fits(int io_bf16, int Dk, int C) {
  return io_bf16 ? fits_io<bf16>(Dk, C) : fits_io<float>(Dk, C);
}

size_t backward_chunk_floats(int C, int Dk, int Dv) {
  return bwd_gs_floats(C, Dk, Dv);
}

}  // namespace kda
