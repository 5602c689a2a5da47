// kda_state.hip -- sequential state pass of the chunked KDA prefill.
//
// Given the chunk-local factors that kda_chunk_prep leaves in the workspace
// (per (batch*head, chunk): -W, Qtil = scale Q*Gam, Ktil^T, P, Gam_C, U; see
// kda_prep_impl.h for their definitions), each chunk n updates
//   Delta = U - W S,   O = Qtil S + P Delta,   S <- diag(Gam_C) S + Ktil^T Delta
// in order, which is the chunked form of the per-token KDA rule (state rows
// are key channels; see include/kda.h for the sources).
//
// Work split.  A workgroup owns one (batch*head) and NS consecutive
// 16-column value slabs, with three wave roles:
//   * four state waves: state wave w computes the Delta rows of token tile w
//     (16 tokens) from its rows of -W and U, and owns the state rows of key
//     unit w (32 keys in bf16, 16 in fp32; units w, w+4, ... when there are
//     more than four), which it updates from its rows of Ktil^T;
//   * four output waves: output wave w computes the O rows of token tile w
//     from its rows of Qtil and P;
//   * one warm-up wave that pulls the blocks of later chunks into L2.
// Every product is split by its output rows, so each wave reads only its
// own share of the chunk's factors.  The products need the whole S (for
// Delta and O) and the whole Delta (for S and O) as the second operand, so
// both are exchanged through LDS in the matrix-core operand layout: two
// barriers per chunk.  O is produced transposed (O^T = S^T Qtil^T +
// Delta^T P^T) so that each lane ends up with four consecutive value
// columns of one token: one vector store per slab.
//
// Each wave fetches its factors straight from global memory into registers
// one chunk ahead (two rotating register sets), the loads interleaved with
// the current chunk's products; only the exchange round trips and the short
// MFMA chains sit on the sequential path.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename IO> struct Vec4T;
template <> struct Vec4T<bf16> {
  typedef uint2 raw;
  __device__ static __forceinline__ f32x4 get(raw r) {
    return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                 __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
  }
  __device__ static __forceinline__ raw put(f32x4 f) {
    bf16x4 v = {(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3]};
    return __builtin_bit_cast(raw, v);
  }
};
template <> struct Vec4T<float> {
  typedef uint4 raw;
  __device__ static __forceinline__ f32x4 get(raw r) {
    return f32x4{__uint_as_float(r.x), __uint_as_float(r.y),
                 __uint_as_float(r.z), __uint_as_float(r.w)};
  }
  __device__ static __forceinline__ raw put(f32x4 f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

// LDS writes done, then the workgroup barrier; outstanding global loads stay
// in flight across it
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave roles of a workgroup: SW state waves (Delta and the state update),
// OW output waves (O), and with STATE_WARM one L2 warm-up wave.
constexpr int SW = 4, OW = 4;
constexpr bool STATE_WARM = true;
constexpr int STATE_PF = 4;  // chunks between warming and use
constexpr int STATE_THREADS = 64 * (SW + OW + (STATE_WARM ? 1 : 0));

template <typename IO, int DK, int C, int NS> struct SP {
  static constexpr int TPU = Mma<IO>::TPU;
  static constexpr int NB = C / 16, NKT = DK / 16;
  static constexpr int NKU = (NKT + TPU - 1) / TPU;  // key units
  static constexpr int NTU = (NB + TPU - 1) / TPU;   // token units
  static constexpr int KUW = (NKU + SW - 1) / SW;    // key units per wave
  static constexpr size_t oSU = 0;                          // [NS][NKU]
  static constexpr size_t oDU = (size_t)NS * NKU * 1024;    // [NS][NTU]
  static constexpr size_t LDS = oDU + (size_t)NS * NTU * 1024;
};

// a state wave's factors of one chunk: its rows of -W and U, and of Ktil^T
// with gamma_C for its key units.  gamma_C comes as one value per lane (lane
// l: entry 16 ((l >> 4) % TPU) + (l & 15) of the unit's 16 TPU entries) and
// is spread to the lanes' state rows by gamma_rows: a wave moves 256 bytes
// for it instead of 16 bytes per lane and key tile
template <typename IO, int DK, int C, int NS> struct SFrag {
  using G = SP<IO, DK, C, NS>;
  typedef typename Mma<IO>::frag frag;
  frag w[G::NKU];
  typename Vec4T<IO>::raw u[NS];
  frag k[G::KUW][G::TPU][G::NTU];
  float gr[G::KUW];
};

// gamma_C of the 4 state rows a lane holds in key tile TPU u + hh (rows
// 16 (TPU u + hh) + 4 g4 + e), read from the lanes that loaded them
__device__ __forceinline__ f32x4 gamma_rows(float gr, int hh, int g4) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = __int_as_float(__builtin_amdgcn_ds_bpermute(
        4 * (16 * hh + 4 * g4 + e), __float_as_int(gr)));
  return r;
}
// an output wave's factors of one chunk: its rows of Qtil and P
template <typename IO, int DK, int C, int NS> struct OFrag {
  using G = SP<IO, DK, C, NS>;
  typedef typename Mma<IO>::frag frag;
  frag q[G::NKU], p[G::NTU];
};

// half 0 of a state wave's factors (-W, U: needed before the Delta
// exchange) or half 1 (Ktil^T, gamma_C)
template <int HALF, typename IO, int DK, int C, int NS>
__device__ __forceinline__ void load_state(SFrag<IO, DK, C, NS> &f,
                                           const char *blk, const WsLayout &W,
                                           int rtc, int w4, int lane, int g4,
                                           int vt0) {
  using G = SP<IO, DK, C, NS>;
  typedef typename Mma<IO>::frag frag;
  typedef typename Vec4T<IO>::raw URaw;
  if (HALF == 0) {
    const frag *Lw = (const frag *)(blk + W.off_negw) + lane;
    const URaw *Lu = (const URaw *)(blk + W.off_u) + lane;
#pragma unroll
    for (int u = 0; u < G::NKU; ++u) f.w[u] = Lw[(rtc * G::NKU + u) * 64];
#pragma unroll
    for (int s = 0; s < NS; ++s) f.u[s] = Lu[((vt0 + s) * G::NB + rtc) * 64];
  } else {
    const frag *Lk = (const frag *)(blk + W.off_ktt) + lane;
    const float *Lg = (const float *)(blk + W.off_gam) + (lane & 15);
#pragma unroll
    for (int j = 0; j < G::KUW; ++j) {
      // gamma_C first: it is needed one phase before the Ktil^T units
      const int tg = min(G::TPU * (w4 + SW * j) + (lane >> 4) % G::TPU,
                         G::NKT - 1);
      f.gr[j] = Lg[16 * tg];
#pragma unroll
      for (int h = 0; h < G::TPU; ++h) {
        // key tile of (unit w4 + SW j, half h), clamped to a valid one
        const int t = min(G::TPU * (w4 + SW * j) + h, G::NKT - 1);
#pragma unroll
        for (int u = 0; u < G::NTU; ++u)
          f.k[j][h][u] = Lk[(t * G::NTU + u) * 64];
      }
    }
  }
}

// half 0 of an output wave's factors (Qtil) or half 1 (P)
template <int HALF, typename IO, int DK, int C, int NS>
__device__ __forceinline__ void load_out(OFrag<IO, DK, C, NS> &f,
                                         const char *blk, const WsLayout &W,
                                         int rtc, int lane) {
  using G = SP<IO, DK, C, NS>;
  typedef typename Mma<IO>::frag frag;
  if (HALF == 0) {
    const frag *Lq = (const frag *)(blk + W.off_qt) + lane;
#pragma unroll
    for (int u = 0; u < G::NKU; ++u) f.q[u] = Lq[(rtc * G::NKU + u) * 64];
  } else {
    // P units above the diagonal are never written by the prep: they are
    // neither loaded nor multiplied (the test is uniform over the wave)
    const frag *Lp = (const frag *)(blk + W.off_p) + lane;
#pragma unroll
    for (int u = 0; u < G::NTU; ++u)
      if (G::NTU == 1 || u <= rtc / G::TPU) f.p[u] = Lp[(rtc * G::NTU + u) * 64];
  }
}

// interleave the next chunk's NL loads with this phase's NM products
template <int NR, int NM, int NL>
__device__ __forceinline__ void interleave_loads() {
  if (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if (NL > NM) __builtin_amdgcn_sched_group_barrier(0x020, NL - NM, 0);
}

template <typename IO, int DK, int C, int NS>
__global__ __launch_bounds__(STATE_THREADS, 1) void kda_state_pass(
    PrefillParams p) {
  using M = Mma<IO>;
  using G = SP<IO, DK, C, NS>;
  using V4 = Vec4T<IO>;
  using SF = SFrag<IO, DK, C, NS>;
  using OF = OFrag<IO, DK, C, NS>;
  typedef typename M::frag frag;
  constexpr int NB = G::NB, NKT = G::NKT, TPU = G::TPU, NKU = G::NKU,
                NTU = G::NTU, KUW = G::KUW;
  __shared__ __attribute__((aligned(1024))) char sm[G::LDS];
  frag *SU = (frag *)(sm + G::oSU);  // S as second operand, [NS][NKU] units
  frag *DU = (frag *)(sm + G::oDU);  // Delta as second operand, [NS][NTU]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // role: uniform
  const int m16 = lane & 15, g4 = lane >> 4;
  const int Dv = p.Dv, H = p.H, T = p.T, BH = p.B * p.H, NC = p.NC;
  const int ng = Dv / (16 * NS);  // workgroups per head
  int bh, grp;
  {
    // keep the workgroups of one head on one XCD (blocks go round-robin over
    // the 8 XCDs), so they share the head's factors through one L2
    const int b = blockIdx.x;
    if (ng > 1 && (BH & 7) == 0) {
      const int x = b & 7, jj = b >> 3;
      bh = (jj / ng) * 8 + x;
      grp = jj % ng;
    } else {
      bh = b / ng;
      grp = b % ng;
    }
  }
  const int bb = bh / H, h = bh % H;
  const int vt0 = grp * NS;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const char *ws0 = p.ws + (size_t)bh * NC * p.wsb;
  const int w4 = wave % 4;                     // index within the role
  const bool rv = (NB >= 4) || w4 < NB;        // owns a token tile
  const int rtc = min(w4, NB - 1);             // (clamped) token tile

  // the upper half of the last token unit stays zero when NB is odd
  for (int i = tid; i < NS * NTU * 256; i += STATE_THREADS)
    ((float *)DU)[i] = 0.f;

  if (wave < SW) {
    // ================= state waves: Delta and the state update ==========
    bool kv[KUW];
#pragma unroll
    for (int j = 0; j < KUW; ++j)
      kv[j] = (NKU % SW == 0) || w4 + SW * j < NKU;
    // state rows owned by this wave: key tiles TPU*u + hh of its units
    f32x4 S[KUW][TPU][NS];
#pragma unroll
    for (int j = 0; j < KUW; ++j)
#pragma unroll
      for (int hh = 0; hh < TPU; ++hh)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          S[j][hh][s] = zero;
          const int t = TPU * (w4 + SW * j) + hh;
          if (p.s0 && kv[j] && t < NKT) {
            const float *s0 = p.s0 + ((size_t)bh * DK + 16 * t + 4 * g4) * Dv +
                              16 * (vt0 + s) + m16;
#pragma unroll
            for (int e = 0; e < 4; ++e) S[j][hh][s][e] = s0[(size_t)e * Dv];
          }
        }
    auto publish_s = [&]() {
#pragma unroll
      for (int j = 0; j < KUW; ++j)
        if (kv[j]) {
          const int u = w4 + SW * j;
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const bool hi = TPU == 2 && TPU * u + 1 < NKT;
            SU[(s * NKU + u) * 64 + lane] =
                M::pack(S[j][0][s], hi ? S[j][TPU - 1][s] : zero);
          }
        }
    };
    publish_s();
    lds_barrier();

    // the state at the start of chunk n, for the backward pass
    auto save_state = [&](int n) {
#pragma unroll
      for (int j = 0; j < KUW; ++j)
#pragma unroll
        for (int hh = 0; hh < TPU; ++hh) {
          const int t = TPU * (w4 + SW * j) + hh;
          if (kv[j] && t < NKT) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              float *so = p.ckpt +
                          (((size_t)bh * NC + n) * DK + 16 * t + 4 * g4) * Dv +
                          16 * (vt0 + s) + m16;
#pragma unroll
              for (int e = 0; e < 4; ++e) so[(size_t)e * Dv] = S[j][hh][s][e];
            }
          }
        }
    };
    auto sstep = [&](int n, const SF &f, SF &nx) {
      if (p.ckpt) save_state(n);
      const char *nblk = ws0 + (size_t)min(n + 1, NC - 1) * p.wsb;
      load_state<0, IO, DK, C, NS>(nx, nblk, W, rtc, w4, lane, g4, vt0);
      frag sb[NS][NKU];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int u = 0; u < NKU; ++u) sb[s][u] = SU[(s * NKU + u) * 64 + lane];
      f32x4 gm[KUW][TPU];
#pragma unroll
      for (int j = 0; j < KUW; ++j)
#pragma unroll
        for (int hh = 0; hh < TPU; ++hh) gm[j][hh] = gamma_rows(f.gr[j], hh, g4);
      // Delta rows of token tile rtc: U - W S  (-W is stored)
      f32x4 d[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) d[s] = V4::get(f.u[s]);
#pragma unroll
      for (int u = 0; u < NKU; ++u)
#pragma unroll
        for (int s = 0; s < NS; ++s) d[s] = M::mma(f.w[u], sb[s][u], d[s]);
      if (rv) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          frag *dst = DU + (s * NTU + rtc / TPU) * 64 + lane;
          if (TPU == 2) {
            // half (rtc & 1) of the token unit: 4 values at byte 8*(rtc&1)
            bf16x4 v4 = {(bf16)d[s][0], (bf16)d[s][1], (bf16)d[s][2],
                         (bf16)d[s][3]};
            *(bf16x4 *)((char *)dst + 8 * (rtc & 1)) = v4;
          } else {
            *(f32x4 *)dst = d[s];
          }
        }
      }
      interleave_loads<NS * NKU, NKU * NS, NKU + NS>();
      lds_barrier();  // Delta complete in DU
      load_state<1, IO, DK, C, NS>(nx, nblk, W, rtc, w4, lane, g4, vt0);
      frag db[NS][NTU];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int u = 0; u < NTU; ++u) db[s][u] = DU[(s * NTU + u) * 64 + lane];
      // S <- diag(gamma_C) S + Ktil^T Delta on the owned key tiles
#pragma unroll
      for (int j = 0; j < KUW; ++j)
#pragma unroll
        for (int hh = 0; hh < TPU; ++hh)
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            f32x4 sn = S[j][hh][s] * gm[j][hh];
#pragma unroll
            for (int u = 0; u < NTU; ++u)
              sn = M::mma(f.k[j][hh][u], db[s][u], sn);
            S[j][hh][s] = sn;
          }
      publish_s();
      interleave_loads<NS * NTU, KUW * TPU * NS * NTU, KUW * (TPU * NTU + 1)>();
      lds_barrier();  // S complete in SU
    };

    SF f0, f1;
    load_state<0, IO, DK, C, NS>(f0, ws0, W, rtc, w4, lane, g4, vt0);
    load_state<1, IO, DK, C, NS>(f0, ws0, W, rtc, w4, lane, g4, vt0);
    for (int n = 0; n < NC; n += 2) {
      sstep(n, f0, f1);
      if (n + 1 >= NC) break;
      sstep(n + 1, f1, f0);
    }
    if (p.s_out) {
#pragma unroll
      for (int j = 0; j < KUW; ++j)
#pragma unroll
        for (int hh = 0; hh < TPU; ++hh) {
          const int t = TPU * (w4 + SW * j) + hh;
          if (kv[j] && t < NKT) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              float *so = p.s_out + ((size_t)bh * DK + 16 * t + 4 * g4) * Dv +
                          16 * (vt0 + s) + m16;
#pragma unroll
              for (int e = 0; e < 4; ++e) so[(size_t)e * Dv] = S[j][hh][s][e];
            }
          }
        }
    }
  } else if (wave < SW + OW) {
    // ================= output waves: O ==================================
    IO *obase = (IO *)p.o + ((size_t)bb * T * H + h) * Dv + 16 * vt0 + 4 * g4;
    const size_t orow = (size_t)H * Dv;  // elements between tokens
    lds_barrier();
    auto ostep = [&](int n, const OF &f, OF &nx) {
      const char *nblk = ws0 + (size_t)min(n + 1, NC - 1) * p.wsb;
      load_out<0, IO, DK, C, NS>(nx, nblk, W, rtc, lane);
      // O^T (value columns x tokens of tile rtc) = S^T Qtil^T + Delta^T P^T,
      // S being the state at the chunk start (SU until the state update)
      frag sb[NS][NKU];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int u = 0; u < NKU; ++u) sb[s][u] = SU[(s * NKU + u) * 64 + lane];
      f32x4 ot[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) ot[s] = zero;
#pragma unroll
      for (int u = 0; u < NKU; ++u)
#pragma unroll
        for (int s = 0; s < NS; ++s) ot[s] = M::mma(sb[s][u], f.q[u], ot[s]);
      interleave_loads<NS * NKU, NKU * NS, NKU>();
      lds_barrier();  // Delta complete in DU
      load_out<1, IO, DK, C, NS>(nx, nblk, W, rtc, lane);
      frag db[NS][NTU];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int u = 0; u < NTU; ++u) db[s][u] = DU[(s * NTU + u) * 64 + lane];
#pragma unroll
      for (int u = 0; u < NTU; ++u) {
        if (NTU > 1 && u > rtc / TPU) continue;  // P is zero there
#pragma unroll
        for (int s = 0; s < NS; ++s) ot[s] = M::mma(db[s][u], f.p[u], ot[s]);
      }
      // lane (g4, m16) holds token 16 rtc + m16, value columns 4 g4 .. 4 g4 + 3
      const int tok = n * C + 16 * rtc + m16;
      if (rv && tok < T) {
        IO *dst = obase + (size_t)tok * orow;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          *(typename V4::raw *)(dst + 16 * s) = V4::put(ot[s]);
      }
      lds_barrier();  // the state update has left SU
    };
    OF f0, f1;
    load_out<0, IO, DK, C, NS>(f0, ws0, W, rtc, lane);
    load_out<1, IO, DK, C, NS>(f0, ws0, W, rtc, lane);
    for (int n = 0; n < NC; n += 2) {
      ostep(n, f0, f1);
      if (n + 1 >= NC) break;
      ostep(n + 1, f1, f0);
    }
  } else {
    // ================= L2 warm-up wave ==================================
    // touches 4 bytes of every 128-byte line of the block of chunk
    // n + STATE_PF while chunk n is computed (the ng workgroups of the head
    // split the lines), as direct-to-LDS loads into a sink so nothing ever
    // waits for them; it takes part in every barrier
    __shared__ __attribute__((aligned(256))) char sink[256];
    const int nline = (int)((p.wsb + 127) / 128);
    const int share = (nline + ng - 1) / ng;
    const int nk = (share + 63) / 64;
    auto warm = [&](int n) {
      const char *blk = ws0 + (size_t)n * p.wsb;
      for (int k = 0; k < nk; ++k) {
        const int ln = min(grp * share + min(64 * k + lane, share - 1),
                           nline - 1);
        __builtin_amdgcn_global_load_lds(
            (const void *)(blk + (size_t)ln * 128),
            (__attribute__((address_space(3))) void *)sink, 4, 0, 0);
      }
    };
    for (int n = 0; n < STATE_PF && n < NC; ++n) warm(n);
    lds_barrier();
    for (int n = 0; n < NC; ++n) {
      if (n + STATE_PF < NC) warm(n + STATE_PF);
      lds_barrier();
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// Concurrent variant: bf16 q/k/v, d_k = d_v = 128, chunk 64, one 16-column
// value slab per workgroup, running at the same time as the chunk prep
// (kda_chunk_prep_d128 in its concurrent mode) on the same CUs.  The prep
// holds one workgroup of eight waves per CU with two waves per SIMD; this
// workgroup has four waves, one per SIMD, and fits beside it: at most 144
// registers per lane (2 x 184 + 144 = 512 per SIMD) and 6 KiB of LDS.
//
// Wave w has both roles of the kernel above for token tile w and key unit
// w: Delta rows (from -W, U), the state rows of key channels 32w .. 32w + 31
// (from Ktil^T, gamma_C) and the O rows (from Qtil, P).  Each group of its
// factors is fetched for the next chunk right after its last use in this
// one, into the same registers, so every fetch has about one chunk step to
// arrive.  The whole S is read from LDS once per chunk, before the Delta
// barrier, and kept for O, so the state update may overwrite SU as soon as
// that barrier is passed: two barriers per chunk, as above.
//
// Before fetching chunk n a wave must know that its ready flag is set: the
// prep sets it after the chunk's (device-coherent) workspace stores have
// completed, and the flags are read with device-coherent loads.  No line of
// the block is touched before that, so the XCD's L2 cannot hold an older
// copy of it (the kernel starts with the L2 invalidated).  The flags of a
// head are contiguous, so one vector load reads 64 of them: a wave polls
// only when it reaches a chunk it does not yet know to be ready, and then
// learns the whole run of ready chunks after it.  The wait is bounded (about
// a second, after which it sets sync[SYNC_TIMEOUT] and stops waiting), so a
// mistake can only give wrong values, never a hang.
//
// Every load of the main loop is issued on every path (indices clamped
// instead of branches): the compiler counts the vector-memory operations
// issued after each load to wait for exactly that load, and a load that is
// skipped on some path would make those counts, and the waits, coarser.
// Once chunk n + PF is known ready, its block is pulled into L2 (4 bytes of
// every line, direct-to-LDS into a sink that nothing reads) so the factor
// loads a few chunks later hit the L2.  That load is written in inline asm:
// as a builtin, the compiler would make later LDS accesses wait for it.  An
// operation the compiler does not count can only make its waits stricter
// (a wait for at most k outstanding operations then also covers one more),
// never looser.
namespace co {
constexpr int DK = 128, DV = 128, C = 64, NB = 4, NKU = 4, NTU = 2;
constexpr int THREADS = 256;
constexpr int PF = 3;                // chunks between warming and use
// polls of about 3 us each (a long sleep between them: a thousand waves
// polling device-coherent lines load the memory side that the prep beside
// them writes to)
constexpr long SPIN_MAX = 1L << 18;
constexpr int POLL_SLEEP = 100;  // s_sleep units of 64 clocks

struct Factors {  // one wave's factors of one chunk
  typedef Mma<bf16>::frag frag;
  frag w[NKU];     // -W, token tile w
  uint2 u;         // U, token tile w, the slab's 16 columns
  frag k[2][NTU];  // Ktil^T, key tiles 2w, 2w + 1
  f32x4 gm[2];     // gamma_C of those key tiles
  frag q[NKU];     // Qtil, token tile w
  frag p[NTU];     // P, token tile w (unit 1 is zero for w < 2)
};
}  // namespace co

__global__ __launch_bounds__(co::THREADS, 1) void kda_state_pass_co(
    PrefillParams p) {
  using namespace co;
  using M = Mma<bf16>;
  using V4 = Vec4T<bf16>;
  typedef M::frag frag;
  constexpr WsLayout W = ws_layout(DK, DV, C, 2);
  __shared__ __attribute__((aligned(1024))) char sm[(NKU + NTU) * 1024];
  __shared__ __attribute__((aligned(256))) char sink[256];  // warm-up only
  frag *SU = (frag *)sm;                 // S as second operand, NKU units
  frag *DU = (frag *)(sm + NKU * 1024);  // Delta as second operand, NTU units

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15, g4 = lane >> 4;
  const int H = p.H, T = p.T, BH = p.B * p.H, NC = p.NC;
  constexpr int ng = DV / 16;
  int bh, grp;
  {
    // a head's slab workgroups on one XCD, as in kda_state_pass
    const int b = blockIdx.x;
    if ((BH & 7) == 0) {
      const int x = b & 7, jj = b >> 3;
      bh = (jj / ng) * 8 + x;
      grp = jj % ng;
    } else {
      bh = b / ng;
      grp = b % ng;
    }
  }
  const int bb = bh / H, h = bh % H, vt = grp;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const char *ws0 = p.ws + (size_t)bh * NC * p.wsb;
  const int *hflags = p.sync + SYNC_FLAGS + (size_t)bh * NC;  // [n]

  // chunks below `ready` are known to be in memory (wave-uniform)
  int ready = 0;
  bool gave_up = false;
  // wait for chunk n (the chunks before it are already known): lane i
  // reads the flag of chunk n + i, and the run of set flags from n on
  // extends `ready`
  auto wait_ready = [&](int n) {
    if (n < ready) return;
    long it = 0;
    while (true) {
      const int f = __hip_atomic_load(hflags + min(n + lane, NC - 1),
                                      __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long set = __ballot(f != 0 || n + lane >= NC);
      const int run = (~set == 0ull) ? 64 : __builtin_ctzll(~set);
      if (run > 0 || gave_up) {
        ready = n + max(run, 1);
        break;
      }
      if (++it > SPIN_MAX) {
        if (lane == 0)
          __hip_atomic_store(p.sync + SYNC_TIMEOUT, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        gave_up = true;
      }
      __builtin_amdgcn_s_sleep(POLL_SLEEP);
    }
    // no load of the block may be moved above the wait
    asm volatile("" ::: "memory");
  };
  // 4 bytes of every 128-byte line of chunk n's block: the head's ng
  // workgroups split the lines, the four waves split a workgroup's share
  const unsigned sink_lds =
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void *)sink;
  auto warm = [&](int n) {
    constexpr int nline = (int)((W.bytes + 127) / 128);
    constexpr int share = (nline + ng - 1) / ng;
    constexpr int per = (share + 3) / 4;
    static_assert(per <= 64, "one load per wave");
    // lanes past the wave's share repeat its last line
    const int i = min(per * w + min(lane, per - 1), share - 1);
    const int line = min(grp * share + i, nline - 1);
    const char *a = ws0 + (size_t)n * p.wsb + (size_t)line * 128;
    int m0save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0save)
        : "v"(a), "s"(sink_lds)
        : "memory");
  };
  auto load_wu = [&](Factors &f, const char *blk) {
    const frag *Lw = (const frag *)(blk + W.off_negw) + lane;
#pragma unroll
    for (int u = 0; u < NKU; ++u) f.w[u] = Lw[(w * NKU + u) * 64];
    f.u = ((const uint2 *)(blk + W.off_u) + lane)[(vt * NB + w) * 64];
  };
  auto load_kg = [&](Factors &f, const char *blk) {
    const frag *Lk = (const frag *)(blk + W.off_ktt) + lane;
    const float *Lg = (const float *)(blk + W.off_gam) + 4 * g4;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int t = 2 * w + h2;
#pragma unroll
      for (int u = 0; u < NTU; ++u) f.k[h2][u] = Lk[(t * NTU + u) * 64];
      f.gm[h2] = *(const f32x4 *)(Lg + 16 * t);
    }
  };
  auto load_qp = [&](Factors &f, const char *blk) {
    const frag *Lq = (const frag *)(blk + W.off_qt) + lane;
#pragma unroll
    for (int u = 0; u < NKU; ++u) f.q[u] = Lq[(w * NKU + u) * 64];
    // P units above the diagonal are never written by the prep: unit 1 of
    // tiles 0 and 1 is loaded (inside the block) but never multiplied
    const frag *Lp = (const frag *)(blk + W.off_p) + lane;
#pragma unroll
    for (int u = 0; u < NTU; ++u) f.p[u] = Lp[(w * NTU + u) * 64];
  };

  // state rows of key tiles 2w, 2w + 1 (accumulator layout)
  f32x4 S[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    S[h2] = zero;
    if (p.s0) {
      const float *s0 = p.s0 + ((size_t)bh * DK + 16 * (2 * w + h2) + 4 * g4) *
                                   DV + 16 * vt + m16;
#pragma unroll
      for (int e = 0; e < 4; ++e) S[h2][e] = s0[(size_t)e * DV];
    }
  }
  SU[w * 64 + lane] = M::pack(S[0], S[1]);

  Factors f;
  wait_ready(0);
  load_wu(f, ws0);
  load_kg(f, ws0);
  load_qp(f, ws0);
  lds_barrier();  // S0 in SU

  bf16 *obase = (bf16 *)p.o + ((size_t)bb * T * H + h) * DV + 16 * vt + 4 * g4;
  const size_t orow = (size_t)H * DV;  // elements between tokens
  for (int n = 0; n < NC; ++n) {
    // the next chunk's block (the last chunk fetches its own again)
    const bool more = n + 1 < NC;
    const char *nb = ws0 + (size_t)(more ? n + 1 : n) * p.wsb;
    // the whole S of the chunk start, for Delta now and for O later
    frag sb[NKU];
#pragma unroll
    for (int u = 0; u < NKU; ++u) sb[u] = SU[u * 64 + lane];
    // Delta rows of token tile w: U - W S
    f32x4 d = V4::get(f.u);
#pragma unroll
    for (int u = 0; u < NKU; ++u) d = M::mma(f.w[u], sb[u], d);
    {
      const bf16x4 v4 = {(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]};
      *(bf16x4 *)((char *)(DU + (w / 2) * 64 + lane) + 8 * (w & 1)) = v4;
    }
    if (more) wait_ready(n + 1);
    load_wu(f, nb);
    lds_barrier();  // Delta complete in DU; every wave has read SU
    frag db[NTU];
#pragma unroll
    for (int u = 0; u < NTU; ++u) db[u] = DU[u * 64 + lane];
    // S <- diag(gamma_C) S + Ktil^T Delta on key tiles 2w, 2w + 1
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x4 sn = S[h2] * f.gm[h2];
#pragma unroll
      for (int u = 0; u < NTU; ++u) sn = M::mma(f.k[h2][u], db[u], sn);
      S[h2] = sn;
    }
    SU[w * 64 + lane] = M::pack(S[0], S[1]);
    load_kg(f, nb);
    // O^T (value columns x tokens of tile w) = S^T Qtil^T + Delta^T P^T
    f32x4 ot = zero;
#pragma unroll
    for (int u = 0; u < NKU; ++u) ot = M::mma(sb[u], f.q[u], ot);
#pragma unroll
    for (int u = 0; u < NTU; ++u)
      if (u <= w / 2) ot = M::mma(db[u], f.p[u], ot);
    // lane (g4, m16): token 16 w + m16, value columns 4 g4 .. 4 g4 + 3
    const int tok = n * C + 16 * w + m16;
    if (tok < T) *(uint2 *)(obase + (size_t)tok * orow) = V4::put(ot);
    load_qp(f, nb);
    // (a chunk already known ready when n + PF is not)
    warm(n + PF < ready ? n + PF : ready - 1);
    lds_barrier();  // S complete in SU; every wave has read DU
  }
  if (p.s_out) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float *so = p.s_out + ((size_t)bh * DK + 16 * (2 * w + h2) + 4 * g4) * DV +
                  16 * vt + m16;
#pragma unroll
      for (int e = 0; e < 4; ++e) so[(size_t)e * DV] = S[h2][e];
    }
  }
  // nothing in flight when the wave ends (the warm-up loads included)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ void kda_sync_clear(int *sync, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) sync[i] = 0;
}

// ---------------------------------------------------------------------------
static int state_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n <= 0)
    return 256;
  return n;
}

template <typename IO, int DK, int C, int NS>
static hipError_t state_ns(const PrefillParams &p, hipStream_t s) {
  const unsigned nblk = (unsigned)(p.B * p.H) * (unsigned)(p.Dv / (16 * NS));
  hipLaunchKernelGGL((kda_state_pass<IO, DK, C, NS>), dim3(nblk),
                     dim3(STATE_THREADS), 0, s, p);
  return hipGetLastError();
}

template <typename IO, int DK, int C>
static hipError_t state_one(const PrefillParams &p, hipStream_t s) {
  // slabs per workgroup: one while that fills the chip, two when the
  // workgroups would otherwise run in several rounds (the second slab reuses
  // the fetched factors); more would not fit the registers
  const long long slabs = p.Dv / 16, units = (long long)p.B * p.H * slabs;
  const long long cus = state_cu_count();
  if constexpr (sizeof(IO) == 2 || DK < 128) {
    if (slabs % 2 == 0 && units >= 2 * cus)
      return state_ns<IO, DK, C, 2>(p, s);
  }
  return state_ns<IO, DK, C, 1>(p, s);
}

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
      case 128064: return FN<IO, 128, 64>(p, s);                            \
    }                                                                       \
    return hipErrorInvalidValue;                                            \
  }

KDA_DISPATCH(state_one)

hipError_t launch_state_pass(const PrefillParams &p, int io_bf16,
                             hipStream_t s) {
  return io_bf16 ? state_one_dk<bf16>(p, s) : state_one_dk<float>(p, s);
}

bool prefill_concurrent_applies(const PrefillParams &p, int io_bf16) {
  // the prep's concurrent mode: the d128 per-channel prep without conv or
  // backward outputs; the state pass: one slab workgroup per CU at most, so
  // every one of them is resident beside a prep workgroup
  return prep_d128_applies(p, io_bf16) && !p.use_conv && !p.ckpt &&
         !p.train_at && p.Dv == co::DV &&
         (long long)p.B * p.H * (co::DV / 16) <= state_cu_count();
}

hipError_t launch_sync_clear(const PrefillParams &p, hipStream_t s) {
  const int n = SYNC_FLAGS + p.B * p.H * p.NC;
  hipLaunchKernelGGL(kda_sync_clear, dim3((n + 255) / 256), dim3(256), 0, s,
                     p.sync, n);
  return hipGetLastError();
}

hipError_t launch_state_pass_concurrent(const PrefillParams &p,
                                        hipStream_t s) {
  const unsigned nblk = (unsigned)(p.B * p.H) * (co::DV / 16);
  hipLaunchKernelGGL(kda_state_pass_co, dim3(nblk), dim3(co::THREADS), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace kda
