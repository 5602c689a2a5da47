// kda_state.hip -- sequential state pass of the chunked KDA prefill.
//
// Given the chunk-local factors that kda_chunk_prep leaves in the workspace
// (per (batch*head, chunk): -W, Qtil = scale Q*Gam, Ktil^T, P, Gam_C, U; see
// kda_prep.hip for their definitions), each chunk n updates
//   Delta = U - W S,   O = Qtil S + P Delta,   S <- diag(Gam_C) S + Ktil^T Delta
// in order, which is the chunked form of the per-token KDA rule (state rows
// are key channels; see include/kda.h for the sources).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------------------
// Sequential state pass.  A workgroup of NW waves owns one (batch*head) and
// NW consecutive 16-column value slabs; wave w carries the state columns of
// slab w in registers as accumulator tiles.  Per chunk, the workgroup needs
// the shared range of the chunk's workspace block plus its own U tiles
// (about 66 KB for d = 128, C = 64, NW = 4).  They reach LDS through a
// register-staged pipeline two chunks deep: at chunk n every thread issues
// the loads of chunk n+2 into one register set, computes chunk n from LDS,
// and then writes the other register set (chunk n+1, loaded one chunk
// earlier) into the free LDS buffer.  Only the MFMA chain and its LDS reads
// sit on the sequential path.
template <typename IO> struct Vec4T;
template <> struct Vec4T<bf16> {
  typedef uint2 raw;
  __device__ static __forceinline__ void get(raw r, float *f) {
    f[0] = __uint_as_float(r.x << 16);
    f[1] = __uint_as_float(r.x & 0xffff0000u);
    f[2] = __uint_as_float(r.y << 16);
    f[3] = __uint_as_float(r.y & 0xffff0000u);
  }
};
template <> struct Vec4T<float> {
  typedef uint4 raw;
  __device__ static __forceinline__ void get(raw r, float *f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};

template <typename IO, int DK, int C, int NW>
struct StateCfg {
  static constexpr size_t SH = ws_shared_bytes(DK, C, (int)sizeof(IO));
  static constexpr size_t UB = (size_t)(C / 16) * 64 * 4 * sizeof(IO);
  static constexpr size_t TOT = SH + NW * UB;         // bytes per chunk
  static constexpr int NL = 2;                        // loader waves
  static constexpr int NKB = (int)((TOT + 1023) / 1024);   // 1 KiB copies
  static constexpr int CPW = (NKB + NL - 1) / NL;     // copies per loader
  static constexpr int NLINE = (int)((SH + 127) / 128 + NW * UB / 128);
  static constexpr int TPW = (NLINE + 64 * NL - 1) / (64 * NL);  // touches
  static constexpr int PF = 3;                        // touch distance
  static constexpr size_t BUF = (size_t)NKB * 1024;
  static constexpr size_t LDS = 2 * BUF + NL * 256;   // + touch sink
  static constexpr bool fits = LDS <= 160 * 1024;
};

__device__ __forceinline__ void dma16(const char *src, char *dst_wave) {
  __builtin_amdgcn_global_load_lds(
      (const void *)src, (__attribute__((address_space(3))) void *)dst_wave,
      16, 0, 0);
}
__device__ __forceinline__ void dma4(const char *src, char *dst_wave) {
  __builtin_amdgcn_global_load_lds(
      (const void *)src, (__attribute__((address_space(3))) void *)dst_wave,
      4, 0, 0);
}

template <typename IO, int DK, int C, int NW>
__global__ __launch_bounds__(64 * (NW + 2), 1) void kda_state_pass(
    PrefillParams p) {
  using M = Mma<IO>;
  using SC = StateCfg<IO, DK, C, NW>;
  typedef typename M::frag frag;
  constexpr int NB = C / 16, NKT = DK / 16, TPU = M::TPU;
  constexpr int NKU = (NKT + TPU - 1) / TPU, NTU = (NB + TPU - 1) / TPU;
  __shared__ __attribute__((aligned(1024))) char sm[SC::LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool loader = wave >= NW;  // waves NW, NW+1 move data
  const int lw = wave - NW;        // loader wave index
  const int m16 = lane & 15, g4 = lane >> 4;
  const int Dv = p.Dv, H = p.H, T = p.T, BH = p.B * p.H, NC = p.NC;
  const int ng = Dv / (16 * NW);  // workgroups per head
  int bh, grp;
  {
    // keep the workgroups of one head on one XCD (blocks go round-robin over
    // the 8 XCDs), so the later reader of the shared factors hits L2
    const int b = blockIdx.x;
    if (ng > 1 && (BH & 7) == 0) {
      const int x = b & 7, j = b >> 3;
      bh = (j / ng) * 8 + x;
      grp = j % ng;
    } else {
      bh = b / ng;
      grp = b % ng;
    }
  }
  const int bb = bh / H, h = bh % H;
  const int slab0 = grp * NW, vt = slab0 + (loader ? 0 : wave);
  const int col = 16 * vt + m16;
  const WsLayout W = ws_layout(DK, Dv, C, (int)sizeof(IO));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const char *ws0 = p.ws + (size_t)bh * NC * p.wsb;
  const size_t uoff = W.off_u + (size_t)slab0 * SC::UB;

  // ---- loader side ---------------------------------------------------------
  // the chunk's byte range is [shared factors | this group's U tiles]; copy
  // block i (1 KiB) of chunk n into LDS buffer `buf`
  auto copy_chunk = [&](int n, int buf) {
    const char *blk = ws0 + (size_t)n * p.wsb;
#pragma unroll
    for (int c = 0; c < SC::CPW; ++c) {
      const int i = lw + c * SC::NL;
      if (i < SC::NKB) {
        const size_t o = (size_t)i * 1024 + lane * 16;
        if (o < SC::TOT)
          dma16(blk + (o < SC::SH ? o : uoff + (o - SC::SH)),
                sm + buf * SC::BUF + (size_t)i * 1024);
      }
    }
  };
  // pull chunk n's lines into L2 (4 bytes per 128-byte line into a sink);
  // every loader wave issues exactly TPW of these
  auto touch_chunk = [&](int n) {
    const char *blk = ws0 + (size_t)n * p.wsb;
    constexpr int NSH = (int)((SC::SH + 127) / 128);
#pragma unroll
    for (int c = 0; c < SC::TPW; ++c) {
      const int ln = min(lw * 64 + lane + c * 64 * SC::NL, SC::NLINE - 1);
      const size_t o = ln < NSH ? (size_t)ln * 128
                                : uoff + (size_t)(ln - NSH) * 128;
      dma4(blk + o, sm + 2 * SC::BUF + lw * 256);
    }
  };
  // s_waitcnt vmcnt(TPW): this wave's copies (issued before its touches)
  // have landed; the touches may still be in flight
  constexpr unsigned WAIT_COPIES = (unsigned)SC::TPW | 0xF70u;

  // ---- compute side: state tiles of slab vt --------------------------------
  f32x4 S[NKT];
  if (!loader && p.s0) {
    const float *s0 = p.s0 + (size_t)bh * DK * Dv + col;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[t][j] = s0[(size_t)(16 * t + 4 * g4 + j) * Dv];
  } else {
#pragma unroll
    for (int t = 0; t < NKT; ++t) S[t] = zero;
  }
  IO *obase = (IO *)p.o + ((size_t)bb * T * H + h) * Dv + col;
  const size_t orow = (size_t)H * Dv;  // elements between tokens

  auto compute = [&](int n) {
    const char *L = sm + (n & 1) * SC::BUF;
    const char *LU = L + SC::SH + (size_t)wave * SC::UB;
    const frag *Lw = (const frag *)(L + W.off_negw) + lane;
    const frag *Lq = (const frag *)(L + W.off_qt) + lane;
    const frag *Lk = (const frag *)(L + W.off_ktt) + lane;
    const frag *Lp = (const frag *)(L + W.off_p) + lane;

    frag Sb[NKU];
#pragma unroll
    for (int u = 0; u < NKU; ++u)
      Sb[u] = M::pack(S[TPU * u], (TPU == 2 && TPU * u + 1 < NKT)
                                      ? S[(TPU * u + 1) % NKT]
                                      : zero);
    // Delta = U - W S0, one row tile at a time (its units read as a batch)
    f32x4 D[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      frag wf[NKU];
#pragma unroll
      for (int u = 0; u < NKU; ++u) wf[u] = Lw[(rt * NKU + u) * 64];
      float u4[4];
      Vec4T<IO>::get(*((const typename Vec4T<IO>::raw *)LU + rt * 64 + lane),
                     u4);
      D[rt] = f32x4{u4[0], u4[1], u4[2], u4[3]};
#pragma unroll
      for (int u = 0; u < NKU; ++u) D[rt] = M::mma(wf[u], Sb[u], D[rt]);
    }
    frag Db[NTU];
#pragma unroll
    for (int u = 0; u < NTU; ++u)
      Db[u] = M::pack(D[TPU * u], (TPU == 2 && TPU * u + 1 < NB)
                                      ? D[(TPU * u + 1) % NB]
                                      : zero);
    // S_C = diag(gamma_C) S0 + K~^T Delta   (the critical path)
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      frag kf[NTU];
#pragma unroll
      for (int u = 0; u < NTU; ++u) kf[u] = Lk[(t * NTU + u) * 64];
      const f32x4 gm =
          *(const f32x4 *)((const float *)(L + W.off_gam) + 16 * t + 4 * g4);
      f32x4 sn = S[t] * gm;
#pragma unroll
      for (int u = 0; u < NTU; ++u) sn = M::mma(kf[u], Db[u], sn);
      S[t] = sn;
    }
    // O = Q~ S0 + P Delta   (S0 survives in Sb)
    const bool full = (n + 1) * C <= T;
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
      frag qf[NKU], pf[NTU];
#pragma unroll
      for (int u = 0; u < NKU; ++u) qf[u] = Lq[(rt * NKU + u) * 64];
#pragma unroll
      for (int u = 0; u < NTU; ++u)
        if (u <= rt / TPU) pf[u] = Lp[(rt * NTU + u) * 64];
      f32x4 O = zero;
#pragma unroll
      for (int u = 0; u < NKU; ++u) O = M::mma(qf[u], Sb[u], O);
#pragma unroll
      for (int u = 0; u < NTU; ++u)
        if (u <= rt / TPU) O = M::mma(pf[u], Db[u], O);
      IO *orow0 = obase + (size_t)(n * C + 16 * rt + 4 * g4) * orow;
      if (full) {
#pragma unroll
        for (int j = 0; j < 4; ++j) orow0[j * orow] = from_f32<IO>(O[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n * C + 16 * rt + 4 * g4 + j < T)
            orow0[j * orow] = from_f32<IO>(O[j]);
      }
    }
  };

  // prologue: chunk 0 in LDS buffer 0, chunks 1..PF-1 heading to L2
  if (loader) {
    copy_chunk(0, 0);
    for (int m = 1; m < SC::PF && m < NC; ++m) touch_chunk(m);
    __builtin_amdgcn_s_waitcnt(0);
  }
  for (int n = 0; n < NC; ++n) {
    __syncthreads();  // buffer n&1 holds chunk n; buffer (n+1)&1 is free
    if (!loader) {
      compute(n);
    } else {
      if (n + 1 < NC) copy_chunk(n + 1, (n + 1) & 1);
      if (n + SC::PF < NC) {
        touch_chunk(n + SC::PF);
        __builtin_amdgcn_s_waitcnt(WAIT_COPIES);
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
    }
  }
  if (!loader && p.s_out) {
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p.s_out[((size_t)bh * DK + 16 * t + 4 * g4 + j) * Dv + col] = S[t][j];
  }
}

// ---------------------------------------------------------------------------
template <typename IO, int DK, int C, int NW>
static hipError_t state_nw(const PrefillParams &p, hipStream_t s) {
  if constexpr (!StateCfg<IO, DK, C, NW>::fits) {
    return hipErrorInvalidValue;
  } else {
    const unsigned nblk = (unsigned)(p.B * p.H) * (unsigned)(p.Dv / (16 * NW));
    hipLaunchKernelGGL((kda_state_pass<IO, DK, C, NW>), dim3(nblk),
                       dim3(64 * (NW + 2)), 0, s, p);
    return hipGetLastError();
  }
}

template <typename IO, int DK, int C>
static hipError_t state_one(const PrefillParams &p, hipStream_t s) {
  // as many 16-column slabs per workgroup (up to 4) as Dv and LDS allow
  const int slabs = p.Dv / 16;
  if (slabs % 4 == 0 && StateCfg<IO, DK, C, 4>::fits)
    return state_nw<IO, DK, C, 4>(p, s);
  if (slabs % 2 == 0 && StateCfg<IO, DK, C, 2>::fits)
    return state_nw<IO, DK, C, 2>(p, s);
  return state_nw<IO, DK, C, 1>(p, s);
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

}  // namespace kda
