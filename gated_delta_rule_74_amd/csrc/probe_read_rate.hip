// probe_read_rate.hip -- how long the state pass's workgroups take to pull
// the chunk factors into registers when they do nothing else (gfx950).
//
// The probe kernel has the state pass's grid (one workgroup per (batch*head,
// 16-column value slab)), its workgroup -> XCD placement (the slab
// workgroups of a head on one XCD, sharing its L2), its per-chunk byte volume
// (the block's shared range -W | Qtil | Ktil^T | P | gamma_C plus the slab's
// U tiles), its staging (16-byte loads per lane straight into registers, one
// chunk ahead, in two halves around two barriers per chunk) and its L2
// warm-up wave (4 bytes of every 128-byte line of the block four chunks
// ahead, the head's workgroups splitting the lines), but no arithmetic: each
// loading wave folds its registers into an xor so the loads stay live.  Its
// time per launch is what the state pass's loads cost on their own, on a
// workspace laid out exactly like the real one.  Measurement only: built into its own library, loaded
// by bench.py, not part of the prefill path.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_device.h"

namespace kda {
namespace probe {

constexpr int NW = 8;     // loading waves, plus one warm-up wave
constexpr int MAXU = 8;   // 1 KiB units per wave per chunk
constexpr int PF = 4;     // chunks between warming and use

struct Args {
  const char *ws;
  size_t wsb, off_u, u_slab;
  int BH, NC, ng, nshared, nu;
  unsigned *sink;
};

// half h of a wave's units of one chunk (the state pass also fetches each
// chunk in two halves, one before each of its two barriers)
constexpr int HU = MAXU / 2;
__device__ __forceinline__ void load_half(const Args &a, const char *blk,
                                          int grp, int wave, int lane, int h,
                                          uint4 (&r)[HU]) {
  const int per = (a.nu + NW - 1) / NW;
#pragma unroll
  for (int i = 0; i < HU; ++i) {
    const int ii = h * HU + i;
    const int j = wave * per + ii;
    if (ii < per && j < a.nu) {
      const size_t off = j < a.nshared
                             ? (size_t)j * 1024
                             : a.off_u + (size_t)grp * a.u_slab +
                                   (size_t)(j - a.nshared) * 1024;
      r[i] = *(const uint4 *)(blk + off + (size_t)lane * 16);
    } else {
      r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

__device__ __forceinline__ unsigned fold(const uint4 (&r)[HU]) {
  unsigned x = 0;
#pragma unroll
  for (int i = 0; i < HU; ++i) x ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
  return x;
}

__global__ __launch_bounds__((NW + 1) * 64, 1) void state_read_probe(Args a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int bh, grp;
  {
    // the state pass's placement: a head's slab workgroups on one XCD
    const int b = blockIdx.x;
    if (a.ng > 1 && (a.BH & 7) == 0) {
      const int x = b & 7, jj = b >> 3;
      bh = (jj / a.ng) * 8 + x;
      grp = jj % a.ng;
    } else {
      bh = b / a.ng;
      grp = b % a.ng;
    }
  }
  const char *ws0 = a.ws + (size_t)bh * a.NC * a.wsb;
  if (wave == NW) {
    // warm-up wave: direct-to-LDS loads into a sink, never waited for
    __shared__ __attribute__((aligned(256))) char sink[256];
    const int nline = (int)((a.wsb + 127) / 128);
    const int share = (nline + a.ng - 1) / a.ng;
    const int nk = (share + 63) / 64;
    auto warm = [&](int n) {
      const char *blk = ws0 + (size_t)n * a.wsb;
      for (int k = 0; k < nk; ++k) {
        const int ln = min(grp * share + min(64 * k + lane, share - 1),
                           nline - 1);
        __builtin_amdgcn_global_load_lds(
            (const void *)(blk + (size_t)ln * 128),
            (__attribute__((address_space(3))) void *)sink, 4, 0, 0);
      }
    };
    for (int n = 0; n < PF && n < a.NC; ++n) warm(n);
    for (int n = 0; n < a.NC; ++n) {
      if (n + PF < a.NC) warm(n + PF);
      __syncthreads();
      __syncthreads();
    }
    return;
  }
  // two register sets in turn (a copy between them would wait for the loads)
  uint4 a0[HU], a1[HU], b0[HU], b1[HU];
  unsigned acc = 0;
  auto step = [&](int n, uint4 (&c0)[HU], uint4 (&c1)[HU], uint4 (&n0)[HU],
                  uint4 (&n1)[HU]) {
    const char *nb = ws0 + (size_t)min(n + 1, a.NC - 1) * a.wsb;
    load_half(a, nb, grp, wave, lane, 0, n0);
    acc ^= fold(c0);
    __syncthreads();
    load_half(a, nb, grp, wave, lane, 1, n1);
    acc ^= fold(c1);
    __syncthreads();
  };
  load_half(a, ws0, grp, wave, lane, 0, a0);
  load_half(a, ws0, grp, wave, lane, 1, a1);
  for (int n = 0; n < a.NC; n += 2) {
    step(n, a0, a1, b0, b1);
    if (n + 1 >= a.NC) break;
    step(n + 1, b0, b1, a0, a1);
  }
  // never true for a workspace the prep wrote; keeps the loads live
  if (acc == 0x9e3779b9u) a.sink[blockIdx.x] = acc;
}

}  // namespace probe
}  // namespace kda

// Time `reps` launches of the probe over a prefill workspace `ws` of
// `ws_bytes` bytes (as kda_prefill_chunk_prep leaves it for bf16 q/k/v) for
// B*H = BH, NC chunks of C tokens, d_k = Dk, d_v = Dv.  Writes the mean
// microseconds per launch and the bytes one workgroup loads per chunk.
// Returns 0, or -1 for a shape it does not cover or a HIP error.
extern "C" int kda_probe_state_reads(const void *ws, size_t ws_bytes, int BH,
                                     int NC, int Dk, int Dv, int C, int reps,
                                     double *us_per_launch,
                                     double *bytes_per_wg_chunk) {
  using namespace kda;
  if (!ws || BH <= 0 || NC <= 0 || reps <= 0 || Dv % 16 || C % 16 || Dk % 16)
    return -1;
  const WsLayout L = ws_layout(Dk, Dv, C, 2);
  if (ws_bytes < (size_t)BH * NC * L.bytes || L.u_slab % 1024) return -1;
  probe::Args a{};
  a.ws = (const char *)ws;
  a.wsb = L.bytes;
  a.off_u = L.off_u;
  a.u_slab = L.u_slab;
  a.BH = BH;
  a.NC = NC;
  a.ng = Dv / 16;
  a.nshared = (int)((L.off_u + 1023) / 1024);
  a.nu = a.nshared + (int)((L.u_slab + 1023) / 1024);
  if ((a.nu + probe::NW - 1) / probe::NW > probe::MAXU) return -1;
  // the last shared unit may run past off_u into the U tiles: still inside
  // the block; the U units of slab grp end at off_u + (grp + 1) u_slab
  if ((size_t)a.nshared * 1024 > L.bytes ||
      L.off_u + (size_t)a.ng * L.u_slab > L.bytes)
    return -1;
  const unsigned nblk = (unsigned)BH * (unsigned)a.ng;
  if (hipMalloc(&a.sink, (size_t)nblk * sizeof(unsigned)) != hipSuccess)
    return -1;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -1;
  if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    for (int i = 0; i < 3; ++i)
      hipLaunchKernelGGL(probe::state_read_probe, dim3(nblk),
                         dim3((probe::NW + 1) * 64), 0, 0, a);
    hipEventRecord(e0, 0);
    for (int i = 0; i < reps; ++i)
      hipLaunchKernelGGL(probe::state_read_probe, dim3(nblk),
                         dim3((probe::NW + 1) * 64), 0, 0, a);
    hipEventRecord(e1, 0);
    float ms = 0.f;
    if (hipEventSynchronize(e1) == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
        hipGetLastError() == hipSuccess) {
      *us_per_launch = (double)ms * 1e3 / reps;
      *bytes_per_wg_chunk = (double)a.nu * 1024.0;
      rc = 0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(a.sink);
  return rc;
}
