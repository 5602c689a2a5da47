// kda_conv.hip -- standalone causal depthwise conv prologue for q, k, v.
//
// For each stream s in {q, k, v} and channel c (see include/kda.h):
//   y[t,c] = sum_{j<W} w[c,j] x[t-W+1+j, c],  x before t = 0 from the conv
//   cache (or zeros);  q, k then divided per head by sqrt(sum y^2 + eps).
// Streaming, no LDS: a group of D / 4 lanes owns a run of tokens (CONV_RUN
// at the smallest head size) of one (batch, head, stream); lane q of the
// group makes channels
// 4q .. 4q + 3.  It keeps the previous W - 1 inputs of its channels in
// registers (a sliding window, filled from the conv cache or zeros before
// the sequence start), reads 8 tokens' inputs at a time with one 8- or
// 16-byte load per token (a group reads whole contiguous rows), applies the
// taps, and stores each token's 4 outputs with one vector store; the
// per-token sum of squares is a butterfly across the group's lanes.  A
// second tiny kernel then rewrites the cache with the last W-1 inputs (it
// runs after the first on the same stream, so reading the old cache and
// writing the new one never race).
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int CONV_RUN = 64;  // tokens per lane group
constexpr int CONV_THREADS = 256;
constexpr int CONV_BATCH = 8;  // tokens loaded ahead at a time

// 4 consecutive values of IO as one vector access, in fp32
template <typename IO> struct Vec4IO;
template <> struct Vec4IO<bf16> {
  __device__ static __forceinline__ f32x4 get(const bf16 *p) {
    const uint2 r = *(const uint2 *)p;
    return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                 __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
  }
  __device__ static __forceinline__ void put(bf16 *p, f32x4 v) {
    *(bf16x4 *)p = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  }
};
template <> struct Vec4IO<float> {
  __device__ static __forceinline__ f32x4 get(const float *p) {
    return *(const f32x4 *)p;
  }
  __device__ static __forceinline__ void put(float *p, f32x4 v) {
    *(f32x4 *)p = v;
  }
};

template <typename IO>
__global__ __launch_bounds__(CONV_THREADS) void kda_conv_fwd(ConvParams p) {
  using V = Vec4IO<IO>;
  const int tid = threadIdx.x;
  const int sidx = blockIdx.z % 3, b = blockIdx.z / 3, h = blockIdx.y;
  const int D = p.D[sidx], W = p.W, T = p.T, H = p.H;
  const int NQ = D / 4;  // lanes per token (a power of two, at most 32)
  const int q4 = tid % NQ, grp = tid / NQ, ngrp = CONV_THREADS / NQ;
  // a workgroup spans tpw tokens (set by the smallest D of the three
  // streams, as the grid is); a stream with a larger D has fewer lane
  // groups, each with a longer run
  const int dmin = min(p.D[0], min(p.D[1], p.D[2]));
  const int tpw = (CONV_THREADS / (dmin / 4)) * CONV_RUN;
  const int run = tpw / ngrp;
  const int t0 = blockIdx.x * tpw + grp * run;
  if (t0 >= T) return;  // a whole lane group at once
  const int t1 = min(t0 + run, T);
  const size_t row = (size_t)H * D;  // elements per token
  const size_t ch0 = (size_t)h * D + 4 * q4;
  const IO *x = (const IO *)p.x[sidx] + (size_t)b * T * row + ch0;
  IO *y = (IO *)p.y[sidx] + (size_t)b * T * row + ch0;
  const bool norm = p.l2 && sidx < 2;

  // tap by lag: y[t] = sum_l wl[l] x[t - l], l < W (zero beyond)
  float wl[4][4];  // [lag][channel]
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const float *w = p.w[sidx] + (ch0 + cc) * W;
#pragma unroll
    for (int l = 0; l < 4; ++l) wl[l][cc] = l < W ? w[W - 1 - l] : 0.f;
  }
  // inputs of tokens t0 - 1, t0 - 2, t0 - 3 (lag 1..3)
  f32x4 win[3];
#pragma unroll
  for (int l = 1; l <= 3; ++l) {
    const int t = t0 - l;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (l < W) {
      if (t >= 0) {
        v = V::get(x + (size_t)t * row);
      } else if (p.state) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          v[cc] = p.state[(((size_t)b * 3 + sidx) * H * p.Dmax + ch0 + cc) *
                              (W - 1) + (W - 1) + t];
      }
    }
    win[l - 1] = v;
  }
  for (int tb = t0; tb < t1; tb += CONV_BATCH) {
    f32x4 xin[CONV_BATCH];
#pragma unroll
    for (int i = 0; i < CONV_BATCH; ++i)
      xin[i] = V::get(x + (size_t)min(tb + i, t1 - 1) * row);
#pragma unroll
    for (int i = 0; i < CONV_BATCH; ++i) {
      f32x4 acc;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        acc[cc] = wl[0][cc] * xin[i][cc] + wl[1][cc] * win[0][cc] +
                  wl[2][cc] * win[1][cc] + wl[3][cc] * win[2][cc];
      win[2] = win[1];
      win[1] = win[0];
      win[0] = xin[i];
      if (norm) {
        float ss = acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] +
                   acc[3] * acc[3];
        for (int off = NQ / 2; off >= 1; off >>= 1)
          ss += __shfl_xor(ss, off, 64);
        acc *= l2_inv_norm(ss + p.eps);
      }
      if (tb + i < t1) V::put(y + (size_t)(tb + i) * row, acc);
    }
  }
}

// new cache[m] = (history ++ x)[T - M + m], m < M = W-1; one thread per
// 4 adjacent channels of one (batch, stream): their 4*M history entries
// are contiguous, so they move as M 16-byte loads and stores.
template <typename IO, int M>
__global__ void kda_conv_cache(ConvParams p) {
  const int T = p.T, H = p.H;
  const size_t C = (size_t)H * p.Dmax;  // history channels per stream
  const size_t i = 4 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= (size_t)p.B * 3 * C) return;
  const int ch = (int)(i % C);
  const size_t bs = i / C;
  const int sidx = (int)(bs % 3), b = (int)(bs / 3);
  const int D = p.D[sidx];
  if (ch >= H * D) return;  // H*D is a multiple of 4: all 4 or none
  f32x4 *st = (f32x4 *)(p.state + i * M);
  float old[4 * M], nw[4 * M];  // entry m of channel ch+c at c*M + m
#pragma unroll
  for (int j = 0; j < M; ++j) *(f32x4 *)&old[4 * j] = st[j];
  const IO *x = (const IO *)p.x[sidx] + (size_t)b * T * H * D + ch;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int tau = T - M + m;
      nw[c * M + m] = tau >= 0 ? to_f32(x[(size_t)tau * H * D + c])
                               : old[c * M + T + m];
    }
  }
#pragma unroll
  for (int j = 0; j < M; ++j) st[j] = *(const f32x4 *)&nw[4 * j];
}

template <typename IO>
static hipError_t cache_t(const ConvParams &p, hipStream_t s) {
  const size_t threads = (size_t)p.B * 3 * p.H * p.Dmax / 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (p.W) {
    case 2: hipLaunchKernelGGL((kda_conv_cache<IO, 1>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((kda_conv_cache<IO, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((kda_conv_cache<IO, 3>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename IO>
static hipError_t conv_t(const ConvParams &p, hipStream_t s) {
  // tokens per workgroup, from the smallest stream D (as in the kernel)
  const int dmin = std::min(p.D[0], std::min(p.D[1], p.D[2]));
  const int tpw = (CONV_THREADS / (dmin / 4)) * CONV_RUN;  // tokens per block
  dim3 grid((unsigned)((p.T + tpw - 1) / tpw), (unsigned)p.H,
            (unsigned)(p.B * 3));
  hipLaunchKernelGGL(kda_conv_fwd<IO>, grid, dim3(CONV_THREADS), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.state) return e;
  return cache_t<IO>(p, s);
}

hipError_t launch_conv(const ConvParams &p, hipStream_t s) {
  return p.io_bf16 ? conv_t<bf16>(p, s) : conv_t<float>(p, s);
}

hipError_t launch_conv_cache(const ConvParams &p, hipStream_t s) {
  return p.io_bf16 ? cache_t<bf16>(p, s) : cache_t<float>(p, s);
}

}  // namespace kda
