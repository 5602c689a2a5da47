// kda_conv.hip -- standalone causal depthwise conv prologue for q, k, v.
//
// For each stream s in {q, k, v} and channel c (see include/kda.h):
//   y[t,c] = sum_{j<W} w[c,j] x[t-W+1+j, c],  x before t = 0 from the conv
//   cache (or zeros);  q, k then divided per head by sqrt(sum y^2 + eps).
// One workgroup per (64-token block, head, batch x stream): the x tile plus
// its W-1 token halo is staged through LDS, each thread makes 4 channels of
// one token, and the per-token sum of squares is a butterfly across the
// lanes that share the token.  A second tiny kernel then rewrites the cache
// with the last W-1 inputs (it runs after the first on the same stream, so
// reading the old cache and writing the new one never race).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int CONV_TB = 64;
constexpr int CONV_THREADS = 256;

template <typename IO>
__global__ __launch_bounds__(CONV_THREADS) void kda_conv_fwd(ConvParams p) {
  __shared__ float xs[(CONV_TB + 3) * 128];
  __shared__ float ws[128 * 4];
  const int tid = threadIdx.x;
  const int sidx = blockIdx.z % 3, b = blockIdx.z / 3, h = blockIdx.y;
  const int tb0 = blockIdx.x * CONV_TB;
  const int D = p.D[sidx], W = p.W, T = p.T, H = p.H;
  const IO *x = (const IO *)p.x[sidx];
  const size_t row = (size_t)H * D;  // elements per token
  const int nrow = CONV_TB + W - 1;

  for (int i = tid; i < D * W; i += CONV_THREADS)
    ws[i] = p.w[sidx][(size_t)h * D * W + i];
  for (int i = tid; i < nrow * D; i += CONV_THREADS) {
    const int tt = i / D, c = i % D;
    const int t = tb0 - (W - 1) + tt;
    float val = 0.f;
    if (t >= 0) {
      if (t < T) val = to_f32(x[((size_t)b * T + t) * row + (size_t)h * D + c]);
    } else if (p.state) {
      const size_t ch = (size_t)h * D + c;
      val = p.state[(((size_t)b * 3 + sidx) * H * p.Dmax + ch) * (W - 1) +
                    (W - 1) + t];
    }
    xs[tt * 128 + c] = val;
  }
  __syncthreads();

  const int NQ = D / 4;              // threads per token (power of two)
  const int tpp = CONV_THREADS / NQ; // tokens per pass
  const int q4 = tid % NQ, tl = tid / NQ;
  const bool norm = p.l2 && sidx < 2;
  IO *y = (IO *)p.y[sidx];
  for (int tt = tl; tt < CONV_TB; tt += tpp) {
    const int t = tb0 + tt;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < W; ++j) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
        acc[cc] += ws[(4 * q4 + cc) * W + j] * xs[(tt + j) * 128 + 4 * q4 + cc];
    }
    if (norm) {
      float ss = acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] +
                 acc[3] * acc[3];
      for (int off = NQ / 2; off >= 1; off >>= 1)
        ss += __shfl_xor(ss, off, 64);
      acc *= l2_inv_norm(ss + p.eps);
    }
    if (t < T) {
      IO *dst = y + ((size_t)b * T + t) * row + (size_t)h * D + 4 * q4;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) dst[cc] = from_f32<IO>(acc[cc]);
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
  dim3 grid((unsigned)((p.T + CONV_TB - 1) / CONV_TB), (unsigned)p.H,
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
