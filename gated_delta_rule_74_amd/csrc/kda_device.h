// kda_device.h -- shared device helpers for the KDA kernels (gfx950).
//
// Fragment convention used by every matrix-core product in this library.
// All products use 16x16 output tiles.  A "fragment unit" is the operand
// one lane holds for one MFMA step, always 16 bytes:
//   bf16: v_mfma_f32_16x16x32_bf16, a unit covers 32 k values, 8 per lane;
//   fp32: 4 x v_mfma_f32_16x16x4_f32, a unit covers 16 k values, 4 per lane.
// Lane l = 16*g + m holds row m (A operand) or column m (B operand) and, in
// unit u, the k values
//   bf16: e < 4 -> k = 32u + 4g + e,   e >= 4 -> k = 32u + 16 + 4g + (e-4)
//   fp32: k = 16u + 4g + e
// This is the k order of the accumulator layout (lane 16*g + n holds column
// n and rows 4g..4g+3 of a 16x16 tile), so an accumulator tile pair (bf16)
// or tile (fp32) IS a B operand unit, and the accumulator of X^T is an A
// operand unit of X -- results move from one product into the next without
// touching LDS.  Any k permutation is a valid contraction as long as the A
// and B operands of one product use the same one, which they do.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Streaming (nontemporal) 8- or 16-byte accesses, for data touched once in
// a kernel: read-once inputs and write-once workspace blocks.  They keep the
// L2 from filling with dirty lines that a following kernel has to write
// back while it runs.
template <typename R>
__device__ __forceinline__ R ld_stream(const void *q) {
  static_assert(sizeof(R) == 8 || sizeof(R) == 16, "8 or 16 bytes");
  if constexpr (sizeof(R) == 16) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(R, __builtin_nontemporal_load((const u4 *)q));
  } else {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(R, __builtin_nontemporal_load((const u2 *)q));
  }
}
template <typename T>
__device__ __forceinline__ void st_stream(void *q, T v) {
  static_assert(sizeof(T) == 8 || sizeof(T) == 16, "8 or 16 bytes");
  if constexpr (sizeof(T) == 16) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u4, v), (u4 *)q);
  } else {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(__builtin_bit_cast(u2, v), (u2 *)q);
  }
}

// A workspace store.  CO = false: the streaming store above.  CO = true:
// also written through to the device-coherent level (sc1), so that a
// workgroup on another XCD whose first read of the line comes after this
// store has completed sees the new value without any cache write-back (the
// chunk prep and the state pass run at the same time in that mode).  Stores
// only; the trailing s_nop covers the wait state that a vector write of the
// data registers needs after a store of more than 8 bytes.
template <bool CO, typename T>
__device__ __forceinline__ void st_ws(void *q, T v) {
  static_assert(sizeof(T) == 8 || sizeof(T) == 16, "8 or 16 bytes");
  if constexpr (!CO) {
    st_stream(q, v);
  } else if constexpr (sizeof(T) == 16) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt\n\ts_nop 1"
                 :: "v"(q), "v"(__builtin_bit_cast(u4, v)));
  } else {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    asm volatile("global_store_dwordx2 %0, %1, off sc1 nt\n\ts_nop 1"
                 :: "v"(q), "v"(__builtin_bit_cast(u2, v)));
  }
}

// workgroup barrier after this wave's LDS accesses are done, leaving its
// global loads in flight (unlike __syncthreads, whose fence also waits for
// them)
__device__ __forceinline__ void barrier_keep_vmem() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 1 / sqrt(x) for the per-head L2 norm, x >= eps > 0: the hardware
// reciprocal square root (within 1 ulp; the correctly rounded sqrt and
// division it replaces cost about 25 instructions)
__device__ __forceinline__ float l2_inv_norm(float x) {
  return __builtin_amdgcn_rsqf(x);
}

// sum over aligned groups of G lanes (G a power of two, at most 32), every
// lane of a group getting the total: DPP moves within a 16-lane row (quad
// swaps, then rotations by 4 and 8 or the half-row mirror), one shuffle
// across the two rows of a 32-lane group
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G == 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (G >= 16) {
    x += dpp_mov<0x124>(x);  // row_ror:4
    x += dpp_mov<0x128>(x);  // row_ror:8
  }
  if constexpr (G >= 32) x += __shfl_xor(x, 16, 64);
  static_assert(G <= 32, "groups of at most 32 lanes");
  return x;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return (bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
}

template <typename IO> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int TPU = 2;  // 16-wide k tiles per unit
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // unit from two accumulator tiles (hi may be absent: zeros)
  __device__ static __forceinline__ frag pack(f32x4 lo, f32x4 hi) {
    frag r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2];
    r[3] = (bf16)lo[3]; r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1];
    r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
  }
  // unit from a k-contiguous row: p points at element k = first k of the
  // unit; `full` = false when only the first 16 k exist (upper half zero)
  __device__ static __forceinline__ frag load_k(const bf16 *p, int g,
                                                bool full = true) {
    bf16x4 lo = *(const bf16x4 *)(p + 4 * g);
    bf16x4 hi;
    if (full) {
      hi = *(const bf16x4 *)(p + 16 + 4 * g);
    } else {
      hi = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    }
    frag r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
  __device__ static __forceinline__ float elem(const frag &f, int e) {
    return (float)f[e];
  }
  __device__ static __forceinline__ void set(frag &f, int e, float x) {
    f[e] = (bf16)x;
  }
  // k offset (within the unit) of element e for lane group g
  __device__ static __forceinline__ int koff(int g, int e) {
    return (e < 4) ? (4 * g + e) : (16 + 4 * g + (e - 4));
  }
  static constexpr int NE = 8;
};

template <> struct Mma<float> {
  static constexpr int TPU = 1;
  typedef f32x4 frag;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ frag pack(f32x4 lo, f32x4) { return lo; }
  __device__ static __forceinline__ frag load_k(const float *p, int g,
                                                bool = true) {
    return *(const f32x4 *)(p + 4 * g);
  }
  __device__ static __forceinline__ float elem(const frag &f, int e) {
    return f[e];
  }
  __device__ static __forceinline__ void set(frag &f, int e, float x) {
    f[e] = x;
  }
  __device__ static __forceinline__ int koff(int g, int e) {
    return 4 * g + e;
  }
  static constexpr int NE = 4;
};

// fp32 16x16x16 product on the matrix cores: D += A(16x16) * B(16x16) with
// A given as rows (lane 16g+m: A[m][4g..4g+3]) and B as the accumulator
// layout (lane 16g+n: B[4g..4g+3][n]).
__device__ __forceinline__ f32x4 mma16_f32(f32x4 a, f32x4 b, f32x4 c) {
  return Mma<float>::mma(a, b, c);
}

// ---------------------------------------------------------------------------
// Prefill workspace: one block per (batch*head, chunk), bh-major.  Layout
//   [ -W | Qtil | Ktil^T | P | gamma_C | U ]
// The first five sections are shared by every value-column slab and form
// one contiguous range [0, off_u); U follows slab-major ([vt][rt]) so each
// 16-column slab's tiles are contiguous too.  Fragment sections are arrays
// of 1 KiB units (64 lanes x 16 B); U tiles are 64 lanes x 4 values.
struct WsLayout {
  int nb, nkt, nvt, tpu, nku, ntu;
  size_t off_negw, off_qt, off_ktt, off_p, off_gam, off_u, u_slab, bytes;
};

__host__ __device__ constexpr size_t ws_align(size_t x) {
  return (x + 255) & ~(size_t)255;
}

// bytes of the shared range [0, off_u)
__host__ __device__ constexpr size_t ws_shared_bytes(int Dk, int C,
                                                     int io_bytes) {
  return ws_align(
      (size_t)(C / 16) * (((Dk / 16) + (io_bytes == 2)) / (1 + (io_bytes == 2))) * 2048 +
      (size_t)(Dk / 16) * (((C / 16) + (io_bytes == 2)) / (1 + (io_bytes == 2))) * 1024 +
      (size_t)(C / 16) * (((C / 16) + (io_bytes == 2)) / (1 + (io_bytes == 2))) * 1024 +
      (size_t)Dk * 4);
}

__host__ __device__ constexpr WsLayout ws_layout(int Dk, int Dv, int C,
                                                 int io_bytes) {
  WsLayout L{};
  L.nb = C / 16;
  L.nkt = Dk / 16;
  L.nvt = Dv / 16;
  L.tpu = (io_bytes == 2) ? 2 : 1;
  L.nku = (L.nkt + L.tpu - 1) / L.tpu;
  L.ntu = (L.nb + L.tpu - 1) / L.tpu;
  size_t o = 0;
  L.off_negw = o; o += (size_t)L.nb * L.nku * 1024;       // -W   [rt][u]
  L.off_qt = o;   o += (size_t)L.nb * L.nku * 1024;       // Qtil [rt][u]
  L.off_ktt = o;  o += (size_t)L.nkt * L.ntu * 1024;      // Ktil^T [ct][u]
  L.off_p = o;    o += (size_t)L.nb * L.ntu * 1024;       // P    [rt][u]
  L.off_gam = o;  o += (size_t)Dk * 4;                    // gamma_C
  o = ws_align(o);
  L.off_u = o;                                            // U [vt][rt]
  L.u_slab = (size_t)L.nb * 64 * 4 * io_bytes;
  o += L.u_slab * L.nvt;
  L.bytes = ws_align(o);
  return L;
}

}  // namespace kda
