// device_common.h - small device helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace colimoe {

// Plain LLVM vector for 16-byte loads: copies of it stay in registers (the
// uint4 class type is copied through memory, which keeps staged data off
// registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes at p (p wave-uniform): loads through it
// take a per-lane offset plus a scalar offset, and loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bits_f(uint32_t v) { return __uint_as_float(v); }
__device__ __forceinline__ uint32_t f_bits(float v) { return __float_as_uint(v); }

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Number of unique experts of a call, clamped to what the buffers can hold.
__device__ __forceinline__ int clamp_nu(const int32_t *n_unique, const Dims &D) {
  int cap = D.T * D.k < D.E ? D.T * D.k : D.E;
  int nu = D.T > 0 ? *n_unique : 0;
  return nu < 0 ? 0 : (nu > cap ? cap : nu);
}

// Work slot s of a call: routed expert ids[s] with pairs [p0, p1) for s < nu,
// else the shared expert (stored after the E routed ones) with tokens
// [0, T).  Caller-supplied union lists are clamped so no access leaves its
// buffer; an out-of-range expert id skips the slot.
__device__ __forceinline__ bool resolve_slot(const Dims &D, const UnionDev &U, int nu, int s, int &e, int &p0,
                                             int &p1) {
  if (s < nu) {
    const int tk = D.T * D.k;
    e = U.ids[s];
    p0 = U.offsets[s];
    p1 = U.offsets[s + 1];
    p0 = p0 < 0 ? 0 : (p0 > tk ? tk : p0);
    p1 = p1 < p0 ? p0 : (p1 > tk ? tk : p1);
    return e >= 0 && e < D.E;
  }
  e = D.E;
  p0 = 0;
  p1 = D.T;
  return D.n_shared > 0;
}

// Pair p of slot s: its token (activation row) and its output row; a token
// outside [0, T) in caller-supplied lists yields orow = -1 (skipped).
__device__ __forceinline__ void slot_token(const Dims &D, const UnionDev &U, int nu, int s, int p, int &t, int &orow) {
  if (s < nu) {
    t = U.pair_token[p];
    orow = p;
  } else {
    t = p;
    orow = D.T * D.k + p;
  }
  if (t < 0 || t >= D.T) {
    t = 0;
    orow = -1;
  }
}

}  // namespace colimoe
