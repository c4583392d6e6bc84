// Shared device types and helpers for the gfx950 BA-Att kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups are dealt round-robin over them

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger
// key); -0 is folded onto +0 so that equal values compare equal.
__device__ __forceinline__ uint32_t float_order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Logical workgroup id with an XCD-aware remap: hardware id w lands on XCD
// w % 8; consecutive logical ids are given to the same XCD so that the
// workgroups of one head share that XCD's L2.  `total` logical ids; the grid
// must hold round_up(total, 8) workgroups; returns -1 for padding groups.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int logical = (w % kNumXcd) * per + (w / kNumXcd);
  return logical < total ? logical : -1;
}

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace ba
