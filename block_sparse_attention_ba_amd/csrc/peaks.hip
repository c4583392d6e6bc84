// Machine-peak microbenchmarks (include/ba_peaks.h): streaming HBM read,
// HBM copy and the bf16 matrix-core rate, measured on the GPU the library
// runs on, as context for the vendor peaks its rooflines are priced against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ba_peaks.h"

namespace ba {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  return NT ? __builtin_nontemporal_load(p) : *p;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                        uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // four loads in flight per thread per round
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = load16<NT>(src + i), b = load16<NT>(src + i + stride), c = load16<NT>(src + i + 2 * stride),
                d = load16<NT>(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += stride) acc ^= load16<NT>(src + i);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(float* __restrict__ sink, int iters, float x) {
  const __bf16 v = (__bf16)x;
  const bf16x8 a = {v, v, v, v, v, v, v, v};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// 32-bit integer mixer (the finalizer of a multiply-xorshift hash): a
// counter-based source of operand bits, so no memory is read in the loop
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// random sign, exponent 2^-2 .. 2^2 and 7-bit mantissa
__device__ __forceinline__ __bf16 random_bf16(uint32_t h) {
  const uint32_t expo = 125u + (h >> 16) % 5u;
  const uint16_t bits = (uint16_t)(((h & 1u) << 15) | (expo << 7) | ((h >> 8) & 0x7Fu));
  return __builtin_bit_cast(__bf16, bits);
}

__global__ __launch_bounds__(kThreads) void mfma_random_kernel(float* __restrict__ sink, int iters, uint32_t seed) {
  bf16x8 a[8], b[8];
  const uint32_t base = seed + (blockIdx.x * kThreads + threadIdx.x) * 128u;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[i][e] = random_bf16(mix32(base + i * 8 + e));
      b[i][e] = random_bf16(mix32(base + 64 + i * 8 + e));
    }
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], c[i & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c[0][r] + c[1][r] + c[2][r] + c[3][r];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace ba

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int finish() { return hipGetLastError() == hipSuccess ? 0 : 4; }

}  // namespace

extern "C" {

int ba_peak_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, int32_t nontemporal,
                 void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || workgroups < 1) return 1;
  const dim3 grid((unsigned)workgroups);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    ba::read_kernel<true><<<grid, ba::kThreads, 0, s>>>(static_cast<const ba::u32x4*>(src), bytes / 16, sink);
  else
    ba::read_kernel<false><<<grid, ba::kThreads, 0, s>>>(static_cast<const ba::u32x4*>(src), bytes / 16, sink);
  return finish();
}

int ba_peak_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst) || workgroups < 1)
    return 1;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (s < d + bytes && d < s + bytes) return 1;  // overlapping
  ba::copy_kernel<<<dim3((unsigned)workgroups), ba::kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const ba::u32x4*>(src), static_cast<ba::u32x4*>(dst), bytes / 16);
  return finish();
}

int ba_peak_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, float x, void* stream) {
  if (!sink || workgroups < 1 || iters < 1) return 1;
  ba::mfma_kernel<<<dim3((unsigned)workgroups), ba::kThreads, 0, static_cast<hipStream_t>(stream)>>>(sink, iters, x);
  return finish();
}

int ba_peak_mfma_bf16_random(float* sink, int32_t workgroups, int32_t iters, uint32_t seed, void* stream) {
  if (!sink || workgroups < 1 || iters < 1) return 1;
  ba::mfma_random_kernel<<<dim3((unsigned)workgroups), ba::kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      sink, iters, seed);
  return finish();
}

}  // extern "C"
