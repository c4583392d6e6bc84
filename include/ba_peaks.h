/* Machine-peak microbenchmarks for the rooflines of libba_att.
 *
 * Not part of the attention operator: kernels that confirm, on the GPU the
 * library runs on, the two constants its rooflines are priced against -- HBM
 * bandwidth (streaming read, and copy) and the bf16 matrix-core rate -- next
 * to the vendor's figures, and the matrix-core rate on random operands, whose
 * switching power lowers the clock.  Built into libba_peaks.so.
 *
 * Conventions as in ba_att.h: device pointers, a hipStream_t passed as void*,
 * the caller owns every buffer, nothing is allocated, arguments are checked
 * before any launch (0 = ok, 1 = invalid argument, 4 = HIP launch error).
 */
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at src once (16-byte vector loads, grid-stride over
 * `workgroups` workgroups of 256 threads; nontemporal != 0: loads marked
 * nontemporal, the streaming hint) and writes one 32-bit XOR digest per
 * thread to sink[workgroups*256], so that no load can be dropped.
 * src 16-byte aligned, bytes a positive multiple of 16. */
int ba_peak_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, int32_t nontemporal,
                 void* stream);

/* Copies `bytes` bytes from src to dst (16-byte vectors, grid-stride).
 * Both 16-byte aligned and not overlapping; bytes a positive multiple of 16. */
int ba_peak_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, void* stream);

/* Every wave of `workgroups` workgroups (4 waves each) issues `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands (2*32*32*16
 * FLOP each, no memory traffic in the loop); operands are x in bf16.  Each
 * thread writes the sum of its accumulators to sink[workgroups*256].
 * FLOPs = workgroups * 4 * iters * 4 * 32768. */
int ba_peak_mfma_bf16(float* sink, int32_t workgroups, int32_t iters, float x, void* stream);

/* As ba_peak_mfma_bf16, but every wave cycles through eight different pairs
 * of register operands, each element a bf16 with a random sign, a random
 * exponent in [-2, 2] and a random 7-bit mantissa drawn from a hash of
 * (seed, thread, element), like the values of attention's Q, K, V and P
 * tiles; every iteration issues the eight products over four independent
 * accumulators.  FLOPs = workgroups * 4 * iters * 8 * 32768. */
int ba_peak_mfma_bf16_random(float* sink, int32_t workgroups, int32_t iters, uint32_t seed, void* stream);

#ifdef __cplusplus
}
#endif
