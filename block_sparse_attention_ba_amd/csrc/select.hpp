// Selection pass of BA-Att on gfx950: block pooling with diagonal
// statistics, the corrected compact score, and the per-row norm sort.
//
// Operation (pith.science review of "Efficient Long-Context Modeling in
// Diffusion Language Models via Block Approximate Sparse Attention", sections
// "What carries the argument" and "Core claim", and the abstract): Q and K
// are downsampled block-wise; the compact block map is scored with a
// correction that uses only the diagonal QK variances; every query-block row
// is sorted and its leading key blocks are kept.
//
// Score reading: with per-block means m and population variances v,
//   S[I,J] = scale*<mq_I, mk_J>
//          + scale^2/2 * sum_c (vq_Ic*vk_Jc + vq_Ic*mk_Jc^2 + mq_Ic^2*vk_Jc),
// i.e. the mean plus half the variance of scale*<q,k> over the block pair
// with covariances cut to their diagonals.  The pooling kernel writes it as
// one bilinear form over augmented 3D-vectors
//   aq_I = [scale*mq, scale^2/2*vq, scale^2/2*mq^2],  ak_J = [mk, vk + mk^2, vk]
// so that S[I,J] = <aq_I, ak_J>.
#pragma once

#include "common.hpp"

namespace ba {

// ---------------------------------------------------------------------------
// Pooling and diagonal statistics: one WAVE per (tensor, b*h, block), four
// blocks per workgroup, no LDS and no barriers.  Lane (c, rg) owns 16-byte
// channel chunk c and rows rg, rg+RG, ... of the block, so every load
// instruction of the wave reads RG consecutive rows = 1 KB of contiguous
// HBM.  The rows stay in registers between the mean and the centred
// variance pass (two-pass statistics); sums over the RG row groups use
// v_permlane16/32_swap (xor 16, 32) and a shuffle for xor 8 (D = 64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_sum(float x, int mask) {
  if (mask == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (mask == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x + wave_shfl_xor(x, mask);
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void pool_stats_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         float* __restrict__ aq,
                                                         float* __restrict__ ak, int N, int n,
                                                         int BH, float scale) {
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RG = 64 / CPR;      // row groups per wave
  constexpr int RPL = BLK / RG;     // rows per lane
  static_assert(BLK % RG == 0, "block must be a multiple of the row groups");

  const int per_tensor = BH * n;
  const int gb = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gb >= 2 * per_tensor) return;
  const int tensor = gb / per_tensor;
  const int rem = gb - tensor * per_tensor;
  const int bh = rem / n;
  const int I = rem - bh * n;
  const int rows = min(BLK, N - I * BLK);
  const uint16_t* X = (tensor == 0 ? q : k) + ((size_t)bh * N + (size_t)I * BLK) * D;

  const int lane = threadIdx.x & 63;
  const int c = lane % CPR;
  const int rg = lane / CPR;

  u32x4 data[RPL];
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    const int row = rg + j * RG;
    data[j] = row < rows ? *reinterpret_cast<const u32x4*>(X + (size_t)row * D + c * 8)
                         : u32x4{0u, 0u, 0u, 0u};
  }

  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s[2 * w] += bf16_lo(data[j][w]);
      s[2 * w + 1] += bf16_hi(data[j][w]);
    }
  }
#pragma unroll
  for (int m = CPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = xor_sum(s[e], m);
  const float inv_rows = 1.0f / (float)rows;
  float mean[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mean[e] = s[e] * inv_rows;

  // The second pass re-derives the fp32 values from the packed rows instead
  // of keeping both forms live: 83 instead of 162 VGPRs at b = 64 and 147
  // instead of 256 at b = 128 (3 instead of 1 wave per SIMD, which moves the
  // 128-token blocks' pooling from 4.3 to 5.4 TB/s).
#pragma unroll
  for (int j = 0; j < RPL; ++j) __asm__ volatile("" : "+v"(data[j]));
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
  for (int j = 0; j < RPL; ++j) {
    if (rg + j * RG < rows) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = bf16_lo(data[j][w]) - mean[2 * w];
        const float b = bf16_hi(data[j][w]) - mean[2 * w + 1];
        s[2 * w] = __builtin_fmaf(a, a, s[2 * w]);
        s[2 * w + 1] = __builtin_fmaf(b, b, s[2 * w + 1]);
      }
    }
  }
#pragma unroll
  for (int m = CPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = xor_sum(s[e], m);

  if (rg == 0) {
    float* out = (tensor == 0 ? aq : ak) + ((size_t)bh * n + I) * (3 * D) + c * 8;
    f32x4 seg[3][2];
    const float hs2 = 0.5f * scale * scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float var = s[e] * inv_rows;
      if (tensor == 0) {
        seg[0][e / 4][e % 4] = scale * mean[e];
        seg[1][e / 4][e % 4] = hs2 * var;
        seg[2][e / 4][e % 4] = hs2 * (mean[e] * mean[e]);
      } else {
        seg[0][e / 4][e % 4] = mean[e];
        seg[1][e / 4][e % 4] = var + mean[e] * mean[e];
        seg[2][e / 4][e % 4] = var;
      }
    }
#pragma unroll
    for (int g = 0; g < 3; ++g) {
      reinterpret_cast<f32x4*>(out + g * D)[0] = seg[g][0];
      reinterpret_cast<f32x4*>(out + g * D)[1] = seg[g][1];
    }
  }
}

// ---------------------------------------------------------------------------
// Compact score and norm sort.  One workgroup per (b*h, 16 query-block
// rows, 16 waves).  S = aq . ak^T is a small fp32 GEMM (K = 3D) done with
// v_mfma_f32_16x16x4_f32: wave w sums half (w % 2) of the dot products for
// the 16x16 output tiles w/2, w/2 + 8, ...; operands are loaded from L2 as
// float4 (lane group g = l/16 takes k = 16m + 4g + e for MFMA step (m, e),
// the same assignment for both operands, so the product is unchanged).  The
// first halves are written to LDS and the second halves added after a
// barrier; then one wave per row selects the `keep` largest scores (ties to
// lower J) by an MSB-first radix select over order-preserving uint32 keys and
// writes mask, ascending idx and cnt.
// ---------------------------------------------------------------------------
constexpr int kScoreRows = 16;
constexpr int kMaxScoreBlocks = 512;  // longest row: 16 rows x n fp32 scores staged in LDS

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

// Wave-wide unsigned max / min, result in every lane: xor-1 / xor-2 within
// quads and rotations by 4 and 8 within rows (DPP), then xor 16 and xor 32
// (v_permlane16/32_swap).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false));  // row_ror 4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false));  // row_ror 8
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r[0], r[1]);
}

// Selects the `keep` largest keys of one row (ties: lower J) held as
// key[i] for J = lane + 64*i; writes mask bytes, ascending idx and the count.
// All control state is wave-uniform (scalar registers); per-bit counts come
// from ballots.
template <int NI>
__device__ __forceinline__ void radix_select_row(const uint32_t (&key)[NI], int n, int keep,
                                                 uint8_t* __restrict__ mask_row,
                                                 int32_t* __restrict__ idx_row,
                                                 int32_t* __restrict__ cnt_out) {
  const int lane = __lane_id();
  uint64_t vmask[NI];  // lanes holding a valid J in slot i
#pragma unroll
  for (int i = 0; i < NI; ++i) vmask[i] = __builtin_amdgcn_ballot_w64(lane + 64 * i < n);
  // Bits above the highest bit where the largest and smallest key differ
  // are shared by every key and need no search.
  uint32_t kmax = 0u, kmin = ~0u;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (lane + 64 * i < n) {
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  kmax = __builtin_amdgcn_readfirstlane(wave_minmax_u32<true>(kmax));
  kmin = __builtin_amdgcn_readfirstlane(wave_minmax_u32<false>(kmin));
  const uint32_t diff = kmax ^ kmin;
  // Invariant: the candidates are the keys whose bits above `bit` equal
  // `prefix`; `remaining` of them are still to be taken (1 <= remaining <=
  // cand).  Every key above the candidate range is taken.
  uint32_t prefix = kmax;
  int remaining = keep;
  int bit = -1;  // bits >= bit+1 of the candidates are fixed
  if (diff != 0u) {
    bit = 31 - __builtin_clz(diff);
    prefix = kmax & ~((bit == 31) ? ~0u : ((2u << bit) - 1u));
    int cand = n;
    for (; bit >= 0; --bit) {
      const uint32_t hi_mask = ~0u << bit;
      const uint32_t want = prefix | (1u << bit);
      int c1 = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        c1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64((key[i] & hi_mask) == want) & vmask[i]);
      if (c1 >= remaining) {
        prefix = want;
        cand = c1;
      } else {
        remaining -= c1;
        cand -= c1;
      }
      if (cand == remaining) break;  // every candidate is taken
    }
  }
  // bit >= 0 (early exit): take every key whose bits >= bit are >= prefix's.
  // bit < 0: keys > prefix, plus the `remaining` lowest-J keys == prefix.
  const uint64_t lt = lanemask_lt();
  const uint32_t cmp_mask = bit >= 0 ? (~0u << bit) : ~0u;
  const uint32_t pre = prefix & cmp_mask;
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int J = lane + 64 * i;
    const bool valid = J < n;
    const uint32_t kk = key[i] & cmp_mask;
    uint64_t km;
    if (bit >= 0) {
      km = __builtin_amdgcn_ballot_w64(kk >= pre) & vmask[i];
    } else {
      const uint64_t eqm = __builtin_amdgcn_ballot_w64(kk == pre) & vmask[i];
      const uint64_t gtm = __builtin_amdgcn_ballot_w64(kk > pre) & vmask[i];
      // the lowest-J equal keys are taken until `remaining` is used up
      uint64_t take = 0;
      int need = remaining - eq_seen;
      uint64_t e = eqm;
      while (need > 0 && e != 0) {
        const uint64_t low = e & (~e + 1);
        take |= low;
        e &= e - 1;
        --need;
      }
      eq_seen += __builtin_popcountll(eqm);
      km = gtm | take;
    }
    const bool kept = (km >> lane) & 1;
    const int pos = base + __builtin_popcountll(km & lt);
    if (kept && pos < keep) idx_row[pos] = J;  // exactly `keep` are kept; the bound is defensive
    base += __builtin_popcountll(km);
    if (valid) mask_row[J] = kept ? 1 : 0;
  }
  if (lane == 0) *cnt_out = base;
}

constexpr int kScoreWaves = 16;
constexpr int kScoreColWaves = 8;  // waves per half of the dot products
constexpr int kMaxColRounds = (kMaxScoreBlocks + 16 * kScoreColWaves - 1) / (16 * kScoreColWaves);

template <int D, int NI>
__global__ __launch_bounds__(kScoreWaves * 64) void score_topk_kernel(const float* __restrict__ aq,
                                                         const float* __restrict__ ak, int n,
                                                         int keep, uint8_t* __restrict__ mask,
                                                         int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ cnt,
                                                         float* __restrict__ score, int total) {
  constexpr int K3 = 3 * D;
  constexpr int KH = K3 / 2;         // each wave takes one half of the 3D-long dot products
  constexpr int KM = KH / 16;        // float4 operand loads per 16x16 tile and half
  constexpr int R = kScoreRows;
  constexpr int AP = K3 + 4;         // padded LDS row pitch of the A tile (floats)
  __shared__ __attribute__((aligned(16))) float Atile[R * AP];
  extern __shared__ float Sbuf[];    // [R][n]

  // the row tiles of one head run on one XCD and share its L2 copy of ak
  const int logical = xcd_remap(blockIdx.x, total);
  if (logical < 0) return;
  const int tiles = (n + R - 1) / R;
  const int bh = logical / tiles;
  const int R0 = (logical - bh * tiles) * R;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int half = wave & 1;               // which half of k this wave sums
  const int cw = wave >> 1;                // column-tile lane of the wave: tiles cw, cw + 8, ...

  // stage the 16 query-block rows of aq once (coalesced float4)
  for (int e = threadIdx.x; e < R * (K3 / 4); e += kScoreWaves * 64) {
    const int row = e / (K3 / 4), k4 = e % (K3 / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (R0 + row < n) v = *reinterpret_cast<const f32x4*>(aq + ((size_t)bh * n + R0 + row) * K3 + 4 * k4);
    *reinterpret_cast<f32x4*>(Atile + row * AP + 4 * k4) = v;
  }

  const int ctiles = (n + 15) / 16;
  auto load_b = [&](int ct, f32x4 (&bfr)[KM]) {
    const int col = ct * 16 + li;
    const float* Bp = ak + ((size_t)bh * n + col) * K3 + half * KH + 4 * lg;
#pragma unroll
    for (int m = 0; m < KM; ++m)
      bfr[m] = col < n ? *reinterpret_cast<const f32x4*>(Bp + 16 * m) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  f32x4 bfr[KM];
  if (cw < ctiles) load_b(cw, bfr);  // in flight while the A tile is staged
  __syncthreads();
  // first half: straight into Sbuf; second half: kept in registers, added
  // after a barrier (a fixed order, so the sum is deterministic)
  f32x4 acc2[kMaxColRounds];
#pragma unroll
  for (int t = 0; t < kMaxColRounds; ++t) {
    const int ct = cw + kScoreColWaves * t;
    acc2[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ct >= ctiles) continue;
    if (t > 0) load_b(ct, bfr);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(Atile + li * AP + half * KH + 16 * m + 4 * lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], bfr[m][e], acc, 0, 0, 0);
    }
    // lane holds column ct*16 + li of rows 4*lg + r
    const int col = ct * 16 + li;
    if (half == 0) {
      if (col < n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Sbuf[(4 * lg + r) * n + col] = acc[r];
      }
    } else {
      acc2[t] = acc;
    }
  }
  __syncthreads();
  if (half == 1) {
#pragma unroll
    for (int t = 0; t < kMaxColRounds; ++t) {
      const int col = (cw + kScoreColWaves * t) * 16 + li;
      if (col < n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Sbuf[(4 * lg + r) * n + col] += acc2[t][r];
      }
    }
  }
  __syncthreads();
  if (score != nullptr) {  // the score map as the selection saw it, row by row
    for (int e = threadIdx.x; e < R * n; e += kScoreWaves * 64) {
      const int row = e / n, col = e - row * n;
      if (R0 + row < n) score[((size_t)bh * n + R0 + row) * n + col] = Sbuf[e];
    }
  }

  for (int r = wave; r < R; r += kScoreWaves) {
    const int I = R0 + r;
    if (I >= n) break;
    uint32_t key[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int J = lane + 64 * i;
      key[i] = (J < n) ? float_order_key(Sbuf[r * n + J]) : 0u;
    }
    const size_t row = (size_t)bh * n + I;
    radix_select_row<NI>(key, n, keep, mask + row * n, idx + row * keep, cnt + row);
  }
}

// ---------------------------------------------------------------------------
// Mask -> ascending index list; one wave per (b*h, query-block) row.
// ---------------------------------------------------------------------------
template <int NI>
__global__ __launch_bounds__(256) void mask_to_index_kernel(const uint8_t* __restrict__ mask,
                                                            int rows, int n, int max_keep,
                                                            int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ cnt) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint8_t* m = mask + (size_t)row * n;
  int32_t* out = idx + (size_t)row * max_keep;
  const uint64_t lt = lanemask_lt();
  int base = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int J = lane + 64 * i;
    const bool kept = (J < n) && (m[J] != 0);
    const uint64_t km = __ballot(kept);
    const int pos = base + __popcll(km & lt);
    if (kept && pos < max_keep) out[pos] = J;
    base += __popcll(km);
  }
  if (lane == 0) cnt[row] = base;
}

}  // namespace ba
