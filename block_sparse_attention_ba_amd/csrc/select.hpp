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
// Pooling and diagonal statistics: one workgroup per (tensor, b*h, block).
// HBM-bound: every Q and K element is read exactly once with 16-byte loads;
// the block's rows stay in registers between the mean and the centred
// variance pass.
// ---------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(256) void pool_stats_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         float* __restrict__ aq,
                                                         float* __restrict__ ak, int N, int n,
                                                         int BH, float scale) {
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;   // rows per pass of the workgroup
  constexpr int PASSES = BLK / RPP;
  static_assert(BLK % RPP == 0, "block must be a multiple of rows per pass");

  __shared__ float red[4][CPR][8];

  const int per_tensor = BH * n;
  const int wg = blockIdx.x;
  const int tensor = wg / per_tensor;
  const int rem = wg - tensor * per_tensor;
  const int bh = rem / n;
  const int I = rem - bh * n;
  const int rows = min(BLK, N - I * BLK);
  const uint16_t* X = (tensor == 0 ? q : k) + ((size_t)bh * N + (size_t)I * BLK) * D;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int c = t % CPR;
  const int r0 = t / CPR;

  u32x4 data[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = r0 + p * RPP;
    if (row < rows) {
      data[p] = *reinterpret_cast<const u32x4*>(X + (size_t)row * D + c * 8);
    } else {
      data[p] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s[2 * w] += bf16_lo(data[p][w]);
      s[2 * w + 1] += bf16_hi(data[p][w]);
    }
  }
#pragma unroll
  for (int m = CPR; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += wave_shfl_xor(s[e], m);
  }
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][c][e] = s[e];
  }
  __syncthreads();
  const float inv_rows = 1.0f / (float)rows;
  float mean[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    mean[e] = (red[0][c][e] + red[1][c][e] + red[2][c][e] + red[3][c][e]) * inv_rows;
  __syncthreads();

  // centred second pass over the rows still held in registers
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    if (r0 + p * RPP < rows) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = bf16_lo(data[p][w]) - mean[2 * w];
        const float b = bf16_hi(data[p][w]) - mean[2 * w + 1];
        s[2 * w] += a * a;
        s[2 * w + 1] += b * b;
      }
    }
  }
#pragma unroll
  for (int m = CPR; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += wave_shfl_xor(s[e], m);
  }
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][c][e] = s[e];
  }
  __syncthreads();
  if (t < CPR) {
    float var[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      var[e] = (red[0][c][e] + red[1][c][e] + red[2][c][e] + red[3][c][e]) * inv_rows;
    float* out = (tensor == 0 ? aq : ak) + ((size_t)bh * n + I) * (3 * D) + c * 8;
    f32x4 seg[3][2];
    if (tensor == 0) {
      const float hs2 = 0.5f * scale * scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        seg[0][e / 4][e % 4] = scale * mean[e];
        seg[1][e / 4][e % 4] = hs2 * var[e];
        seg[2][e / 4][e % 4] = hs2 * (mean[e] * mean[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        seg[0][e / 4][e % 4] = mean[e];
        seg[1][e / 4][e % 4] = var[e] + mean[e] * mean[e];
        seg[2][e / 4][e % 4] = var[e];
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
// rows).  S = aq . ak^T in fp32 (VALU, LDS-tiled: 2x4 outputs per thread,
// k-chunks of 32), staged row-major in LDS; then one wave per row selects
// the `keep` largest scores (ties to lower J) with an MSB-first radix select
// over order-preserving uint32 keys and writes mask, ascending idx and cnt.
// ---------------------------------------------------------------------------
constexpr int kScoreRows = 16;
constexpr int kScoreCols = 128;
constexpr int kScoreKC = 32;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

// Selects the `keep` largest keys of one row (ties: lower J) held as
// key[i] for J = lane + 64*i; writes mask bytes, ascending idx and the count.
template <int NI>
__device__ __forceinline__ void radix_select_row(const uint32_t (&key)[NI], int n, int keep,
                                                 uint8_t* __restrict__ mask_row,
                                                 int32_t* __restrict__ idx_row,
                                                 int32_t* __restrict__ cnt_out) {
  const int lane = __lane_id();
  // bits shared by every valid key need no search
  uint32_t kor = 0u, kand = ~0u;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (lane + 64 * i < n) {
      kor |= key[i];
      kand &= key[i];
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    kor |= (uint32_t)__shfl_xor((int)kor, m, 64);
    kand &= (uint32_t)__shfl_xor((int)kand, m, 64);
  }
  const uint32_t diff = kor ^ kand;
  uint32_t prefix = kand;  // correct on every bit above the highest differing one
  int remaining = keep;
  if (diff != 0u) {
    const int top = 31 - __clz(diff);
    prefix = kand & ~((top == 31) ? ~0u : ((2u << top) - 1u));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t hi_mask = ~0u << bit;
      const uint32_t want = prefix | (1u << bit);
      int c1 = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool hit = (lane + 64 * i < n) && ((key[i] & hi_mask) == want);
        c1 += __popcll(__ballot(hit));
      }
      if (c1 >= remaining) {
        prefix = want;
      } else {
        remaining -= c1;
      }
    }
  }
  // keys > prefix are all kept; of the keys == prefix the `remaining` with
  // the lowest J are kept
  const uint64_t lt = lanemask_lt();
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int J = lane + 64 * i;
    const bool valid = J < n;
    const bool gt = valid && key[i] > prefix;
    const bool eq = valid && key[i] == prefix;
    const uint64_t eqm = __ballot(eq);
    const int eq_rank = eq_seen + __popcll(eqm & lt);
    eq_seen += __popcll(eqm);
    const bool kept = gt || (eq && eq_rank < remaining);
    const uint64_t km = __ballot(kept);
    const int pos = base + __popcll(km & lt);
    if (kept && pos < keep) idx_row[pos] = J;  // exactly `keep` are kept; the bound is defensive
    base += __popcll(km);
    if (valid) mask_row[J] = kept ? 1 : 0;
  }
  if (lane == 0) *cnt_out = base;
}

template <int D, int NI>
__global__ __launch_bounds__(256) void score_topk_kernel(const float* __restrict__ aq,
                                                         const float* __restrict__ ak, int n,
                                                         int keep, uint8_t* __restrict__ mask,
                                                         int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ cnt,
                                                         float* __restrict__ score) {
  constexpr int K3 = 3 * D;
  constexpr int R = kScoreRows, C = kScoreCols, KC = kScoreKC;
  __shared__ float Qs[KC][R];
  __shared__ float Ks[KC][C + 4];
  extern __shared__ float Sbuf[];  // [R][n]

  const int tiles = (n + R - 1) / R;
  const int bh = blockIdx.x / tiles;
  const int R0 = (blockIdx.x - bh * tiles) * R;
  const float* A = aq + (size_t)bh * n * K3;
  const float* Bm = ak + (size_t)bh * n * K3;
  const int t = threadIdx.x;
  const int rp = t / 32;  // rows 2rp, 2rp+1
  const int cq = t % 32;  // cols 4cq .. 4cq+3

  for (int C0 = 0; C0 < n; C0 += C) {
    float acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

    for (int k0 = 0; k0 < K3; k0 += KC) {
      if (t < R * KC / 4) {
        const int row = t / (KC / 4), k4 = t % (KC / 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (R0 + row < n) v = *reinterpret_cast<const f32x4*>(A + (size_t)(R0 + row) * K3 + k0 + 4 * k4);
#pragma unroll
        for (int j = 0; j < 4; ++j) Qs[4 * k4 + j][row] = v[j];
      }
#pragma unroll
      for (int i = 0; i < C * KC / 4 / 256; ++i) {
        const int e = t + 256 * i;
        const int col = e / (KC / 4), k4 = e % (KC / 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (C0 + col < n) v = *reinterpret_cast<const f32x4*>(Bm + (size_t)(C0 + col) * K3 + k0 + 4 * k4);
#pragma unroll
        for (int j = 0; j < 4; ++j) Ks[4 * k4 + j][col] = v[j];
      }
      __syncthreads();
#pragma unroll 8
      for (int kk = 0; kk < KC; ++kk) {
        const f32x2 a = *reinterpret_cast<const f32x2*>(&Qs[kk][2 * rp]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&Ks[kk][4 * cq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[0][j] = __builtin_fmaf(a[0], b[j], acc[0][j]);
          acc[1][j] = __builtin_fmaf(a[1], b[j], acc[1][j]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int row = 2 * rp + a;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = C0 + 4 * cq + j;
        if (col < n) Sbuf[row * n + col] = acc[a][j];
      }
      if (score != nullptr && R0 + row < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = C0 + 4 * cq + j;
          if (col < n) score[((size_t)bh * n + R0 + row) * n + col] = acc[a][j];
        }
      }
    }
  }
  __syncthreads();

  const int wave = t >> 6, lane = t & 63;
  for (int r = wave; r < R; r += 4) {
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
