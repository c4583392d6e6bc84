// Selection-quality diagnostics for gfx950: how well the pre-downsampled
// block scores rank key blocks against the exact post-downsample map.
//
// The pith.science review of "Efficient Long-Context Modeling in Diffusion
// Language Models via Block Approximate Sparse Attention" states ("Core
// claim", abstract) that the diagonal-variance correction stands in for the
// full covariance and that the pre-downsampled scores stand in for the
// post-downsample attention map; its referee report notes that neither
// approximation is quantified.  These kernels compute, on the device:
//
//  * block_map_kernel -- the exact post-downsample maps of every (b, h):
//      M_lme[I,J]  = ln( mean_{s in I, t in J} e^{x_st} ),
//      M_prob[I,J] = mean_{s in I, t in J} e^{x_st - LSE_s},
//    x = scale <q_s, k_t>, LSE_s the row's log-normaliser over all keys.
//  * moments_kernel + gemm_nt_f32_kernel + sum_parts_kernel -- the
//    second-cumulant score with FULL block covariances,
//      S_full[I,J] = scale <qm,km> + scale^2/2 (<Cq,Ck>_F + km'Cq km + qm'Ck qm),
//    and the uncorrected score S_mean = scale <qm, km>.
//  * rank_agree_kernel -- per row of two maps: block recall of the kept
//    sets (norm-sort rule: value descending, lower index first) and
//    Spearman's rho of tie-averaged ranks.
#pragma once

#include "attention.hpp"

namespace ba {

// 32-lane reductions: lanes l and l^32 hold the same query in the S^T
// layout, so a reduction over one 32-lane half covers a wave's 32 queries.
// DPP xor-1 / xor-2 in quads, rotations by 4 and 8 in rows of 16, then
// v_permlane16_swap across the two rows of the half.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <bool MAX>
__device__ __forceinline__ float half_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_f32<0xB1>(x));   // quad_perm 1,0,3,2
  x = op(x, dpp_f32<0x4E>(x));   // quad_perm 2,3,0,1
  x = op(x, dpp_f32<0x124>(x));  // row_ror 4
  x = op(x, dpp_f32<0x128>(x));  // row_ror 8
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// Exact post-downsample maps.  One workgroup per query block I of one (b, h)
// (32*WAVES = BLK rows, one wave per 32 queries) walks every 64-key chunk:
// S^T = K Q^T as in the attention kernel (K copied to LDS by direct-to-LDS
// loads, Q^T in registers).  Per lane (one query s) and key block J the
// kernel keeps lse2_sJ = log2 sum_{t in J} 2^{x_st log2 e}; at the end of J
// it reduces over the wave's valid queries
//   M = max_s lse2_sJ,  Z = sum_s 2^{lse2_sJ - M},  P = sum_s 2^{lse2_sJ - LSE2_s}
// and parks (M, Z, P) per wave in LDS; after the walk the waves' parts are
// combined per J and both maps are written as coalesced rows.
// ---------------------------------------------------------------------------
struct MapParams {
  const uint16_t* q;
  const uint16_t* k;
  const float* lse;  // natural-log row LSE over all keys [BH, N], or null
  float* m_lme;      // [BH, n, n]
  float* m_prob;     // [BH, n, n], written only with lse
  int N;
  int n_blocks;
  int total;         // BH * n_blocks
  float scale_log2;
};

template <int D, int WAVES, int BLK>
__global__ __launch_bounds__(WAVES * 64, 2) void block_map_kernel(MapParams p) {
  constexpr int KSTEPS = D / 16;
  constexpr int CPR = D / 8;
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kChunk * ROW_BYTES;
  constexpr int DMA = (kChunk * CPR) / (64 * WAVES);
  constexpr int SUBS = BLK / kChunk;  // chunks per key block
  static_assert(WAVES * 32 == BLK, "one wave per 32 queries of the block");
  static_assert((kChunk * CPR) % (64 * WAVES) == 0, "tile must split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) uint8_t Ktile[TILE_BYTES];
  extern __shared__ float parts[];  // [n_blocks][WAVES][3]

  const int logical = xcd_remap(blockIdx.x, p.total);
  if (logical < 0) return;
  const int n = p.n_blocks;
  const int bh = logical / n;
  const int I = logical - bh * n;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;
  const int lq = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = p.q + head;
  const uint16_t* Kh = p.k + head;
  const float sl2 = p.scale_log2;

  uint32_t voff[DMA];
#pragma unroll
  for (int j = 0; j < DMA; ++j) {
    const int slot = (j * WAVES + wave) * 64 + lane;
    const int r = slot / CPR, s = slot % CPR;
    voff[j] = r * ROW_BYTES + k_slot<CPR>(r, s) * 16;
  }
  auto k_rsrc = [&](int k0) {
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kChunk, N - k0)));
    return make_rsrc(Kh + (size_t)k0 * D, rows * ROW_BYTES);
  };

  const int qrow = I * BLK + wave * 32 + lq;
  const bool qvalid = qrow < N;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qvalid) w = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }
  const bool with_prob = p.lse != nullptr;
  const float lse2_row = (with_prob && qvalid) ? p.lse[(size_t)bh * N + qrow] * 1.44269504088896340736f : 0.f;

  auto read_k = [&](int kt, int ks) -> bf16x8 {
    const int r = kt * 32 + lq;
    return *reinterpret_cast<const bf16x8*>(Ktile + r * ROW_BYTES + k_slot<CPR>(r, ks * 2 + g) * 16);
  };

  const int n_chunks = (N + kChunk - 1) / kChunk;
  dma_tile<DMA, WAVES>(k_rsrc(0), Ktile, wave, voff);
  float mJ = -__builtin_inff(), zJ = 0.f;  // running log2-sum-exp of this lane's query over block J
  for (int c = 0; c < n_chunks; ++c) {
    const int k0 = c * kChunk;
    const int valid = min(kChunk, N - k0);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K(c) landed
    __syncthreads();
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_k(0, ks), qf[ks], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_k(1, ks), qf[ks], sacc[1], 0, 0, 0);
    }
    __syncthreads();  // every wave has read K(c)
    if (c + 1 < n_chunks) dma_tile<DMA, WAVES>(k_rsrc(k0 + kChunk), Ktile, wave, voff);

    if (valid < kChunk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= valid) sacc[kt][r] = -__builtin_inff();
        }
    }
    float ma = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
    float mb = fmaxf(fmaxf(sacc[1][0], sacc[1][1]), sacc[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = fmaxf(fmaxf(ma, sacc[0][r]), sacc[0][r + 1]);
      mb = fmaxf(fmaxf(mb, sacc[1][r]), sacc[1][r + 1]);
    }
    const float mc = pair_max(fmaxf(fmaxf(ma, sacc[0][15]), fmaxf(mb, sacc[1][15]))) * sl2;  // finite: valid >= 1
    float zc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) zc += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], sl2, -mc));
    zc = pair_sum(zc);
    // fold this chunk into the running sum of its key block
    const float m_new = fmaxf(mJ, mc);
    zJ = zJ * __builtin_amdgcn_exp2f(mJ - m_new) + zc * __builtin_amdgcn_exp2f(mc - m_new);
    mJ = m_new;

    if (c % SUBS == SUBS - 1 || c + 1 == n_chunks) {
      const int J = c / SUBS;
      const float l2 = mJ + __builtin_amdgcn_logf(zJ);  // log2 sum over the block's keys
      const float v = qvalid ? l2 : -__builtin_inff();
      const float M = half_reduce<true>(v);
      const float Z = M == -__builtin_inff() ? 0.f : half_reduce<false>(__builtin_amdgcn_exp2f(v - M));
      const float P = half_reduce<false>(qvalid && with_prob ? __builtin_amdgcn_exp2f(l2 - lse2_row) : 0.f);
      if (lane == 0) {
        float* dst = parts + (J * WAVES + wave) * 3;
        dst[0] = M;
        dst[1] = Z;
        dst[2] = P;
      }
      mJ = -__builtin_inff();
      zJ = 0.f;
    }
  }
  __syncthreads();

  // combine the waves' parts: row I of both maps
  const int nI = min(BLK, N - I * BLK);
  const size_t row = ((size_t)bh * n + I) * n;
  for (int J = threadIdx.x; J < n; J += WAVES * 64) {
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, parts[(J * WAVES + w) * 3]);
    float Z = 0.f, P = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float* src = parts + (J * WAVES + w) * 3;
      if (src[0] != -__builtin_inff()) Z += src[1] * __builtin_amdgcn_exp2f(src[0] - M);
      P += src[2];
    }
    const int nJ = min(BLK, N - J * BLK);
    const float cnt = (float)nI * (float)nJ;
    p.m_lme[row + J] = (M + __builtin_amdgcn_logf(Z)) * 0.69314718055994530942f - logf(cnt);
    if (with_prob) p.m_prob[row + J] = P / cnt;
  }
}

// ---------------------------------------------------------------------------
// Block moments.  One workgroup (4 waves) per (tensor, b*h, block): the
// block's tokens X [<= BLK, D] bf16 are copied to LDS (rows past N read as
// zero) and M = X^T X is formed with v_mfma_f32_32x32x16_bf16; both operands
// come from the same row-major tile through transposing reads, since the A
// operand of X^T and the B operand of X share one register layout.  With
// the channel means m and T = D(D+1)/2 upper-triangle entries (i <= j,
// row-major), the rows of the augmented operands are written directly:
//   query side: [ scale*m | s2*w_ij*(M_ij/|I| - m_i m_j) | s2*w_ij*m_i m_j ]
//   key side:   [ m       | M_ij/|J|                     | M_ij/|J| - m_i m_j ]
// with s2 = scale^2/2 and w_ij = 1 on the diagonal, 2 off it, so that one
// dot product over D + 2T entries is
//   scale<qm,km> + s2*(<Cq, Ck + km km'> + <qm qm', Ck>) = S_full.
// ---------------------------------------------------------------------------
template <int D>
constexpr int kFullWidth = D + D * (D + 1);  // D + 2T

// Transposing read of channel tile `dt` of a row-major [tokens, D] LDS tile
// (V-tile swizzle): lane l receives X[t][dt*32 + l%32] for the tokens
// t = 16*step + {4g..4g+3, 8+4g..8+4g+3}, g = l/32 -- the A layout of X^T
// and, equally, the B layout of X for v_mfma_f32_32x32x16_bf16.
template <int D>
__device__ __forceinline__ bf16x8 read_tile_t(const uint8_t* X, int lane, int step, int dt) {
  constexpr int CPR = D / 8;
  constexpr int ROW_BYTES = D * 2;
  const int grp = lane >> 4, li = lane & 15;
  const int dd = dt * 32 + 16 * (grp & 1) + 4 * (li & 3);
  const int r0 = step * 16 + 4 * (grp >> 1) + (li >> 2), r1 = r0 + 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (BA_LDS i16x4*)(X + r0 * ROW_BYTES + v_slot<CPR>(r0, dd >> 3) * 16 + (dd & 7) * 2));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (BA_LDS i16x4*)(X + r1 * ROW_BYTES + v_slot<CPR>(r1, dd >> 3) * 16 + (dd & 7) * 2));
  const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, a8);
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void moments_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ k,
                                                      float* __restrict__ aqf, float* __restrict__ akf,
                                                      int N, int n, int BH, float scale) {
  constexpr int WAVES = 4;
  constexpr int CPR = D / 8;
  constexpr int ROW_BYTES = D * 2;
  constexpr int DMA = (BLK * CPR) / (64 * WAVES);
  constexpr int DT = D / 32;          // 32-wide channel tiles
  constexpr int TPW = DT * DT / WAVES;  // output tiles per wave
  constexpr int T = D * (D + 1) / 2;
  constexpr int KF = kFullWidth<D>;
  static_assert((BLK * CPR) % (64 * WAVES) == 0, "tile must split evenly over the waves");
  static_assert((DT * DT) % WAVES == 0, "tiles must split evenly over the waves");

  __shared__ __attribute__((aligned(1024))) uint8_t X[BLK * ROW_BYTES];
  __shared__ float mean[D];

  const int item = blockIdx.x;  // (tensor, bh, block)
  const int tensor = item / (BH * n);
  const int rem = item - tensor * BH * n;
  const int bh = rem / n;
  const int blk = rem - bh * n;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* src = (tensor == 0 ? q : k) + ((size_t)bh * N + (size_t)blk * BLK) * D;
  const int rows = __builtin_amdgcn_readfirstlane(min(BLK, N - blk * BLK));
  uint32_t voff[DMA];
#pragma unroll
  for (int j = 0; j < DMA; ++j) {
    const int slot = (j * WAVES + wave) * 64 + lane;
    const int r = slot / CPR, s = slot % CPR;
    voff[j] = r * ROW_BYTES + v_slot<CPR>(r, s) * 16;
  }
  // (through dma_tile: the buffer-to-LDS builtin called from a kernel
  // template's body makes the host pass drop the kernel's launch stub)
  dma_tile<DMA, WAVES>(make_rsrc(src, rows * ROW_BYTES), X, wave, voff);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // channel means (zero rows past N add nothing)
  const float inv = 1.0f / (float)rows;
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float acc = 0.f;
    for (int r = 0; r < BLK; ++r) {
      const uint16_t bits = *reinterpret_cast<const uint16_t*>(X + r * ROW_BYTES + v_slot<CPR>(r, d >> 3) * 16 + (d & 7) * 2);
      acc += __uint_as_float((uint32_t)bits << 16);
    }
    mean[d] = acc * inv;
  }

  f32x16 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x16{};
#pragma unroll
  for (int step = 0; step < BLK / 16; ++step) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tile = wave * TPW + t;
      const int ti = tile / DT, tj = tile % DT;
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tile_t<D>(X, lane, step, ti),
                                                       read_tile_t<D>(X, lane, step, tj), acc[t], 0, 0, 0);
    }
  }
  __syncthreads();  // means visible

  float* out = (tensor == 0 ? aqf : akf) + ((size_t)bh * n + blk) * KF;
  const float s2 = 0.5f * scale * scale;
  if (threadIdx.x < D) out[threadIdx.x] = tensor == 0 ? scale * mean[threadIdx.x] : mean[threadIdx.x];
  const int g = lane >> 5;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave * TPW + t;
    const int ti = tile / DT, tj = tile % DT;
    if (ti > tj) continue;  // upper-triangle tiles only (wave-uniform)
    const int j = tj * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ti * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (i > j) continue;
      const int pos = i * D - i * (i - 1) / 2 + (j - i);
      const float second = acc[t][r] * inv;  // M_ij / |block|
      const float outer = mean[i] * mean[j];
      if (tensor == 0) {
        const float w = i == j ? s2 : 2.f * s2;
        out[D + pos] = w * (second - outer);
        out[D + T + pos] = w * outer;
      } else {
        out[D + pos] = second;
        out[D + T + pos] = second - outer;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K product of the augmented rows: part p of
//   S[bh, I, J] = sum_k A[bh, I, k] * B[bh, J, k]
// over k in [k_lo(p), k_hi(p)), fp32 v_mfma_f32_32x32x2_f32.  A workgroup
// (4 waves) owns a 64 x 64 output tile, a wave one 32 x 32 quarter.  Lane
// (i, g) loads float4 A[I0+i][k0+4g .. +3] and B[J0+i][k0+4g .. +3]; MFMA e
// of the step pairs k0+e (g = 0) with k0+4+e (g = 1) in both operands, so
// the 4 MFMAs of a step sum k0 .. k0+7 exactly once.  Parts are written to
// their own slices and summed in a fixed order (deterministic).
// ---------------------------------------------------------------------------
struct GemmParams {
  const float* a;  // [BH, n, K]
  const float* b;  // [BH, n, K]
  float* parts;    // [P, BH, n, n]
  int n, K, BH, n_tiles;  // tiles per head side = ceil(n / 64)
  int k_first;            // part 0 covers [0, k_first)
  int k_chunk;            // parts 1.. cover k_chunk each (multiple of 8) from k_first
  int P;
};

__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tiles2 = p.n_tiles * p.n_tiles;
  int item = blockIdx.x;
  const int part = item / (p.BH * tiles2);
  item -= part * p.BH * tiles2;
  const int bh = item / tiles2;
  const int t = item - bh * tiles2;
  const int I0 = (t / p.n_tiles) * 64 + (wave >> 1) * 32;
  const int J0 = (t % p.n_tiles) * 64 + (wave & 1) * 32;
  const int k_lo = part == 0 ? 0 : p.k_first + (part - 1) * p.k_chunk;
  const int k_hi = part == 0 ? p.k_first : min(p.K, k_lo + p.k_chunk);
  const int i = lane & 31, g = lane >> 5;
  const int ra = I0 + i, rb = J0 + i;
  const float* A = p.a + ((size_t)bh * p.n + min(ra, p.n - 1)) * p.K + 4 * g;
  const float* B = p.b + ((size_t)bh * p.n + min(rb, p.n - 1)) * p.K + 4 * g;
  const bool va = ra < p.n, vb = rb < p.n;

  f32x16 acc = f32x16{};
  constexpr int U = 4;  // steps of 8 k in flight
  int k0 = k_lo;
  for (; k0 + 8 * U <= k_hi; k0 += 8 * U) {
    f32x4 av[U], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      av[u] = *reinterpret_cast<const f32x4*>(A + k0 + 8 * u);
      bv[u] = *reinterpret_cast<const f32x4*>(B + k0 + 8 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(va ? av[u][e] : 0.f, vb ? bv[u][e] : 0.f, acc, 0, 0, 0);
  }
  for (; k0 < k_hi; k0 += 8) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(A + k0);
    const f32x4 bv = *reinterpret_cast<const f32x4*>(B + k0);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(va ? av[e] : 0.f, vb ? bv[e] : 0.f, acc, 0, 0, 0);
  }
  // C layout: lane (j, g), register r -> row 8*(r/4) + 4g + r%4, column j
  const int j = J0 + (lane & 31);
  if (j >= p.n) return;
  float* out = p.parts + ((size_t)part * p.BH + bh) * p.n * p.n;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = I0 + 8 * (r >> 2) + 4 * g + (r & 3);
    if (row < p.n) out[(size_t)row * p.n + j] = acc[r];
  }
}

// full = sum of the P parts in order; mean (optional) = part 0
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ parts, int P, size_t count,
                                                        float* __restrict__ full, float* __restrict__ mean) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < count; e += (size_t)gridDim.x * 256) {
    float s = parts[e];
    if (mean != nullptr) mean[e] = s;
    for (int q = 1; q < P; ++q) s += parts[(size_t)q * count + e];
    full[e] = s;
  }
}

// ---------------------------------------------------------------------------
// Rank agreement of two maps, one wave per row (four rows per workgroup).
// For entry i of a row (lane i%64, slot i/64): less/equal counts over the
// row give the doubled tie-averaged rank 2*rank = 2*less + equal + 1, and
// the norm-sort position #{x_j > x_i} + #{j < i : x_j = x_i} decides
// membership of the kept set (position < keep).  Centred doubled ranks are
// integers, so the sums of Spearman's rho are exact (int64) and only the
// final ratio rounds; recall = |kept(x) & kept(r)| / keep.
// ---------------------------------------------------------------------------
constexpr int kAgreeMaxN = 512;

template <int NE>
__global__ __launch_bounds__(256) void rank_agree_kernel(const float* __restrict__ x, const float* __restrict__ r,
                                                         int rows, int n, int keep, float* __restrict__ recall,
                                                         float* __restrict__ rho) {
  __shared__ float xs[4][kAgreeMaxN];
  __shared__ float rs[4][kAgreeMaxN];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= rows) return;  // wave-uniform; no barrier below
  const float* xr = x + (size_t)row * n;
  const float* rr = r + (size_t)row * n;
  for (int i = lane; i < n; i += 64) {
    xs[w][i] = xr[i];
    rs[w][i] = rr[i];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();

  float xv[NE], rv[NE];
  int lx[NE], ex[NE], px[NE], lr[NE], er[NE], pr[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int i = lane + 64 * e;
    xv[e] = i < n ? xs[w][i] : 0.f;
    rv[e] = i < n ? rs[w][i] : 0.f;
    lx[e] = ex[e] = px[e] = lr[e] = er[e] = pr[e] = 0;
  }
  for (int jj = 0; jj < n; ++jj) {
    const float xj = xs[w][jj], rj = rs[w][jj];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int i = lane + 64 * e;
      lx[e] += xj < xv[e];
      ex[e] += xj == xv[e];
      px[e] += (xj > xv[e]) | ((xj == xv[e]) & (jj < i));
      lr[e] += rj < rv[e];
      er[e] += rj == rv[e];
      pr[e] += (rj > rv[e]) | ((rj == rv[e]) & (jj < i));
    }
  }
  long long sab = 0, saa = 0, sbb = 0;
  int both = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int i = lane + 64 * e;
    if (i >= n) continue;
    const long long a = 2 * lx[e] + ex[e] + 1 - (n + 1);  // centred doubled ranks
    const long long b = 2 * lr[e] + er[e] + 1 - (n + 1);
    sab += a * b;
    saa += a * a;
    sbb += b * b;
    both += (px[e] < keep) & (pr[e] < keep);
  }
  for (int m = 32; m >= 1; m >>= 1) {
    sab += __shfl_xor(sab, m, 64);
    saa += __shfl_xor(saa, m, 64);
    sbb += __shfl_xor(sbb, m, 64);
    both += __shfl_xor(both, m, 64);
  }
  if (lane == 0) {
    const double den = sqrt((double)saa * (double)sbb);
    rho[row] = den > 0.0 ? (float)((double)sab / den) : 0.f;
    recall[row] = (float)((double)both / (double)keep);
  }
}

}  // namespace ba
