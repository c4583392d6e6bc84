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

// One wave pools block gb of the 2*BH*n (tensor, head, block) triples.
template <int D, int BLK, bool NT>
__device__ __forceinline__ void pool_block(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                           float* __restrict__ aq, float* __restrict__ ak, int N, int n,
                                           int BH, float scale, int gb) {
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RG = 64 / CPR;      // row groups per wave
  constexpr int RPL = BLK / RG;     // rows per lane
  static_assert(BLK % RG == 0, "block must be a multiple of the row groups");

  const int per_tensor = BH * n;
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
    // inputs larger than the last-level cache are streamed with nontemporal
    // loads (measured: 7.1 against 6.0 TB/s for plain loads); smaller ones
    // are read with plain loads, which leave them cached for the next call
    const u32x4* src = reinterpret_cast<const u32x4*>(X + (size_t)row * D + c * 8);
    data[j] = row < rows ? (NT ? __builtin_nontemporal_load(src) : *src) : u32x4{0u, 0u, 0u, 0u};
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

  // stored: aq = [scale * mean, scale^2 / 2 * var], ak = [mean, var]; the
  // third segment of each augmented vector follows from these two and is
  // formed by the score kernel
  if (rg == 0) {
    float* out = (tensor == 0 ? aq : ak) + ((size_t)bh * n + I) * (2 * D) + c * 8;
    f32x4 seg[2][2];
    const float hs2 = 0.5f * scale * scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float var = s[e] * inv_rows;
      seg[0][e / 4][e % 4] = tensor == 0 ? scale * mean[e] : mean[e];
      seg[1][e / 4][e % 4] = tensor == 0 ? hs2 * var : var;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      reinterpret_cast<f32x4*>(out + g * D)[0] = seg[g][0];
      reinterpret_cast<f32x4*>(out + g * D)[1] = seg[g][1];
    }
  }
}

template <int D, int BLK, bool NT>
__global__ __launch_bounds__(256) void pool_stats_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         float* __restrict__ aq,
                                                         float* __restrict__ ak, int N, int n,
                                                         int BH, float scale) {
  const int gb = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gb >= 2 * BH * n) return;
  pool_block<D, BLK, NT>(q, k, aq, ak, N, n, BH, scale, gb);
}

// ---------------------------------------------------------------------------
// Compact score and norm sort.  One workgroup of 16 waves per (b*h, R
// consecutive query-block rows), R in {16, 32, 64} chosen by the host: every
// workgroup reads its head's ak once, so larger R means fewer re-reads of ak,
// and two workgroups resident on a compute unit overlap one's selections with
// the other's products.
//
// S = aq . ak^T is a small fp32 GEMM (K = 3D) done with
// v_mfma_f32_16x16x4_f32 on 16x16 output tiles.  Wave w owns the column
// tiles w, w + 16, ... and every row tile of them, so the B operand (ak,
// streamed from L2 as float4 buffer loads per lane) is read once per
// workgroup and reused for the R/16 row tiles; the A operand (aq) is staged
// whole in LDS, its float4 slots XOR-swizzled by the row so that the 16 rows
// of a tile hit distinct banks.  Lane group g takes k = 16m + 4g + e for MFMA
// step (m, e) in both operands (a permutation of k, so the product is
// unchanged); every tile accumulates its K steps in the same order whatever
// R is, so S does not depend on R.  The accumulators then go to an LDS row
// buffer [R][n + 4] that reuses the A tile's memory; each wave selects the
// `keep` largest scores (ties to lower J) of its rows, several rows per
// search, by an MSB-first radix select over order-preserving uint32 keys and
// writes mask, ascending idx and cnt.
// ---------------------------------------------------------------------------
constexpr int kMaxScoreBlocks = 2048;  // longest row
constexpr int kScoreWaves = 16;
constexpr int kScoreLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup

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

// Selects the `keep` largest keys (ties: lower J) of each of P rows, row p
// held as key[p][i] for J = lane + 64*i with key 0 in the slots J >= n;
// writes mask bytes, ascending idx and the count of every row with
// live[p].  All control state is wave-uniform (scalar registers) and
// per-bit counts come from ballots.  The P searches advance together, one
// bit per pass with no branch per row, so their dependency chains overlap.
template <int NI, int P>
__device__ __forceinline__ void radix_select_rows(const uint32_t (&key)[P][NI], const bool (&live)[P], int n,
                                                  int keep, uint8_t* const (&mask_row)[P],
                                                  int32_t* const (&idx_row)[P], int32_t* const (&cnt_out)[P]) {
  const int lane = __lane_id();
  uint64_t vmask[NI];  // lanes holding a valid J in slot i
#pragma unroll
  for (int i = 0; i < NI; ++i) vmask[i] = __builtin_amdgcn_ballot_w64(lane + 64 * i < n);
  // Invariant per row: the candidates are the keys whose bits above `bit`
  // equal `prefix`; `remaining` of them are still to be taken (1 <=
  // remaining <= cand).  Every key above the candidate range is taken.
  // Bits above the highest bit where the row's largest and smallest key
  // differ are shared by every key and need no search.
  uint32_t prefix[P];
  int remaining[P], bit[P], cand[P];
  bool act[P];
  bool any = false;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    uint32_t kmax = 0u, kmin = ~0u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (lane + 64 * i < n) {
        kmax = key[p][i] > kmax ? key[p][i] : kmax;
        kmin = key[p][i] < kmin ? key[p][i] : kmin;
      }
    }
    kmax = __builtin_amdgcn_readfirstlane(wave_minmax_u32<true>(kmax));
    kmin = __builtin_amdgcn_readfirstlane(wave_minmax_u32<false>(kmin));
    const uint32_t diff = kmax ^ kmin;
    const int top = diff != 0u ? 31 - __builtin_clz(diff) : -1;
    bit[p] = top;
    prefix[p] = top < 0 ? kmax : kmax & ~((top == 31) ? ~0u : ((2u << top) - 1u));
    remaining[p] = keep;
    cand[p] = n;
    act[p] = top >= 0;
    any = any || act[p];
  }
  while (any) {
    any = false;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int b = act[p] ? bit[p] : 0;
      const uint32_t hi_mask = ~0u << b;
      const uint32_t want = prefix[p] | (1u << b);
      // keys of invalid slots are 0, which never equals `want` (bit b is set)
      int c1 = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        c1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64((key[p][i] & hi_mask) == want));
      const bool take = c1 >= remaining[p];
      const uint32_t np = take ? want : prefix[p];
      const int nc = take ? c1 : cand[p] - c1;
      const int nr = take ? remaining[p] : remaining[p] - c1;
      const bool fin = nc == nr;  // every candidate is taken: stop at this bit
      prefix[p] = act[p] ? np : prefix[p];
      cand[p] = act[p] ? nc : cand[p];
      remaining[p] = act[p] ? nr : remaining[p];
      bit[p] = act[p] && !fin ? bit[p] - 1 : bit[p];
      act[p] = act[p] && !fin && bit[p] >= 0;
      any = any || act[p];
    }
  }
  // bit >= 0 (early exit): take every key whose bits >= bit are >= prefix's.
  // bit < 0: keys > prefix, plus the `remaining` lowest-J keys == prefix.
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (!live[p]) continue;
    const uint32_t cmp_mask = bit[p] >= 0 ? (~0u << bit[p]) : ~0u;
    const uint32_t pre = prefix[p] & cmp_mask;
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int J = lane + 64 * i;
      const bool valid = J < n;
      const uint32_t kk = key[p][i] & cmp_mask;
      uint64_t km;
      if (bit[p] >= 0) {
        km = __builtin_amdgcn_ballot_w64(kk >= pre) & vmask[i];
      } else {
        const uint64_t eqm = __builtin_amdgcn_ballot_w64(kk == pre) & vmask[i];
        const uint64_t gtm = __builtin_amdgcn_ballot_w64(kk > pre) & vmask[i];
        // the lowest-J equal keys are taken until `remaining` is used up
        uint64_t take = 0;
        int need = remaining[p] - eq_seen;
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
      if (kept && pos < keep) idx_row[p][pos] = J;  // exactly `keep` are kept; the bound is defensive
      base += __builtin_popcountll(km);
      if (valid) mask_row[p][J] = kept ? 1 : 0;
    }
    if (lane == 0) *cnt_out[p] = base;
  }
}

// LDS bytes of one score workgroup: the A tile as three bf16 planes
// [3][R][3D] while the products run, then, in the same memory, the score
// rows [R][n + 4] (fp32).
__host__ __device__ constexpr int score_lds_bytes(int D, int R, int n) {
  return 3 * R * 3 * D * 2 > R * (n + 4) * 4 ? 3 * R * 3 * D * 2 : R * (n + 4) * 4;
}

// An fp32 value as the sum of three bf16, h + m + l: h rounds x, m rounds
// the remainder x - h, l the remainder after m.  Each remainder is exact in
// fp32, so the three carry x's 24 significant bits.
__device__ __forceinline__ void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
  h = (__bf16)x;
  const float r1 = x - (float)h;
  m = (__bf16)r1;
  l = (__bf16)(r1 - (float)m);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// eight values, lo then hi
__device__ __forceinline__ void split3(const f32x4 lo, const f32x4 hi, bf16x8& h, bf16x8& m, bf16x8& l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 a, b, c;
    split3(e < 4 ? lo[e] : hi[e - 4], a, b, c);
    h[e] = a;
    m[e] = b;
    l[e] = c;
  }
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3): loads past
// the end return zero, which stands for the rows and columns beyond n.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t score_rsrc(const float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 load_f32x4(__amdgpu_buffer_rsrc_t rs, int byte_offset) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_offset, 0, 0));
}

// Rows R0 .. R0+R-1 of head bh, by a workgroup of W waves whose LDS starts at lds.
//
// S = A . B^T over the augmented 3D-vectors A = [aq0, aq1, aq0^2 / 2] and
// B = [ak0, ak1 + ak0^2, ak1], from the two stored segments of aq and ak.  It
// is formed on the bf16 matrix cores: each fp32 operand is the sum of three
// bf16 (split3), and the six products of pieces down to 2^-24 relative are
// summed into fp32 accumulators (l.h, m.m, m.h, h.l, h.m, h.h: the two
// smallest first, the largest last) -- the accuracy of an fp32 product at
// 6/16 of its matrix-core time.  The whole A tile is formed and
// split once into three bf16 planes in LDS, with every load in flight before
// the first write.  B streams through registers in 32-wide blocks of d: a
// block's two stored segments give all three of its augmented segments,
// each split as it is used, and each stored segment's registers take the
// next block's loads as soon as its last use is split.  Buffer loads return
// zero past row/column n, so no load is predicated and the compiler can wait
// for each one by count instead of for all of them.
template <int D, int NI, int R, int W>
__device__ __forceinline__ void score_tile(const float* __restrict__ aq, const float* __restrict__ ak, int n,
                                           int keep, uint8_t* __restrict__ mask, int32_t* __restrict__ idx,
                                           int32_t* __restrict__ cnt, float* __restrict__ score, int bh, int R0,
                                           float* lds) {
  constexpr int K2 = 2 * D;           // stored values per row
  constexpr int K3 = 3 * D;           // augmented values per row
  constexpr int F4 = K2 / 4;          // float4 slots per stored A row
  constexpr int F8 = K3 / 8;          // 16-byte slots per A row and plane (bf16)
  constexpr int SWZ = F8 % 16 == 0 ? 15 : 7;  // slot swizzle within aligned groups of SWZ + 1 slots
  static_assert(F8 % (SWZ + 1) == 0, "swizzle must stay inside the row");
  constexpr int DB = D / 32;          // 32-wide blocks of d: eight values per lane and segment
  constexpr int RT = R / 16;          // row tiles
  constexpr int CTW = (4 * NI + W - 1) / W;  // column tiles per wave (4*NI tiles cover 64*NI columns)
  constexpr int STEPS = CTW * DB;
  constexpr int T = W * 64;
  constexpr int AL = (R * F4 + T - 1) / T;  // A float4 loads per thread
  constexpr int PLANE = R * K3;             // bf16 elements per plane
  static_assert(RT * CTW <= 8, "accumulators of a wave");
  __bf16* const Abuf = reinterpret_cast<__bf16*>(lds);  // [3][R][K3]; slot j of row r at j ^ (r & SWZ)
  float* const Sbuf = lds;  // [R][SP], once every wave is done with Abuf
  const int SP = n + 4;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int ctiles = (n + 15) / 16;
  const int rows_here = min(R, n - R0);
  const auto a_rs = score_rsrc(aq + ((size_t)bh * n + R0) * K2, rows_here * K2 * 4);
  const auto b_rs = score_rsrc(ak + (size_t)bh * n * K2, n * K2 * 4);
  // step s = (column tile t of this wave, d block m); lane (li, lg) takes
  // d = 32m + 8lg + e for element e, in both operands and every segment
  auto b_offset = [&](int s) {
    const int t = s / DB, m = s - t * DB;
    return (((wave + W * t) * 16 + li) * K2 + 32 * m + 8 * lg) * 4;
  };
  // the eight values of stored segment g (ak0 or ak1) for step s
  auto load_b = [&](int s, int g, f32x4 (&dst)[2]) {
    const int o = b_offset(s) + g * 4 * D;
    dst[0] = load_f32x4(b_rs, o);
    dst[1] = load_f32x4(b_rs, o + 16);
  };
  // three bf16 planes of the augmented value v at augmented index k of row
  auto put_a = [&](int row, int k, const f32x4 v) {
    const int off = row * K3 + 8 * ((k >> 3) ^ (row & SWZ)) + (k & 7);
    bf16x4 h, m, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __bf16 a, b, c;
      split3(v[q], a, b, c);
      h[q] = a;
      m[q] = b;
      l[q] = c;
    }
    *reinterpret_cast<bf16x4*>(Abuf + off) = h;
    *reinterpret_cast<bf16x4*>(Abuf + PLANE + off) = m;
    *reinterpret_cast<bf16x4*>(Abuf + 2 * PLANE + off) = l;
  };

  f32x4 av[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) av[i] = load_f32x4(a_rs, (threadIdx.x + i * T) * 16);
  f32x4 x0[2], x1[2];  // ak0 and ak1 of the current block
  load_b(0, 0, x0);
  load_b(0, 1, x1);
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int e = threadIdx.x + i * T;
    if ((R * F4) % T == 0 || e < R * F4) {
      const int row = e / F4, k = 4 * (e - row * F4);  // stored values k .. k+3 of the row
      put_a(row, k, av[i]);                            // aq0 or aq1 at the same index
      if (k < D) put_a(row, 2 * D + k, av[i] * av[i] * 0.5f);  // aq0^2 / 2
    }
  }
  __syncthreads();

  f32x4 acc[CTW][RT];
#pragma unroll
  for (int t = 0; t < CTW; ++t)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the six piece products of augmented segment g of this block (l.h, m.m,
  // m.h, h.l, h.m, h.h), each A plane read just before its products; row
  // tiles innermost, so that consecutive MFMAs of a wave use different
  // accumulators
  auto products = [&](int t, int m, int g, const bf16x8& bh, const bf16x8& bm, const bf16x8& bl) {
    const int slot = g * (D / 8) + 4 * m + lg;
    auto plane = [&](int p, int r) {
      const int row = r * 16 + li;
      return *reinterpret_cast<const bf16x8*>(Abuf + p * PLANE + row * K3 + 8 * (slot ^ (row & SWZ)));
    };
    bf16x8 a[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) a[r] = plane(2, r);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bh, acc[t][r], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < RT; ++r) a[r] = plane(1, r);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bm, acc[t][r], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bh, acc[t][r], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < RT; ++r) a[r] = plane(0, r);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bl, acc[t][r], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bm, acc[t][r], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bh, acc[t][r], 0, 0, 0);
  };
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int t = s / DB, m = s - t * DB;
    const bool on = wave + W * t < ctiles;
    bf16x8 bh, bm, bl;
    // segment 0: ak0
    split3(x0[0], x0[1], bh, bm, bl);
    if (on) products(t, m, 0, bh, bm, bl);
    // segment 1: ak1 + ak0^2, formed in ak0's registers, which then take the
    // next block's ak0
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int q = 0; q < 4; ++q) x0[h2][q] = __builtin_fmaf(x0[h2][q], x0[h2][q], x1[h2][q]);
    split3(x0[0], x0[1], bh, bm, bl);
    if (s + 1 < STEPS) load_b(s + 1, 0, x0);
    if (on) products(t, m, 1, bh, bm, bl);
    // segment 2: ak1, whose registers then take the next block's ak1
    split3(x1[0], x1[1], bh, bm, bl);
    if (s + 1 < STEPS) load_b(s + 1, 1, x1);
    if (on) products(t, m, 2, bh, bm, bl);
  }
  __syncthreads();  // the score rows overwrite the A tile
  // lane holds column ct*16 + li of rows r*16 + 4*lg + {0..3}
#pragma unroll
  for (int t = 0; t < CTW; ++t) {
    const int ct = wave + W * t;
    const int col = ct * 16 + li;
    if (ct < ctiles && col < n) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) Sbuf[(r * 16 + 4 * lg + q) * SP + col] = acc[t][r][q];
    }
  }
  __syncthreads();
  if (score != nullptr) {  // the score map as the selection saw it, row by row
    for (int e = threadIdx.x; e < R * n; e += W * 64) {
      const int row = e / n, col = e - row * n;
      if (R0 + row < n) score[((size_t)bh * n + R0 + row) * n + col] = Sbuf[row * SP + col];
    }
  }

  // wave w selects rows w, w + W, ...: RP of them at a time
  constexpr int RW = (R + W - 1) / W;
  constexpr int RP = NI <= 8 ? (RW < 4 ? RW : 4) : 1;
  for (int r0 = wave; r0 < R; r0 += W * RP) {
    if (R0 + r0 >= n) break;
    uint32_t key[RP][NI];
    bool live[RP];
    uint8_t* mrow[RP];
    int32_t* irow[RP];
    int32_t* crow[RP];
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      const int r = min(r0 + W * p, R - 1);
      const int I = R0 + r;
      live[p] = r0 + W * p < R && I < n;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int J = lane + 64 * i;
        const uint32_t k = float_order_key(Sbuf[r * SP + min(J, n - 1)]);
        key[p][i] = J < n ? k : 0u;
      }
      const size_t row = (size_t)bh * n + min(I, n - 1);
      mrow[p] = mask + row * n;
      irow[p] = idx + row * keep;
      crow[p] = cnt + row;
    }
    radix_select_rows<NI, RP>(key, live, n, keep, mrow, irow, crow);
  }
}

template <int D, int NI, int R>
__global__ __launch_bounds__(kScoreWaves * 64) void score_topk_kernel(const float* __restrict__ aq,
                                                         const float* __restrict__ ak, int n,
                                                         int keep, uint8_t* __restrict__ mask,
                                                         int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ cnt,
                                                         float* __restrict__ score, int total) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  // the row tiles of one head run on one XCD and share its L2 copy of ak
  const int logical = xcd_remap(blockIdx.x, total);
  if (logical < 0) return;
  const int tiles = (n + R - 1) / R;
  const int bh = logical / tiles;
  score_tile<D, NI, R, kScoreWaves>(aq, ak, n, keep, mask, idx, cnt, score, bh, (logical - bh * tiles) * R, lds);
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
