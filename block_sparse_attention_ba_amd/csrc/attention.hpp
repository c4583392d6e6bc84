// Block-sparse and dense flash-attention forward for gfx950 (bf16 MFMA).
//
// Operation (pith.science review of "Efficient Long-Context Modeling in
// Diffusion Language Models via Block Approximate Sparse Attention", "The
// pith"): exact softmax attention of every query restricted to the tokens of
// its kept key blocks; the dense variant keeps every block and is the
// comparator of the review's "If this is right" speedup claim.
//
// Design (per workgroup: one tile of 32*WAVES query rows of one (b, h)):
//  * Each wave owns 32 query rows.  Scores are formed TRANSPOSED,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 d from LDS,
//    B = Q^T from registers (Q is loaded once).  In the 32x32 accumulator
//    layout lane l then holds column l%32 -- a single query -- so the
//    running max/sum of a query live in one lane pair (l, l^32) and need one
//    cross-lane exchange per key chunk.
//  * The output is accumulated transposed too, O^T = V^T P^T: B = P^T comes
//    straight from the score registers (fp32 -> bf16), A = V^T is read from a
//    transposed V tile in LDS.  Every O register of a lane belongs to that
//    lane's query, so the online-softmax rescale is lane-local.
//  * Keys are processed in chunks of 64 (one block of 64, or half a block of
//    128).  K (row-major, padded) and V^T (padded) are staged through LDS;
//    the next chunk's global loads are in flight while the current chunk is
//    computed.
//  * The sparse variant walks the compacted block-index list of its query
//    block; the dense variant walks all keys.  Keys >= N are masked to -inf.
//  * Softmax runs in the log2 domain in fp32: p = exp2(s*scale*log2(e) - m).
#pragma once

#include "common.hpp"

namespace ba {

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;  // sparse: [BH, n, max_keep]
  const int32_t* cnt;  // sparse: [BH, n]
  void* o;
  float* lse;
  int N;
  int n_blocks;   // key blocks (sparse) -- also the number of query blocks
  int n_qtiles;   // query tiles per head
  int total;      // BH * n_qtiles
  int max_keep;
  float scale_log2;  // softmax scale * log2(e)
};

constexpr int kChunk = 64;  // keys per LDS chunk

template <int D>
struct AttnSmem {
  static constexpr int KP = D + 8;        // K row pitch (bf16 elements)
  static constexpr int VP = kChunk + 4;   // V^T row pitch (bf16 elements)
  static constexpr int K_ELEMS = kChunk * KP;
  static constexpr int V_ELEMS = D * VP;
  static constexpr int BYTES = (K_ELEMS + V_ELEMS) * 2;
};

template <int D, int WAVES, int BLK, bool SPARSE, bool OUT_F32>
__global__ __launch_bounds__(WAVES * 64) void attn_fwd_kernel(AttnParams p) {
  constexpr int NT = WAVES * 64;
  constexpr int ROWS = WAVES * 32;
  constexpr int KSTEPS = D / 16;          // MFMA k-steps of the score product
  constexpr int DT = D / 32;              // 32-wide d tiles of the output
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int K_LOADS = (kChunk * CPR + NT - 1) / NT;
  constexpr int V_ITEMS_TOTAL = (kChunk / 4) * CPR;  // items of 4 keys x 8 d
  constexpr int V_ITEMS = (V_ITEMS_TOTAL + NT - 1) / NT;
  constexpr int SUBS = SPARSE ? BLK / kChunk : 1;  // chunks per listed block
  using Sm = AttnSmem<D>;
  static_assert(!SPARSE || ROWS == BLK, "sparse tile must be one query block");

  __shared__ __attribute__((aligned(16))) uint16_t smem[Sm::K_ELEMS + Sm::V_ELEMS];
  uint16_t* Ks = smem;
  uint16_t* Vt = smem + Sm::K_ELEMS;

  const int logical = xcd_remap(blockIdx.x, p.total);
  if (logical < 0) return;
  const int bh = logical / p.n_qtiles;
  const int qt = logical - bh * p.n_qtiles;
  const int N = p.N;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 5;    // lane half
  const int lq = lane & 31;   // query column of this lane

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = p.q + head;
  const uint16_t* Kh = p.k + head;
  const uint16_t* Vh = p.v + head;

  // ---- chunk schedule
  int n_chunks;
  const int32_t* idx_row = nullptr;
  if constexpr (SPARSE) {
    const int row = bh * p.n_blocks + qt;
    int c = p.cnt[row];
    c = c < 0 ? 0 : (c > p.max_keep ? p.max_keep : c);
    n_chunks = c * SUBS;
    idx_row = p.idx + (size_t)row * p.max_keep;
  } else {
    n_chunks = (N + kChunk - 1) / kChunk;
  }
  auto chunk_start = [&](int c) -> int {  // first key of chunk c, or -1 if skipped
    if constexpr (SPARSE) {
      const int J = idx_row[c / SUBS];
      if (J < 0 || J >= p.n_blocks) return -1;
      return J * BLK + (c % SUBS) * kChunk;
    } else {
      return c * kChunk;
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T), loaded once
  const int qrow = qt * ROWS + wave * 32 + lq;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < N) w = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }

  // ---- register staging of one chunk
  u32x4 kreg[K_LOADS];
  u32x4 vreg[V_ITEMS][4];
  auto load_chunk = [&](int c) {
    const int k0 = chunk_start(c);
    const int valid = k0 < 0 ? 0 : min(kChunk, N - k0);
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int e = t + i * NT;
      const int row = e / CPR, col = e % CPR;
      kreg[i] = u32x4{0u, 0u, 0u, 0u};
      if ((K_LOADS * NT == kChunk * CPR || e < kChunk * CPR) && row < valid)
        kreg[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)(k0 + row) * D + col * 8);
    }
#pragma unroll
    for (int i = 0; i < V_ITEMS; ++i) {
      const int e = t + i * NT;
      const int c8 = e % CPR, kg = e / CPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vreg[i][r] = u32x4{0u, 0u, 0u, 0u};
        const int key = kg * 4 + r;
        if ((V_ITEMS * NT == V_ITEMS_TOTAL || e < V_ITEMS_TOTAL) && key < valid)
          vreg[i][r] = *reinterpret_cast<const u32x4*>(Vh + (size_t)(k0 + key) * D + c8 * 8);
      }
    }
    return valid;
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int e = t + i * NT;
      if (K_LOADS * NT == kChunk * CPR || e < kChunk * CPR) {
        const int row = e / CPR, col = e % CPR;
        *reinterpret_cast<u32x4*>(Ks + row * Sm::KP + col * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_ITEMS; ++i) {
      const int e = t + i * NT;
      if (V_ITEMS * NT == V_ITEMS_TOTAL || e < V_ITEMS_TOTAL) {
        const int c8 = e % CPR, kg = e / CPR;
        // transpose 4 keys x 8 d into 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // d = 8*c8 + 2w (low halves) and 2w+1 (high halves)
          const uint32_t a0 = vreg[i][0][w], a1 = vreg[i][1][w];
          const uint32_t a2 = vreg[i][2][w], a3 = vreg[i][3][w];
          u32x2 lo, hi;
          lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // (a0.lo, a1.lo)
          lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);
          hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // (a0.hi, a1.hi)
          hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
          const int d0 = 8 * c8 + 2 * w;
          *reinterpret_cast<u32x2*>(Vt + d0 * Sm::VP + kg * 4) = lo;
          *reinterpret_cast<u32x2*>(Vt + (d0 + 1) * Sm::VP + kg * 4) = hi;
        }
      }
    }
  };

  // ---- running state of this lane's query
  f32x16 oacc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) oacc[d] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float sl2 = p.scale_log2;

  int valid_next = 0;
  if (n_chunks > 0) valid_next = load_chunk(0);
  for (int c = 0; c < n_chunks; ++c) {
    const int valid = valid_next;
    store_chunk();
    __syncthreads();
    if (c + 1 < n_chunks) valid_next = load_chunk(c + 1);

    // S^T (64 keys x 32 queries) = K Q^T
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kt * 32 + lq) * Sm::KP + ks * 16 + g * 8);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[kt], 0, 0, 0);
      }
    }
    // keys past the end of the sequence (or of a skipped entry)
    if (valid < kChunk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= valid) sacc[kt][r] = -__builtin_inff();
        }
    }
    float mloc = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kt][r]);
    mloc = fmaxf(mloc, wave_shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc * sl2);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    float psum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * s + 2 * e], sl2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * s + 2 * e + 1], sl2, -m_use));
          psum += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[kt][s] = __builtin_bit_cast(bf16x8, w);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < DT; ++d) oacc[d] *= alpha;

    // O^T (D x 32 queries) += V^T P^T
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kb = kt * 32 + s * 16 + 4 * g;
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const uint16_t* vrow = Vt + (d * 32 + lq) * Sm::VP + kb;
          u32x4 w;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[kt][s], oacc[d], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue
  const float l_tot = l_run + wave_shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < N) {
    if (p.lse != nullptr && g == 0) {
      p.lse[(size_t)bh * N + qrow] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -__builtin_inff();
    }
    if constexpr (OUT_F32) {
      float* Orow = reinterpret_cast<float*>(p.o) + head + (size_t)qrow * D;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v4 = {oacc[d][4 * j] * inv, oacc[d][4 * j + 1] * inv, oacc[d][4 * j + 2] * inv,
                      oacc[d][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(Orow + d * 32 + 8 * j + 4 * g) = v4;
        }
    } else {
      uint16_t* Orow = reinterpret_cast<uint16_t*>(p.o) + head + (size_t)qrow * D;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[d][4 * j] * inv, oacc[d][4 * j + 1] * inv);
          w[1] = pack_bf16x2(oacc[d][4 * j + 2] * inv, oacc[d][4 * j + 3] * inv);
          *reinterpret_cast<u32x2*>(Orow + d * 32 + 8 * j + 4 * g) = w;
        }
    }
  }
}

}  // namespace ba
