// Block-sparse and dense flash-attention forward for gfx950 (bf16 MFMA).
//
// Operation (pith.science review of "Efficient Long-Context Modeling in
// Diffusion Language Models via Block Approximate Sparse Attention", "The
// pith"): exact softmax attention of every query restricted to the tokens of
// its kept key blocks; the dense variant keeps every block and is the
// comparator of the review's "If this is right" speedup claim.
//
// Design (one workgroup = one tile of 32*WAVES query rows of one (b, h)):
//  * Each wave owns 32 query rows.  Scores are formed TRANSPOSED,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 d from LDS,
//    B = Q^T held in registers for the whole kernel).  In the 32x32
//    accumulator layout lane l then holds column l%32 -- one query -- so the
//    running max/sum of a query live in the lane pair (l, l^32).
//  * The output is accumulated transposed too, O^T = V^T P^T: B = P^T comes
//    straight from the score registers (fp32 -> bf16), A = V^T is read from a
//    row-major V tile with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16).  Every O register of a lane belongs to that lane's
//    query, so the online-softmax rescale is lane-local.
//  * Keys are processed in chunks of 64.  K and V chunks are copied HBM/L2 ->
//    LDS by direct-to-LDS buffer loads (no register staging; loads past the
//    sequence end return zero) into one K and one V buffer used in
//    ping-pong: V(c) streams in while S^T(c) and the row maxima are formed
//    (and, in four-wave tiles, the whole softmax), K(c+1) streams in while
//    O^T += V(c) P^T runs.  16-byte chunks of every row are
//    XOR-swizzled so that both the row reads of K and the transposing reads
//    of V are free of bank conflicts.  MFMA operands are read from LDS one
//    step ahead of their use.
//  * Online softmax in the log2 domain, fp32, with the exact running max.  The
//    accumulators of a wave are rescaled only in chunks where some query of
//    the wave finds a new maximum (a wave-uniform branch).
//  * The sparse variant walks the compacted block-index list of its query
//    block; the dense variant walks all keys.  Keys >= N are masked to -inf.
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
  int total;      // BH * n_qtiles * n_split
  int max_keep;
  float scale_log2;  // softmax scale * log2(e)
  // split key lists: every row's chunk list is cut into n_split contiguous
  // parts; part p writes its (O, LSE) at o + p*o_part_stride and
  // lse + p*lse_part_stride (elements).  n_split = 1: no split.
  int n_split;
  size_t o_part_stride;
  size_t lse_part_stride;
  // optional external contribution (fp32 O [BH,N,D], natural-log LSE [BH,N])
  // over another key set, merged into the result in log space
  const float* o_ext;
  const float* lse_ext;
};

constexpr int kChunk = 64;  // keys per LDS chunk

#define BA_LDS __attribute__((address_space(3)))
typedef short i16x4 __attribute__((ext_vector_type(4)));

// 16-byte slot of logical chunk c in row r of a K tile / a V tile
template <int CPR>
__device__ __forceinline__ int k_slot(int r, int c) { return c ^ (r % CPR); }
// V: a transposing read serves 32 lanes = 4 key rows x 4 consecutive chunks
// per cycle; XOR-ing 4*(row%4) (or, with 8 chunks per row, 4*((row/2)%2)
// while consecutive rows fall in opposite bank halves) spreads them over all
// 64 banks.
template <int CPR>
__device__ __forceinline__ int v_slot(int r, int c) {
  return CPR >= 16 ? (c ^ ((r & 3) << 2)) : (c ^ (((r >> 1) & 1) << 2));
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3): loads past
// the end return zero, which pads partial and skipped key chunks.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// max / sum of x over the lane pair (l, l^32) with one v_permlane32_swap
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copy j of a 64-key tile: lane `lane` of wave `wave` fills LDS slot
// (j*WAVES + wave)*64 + lane (16 bytes) from byte offset voff[j] of the tile.
template <int DMA, int WAVES>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, int wave,
                                         const uint32_t* voff) {
#pragma unroll
  for (int j = 0; j < DMA; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (BA_LDS void*)(dst + (j * WAVES + wave) * 64 * 16),
                                             16, voff[j], 0, 0, 0);
}

template <int D, int WAVES, int BLK, bool SPARSE, bool OUT_F32>
__global__ __launch_bounds__(WAVES * 64, 2) void attn_fwd_kernel(AttnParams p) {
  constexpr int ROWS = WAVES * 32;
  constexpr int KSTEPS = D / 16;          // MFMA k-steps of the score product
  constexpr int DT = D / 32;              // 32-wide d tiles of the output
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kChunk * ROW_BYTES;
  constexpr int DMA = (kChunk * CPR) / (64 * WAVES);  // 16-byte loads per lane per tile
  constexpr int SUBS = SPARSE ? BLK / kChunk : 1;     // chunks per listed block
  static_assert(!SPARSE || ROWS == BLK, "sparse tile must be one query block");
  static_assert((kChunk * CPR) % (64 * WAVES) == 0, "tile must split evenly over the waves");

  // two separate arrays: the compiler then sees that a copy into one does not
  // write the other, and does not make the reads of V wait for the copy of K
  __shared__ __attribute__((aligned(1024))) uint8_t Ktile[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Vtile[TILE_BYTES];
  uint8_t* const Kbuf = Ktile;
  uint8_t* const Vbuf = Vtile;

  const int logical = xcd_remap(blockIdx.x, p.total);
  if (logical < 0) return;
  const int tile = logical / p.n_split;      // the parts of a tile are neighbours
  const int part = logical - tile * p.n_split;
  const int bh = tile / p.n_qtiles;
  const int qt = tile - bh * p.n_qtiles;
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;    // lane half
  const int lq = lane & 31;   // query column of this lane

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = p.q + head;
  const uint16_t* Kh = p.k + head;
  const uint16_t* Vh = p.v + head;

  // ---- chunk schedule; the block lists are read through the constant
  // address space (scalar loads, which never wait for the tile copies)
  typedef const __attribute__((address_space(4))) int32_t* cidx_t;
  int n_chunks;
  cidx_t idx_row = nullptr;
  if constexpr (SPARSE) {
    const int row = bh * p.n_blocks + qt;
    int c = ((cidx_t)p.cnt)[row];
    c = c < 0 ? 0 : (c > p.max_keep ? p.max_keep : c);
    n_chunks = c * SUBS;
    idx_row = (cidx_t)p.idx + (size_t)row * p.max_keep;
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

  // ---- direct-to-LDS tile copies: lane `lane` of wave `wave` fills LDS slot
  // p = (j*WAVES + wave)*64 + lane (16 bytes) of copy j; the slot holds
  // logical chunk c of row r under the tile's swizzle.  Byte offsets of the
  // source chunks are loop-invariant.
  uint32_t voff_k[DMA], voff_v[DMA];
#pragma unroll
  for (int j = 0; j < DMA; ++j) {
    const int slot = (j * WAVES + wave) * 64 + lane;
    const int r = slot / CPR, s = slot % CPR;
    voff_k[j] = r * ROW_BYTES + k_slot<CPR>(r, s) * 16;
    voff_v[j] = r * ROW_BYTES + v_slot<CPR>(r, s) * 16;
  }
  auto tile_rsrc = [&](const uint16_t* src, int k0) {
    // (a chunk may start past N: the second half of a 128-key tail block with
    // at most 64 rows; its count must clamp at 0, as a negative count would
    // wrap to an unbounded resource)
    // The values are wave-uniform, but the clamp is selected as a vector
    // med3; readfirstlane puts them back in scalar registers, else every copy
    // is wrapped in a loop that re-establishes a uniform resource.
    const int rows = __builtin_amdgcn_readfirstlane(k0 < 0 ? 0 : max(0, min(kChunk, N - k0)));
    const int first = __builtin_amdgcn_readfirstlane(k0 < 0 ? 0 : k0);
    return make_rsrc(src + (size_t)first * D, rows * ROW_BYTES);
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

  // ---- LDS operand reads
  auto read_k = [&](int kt, int ks) -> bf16x8 {  // A of S^T: key kt*32+lq, d = 16ks+8g..+8
    const int r = kt * 32 + lq;
    return *reinterpret_cast<const bf16x8*>(Kbuf + r * ROW_BYTES + k_slot<CPR>(r, ks * 2 + g) * 16);
  };
  // A of O^T for d tile `dtile`, keys base+4g+{0..3} and base+8+4g+{0..3},
  // base = 16*step: two transposing reads of the row-major V tile
  const int grp = lane >> 4, li = lane & 15;
  const int dl = 16 * (grp & 1) + 4 * (li & 3);  // d of this lane's 8-byte read
  const int kr = 4 * (grp >> 1) + (li >> 2);      // key row of this lane's read within a step
  auto read_v = [&](int step, int dtile) -> bf16x8 {
    const int dd = dtile * 32 + dl;
    const int r0 = step * 16 + kr, r1 = r0 + 8;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (BA_LDS i16x4*)(Vbuf + r0 * ROW_BYTES + v_slot<CPR>(r0, dd >> 3) * 16 + (dd & 7) * 2));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (BA_LDS i16x4*)(Vbuf + r1 * ROW_BYTES + v_slot<CPR>(r1, dd >> 3) * 16 + (dd & 7) * 2));
    const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                           hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, a8);
  };

  // ---- running state of this lane's query
  f32x16 oacc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) oacc[d] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float sl2 = p.scale_log2;

  // this workgroup's part of the chunk list
  const int per_part = (n_chunks + p.n_split - 1) / p.n_split;
  const int c_begin = min(n_chunks, part * per_part);
  const int c_end = min(n_chunks, c_begin + per_part);

  int k0_next = c_begin < c_end ? chunk_start(c_begin) : 0;
  if (c_begin < c_end) dma_tile<DMA, WAVES>(tile_rsrc(Kh, k0_next), Kbuf, wave, voff_k);

  for (int c = c_begin; c < c_end; ++c) {
    const int k0 = k0_next;
    const int valid = k0 < 0 ? 0 : max(0, min(kChunk, N - k0));
    if (c + 1 < c_end) k0_next = chunk_start(c + 1);

    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K(c) landed
    __syncthreads();  // K(c) visible to all waves; every wave is done with V(c-1)
    dma_tile<DMA, WAVES>(tile_rsrc(Vh, k0), Vbuf, wave, voff_v);

    // S^T (64 keys x 32 queries) = K Q^T, K operands read one k-step ahead
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    bf16x8 kcur[2] = {read_k(0, 0), read_k(1, 0)};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      bf16x8 knext[2];
      if (ks + 1 < KSTEPS) {
        knext[0] = read_k(0, ks + 1);
        knext[1] = read_k(1, ks + 1);
      }
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[0], qf[ks], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[1], qf[ks], sacc[1], 0, 0, 0);
      if (ks + 1 < KSTEPS) {
        kcur[0] = knext[0];
        kcur[1] = knext[1];
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
    // two chains of three-input maxima (v_max3_f32): 17 instructions for 32 values
    float ma = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
    float mb = fmaxf(fmaxf(sacc[1][0], sacc[1][1]), sacc[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = fmaxf(fmaxf(ma, sacc[0][r]), sacc[0][r + 1]);
      mb = fmaxf(fmaxf(mb, sacc[1][r]), sacc[1][r + 1]);
    }
    float mloc = fmaxf(fmaxf(ma, sacc[0][15]), fmaxf(mb, sacc[1][15]));
    mloc = pair_max(mloc) * sl2;
    if (__any(mloc > m_run)) {  // exact running max: a row's largest probability is 1
      const float m_new = fmaxf(m_run, mloc);
      if (m_new != -__builtin_inff()) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DT; ++d) oacc[d] *= alpha;
        m_run = m_new;
      }
    }
    const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;

    float psum = 0.f;
    bf16x8 pf[4];  // P^T operand of each 16-key step
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
        pf[2 * kt + s] = __builtin_bit_cast(bf16x8, w);
      }
    }
    l_run += psum;
    // Four-wave tiles: keep the softmax ahead of the wait for V(c) so that it
    // covers the copy (without the fence the compiler sinks it past the
    // barrier, next to its use in O^T += V^T P^T).  Two-wave tiles are faster
    // with the sunk form, where the exponentials fill the gaps between the
    // PV MFMAs and the copy of K(c+1) starts earlier.
    if constexpr (WAVES == 4)
      __asm__ volatile("" : "+v"(pf[0]), "+v"(pf[1]), "+v"(pf[2]), "+v"(pf[3]), "+v"(l_run));

    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // V(c) landed
    __syncthreads();  // V(c) visible; every wave is done with K(c)
    if (c + 1 < c_end) dma_tile<DMA, WAVES>(tile_rsrc(Kh, k0_next), Kbuf, wave, voff_k);

    // O^T (D x 32 queries) += V^T P^T, V operands read one step ahead
    bf16x8 vcur[DT];
#pragma unroll
    for (int d = 0; d < DT; ++d) vcur[d] = read_v(0, d);
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      bf16x8 vnext[DT];
      if (step + 1 < 4) {
#pragma unroll
        for (int d = 0; d < DT; ++d) vnext[d] = read_v(step + 1, d);
      }
#pragma unroll
      for (int d = 0; d < DT; ++d)
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur[d], pf[step], oacc[d], 0, 0, 0);
      if (step + 1 < 4) {
#pragma unroll
        for (int d = 0; d < DT; ++d) vcur[d] = vnext[d];
      }
    }
  }

  // ---- epilogue: LSE (log2 domain) and the factor of oacc in the output
  const float l_tot = pair_sum(l_run);
  float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -__builtin_inff();
  float w_own = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  float w_ext = 0.f;
  const size_t row = (size_t)bh * N + qrow;
  if (p.o_ext != nullptr && qrow < N) {
    // merge with the external (O, LSE): weights Z_own/Z and Z_ext/Z
    const float le2 = p.lse_ext[row] * 1.44269504088896340736f;
    const float M = fmaxf(lse2, le2);
    if (M != -__builtin_inff()) {
      const float a = lse2 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(lse2 - M);
      const float b = le2 == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(le2 - M);
      const float L = a + b;
      w_own *= a / L;
      w_ext = b / L;
      lse2 = M + log2f(L);
    }
  }
  if (qrow < N) {
    if (p.lse != nullptr && g == 0)
      p.lse[part * p.lse_part_stride + row] = lse2 * 0.69314718055994530942f;  // -inf stays -inf
    // this lane's 4-value groups: d = dt*32 + 8j + 4g .. +3 (no lambda here:
    // capturing oacc, sized by a template parameter, drops the launch stub)
    const float* Erow = w_ext != 0.f ? p.o_ext + row * D : nullptr;
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dd = d * 32 + 8 * j + 4 * g;
        f32x4 v4 = {oacc[d][4 * j] * w_own, oacc[d][4 * j + 1] * w_own, oacc[d][4 * j + 2] * w_own,
                    oacc[d][4 * j + 3] * w_own};
        if (Erow != nullptr) v4 += *reinterpret_cast<const f32x4*>(Erow + dd) * w_ext;
        if constexpr (OUT_F32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + part * p.o_part_stride + row * D + dd) = v4;
        } else {
          u32x2 w;
          w[0] = pack_bf16x2(v4[0], v4[1]);
          w[1] = pack_bf16x2(v4[2], v4[3]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + part * p.o_part_stride + row * D + dd) = w;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Exact log-space merge of P attention results over disjoint key sets:
//   LSE = ln sum_p e^{LSE_p},  O = sum_p e^{LSE_p - LSE} O_p
// (a part with LSE_p = -inf weighs 0; all parts empty: O = 0, LSE = -inf).
// One wave per row; lanes hold consecutive fp32 pairs (D = 128) or single
// values (D = 64) of the row, so every part's row is one coalesced read.
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts, int n_parts,
                                                    size_t rows, void* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int E = D / 64;  // values per lane
  const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  float M = -__builtin_inff();
  for (int q = 0; q < n_parts; ++q) M = fmaxf(M, lse_parts[q * rows + r]);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int q = 0; q < n_parts; ++q) {
      const float lq = lse_parts[q * rows + r];
      if (lq == -__builtin_inff()) continue;
      const float w = __builtin_amdgcn_exp2f((lq - M) * 1.44269504088896340736f);
      L += w;
      const float* src = o_parts + (q * rows + r) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(w, src[e], acc[e]);
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  if (lse != nullptr && lane == 0) lse[r] = L > 0.f ? M + logf(L) : -__builtin_inff();
  if constexpr (OUT_F32) {
    float* dst = reinterpret_cast<float*>(o) + r * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = acc[e] * inv;
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(o) + r * D + lane * E;
    if constexpr (E == 2) {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      dst[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
    }
  }
}

}  // namespace ba
