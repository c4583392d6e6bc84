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
//  * The sparse walk visits a row's kept blocks in one order shared by every
//    row (increasing (J * g) mod n, g near n/phi): each kept set is spread
//    evenly over that order, so the walks of the workgroups resident on an
//    XCD advance together and read each shared key block from L2 at about
//    the same time.  Ascending walks would not: kept blocks cluster around
//    each row's own diagonal band and key runs, so concurrent rows sit at
//    different keys.
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
  // sparse walk order: a row's kept blocks are visited in increasing
  // (J * walk_mul) mod n_blocks, one order shared by every row of every head
  // (0: the list's own order); walk_inv is its inverse mod n_blocks
  int walk_mul;
  int walk_inv;
};

// Longest block list a workgroup reorders (longer lists are walked as given).
constexpr int kMaxOrdered = 1024;

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

// A wave-uniform int32 read through the scalar cache.  The load is written
// out, with its wait, so that the compiler neither treats the (written)
// memory as constant nor lets the read move above the writes before it.
__device__ __forceinline__ int scalar_load_i32(const int32_t* ptr) {
  int v;
  __asm__ volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// Keys of the 64-key chunk starting at k0 that lie before the sequence end N
// (0 for a skipped entry, k0 < 0), formed in the scalar unit: written as
// min/max the compiler would form the clamp as a vector med3 of scalars and
// read it back with readfirstlane, in every copy of every chunk.
__device__ __forceinline__ int chunk_rows(int k0, int N) {
  int r;
  __asm__("s_sub_i32 %0, %1, %2\n\t"
          "s_min_i32 %0, %0, %3\n\t"
          "s_max_i32 %0, %0, 0\n\t"
          "s_cmp_lt_i32 %2, 0\n\t"
          "s_cselect_b32 %0, 0, %0"
          : "=&s"(r)
          : "s"(N), "s"(k0), "i"(kChunk)
          : "scc");
  return r;
}
__device__ __forceinline__ int chunk_first(int k0) {
  int r;
  __asm__("s_max_i32 %0, %1, 0" : "=s"(r) : "s"(k0) : "scc");
  return r;
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

// LDS bytes of one K or V tile (64 keys of D bf16 values)
template <int D>
constexpr int attn_tile_bytes() { return kChunk * D * 2; }

// One tile of the forward: query tile `logical` (tile-major, then key-list
// part) of the launch described by p, with the workgroup's K and V LDS tiles.
// Every wave of the workgroup calls it with the same `logical`; tid is the
// thread's index in the workgroup.
// REMAT: which of the lane's addresses are formed again in every chunk
// instead of held across the chunk loop (fewer live registers): bit 0 the
// tile-copy offsets, bit 1 the K operand reads, bit 2 the V operand reads.
template <int D, int WAVES, int BLK, bool SPARSE, bool OUT_F32, int REMAT = 0>
__device__ __forceinline__ void attn_tile(AttnParams p, int logical, int tid, uint8_t* Ktile,
                                          uint8_t* Vtile) {
  constexpr int ROWS = WAVES * 32;
  constexpr int KSTEPS = D / 16;          // MFMA k-steps of the score product
  constexpr int DT = D / 32;              // 32-wide d tiles of the output
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kChunk * ROW_BYTES;
  constexpr int DMA = (kChunk * CPR) / (64 * WAVES);  // 16-byte loads per lane per tile
  constexpr int SUBS = SPARSE ? BLK / kChunk : 1;     // chunks per listed block
  // a sparse tile is one query block, or (PAIR) two neighbouring ones
  constexpr bool PAIR = SPARSE && ROWS == 2 * BLK;
  static_assert(!SPARSE || ROWS == BLK || PAIR, "sparse tile must be one or two query blocks");
  static_assert((kChunk * CPR) % (64 * WAVES) == 0, "tile must split evenly over the waves");

  uint8_t* const Kbuf = Ktile;
  uint8_t* const Vbuf = Vtile;

  const int tile = logical / p.n_split;      // the parts of a tile are neighbours
  const int part = logical - tile * p.n_split;
  const int bh = tile / p.n_qtiles;
  const int qt = tile - bh * p.n_qtiles;
  const int N = p.N;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;    // lane half
  const int lq = lane & 31;   // query column of this lane

  const size_t head = (size_t)bh * N * D;
  const uint16_t* Qh = p.q + head;
  const uint16_t* Kh = p.k + head;
  const uint16_t* Vh = p.v + head;

  // ---- Q fragments (B operand of S^T = K Q^T), loaded once; in flight
  // while the block list is reordered
  const int qrow = qt * ROWS + wave * 32 + lq;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < N) w = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, w);
  }

  // ---- chunk schedule: block-list entries are read with scalar loads
  // (which never wait for the tile copies)
  int n_chunks;
  const int32_t* listA = nullptr;  // caller's list of the (first) query block
  const int32_t* listB = nullptr;  // caller's list of the second block of a pair
  const int32_t* walk = nullptr;   // a built walk: (owner bits << 16) | J per entry
  int cA = 0;
  int my_bit = 1;                  // owner bit of this wave's query block
  if constexpr (SPARSE) {
    typedef const __attribute__((address_space(4))) int32_t* cidx_t;
    const int n = p.n_blocks;
    const int qb = PAIR ? 2 * qt : qt;
    const int rowA = bh * n + qb;
    auto clamp_cnt = [&](int c) { return c < 0 ? 0 : (c > p.max_keep ? p.max_keep : c); };
    cA = clamp_cnt(((cidx_t)p.cnt)[rowA]);
    listA = p.idx + (size_t)rowA * p.max_keep;
    int cB = 0;
    if constexpr (PAIR) {
      my_bit = wave < WAVES / 2 ? 1 : 2;
      if (qb + 1 < n) {
        cB = clamp_cnt(((cidx_t)p.cnt)[rowA + 1]);
        listB = listA + p.max_keep;
      }
    }
    const int tot = cA + cB;
    n_chunks = tot * SUBS;  // as given: the first block's entries, then the second's
    // Walk order.  The kept blocks of one row cluster (a band around the
    // diagonal, runs of similar keys), so ascending walks of the rows that
    // are resident together sit at different keys at any moment and share
    // little of L2.  In the order of increasing (J * walk_mul) mod n -- a
    // golden-ratio stride, the same for every row -- any kept set is spread
    // evenly, so the walks advance together and a block kept by many rows is
    // read by all of them at about the same time.  A pair of query blocks
    // walks the union of its two lists in that order, each entry tagged with
    // the blocks that keep it, so a block both keep is copied to LDS once.
    //
    // The walk is built by a rank sort of packed words
    // (key << 16 | list << 15 | position).  The key fixes the block (J is
    // key * walk_mul^-1 mod n), so the words order the entries by key, then
    // the first list before the second, then list position; the position
    // makes every word unique, so an entry's rank is the number of smaller
    // words.  Merging each entry of the second list into an entry of the
    // first for the same block just before it keeps repeated entries'
    // multiplicity; entries outside [0, n) take key 0xFFFF and sort last.  It is stored in this tile's own output rows, which hold
    // nothing else until the epilogue: every wave passes two barriers after
    // its last walk read before any output is written.  Full lists keep
    // ascending order (then the walk equals the dense one); a walk longer
    // than 2*kMaxOrdered, or than the output rows hold, is taken as given.
    const size_t out_elem = OUT_F32 ? 4 : 2;
    const int rows_here = min(ROWS, N - qt * ROWS);
    const bool full = cA == n && (!PAIR || qb + 1 >= n || cB == n);
    const bool build = p.walk_mul > 0 && tot > 1 && tot <= 2 * kMaxOrdered &&
                       (size_t)tot * 4 <= (size_t)rows_here * D * out_elem && (PAIR || !full);
    if (build) {
      constexpr int T = WAVES * 64;
      static_assert(TILE_BYTES >= 2 * kMaxOrdered * 4, "a tile holds the packed walk");
      // K and V tiles are free until their first copies
      uint32_t* const keys = reinterpret_cast<uint32_t*>(Vtile);
      uint32_t* const sorted = reinterpret_cast<uint32_t*>(Ktile);
      int* const scan = reinterpret_cast<int*>(Vtile);  // reused once the keys are ranked
      int32_t* const out = reinterpret_cast<int32_t*>(
          reinterpret_cast<uint8_t*>(p.o) +
          (part * p.o_part_stride + ((size_t)bh * N + (size_t)qt * ROWS) * D) * out_elem);
      // the packed words, padded to whole 16-byte groups with all-ones words,
      // which are above every word and add to no rank
      const int tot4 = (tot + 3) >> 2;
      for (int e = tid; e < 4 * tot4; e += T) {
        uint32_t w = 0xFFFFFFFFu;
        if (e < tot) {
          const bool inB = e >= cA;
          const int J = inB ? listB[e - cA] : listA[e];
          const uint32_t own = inB ? 1u : 0u;
          const uint32_t key = full ? (uint32_t)J : (uint32_t)J * (uint32_t)p.walk_mul % (uint32_t)n;
          w = ((J >= 0 && J < n) ? key << 16 : 0xFFFF0000u) | (own << 15) | (uint32_t)e;
        }
        keys[e] = w;
      }
      __syncthreads();
      // rank = number of smaller words; every lane reads the same 16 bytes
      // (a broadcast), several in flight
      const u32x4* const keys4 = reinterpret_cast<const u32x4*>(keys);
      for (int e = tid; e < tot; e += T) {
        const uint32_t v = keys[e];
        int rank = 0;
#pragma unroll 4
        for (int j4 = 0; j4 < tot4; ++j4) {
          const u32x4 w = keys4[j4];
#pragma unroll
          for (int i = 0; i < 4; ++i) rank += w[i] < v;
        }
        sorted[rank] = v;
      }
      __syncthreads();
      // an entry of the second list merges into an entry of the first for
      // the same key just before it; every other sorted entry starts a walk
      // entry
      auto starts = [&](int r) -> bool {
        if (r == 0) return true;
        const uint32_t v = sorted[r], u = sorted[r - 1];
        return !((v >> 16) == (u >> 16) && ((v >> 15) & 1u) && !((u >> 15) & 1u));
      };
      const int seg = (tot + T - 1) / T;
      const int s0 = min(tot, (int)tid * seg), s1 = min(tot, s0 + seg);
      int mine_starts = 0;
      for (int r = s0; r < s1; ++r) mine_starts += starts(r);
      // exclusive scan of the per-thread counts: within each wave by lane
      // shuffles, then over the waves' totals
      int incl = mine_starts;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (lane == 63) scan[wave] = incl;
      __syncthreads();
      int pos = incl - mine_starts, walk_len = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const int t = scan[w];
        if (w < wave) pos += t;
        walk_len += t;
      }
      for (int r = s0; r < s1; ++r) {
        if (!starts(r)) continue;
        const uint32_t v = sorted[r], key = v >> 16;
        uint32_t own_bits = 1u << ((v >> 15) & 1u);
        if (r + 1 < tot && !starts(r + 1)) own_bits |= 2u;
        const uint32_t J = key == 0xFFFFu ? 0x7FFFu : full ? key : key * (uint32_t)p.walk_inv % (uint32_t)n;
        out[pos++] = (int32_t)((own_bits << 16) | J);
      }
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the walk is in L2
      __syncthreads();
      n_chunks = __builtin_amdgcn_readfirstlane(walk_len) * SUBS;
      walk = out;
    }
  } else {
    n_chunks = (N + kChunk - 1) / kChunk;
  }
  // first key of chunk c (-1: skipped) and the owner bits of its block
  auto chunk_entry = [&](int c, int& own) -> int {
    if constexpr (SPARSE) {
      const int i = c / SUBS;
      int J;
      if (walk != nullptr) {
        const int raw = scalar_load_i32(walk + i);
        J = raw & 0xFFFF;
        own = raw >> 16;
      } else if (i < cA) {
        J = scalar_load_i32(listA + i);
        own = 1;
      } else {
        J = scalar_load_i32(listB + (i - cA));
        own = 2;
      }
      if (J < 0 || J >= p.n_blocks) return -1;
      return J * BLK + (c % SUBS) * kChunk;
    } else {
      own = 3;
      return c * kChunk;
    }
  };

  // ---- direct-to-LDS tile copies: lane `lane` of wave `wave` fills LDS slot
  // p = (j*WAVES + wave)*64 + lane (16 bytes) of copy j; the slot holds
  // logical chunk c of row r under the tile's swizzle.  Byte offsets of the
  // source chunks are loop-invariant.
  // (lane_c is the lane index these addresses are formed from: with REMAT
  // it is made opaque in every chunk, so they are formed again there)
  int lane_c = lane;   // copy offsets
  int lane_k = lane;   // K operand reads
  int lane_v = lane;   // V operand reads
  auto copy_offsets = [&](uint32_t* vk, uint32_t* vv) {
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
      const int slot = (j * WAVES + wave) * 64 + lane_c;
      const int r = slot / CPR, s = slot % CPR;
      if (vk) vk[j] = r * ROW_BYTES + k_slot<CPR>(r, s) * 16;
      if (vv) vv[j] = r * ROW_BYTES + v_slot<CPR>(r, s) * 16;
    }
  };
  uint32_t voff_k[DMA], voff_v[DMA];
  copy_offsets(voff_k, voff_v);
  auto copy_k = [&](const __amdgpu_buffer_rsrc_t& rs) {
    if constexpr ((REMAT & 1) != 0) {
      uint32_t vo[DMA];
      copy_offsets(vo, nullptr);
      dma_tile<DMA, WAVES>(rs, Kbuf, wave, vo);
    } else {
      dma_tile<DMA, WAVES>(rs, Kbuf, wave, voff_k);
    }
  };
  auto copy_v = [&](const __amdgpu_buffer_rsrc_t& rs) {
    if constexpr ((REMAT & 1) != 0) {
      uint32_t vo[DMA];
      copy_offsets(nullptr, vo);
      dma_tile<DMA, WAVES>(rs, Vbuf, wave, vo);
    } else {
      dma_tile<DMA, WAVES>(rs, Vbuf, wave, voff_v);
    }
  };
  auto tile_rsrc = [&](const uint16_t* src, int k0) {
    // (a chunk may start past N: the second half of a 128-key tail block with
    // at most 64 rows; its count must clamp at 0, as a negative count would
    // wrap to an unbounded resource)
    // (formed in scalar registers: a resource held in vector registers would
    // wrap every copy in a loop that re-establishes a uniform resource)
    const int rows = chunk_rows(k0, N);
    const int first = chunk_first(k0);
    return make_rsrc(src + (size_t)first * D, rows * ROW_BYTES);
  };

  // ---- LDS operand reads
  auto read_k = [&](int kt, int ks) -> bf16x8 {  // A of S^T: key kt*32+lq, d = 16ks+8g..+8
    if constexpr ((REMAT & 2) != 0 && CPR == 16) {
      // Row r = kt*32 + lq holds chunk c at slot c ^ (lq & 15), so the read
      // of chunk 2ks+g is at A ^ (32*ks) (+ 8192 for kt = 1), with
      // A = 256*lq + 16*((lq & 15) ^ g): the XOR only flips bits 5-7, which
      // the other terms of A leave clear (the tile is 1 KB aligned).  One
      // lane constant and one XOR per k-step when addresses are re-formed.
      const int lqk = lane_k & 31;
      const int a = lqk * ROW_BYTES + (((lqk & 15) ^ (lane_k >> 5)) << 4);
      return *reinterpret_cast<const bf16x8*>(Kbuf + kt * 32 * ROW_BYTES + (a ^ (ks << 5)));
    } else {
      const int r = kt * 32 + (lane_k & 31);
      return *reinterpret_cast<const bf16x8*>(Kbuf + r * ROW_BYTES + k_slot<CPR>(r, ks * 2 + (lane_k >> 5)) * 16);
    }
  };
  // A of O^T for d tile `dtile`, keys base+4g+{0..3} and base+8+4g+{0..3},
  // base = 16*step: two transposing reads of the row-major V tile
  auto read_v = [&](int step, int dtile) -> bf16x8 {
    const int grp = lane_v >> 4, li = lane_v & 15;
    const int dl = 16 * (grp & 1) + 4 * (li & 3);  // d of this lane's 8-byte read
    const int kr = 4 * (grp >> 1) + (li >> 2);      // key row of this lane's read within a step
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
  // running max (log2 units).  It starts at a finite floor below any score
  // rather than -inf: a chunk whose keys are all masked (max -inf) leaves it,
  // the first real maximum then rescales by exp2(floor - m) = 0 exactly as
  // from -inf, and no chunk needs a test for an infinite max.  (A row whose
  // scores all lie below the floor, which takes inputs whose products
  // overflow fp32, would count as empty.)
  float m_run = -1e30f;
  float l_run = 0.f;
  const float sl2 = p.scale_log2;

  // this workgroup's part of the chunk list
  const int per_part = (n_chunks + p.n_split - 1) / p.n_split;
  const int c_begin = min(n_chunks, part * per_part);
  const int c_end = min(n_chunks, c_begin + per_part);

  int own_next = 0;
  int k0_next = c_begin < c_end ? chunk_entry(c_begin, own_next) : 0;
  if (c_begin < c_end) copy_k(tile_rsrc(Kh, k0_next));

  for (int c = c_begin; c < c_end; ++c) {
    if constexpr ((REMAT & 1) != 0) __asm__ volatile("" : "+v"(lane_c));
    if constexpr ((REMAT & 2) != 0) __asm__ volatile("" : "+v"(lane_k));
    if constexpr ((REMAT & 4) != 0) __asm__ volatile("" : "+v"(lane_v));
    const int k0 = k0_next;
    // in a pair, a wave works only on the blocks its own query block keeps;
    // it still copies its share of every tile and meets every barrier
    const bool mine = !PAIR || (own_next & my_bit) != 0;
    const int valid = chunk_rows(k0, N);
    if (c + 1 < c_end) k0_next = chunk_entry(c + 1, own_next);

    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K(c) landed
    __syncthreads();  // K(c) visible to all waves; every wave is done with V(c-1)
    copy_v(tile_rsrc(Vh, k0));

    bf16x8 pf[4];  // P^T operand of each 16-key step
    if (mine) {
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
      // (key kt*32 + 8(r/4) + 4g + r%4 is past the end when its constant part
      // reaches valid - 4g: one register per chunk, not one per key)
      if (valid < kChunk) {
        const int lim = valid - 4 * g;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kt * 32 + 8 * (r >> 2) + (r & 3) >= lim) sacc[kt][r] = -__builtin_inff();
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
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 from the floor
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DT; ++d) oacc[d] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run;

      // (the sum starts from the first pair: 0 + x is not folded away, as
      // -0 + 0 would not be -0; every pair sum here is >= 0, so the bits
      // are those of a sum started at 0)
      float psum;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * s + 2 * e], sl2, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * s + 2 * e + 1], sl2, -m_use));
            if (kt == 0 && s == 0 && e == 0) psum = p0 + p1;
            else psum += p0 + p1;
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
    }

    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // V(c) landed
    __syncthreads();  // V(c) visible; every wave is done with K(c)
    if (c + 1 < c_end) copy_k(tile_rsrc(Kh, k0_next));

    if (!mine) continue;
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

template <int D, int WAVES, int BLK, bool SPARSE, bool OUT_F32>
__global__ __launch_bounds__(WAVES * 64, 2) void attn_fwd_kernel(AttnParams p) {
  // two separate arrays: the compiler then sees that a copy into one does not
  // write the other, and does not make the reads of V wait for the copy of K
  __shared__ __attribute__((aligned(1024))) uint8_t Ktile[attn_tile_bytes<D>()];
  __shared__ __attribute__((aligned(1024))) uint8_t Vtile[attn_tile_bytes<D>()];
  const int logical = xcd_remap(blockIdx.x, p.total);
  if (logical < 0) return;
  attn_tile<D, WAVES, BLK, SPARSE, OUT_F32>(p, logical, threadIdx.x, Ktile, Vtile);
}

// ---------------------------------------------------------------------------
// Work-queue form of the sparse forward.  The grid holds only as many
// workgroups as the device keeps resident; each takes query tiles from a
// queue until none is left.  The tiles are dealt into one queue per XCD, a
// contiguous range in head order (the ranges xcd_remap gives the one-tile
// launch), so the workgroups of an XCD share its L2 as before.  A workgroup
// whose own queue is empty takes tiles from the other XCDs' queues, so an
// XCD that runs faster (the XCDs' clocks differ under the power limit) or
// draws cheaper tiles (pair tiles walk unions of different sizes) ends with
// the others instead of idling while they drain.  Running tiles back to back
// in one workgroup costs a few percent against the one-tile launch, so the
// queues pay off only where the XCDs' shares differ: lists whose kept counts
// vary from head to head, not the selection pass's equal rows.
//
// queue: kQueueWords words, zero when the launch starts.  Words 0..7 count
// the tickets drawn from each XCD's range, word 8 the workgroups that have
// left the loop; the last workgroup to leave sets them back to zero, so the
// same queue serves the next launch on the stream.  Every draw increments a
// counter, so a workgroup leaves after at most 8 failed draws whatever the
// queue held; a queue not at zero only makes the results wrong (stale
// tickets skip tiles, a stale leaver count clears the queue early and tiles
// are drawn again), and every list entry read back is range-checked.
// ---------------------------------------------------------------------------
constexpr int kQueueWords = 16;
// The loop keeps the tile code's state live across tiles, so the K operand
// addresses are formed in every chunk: the kernel then fits the 168 VGPRs
// of three waves per SIMD, as the one-tile kernel does, with its few spills
// outside the chunk loop.
constexpr int kQueuedRemat = 2;

template <int D, int WAVES, int BLK, bool OUT_F32>
__global__ __launch_bounds__(WAVES * 64, 3) void attn_fwd_queued_kernel(AttnParams p, uint32_t* queue) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ktile[attn_tile_bytes<D>()];
  __shared__ __attribute__((aligned(1024))) uint8_t Vtile[attn_tile_bytes<D>()];
  // next tile, in a slot per iteration parity: a slot is rewritten two
  // iterations later, after a barrier every wave passes once it has read it
  __shared__ int next_tile[2];
  const int xcd = blockIdx.x % kNumXcd;  // workgroups are dealt round-robin over the XCDs
  const int per = (p.total + kNumXcd - 1) / kNumXcd;
  uint32_t open = (1u << kNumXcd) - 1;  // queues this workgroup has not yet found empty
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) {
      int t = -1;
      for (int i = 0; i < kNumXcd && t < 0; ++i) {
        const int y = (xcd + i) % kNumXcd;
        if (!((open >> y) & 1u)) continue;
        const int lo = y * per;
        const int len = min(per, p.total - lo);
        const uint32_t ticket = len > 0 ? atomicAdd(&queue[y], 1u) : 0xFFFFFFFFu;
        if (len > 0 && ticket < (uint32_t)len) t = lo + (int)ticket;
        else open &= ~(1u << y);
      }
      next_tile[it & 1] = t;
    }
    __syncthreads();
    const int logical = __builtin_amdgcn_readfirstlane(next_tile[it & 1]);
    if (logical < 0) break;  // uniform: every wave read the same slot
    // the thread index, opaque to the compiler in each iteration: values
    // derived from it are then formed inside each tile as in the one-tile
    // kernel, not hoisted out of this loop and held live across every tile
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    attn_tile<D, WAVES, BLK, true, OUT_F32, kQueuedRemat>(p, logical, tid, Ktile, Vtile);
  }
  if (threadIdx.x == 0) {
    // every ticket this workgroup draws precedes its count of leaving
    const uint32_t left =
        __hip_atomic_fetch_add(&queue[kNumXcd], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (left == gridDim.x - 1) {
      for (int i = 0; i <= kNumXcd; ++i)
        __hip_atomic_store(&queue[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
