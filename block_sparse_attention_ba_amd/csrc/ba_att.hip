// C-ABI entry points of the gfx950 BA-Att library (declared in ba_att.h).
//
// Host code only validates arguments, carves the caller's workspace and
// enqueues kernels on the caller's stream.  Nothing is allocated and nothing
// synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <math.h>
#include <mutex>
#include <stdint.h>

#include "ba_att.h"
#include "attention.hpp"
#include "diagnostics.hpp"
#include "select.hpp"

namespace {

constexpr int kMaxN = 1 << 20;
constexpr int kMaxBlocksPerRow = 2048;  // mask -> index rows
constexpr int kMaxSelectBlocks = ba::kMaxScoreBlocks;
constexpr int kMaxFullScoreBlocks = 512;  // the full-covariance diagnostic

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int num_blocks(int N, int block) { return (N + block - 1) / block; }

// Shape checks shared by every entry point that takes Q/K/V.
ba_status check_shape(int B, int H, int N, int D) {
  if (B < 1 || H < 1 || N < 1 || D < 1) return BA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return BA_ERR_UNSUPPORTED;
  if (N > kMaxN) return BA_ERR_UNSUPPORTED;
  const long long elems = (long long)B * H * N * D;
  if (elems >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  return BA_OK;
}

float resolve_scale(float scale, int D) { return scale > 0.f ? scale : 1.0f / sqrtf((float)D); }

int round_up8(int x) { return (x + 7) / 8 * 8; }

// keep = n - floor(sparsity*n + 1e-9), clamped to [1, n] (valid n, sparsity)
int keep_count(int n, double sparsity) {
  const long long drop = (long long)floor(sparsity * (double)n + 1e-9);
  return (int)std::min<long long>(n, std::max<long long>(1, (long long)n - drop));
}

ba_status finish_launch() {
  return hipGetLastError() == hipSuccess ? BA_OK : BA_ERR_HIP;
}

int ni_for(int n) {  // elements per lane for a row of n blocks: 1, 2, 4, ..., 32
  int ni = 1;
  while (ni * 64 < n) ni *= 2;
  return ni;
}

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  return cus;
}

template <int D>
void launch_pool(int BH, int N, int n, int block, float scale, const uint16_t* q, const uint16_t* k,
                 float* aq, float* ak, hipStream_t s) {
  const dim3 grid((2 * BH * n + 3) / 4);  // one wave per (tensor, head, block)
  // Q and K larger than the 256 MB last-level cache (MALL) are streamed
  const bool nt = 2.0 * BH * N * D * sizeof(uint16_t) > 256.0 * (1 << 20);
  if (block == 64) {
    if (nt) ba::pool_stats_kernel<D, 64, true><<<grid, 256, 0, s>>>(q, k, aq, ak, N, n, BH, scale);
    else ba::pool_stats_kernel<D, 64, false><<<grid, 256, 0, s>>>(q, k, aq, ak, N, n, BH, scale);
  } else {
    if (nt) ba::pool_stats_kernel<D, 128, true><<<grid, 256, 0, s>>>(q, k, aq, ak, N, n, BH, scale);
    else ba::pool_stats_kernel<D, 128, false><<<grid, 256, 0, s>>>(q, k, aq, ak, N, n, BH, scale);
  }
}

// Rows per score workgroup: the largest R with a kernel for this row length
// (64 up to n = 256, 32 up to n = 1024, else 16) whose grid of
// B*H*ceil(n/R) workgroups covers every compute unit twice, else the largest
// that covers it once, else 16; R must fit the accumulators and the LDS.
// Each workgroup reads its head's ak once, so taller workgroups re-read it
// less.  Up to n = 256 the kernels keep to 64 VGPRs, so two workgroups share
// a compute unit and one's row selections (scalar-bound) overlap the other's
// fp32 products; longer rows take more registers and only the single cover
// applies.
int score_rows(int BH, int n, int D, int NI) {
  const int cus = device_cus();
  for (int cover : {2, 1}) {
    if (cover == 2 && NI > 4) continue;
    for (int R : {64, 32, 16}) {
      if ((R == 64 && NI > 4) || (R == 32 && NI > 16)) continue;
      const int ctw = NI >= 4 ? NI / 4 : 1;
      if ((R / 16) * ctw > 8 || cover * ba::score_lds_bytes(D, R, n) > ba::kScoreLdsBytes) continue;
      if ((long long)BH * ((n + R - 1) / R) >= (long long)cover * cus) return R;
    }
  }
  return 16;
}

template <int D, int NI, int R>
void launch_score_r(int BH, int n, int keep, const float* aq, const float* ak, uint8_t* mask,
                    int32_t* idx, int32_t* cnt, float* score, hipStream_t s) {
  const int total = BH * ((n + R - 1) / R);
  const size_t smem = (size_t)ba::score_lds_bytes(D, R, n);
  if (smem > 65536)  // beyond the default dynamic-LDS limit of a launch
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&ba::score_topk_kernel<D, NI, R>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  ba::score_topk_kernel<D, NI, R><<<dim3(round_up8(total)), ba::kScoreWaves * 64, smem, s>>>(
      aq, ak, n, keep, mask, idx, cnt, score, total);
}

template <int D, int NI>
void launch_score_ni(int BH, int n, int keep, const float* aq, const float* ak, uint8_t* mask,
                     int32_t* idx, int32_t* cnt, float* score, hipStream_t s) {
  const int R = score_rows(BH, n, D, NI);
  if constexpr (NI <= 4) {
    if (R == 64) return launch_score_r<D, NI, 64>(BH, n, keep, aq, ak, mask, idx, cnt, score, s);
  }
  if constexpr (NI <= 16) {
    if (R == 32) return launch_score_r<D, NI, 32>(BH, n, keep, aq, ak, mask, idx, cnt, score, s);
  }
  launch_score_r<D, NI, 16>(BH, n, keep, aq, ak, mask, idx, cnt, score, s);
}

template <int D>
void launch_score(int BH, int n, int keep, const float* aq, const float* ak, uint8_t* mask,
                  int32_t* idx, int32_t* cnt, float* score, hipStream_t s) {
  switch (ni_for(n)) {
    case 1: launch_score_ni<D, 1>(BH, n, keep, aq, ak, mask, idx, cnt, score, s); break;
    case 2: launch_score_ni<D, 2>(BH, n, keep, aq, ak, mask, idx, cnt, score, s); break;
    case 4: launch_score_ni<D, 4>(BH, n, keep, aq, ak, mask, idx, cnt, score, s); break;
    case 8: launch_score_ni<D, 8>(BH, n, keep, aq, ak, mask, idx, cnt, score, s); break;
    case 16: launch_score_ni<D, 16>(BH, n, keep, aq, ak, mask, idx, cnt, score, s); break;
    default: launch_score_ni<D, 32>(BH, n, keep, aq, ak, mask, idx, cnt, score, s); break;
  }
}

template <int D, int WAVES, int BLK, bool SPARSE>
void launch_attn(const ba::AttnParams& p, bool out_f32, hipStream_t s) {
  const dim3 grid(round_up8(p.total));
  if (out_f32)
    ba::attn_fwd_kernel<D, WAVES, BLK, SPARSE, true><<<grid, WAVES * 64, 0, s>>>(p);
  else
    ba::attn_fwd_kernel<D, WAVES, BLK, SPARSE, false><<<grid, WAVES * 64, 0, s>>>(p);
}

// Work-queue sparse forward: as many workgroups as the device keeps
// resident (a multiple of the XCD count), each taking tiles from the queue.
template <int D, int WAVES, int BLK, bool OUT_F32>
ba_status launch_attn_queued_t(const ba::AttnParams& p, uint32_t* queue, hipStream_t s) {
  auto kern = ba::attn_fwd_queued_kernel<D, WAVES, BLK, OUT_F32>;
  // resident workgroups per compute unit, asked once (a property of the
  // kernel's resources on this architecture)
  static std::atomic<int> per_cu_cached{0};
  int per_cu = per_cu_cached.load();
  if (per_cu < 1) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WAVES * 64, 0) != hipSuccess || per_cu < 1)
      return BA_ERR_HIP;
    per_cu_cached.store(per_cu);
  }
  const long long resident = (long long)device_cus() * per_cu / ba::kNumXcd * ba::kNumXcd;
  const long long wgs = std::max<long long>(ba::kNumXcd, std::min<long long>(resident, round_up8(p.total)));
  kern<<<dim3((unsigned)wgs), WAVES * 64, 0, s>>>(p, queue);
  return BA_OK;
}

template <int D, int WAVES, int BLK>
ba_status launch_attn_queued(const ba::AttnParams& p, bool out_f32, uint32_t* queue, hipStream_t s) {
  return out_f32 ? launch_attn_queued_t<D, WAVES, BLK, true>(p, queue, s)
                 : launch_attn_queued_t<D, WAVES, BLK, false>(p, queue, s);
}

// Workspace of the selection pass: the pooled statistics aq, ak (fp32
// [B*H, n, 2D] each).
size_t select_workspace_bytes(int BH, int n, int D) { return 2 * (size_t)BH * n * 2 * D * sizeof(float); }

// Checks of ba_att_select's arguments other than its workspace.
ba_status check_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, double sparsity,
                       const void* q, const void* k, const uint8_t* block_mask, const int32_t* block_idx,
                       const int32_t* block_cnt, const float* score) {
  ba_status st = check_shape(B, H, N, D);
  if (st != BA_OK) return st;
  if (!q || !k || !block_mask || !block_idx || !block_cnt) return BA_ERR_INVALID_ARG;
  if (!(sparsity >= 0.0 && sparsity < 1.0)) return BA_ERR_INVALID_ARG;
  if (block != 64 && block != 128) return BA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(block_idx, 4) || !aligned(block_cnt, 4) ||
      (score && !aligned(score, 4)))
    return BA_ERR_INVALID_ARG;
  if (num_blocks(N, block) > kMaxSelectBlocks) return BA_ERR_UNSUPPORTED;
  return BA_OK;
}

// The selection pass with the pooled statistics at ws: aq [B*H, n, 2D] then
// ak [B*H, n, 2D], fp32 (checked arguments).
ba_status launch_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                        double sparsity, const void* q, const void* k, uint8_t* block_mask,
                        int32_t* block_idx, int32_t* block_cnt, float* score, float* ws, hipStream_t s) {
  const int n = num_blocks(N, block);
  const int keep = keep_count(n, sparsity);
  const int BH = B * H;
  const float sc = resolve_scale(scale, D);
  float* aq = ws;
  float* ak = aq + (size_t)BH * n * 2 * D;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  if (D == 128) {
    launch_pool<128>(BH, N, n, block, sc, q16, k16, aq, ak, s);
    launch_score<128>(BH, n, keep, aq, ak, block_mask, block_idx, block_cnt, score, s);
  } else {
    launch_pool<64>(BH, N, n, block, sc, q16, k16, aq, ak, s);
    launch_score<64>(BH, n, keep, aq, ak, block_mask, block_idx, block_cnt, score, s);
  }
  return finish_launch();
}

}  // namespace

extern "C" {

int32_t ba_att_num_blocks(int32_t N, int32_t block) {
  if (N < 1 || block < 1) return -1;
  return num_blocks(N, block);
}

int32_t ba_att_keep_count(int32_t n_blocks, double sparsity) {
  if (n_blocks < 1 || !(sparsity >= 0.0 && sparsity < 1.0)) return -1;
  return keep_count(n_blocks, sparsity);
}

size_t ba_att_select_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block) {
  if (check_shape(B, H, N, D) != BA_OK || block < 1) return 0;
  return select_workspace_bytes(B * H, num_blocks(N, block), D);
}

int ba_att_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                  double sparsity, const void* q, const void* k, uint8_t* block_mask,
                  int32_t* block_idx, int32_t* block_cnt, float* score, void* workspace,
                  size_t workspace_bytes, void* stream) {
  ba_status st = check_select(B, H, N, D, block, sparsity, q, k, block_mask, block_idx, block_cnt, score);
  if (st != BA_OK) return st;
  const size_t need = ba_att_select_workspace_bytes(B, H, N, D, block);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return BA_ERR_WORKSPACE;
  return launch_select(B, H, N, D, block, scale, sparsity, q, k, block_mask, block_idx, block_cnt, score,
                       static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------- no-allocation
// Fixed device scratch of ba_att_select_noalloc: the pooled statistics of
// the selection pass for callers that cannot allocate.  One copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): it uses the
// per-device address from hipGetSymbolAddress.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// Address of the current device's scratch, looked up once per device.
ba_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BA_OK;
}
}  // namespace

extern "C" {

int ba_att_select_noalloc(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                          double sparsity, const void* q, const void* k, uint8_t* block_mask,
                          int32_t* block_idx, int32_t* block_cnt, float* score, void* stream) {
  ba_status st = check_select(B, H, N, D, block, sparsity, q, k, block_mask, block_idx, block_cnt, score);
  if (st != BA_OK) return st;
  if (ba_att_select_workspace_bytes(B, H, N, D, block) > kScratchBytes) return BA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != BA_OK) return st;
  return launch_select(B, H, N, D, block, scale, sparsity, q, k, block_mask, block_idx, block_cnt, score,
                       static_cast<float*>(ws), static_cast<hipStream_t>(stream));
}

int ba_att_mask_to_index(int32_t B, int32_t H, int32_t n_blocks, const uint8_t* block_mask,
                         int32_t max_keep, int32_t* block_idx, int32_t* block_cnt, void* stream) {
  if (B < 1 || H < 1 || n_blocks < 1 || max_keep < 1) return BA_ERR_INVALID_ARG;
  if (!block_mask || !block_idx || !block_cnt) return BA_ERR_INVALID_ARG;
  if (!aligned(block_idx, 4) || !aligned(block_cnt, 4)) return BA_ERR_INVALID_ARG;
  if (n_blocks > kMaxBlocksPerRow) return BA_ERR_UNSUPPORTED;
  const long long rows = (long long)B * H * n_blocks;
  if (rows * n_blocks >= (1ll << 31) || rows * max_keep >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((rows + 3) / 4));
  switch (ni_for(n_blocks)) {
    case 1: ba::mask_to_index_kernel<1><<<grid, 256, 0, s>>>(block_mask, (int)rows, n_blocks, max_keep, block_idx, block_cnt); break;
    case 2: ba::mask_to_index_kernel<2><<<grid, 256, 0, s>>>(block_mask, (int)rows, n_blocks, max_keep, block_idx, block_cnt); break;
    case 4: ba::mask_to_index_kernel<4><<<grid, 256, 0, s>>>(block_mask, (int)rows, n_blocks, max_keep, block_idx, block_cnt); break;
    case 8: ba::mask_to_index_kernel<8><<<grid, 256, 0, s>>>(block_mask, (int)rows, n_blocks, max_keep, block_idx, block_cnt); break;
    case 16: ba::mask_to_index_kernel<16><<<grid, 256, 0, s>>>(block_mask, (int)rows, n_blocks, max_keep, block_idx, block_cnt); break;
    default: ba::mask_to_index_kernel<32><<<grid, 256, 0, s>>>(block_mask, (int)rows, n_blocks, max_keep, block_idx, block_cnt); break;
  }
  return finish_launch();
}

}  // extern "C"

namespace {

constexpr int kMaxSplit = 64;

// The forward sorts packed words (key << 16) | (list << 15) | position, with
// key 0xFFFF for an invalid entry, and stores a walk entry's block index in
// 15 bits with 0x7FFF for an invalid one, so every block index must fit in
// 15 bits below 0x7FFF.
static_assert(kMaxN / 64 < 0x7FFF, "block indices of the walk fit 15 bits");
static_assert(BA_ATT_QUEUE_WORDS == ba::kQueueWords, "queue size in the header and the kernel agree");

// Multiplier of the sparse walk order: the integer nearest n/phi (phi the
// golden ratio) that is coprime with n, so that J -> J*g mod n permutes the
// blocks and scatters neighbouring blocks across the walk.
int walk_multiplier(int n) {
  if (n <= 2) return 1;
  auto gcd = [](int a, int b) { while (b) { const int t = a % b; a = b; b = t; } return a; };
  const int g0 = (int)lround(n * 0.6180339887498949);
  for (int d = 0; d < n; ++d) {
    if (g0 - d >= 1 && gcd(g0 - d, n) == 1) return g0 - d;
    if (g0 + d < n && gcd(g0 + d, n) == 1) return g0 + d;
  }
  return 1;
}

// Inverse of the walk multiplier mod n (extended Euclid; the multiplier is
// coprime with n), so that the block of a walk key is key * inverse mod n.
int walk_inverse(int m, int n) {
  if (n <= 1) return 0;
  long long r0 = n, r1 = m % n, t0 = 0, t1 = 1;
  while (r1 != 0) {
    const long long q = r0 / r1, r2 = r0 - q * r1, t2 = t0 - q * t1;
    r0 = r1; r1 = r2; t0 = t1; t1 = t2;
  }
  return (int)(((t0 % n) + n) % n);
}

// Checks of the arguments every forward variant shares.
ba_status check_forward(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, const void* q,
                        const void* k, const void* v, const int32_t* block_idx, const int32_t* block_cnt,
                        int32_t max_keep) {
  ba_status st = check_shape(B, H, N, D);
  if (st != BA_OK) return st;
  if (!q || !k || !v || !block_idx || !block_cnt) return BA_ERR_INVALID_ARG;
  if (block != 64 && block != 128) return BA_ERR_UNSUPPORTED;
  if (max_keep < 1) return BA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(block_idx, 4) ||
      !aligned(block_cnt, 4))
    return BA_ERR_INVALID_ARG;
  if ((long long)B * H * num_blocks(N, block) * max_keep >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  return BA_OK;
}

// Sparse forward into o (o_f32: fp32, else bf16) and lse, cutting every
// row's chunk list into n_split parts written at the given strides, and
// merging an optional external contribution.
ba_status launch_forward(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                         const void* q, const void* k, const void* v, const int32_t* block_idx,
                         const int32_t* block_cnt, int32_t max_keep, int n_split, void* o, bool o_f32,
                         float* lse, size_t o_stride, size_t lse_stride, const float* o_ext,
                         const float* lse_ext, hipStream_t s, uint32_t* queue = nullptr) {
  const int n = num_blocks(N, block);
  // block 128: one four-wave tile per query block; block 64: one four-wave
  // tile per pair of neighbouring query blocks
  const int n_qtiles = block == 64 ? (n + 1) / 2 : n;
  const long long total = (long long)B * H * n_qtiles * n_split;
  if (total >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  ba::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.idx = block_idx;
  p.cnt = block_cnt;
  p.o = o;
  p.lse = lse;
  p.N = N;
  p.n_blocks = n;
  p.n_qtiles = n_qtiles;
  p.total = (int)total;
  p.max_keep = max_keep;
  p.scale_log2 = resolve_scale(scale, D) * 1.44269504088896340736f;
  p.n_split = n_split;
  p.o_part_stride = o_stride;
  p.lse_part_stride = lse_stride;
  p.o_ext = o_ext;
  p.lse_ext = lse_ext;
  p.walk_mul = walk_multiplier(n);
  p.walk_inv = walk_inverse(p.walk_mul, n);
  if (queue != nullptr) {
    ba_status st;
    if (D == 128) st = block == 64 ? launch_attn_queued<128, 4, 64>(p, o_f32, queue, s)
                                   : launch_attn_queued<128, 4, 128>(p, o_f32, queue, s);
    else st = block == 64 ? launch_attn_queued<64, 4, 64>(p, o_f32, queue, s)
                          : launch_attn_queued<64, 4, 128>(p, o_f32, queue, s);
    if (st != BA_OK) return st;
    return finish_launch();
  }
  if (D == 128) {
    if (block == 64) launch_attn<128, 4, 64, true>(p, o_f32, s);
    else launch_attn<128, 4, 128, true>(p, o_f32, s);
  } else {
    if (block == 64) launch_attn<64, 4, 64, true>(p, o_f32, s);
    else launch_attn<64, 4, 128, true>(p, o_f32, s);
  }
  return finish_launch();
}

template <int D>
void launch_merge_d(const float* o_parts, const float* lse_parts, int n_parts, size_t rows, void* o,
                    bool o_f32, float* lse, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (o_f32)
    ba::merge_kernel<D, true><<<grid, 256, 0, s>>>(o_parts, lse_parts, n_parts, rows, o, lse);
  else
    ba::merge_kernel<D, false><<<grid, 256, 0, s>>>(o_parts, lse_parts, n_parts, rows, o, lse);
}

void launch_merge(int D, const float* o_parts, const float* lse_parts, int n_parts, size_t rows, void* o,
                  bool o_f32, float* lse, hipStream_t s) {
  if (D == 128) launch_merge_d<128>(o_parts, lse_parts, n_parts, rows, o, o_f32, lse, s);
  else launch_merge_d<64>(o_parts, lse_parts, n_parts, rows, o, o_f32, lse, s);
}

}  // namespace

extern "C" {

int ba_att_forward(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                   const void* q, const void* k, const void* v, const int32_t* block_idx,
                   const int32_t* block_cnt, int32_t max_keep, void* o, int32_t o_dtype,
                   float* lse, void* stream) {
  ba_status st = check_forward(B, H, N, D, block, q, k, v, block_idx, block_cnt, max_keep);
  if (st != BA_OK) return st;
  if (!o || (o_dtype != BA_BF16 && o_dtype != BA_F32)) return BA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || (lse && !aligned(lse, 4))) return BA_ERR_INVALID_ARG;
  return launch_forward(B, H, N, D, block, scale, q, k, v, block_idx, block_cnt, max_keep, 1, o,
                        o_dtype == BA_F32, lse, 0, 0, nullptr, nullptr, static_cast<hipStream_t>(stream));
}

int ba_att_forward_queued(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                          const void* q, const void* k, const void* v, const int32_t* block_idx,
                          const int32_t* block_cnt, int32_t max_keep, void* o, int32_t o_dtype,
                          float* lse, uint32_t* queue, void* stream) {
  ba_status st = check_forward(B, H, N, D, block, q, k, v, block_idx, block_cnt, max_keep);
  if (st != BA_OK) return st;
  if (!o || (o_dtype != BA_BF16 && o_dtype != BA_F32)) return BA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || (lse && !aligned(lse, 4))) return BA_ERR_INVALID_ARG;
  if (!queue || !aligned(queue, 64)) return BA_ERR_WORKSPACE;
  return launch_forward(B, H, N, D, block, scale, q, k, v, block_idx, block_cnt, max_keep, 1, o,
                        o_dtype == BA_F32, lse, 0, 0, nullptr, nullptr, static_cast<hipStream_t>(stream),
                        queue);
}

size_t ba_att_forward_split_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t n_split) {
  if (check_shape(B, H, N, D) != BA_OK || n_split < 1 || n_split > kMaxSplit) return 0;
  return (size_t)n_split * B * H * N * (size_t)(D + 1) * sizeof(float);
}

int32_t ba_att_forward_split_parts(int32_t B, int32_t H, int32_t N, int32_t block, int32_t max_keep) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN || max_keep < 1 || (block != 64 && block != 128)) return 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 0;
  // resident attention workgroups per compute unit: three four-wave tiles
  // (one query block at block 128, a pair of them at block 64)
  const long long resident = (long long)cus * 3;
  const int n = num_blocks(N, block);
  const long long tiles = (long long)B * H * (block == 64 ? (n + 1) / 2 : n);
  long long parts = resident / tiles;  // the largest count that still fits one round
  parts = std::min(parts, (long long)max_keep * (block / ba::kChunk));
  parts = std::min(parts, (long long)kMaxSplit);
  return (int32_t)std::max(parts, 1ll);
}

int ba_att_forward_split(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                         const void* q, const void* k, const void* v, const int32_t* block_idx,
                         const int32_t* block_cnt, int32_t max_keep, int32_t n_split, void* o,
                         int32_t o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  ba_status st = check_forward(B, H, N, D, block, q, k, v, block_idx, block_cnt, max_keep);
  if (st != BA_OK) return st;
  if (!o || (o_dtype != BA_BF16 && o_dtype != BA_F32)) return BA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || (lse && !aligned(lse, 4))) return BA_ERR_INVALID_ARG;
  if (n_split < 1 || n_split > kMaxSplit) return BA_ERR_INVALID_ARG;
  const size_t need = ba_att_forward_split_workspace_bytes(B, H, N, D, n_split);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return BA_ERR_WORKSPACE;
  const size_t rows = (size_t)B * H * N;
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = o_parts + (size_t)n_split * rows * D;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_forward(B, H, N, D, block, scale, q, k, v, block_idx, block_cnt, max_keep, n_split, o_parts,
                      true, lse_parts, rows * D, rows, nullptr, nullptr, s);
  if (st != BA_OK) return st;
  launch_merge(D, o_parts, lse_parts, n_split, rows, o, o_dtype == BA_F32, lse, s);
  return finish_launch();
}

int ba_att_merge(int32_t B, int32_t H, int32_t N, int32_t D, int32_t n_parts, const float* o_parts,
                 const float* lse_parts, void* o, int32_t o_dtype, float* lse, void* stream) {
  ba_status st = check_shape(B, H, N, D);
  if (st != BA_OK) return st;
  if (n_parts < 1 || n_parts > kMaxSplit || !o_parts || !lse_parts || !o) return BA_ERR_INVALID_ARG;
  if (o_dtype != BA_BF16 && o_dtype != BA_F32) return BA_ERR_INVALID_ARG;
  if (!aligned(o_parts, 16) || !aligned(lse_parts, 4) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
    return BA_ERR_INVALID_ARG;
  if ((long long)n_parts * B * H * N * D >= (1ll << 40)) return BA_ERR_UNSUPPORTED;
  launch_merge(D, o_parts, lse_parts, n_parts, (size_t)B * H * N, o, o_dtype == BA_F32, lse,
               static_cast<hipStream_t>(stream));
  return finish_launch();
}

int ba_att_forward_ext(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                       const void* q, const void* k, const void* v, const int32_t* block_idx,
                       const int32_t* block_cnt, int32_t max_keep, const float* o_ext,
                       const float* lse_ext, void* o, int32_t o_dtype, float* lse, void* stream) {
  ba_status st = check_forward(B, H, N, D, block, q, k, v, block_idx, block_cnt, max_keep);
  if (st != BA_OK) return st;
  if (!o || (o_dtype != BA_BF16 && o_dtype != BA_F32) || !o_ext || !lse_ext) return BA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || (lse && !aligned(lse, 4)) || !aligned(o_ext, 16) || !aligned(lse_ext, 4))
    return BA_ERR_INVALID_ARG;
  return launch_forward(B, H, N, D, block, scale, q, k, v, block_idx, block_cnt, max_keep, 1, o,
                        o_dtype == BA_F32, lse, 0, 0, o_ext, lse_ext, static_cast<hipStream_t>(stream));
}

int ba_att_dense(int32_t B, int32_t H, int32_t N, int32_t D, float scale, const void* q,
                 const void* k, const void* v, void* o, int32_t o_dtype, float* lse, void* stream) {
  ba_status st = check_shape(B, H, N, D);
  if (st != BA_OK) return st;
  if (!q || !k || !v || !o) return BA_ERR_INVALID_ARG;
  if (o_dtype != BA_BF16 && o_dtype != BA_F32) return BA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return BA_ERR_INVALID_ARG;
  ba::AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.N = N;
  p.n_blocks = 0;
  p.n_qtiles = (N + 127) / 128;
  p.total = B * H * p.n_qtiles;
  p.max_keep = 0;
  p.scale_log2 = resolve_scale(scale, D) * 1.44269504088896340736f;
  p.n_split = 1;
  const bool f32 = o_dtype == BA_F32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) launch_attn<128, 4, 64, false>(p, f32, s);
  else launch_attn<64, 4, 64, false>(p, f32, s);
  return finish_launch();
}

}  // extern "C"

// ------------------------------------------------------------ diagnostics
namespace {

constexpr int kMaxMapParts = 4096;  // n * waves per workgroup: 12 bytes each of LDS

template <int D, int WAVES, int BLK>
void launch_block_map(const ba::MapParams& p, hipStream_t s) {
  const size_t smem = (size_t)p.n_blocks * WAVES * 3 * sizeof(float);
  ba::block_map_kernel<D, WAVES, BLK><<<dim3(round_up8(p.total)), WAVES * 64, smem, s>>>(p);
}

// Split of the full-covariance product: part 0 covers the D mean channels
// (so it is the uncorrected score), parts 1..P-1 the 2T moment entries in
// chunks of k_chunk (a multiple of 8), enough parts for ~2048 workgroups.
struct FullPlan {
  int kf, k_chunk, parts, tiles;
};

FullPlan full_plan(int BH, int n, int D) {
  FullPlan f;
  f.kf = D + D * (D + 1);
  f.tiles = (n + 63) / 64;
  const long long tiles = (long long)BH * f.tiles * f.tiles;
  long long split = (2048 + tiles - 1) / tiles;
  if (split < 1) split = 1;
  if (split > 16) split = 16;
  const int rest = f.kf - D;
  f.k_chunk = (int)(((rest + split - 1) / split + 7) / 8 * 8);
  f.parts = 1 + (rest + f.k_chunk - 1) / f.k_chunk;
  return f;
}

template <int D>
void launch_moments(int BH, int N, int n, int block, float scale, const uint16_t* q, const uint16_t* k,
                    float* aqf, float* akf, hipStream_t s) {
  const dim3 grid((unsigned)(2 * BH * n));
  if (block == 64)
    ba::moments_kernel<D, 64><<<grid, 256, 0, s>>>(q, k, aqf, akf, N, n, BH, scale);
  else
    ba::moments_kernel<D, 128><<<grid, 256, 0, s>>>(q, k, aqf, akf, N, n, BH, scale);
}

}  // namespace

extern "C" {

int ba_att_block_map(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                     const void* q, const void* k, const float* lse, float* m_lme, float* m_prob,
                     void* stream) {
  ba_status st = check_shape(B, H, N, D);
  if (st != BA_OK) return st;
  if (!q || !k || !m_lme || ((lse == nullptr) != (m_prob == nullptr))) return BA_ERR_INVALID_ARG;
  if (block != 64 && block != 128) return BA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(m_lme, 4) || (lse && !aligned(lse, 4)) ||
      (m_prob && !aligned(m_prob, 4)))
    return BA_ERR_INVALID_ARG;
  const int n = num_blocks(N, block);
  const int waves = block / 32;
  if ((long long)n * waves > kMaxMapParts) return BA_ERR_UNSUPPORTED;
  const long long total = (long long)B * H * n;
  if (total * n >= (1ll << 40) || total >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  ba::MapParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.lse = lse;
  p.m_lme = m_lme;
  p.m_prob = m_prob;
  p.N = N;
  p.n_blocks = n;
  p.total = (int)total;
  p.scale_log2 = resolve_scale(scale, D) * 1.44269504088896340736f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) {
    if (block == 64) launch_block_map<128, 2, 64>(p, s);
    else launch_block_map<128, 4, 128>(p, s);
  } else {
    if (block == 64) launch_block_map<64, 2, 64>(p, s);
    else launch_block_map<64, 4, 128>(p, s);
  }
  return finish_launch();
}

size_t ba_att_score_full_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block) {
  if (check_shape(B, H, N, D) != BA_OK || (block != 64 && block != 128)) return 0;
  const int n = num_blocks(N, block);
  if (n > kMaxFullScoreBlocks) return 0;
  const int BH = B * H;
  const FullPlan f = full_plan(BH, n, D);
  return (2 * (size_t)BH * n * f.kf + (size_t)f.parts * BH * n * n) * sizeof(float);
}

int ba_att_score_full(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                      const void* q, const void* k, float* s_full, float* s_mean, void* workspace,
                      size_t workspace_bytes, void* stream) {
  ba_status st = check_shape(B, H, N, D);
  if (st != BA_OK) return st;
  if (!q || !k || !s_full) return BA_ERR_INVALID_ARG;
  if (block != 64 && block != 128) return BA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(s_full, 4) || (s_mean && !aligned(s_mean, 4)))
    return BA_ERR_INVALID_ARG;
  const int n = num_blocks(N, block);
  if (n > kMaxFullScoreBlocks) return BA_ERR_UNSUPPORTED;
  const size_t need = ba_att_score_full_workspace_bytes(B, H, N, D, block);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return BA_ERR_WORKSPACE;
  const int BH = B * H;
  const FullPlan f = full_plan(BH, n, D);
  float* aqf = static_cast<float*>(workspace);
  float* akf = aqf + (size_t)BH * n * f.kf;
  float* parts = akf + (size_t)BH * n * f.kf;
  const float sc = resolve_scale(scale, D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  if (D == 128) launch_moments<128>(BH, N, n, block, sc, q16, k16, aqf, akf, s);
  else launch_moments<64>(BH, N, n, block, sc, q16, k16, aqf, akf, s);
  ba::GemmParams g{};
  g.a = aqf;
  g.b = akf;
  g.parts = parts;
  g.n = n;
  g.K = f.kf;
  g.BH = BH;
  g.n_tiles = f.tiles;
  g.k_first = D;
  g.k_chunk = f.k_chunk;
  g.P = f.parts;
  const long long wgs = (long long)f.parts * BH * f.tiles * f.tiles;
  if (wgs >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  ba::gemm_nt_f32_kernel<<<dim3((unsigned)wgs), 256, 0, s>>>(g);
  const size_t count = (size_t)BH * n * n;
  const unsigned grid = (unsigned)((count + 255) / 256 < 4096 ? (count + 255) / 256 : 4096);
  ba::sum_parts_kernel<<<dim3(grid), 256, 0, s>>>(parts, f.parts, count, s_full, s_mean);
  return finish_launch();
}

int ba_att_rank_agreement(int32_t B, int32_t H, int32_t n_blocks, int32_t keep, const float* x,
                          const float* r, float* recall, float* rho, void* stream) {
  if (B < 1 || H < 1 || n_blocks < 1 || keep < 1 || keep > n_blocks) return BA_ERR_INVALID_ARG;
  if (!x || !r || !recall || !rho) return BA_ERR_INVALID_ARG;
  if (!aligned(x, 4) || !aligned(r, 4) || !aligned(recall, 4) || !aligned(rho, 4)) return BA_ERR_INVALID_ARG;
  if (n_blocks > ba::kAgreeMaxN) return BA_ERR_UNSUPPORTED;
  const long long rows = (long long)B * H * n_blocks;
  if (rows * n_blocks >= (1ll << 40) || rows >= (1ll << 31)) return BA_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ne = (n_blocks + 63) / 64;
  if (ne <= 1) ba::rank_agree_kernel<1><<<grid, 256, 0, s>>>(x, r, (int)rows, n_blocks, keep, recall, rho);
  else if (ne <= 2) ba::rank_agree_kernel<2><<<grid, 256, 0, s>>>(x, r, (int)rows, n_blocks, keep, recall, rho);
  else if (ne <= 4) ba::rank_agree_kernel<4><<<grid, 256, 0, s>>>(x, r, (int)rows, n_blocks, keep, recall, rho);
  else ba::rank_agree_kernel<8><<<grid, 256, 0, s>>>(x, r, (int)rows, n_blocks, keep, recall, rho);
  return finish_launch();
}

const char* ba_att_status_string(int status) {
  switch (status) {
    case BA_OK: return "ok";
    case BA_ERR_INVALID_ARG: return "invalid argument";
    case BA_ERR_UNSUPPORTED: return "unsupported shape or size";
    case BA_ERR_WORKSPACE: return "workspace or work queue missing, misaligned or too small";
    case BA_ERR_HIP: return "HIP launch failed";
    case BA_ERR_SCRATCH: return "shape needs more than the 64 MiB fixed scratch of ba_att_select_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
