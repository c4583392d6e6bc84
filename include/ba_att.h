/*
 * ba_att.h -- C ABI of the MI355X (gfx950) Block Approximate Sparse Attention
 * (BA-Att) operator.
 *
 * The operator is the one described in the pith.science review of
 * "Efficient Long-Context Modeling in Diffusion Language Models via Block
 * Approximate Sparse Attention" (arXiv 2605.19726), sections "The pith",
 * "Core claim", "What carries the argument" and the abstract: attention for a
 * bidirectional layer is computed in two passes,
 *
 *   1. selection -- pool Q and K per block (mean and diagonal variance),
 *      score the compact block map with a correction built from the diagonal
 *      QK variances, and norm-sort every query-block row to keep a fixed
 *      number of key blocks (ba_att_select);
 *   2. attention -- exact softmax attention of every query restricted to the
 *      tokens of the kept key blocks (ba_att_forward).
 *
 * ba_att_dense is the full-attention comparator the speedup is quoted
 * against (same review, "If this is right": acceleration over
 * FlashAttention).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are contiguous, row-major [B, H, N, D] (D fastest); Q, K, V are
 *    bf16 (raw 16-bit patterns), O is bf16 or fp32, LSE is fp32 [B, H, N].
 *  - Blocks: n = ceil(N / block); block I holds tokens
 *    [I*block, min((I+1)*block, N)); the last block may be partial.
 *  - Block masks are uint8 [B, H, n, n] (row = query block, column = key
 *    block, 1 = kept).  Block index lists are int32 [B, H, n, max_keep]
 *    (kept key-block indices of each row, ascending) with int32 counts
 *    [B, H, n].
 *  - scale <= 0 selects the default softmax scale 1/sqrt(D).
 *  - Supported: D in {64, 128}; block in {64, 128}; 1 <= N <= 2^20;
 *    B*H*N*D < 2^31 elements.  The selection pass (ba_att_select) and
 *    ba_att_mask_to_index further need n <= 2048 key blocks per row
 *    (N <= 131072 at block 64, N <= 262144 at block 128); the diagnostics
 *    state their own limits.  Shapes beyond a limit return
 *    BA_ERR_UNSUPPORTED.
 *  - Every pointer argument is a DEVICE pointer on the current HIP device,
 *    16-byte aligned (the mask, idx and cnt buffers 4-byte aligned), owned by
 *    the caller.  The library allocates nothing and never synchronises the
 *    host: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and completes asynchronously.  Results depend on no state kept
 *    between calls (the library caches only device properties, such as the
 *    resident workgroups per compute unit of ba_att_forward_queued's kernel;
 *    ba_att_select_noalloc's fixed scratch is described there).
 *  - Errors: every argument is checked on the host before anything is
 *    launched; a failed check returns a nonzero ba_status and enqueues
 *    nothing.  After the launches hipGetLastError() is checked and a launch
 *    failure returns BA_ERR_HIP.  Faults during execution surface at the
 *    caller's next synchronisation.
 */
#ifndef BA_ATT_H
#define BA_ATT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_OK = 0,
  BA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, sparsity outside [0,1), misalignment */
  BA_ERR_UNSUPPORTED = 2, /* D or block outside the supported set, sizes too large */
  BA_ERR_WORKSPACE = 3,   /* workspace or work queue missing, misaligned or too small */
  BA_ERR_HIP = 4,         /* a HIP launch failed */
  BA_ERR_SCRATCH = 5      /* ba_att_select_noalloc: the shape needs more than its fixed scratch */
} ba_status;

typedef enum { BA_BF16 = 0, BA_F32 = 1 } ba_dtype;

/* Number of blocks n = ceil(N / block) (block partition of the review's
 * "The pith": the attention space is downsampled block-wise).  Returns -1
 * when N < 1 or block < 1. */
int32_t ba_att_num_blocks(int32_t N, int32_t block);

/* Kept key blocks per query-block row at a block-sparsity ratio (review,
 * "Core claim": half the blocks are dropped at 50% sparsity).  Fixed count
 * keep = n - floor(sparsity*n + 1e-9), clamped to [1, n].  Returns -1 when
 * n_blocks < 1 or sparsity is outside [0, 1). */
int32_t ba_att_keep_count(int32_t n_blocks, double sparsity);

/* Bytes of device workspace ba_att_select needs: the pooled block statistics
 * of Q and K, 2 * B*H*n * 2*D fp32.  Returns 0 for invalid sizes.  (A helper
 * of this interface; the pages define no workspace.) */
size_t ba_att_select_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block);

/* Selection pass (review, "What carries the argument": block-wise
 * pre-downsampling, norm sorting and the diagonal-variance correction).
 *
 * For every (b, h) and block, means m and population variances v of Q and
 * K over the block's valid tokens; then the corrected compact score
 *   S[I,J] = scale*<mq_I, mk_J>
 *          + scale^2/2 * sum_c (vq_Ic*vk_Jc + vq_Ic*mk_Jc^2 + mq_Ic^2*vk_Jc)
 * and, per query-block row, the keep = ba_att_keep_count(n, sparsity) key
 * blocks of largest S (ties: lower J first).
 *
 *   q, k        bf16 [B,H,N,D]                                     (in)
 *   block_mask  uint8 [B,H,n,n], 1 = kept                          (out)
 *   block_idx   int32 [B,H,n,keep], kept J ascending               (out)
 *   block_cnt   int32 [B,H,n], all equal to keep                   (out)
 *   score       fp32 [B,H,n,n] (the map S), or NULL to skip        (out)
 *   workspace   >= ba_att_select_workspace_bytes(...) bytes        (scratch)
 * Supported: n <= 2048 (otherwise BA_ERR_UNSUPPORTED). */
int ba_att_select(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                  double sparsity, const void* q, const void* k, uint8_t* block_mask,
                  int32_t* block_idx, int32_t* block_cnt, float* score, void* workspace,
                  size_t workspace_bytes, void* stream);

/* ba_att_select without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace),
 * checks and results as ba_att_select, bit for bit.  The pooled statistics
 * go to a fixed scratch array in the library's device code: 64 MiB per GPU,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends.  A shape whose ba_att_select_workspace_bytes exceeds
 * 64 MiB (67108864 bytes) returns BA_ERR_SCRATCH and launches nothing.  The
 * call allocates nothing.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (concurrent streams, or host threads on the
 * same device) race and must be serialised by the caller; consecutive calls
 * on one stream are safe, since each call writes every scratch entry it
 * reads. */
int ba_att_select_noalloc(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                          double sparsity, const void* q, const void* k, uint8_t* block_mask,
                          int32_t* block_idx, int32_t* block_cnt, float* score, void* stream);

/* Compacts a block mask into index lists, so a caller's own mask can drive
 * ba_att_forward.  (A helper of this interface, not an operation of the
 * pages: the block mask is their statement of the selection, the index list
 * is this library's compacted form of it.)  Per row: block_cnt = number of
 * ones; block_idx holds the ascending indices of the first
 * min(cnt, max_keep) ones (a row with more than max_keep ones is truncated,
 * detectable as cnt > max_keep).
 *   block_mask uint8 [B,H,n,n] (in); block_idx int32 [B,H,n,max_keep],
 *   block_cnt int32 [B,H,n] (out).  Supported: n <= 2048. */
int ba_att_mask_to_index(int32_t B, int32_t H, int32_t n_blocks, const uint8_t* block_mask,
                         int32_t max_keep, int32_t* block_idx, int32_t* block_cnt, void* stream);

/* Block-sparse attention pass (review, "The pith": attention only over the
 * selected blocks).  For every valid query s of block I, exact softmax over
 * the tokens t < N of the key blocks block_idx[b,h,I,0:cnt) with
 * cnt = min(block_cnt[b,h,I], max_keep):
 *   LSE_s = ln sum_t exp(scale*<q_s,k_t>),  O_s = sum_t exp(scale*<q_s,k_t> - LSE_s) v_t.
 * Entries outside [0, n) are skipped; entries must be distinct (a repeated
 * entry is counted twice).  A row with no valid entry gives O = 0 and
 * LSE = -inf.  The entries may come in any order: the kernel visits them in
 * an order of its own (one shared by every row), so results equal the
 * oracle's up to fp32 rounding order.  o must not overlap any input: the
 * kernel keeps its reordered list in a row's own output rows until it
 * writes them.
 *   q, k, v  bf16 [B,H,N,D] (in); block_idx/block_cnt as above (in);
 *   o        [B,H,N,D] of o_dtype (BA_BF16 or BA_F32) (out);
 *   lse      fp32 [B,H,N] natural log including the scale, or NULL (out). */
int ba_att_forward(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                   const void* q, const void* k, const void* v, const int32_t* block_idx,
                   const int32_t* block_cnt, int32_t max_keep, void* o, int32_t o_dtype,
                   float* lse, void* stream);

/* Words of the work queue of ba_att_forward_queued (64 bytes). */
#define BA_ATT_QUEUE_WORDS 16

/* ba_att_forward with its tiles dealt from a work queue: the persistent,
 * XCD-aware form of the block-sparse attention pass.  The operation is
 * ba_att_forward's (review, "The pith": attention over the selected blocks
 * only); the scheduling is this library's, not the pages'.  The launch holds only
 * the workgroups the device keeps resident; each takes query tiles from one
 * queue per XCD (a contiguous range of tiles in head order, so an XCD's
 * workgroups share its L2) and, once that is empty, from the other XCDs'
 * queues, so XCDs that run faster or draw cheaper tiles take more of them.
 * Every row is computed by the same code as in ba_att_forward, so results
 * are bit-identical to ba_att_forward's.  ba_att_forward deals every XCD an
 * equal range of heads, so it is the faster call when every row keeps the
 * same number of blocks (ba_att_select's lists); this call is the faster
 * one when the kept counts vary from head to head.
 *   queue  uint32 [BA_ATT_QUEUE_WORDS], device memory, 64-byte aligned,
 *          caller-owned.  It must hold zeros when the call's kernel starts,
 *          and the kernel leaves it zero when it ends: zero it once when it
 *          is allocated, then reuse it for every call on one stream.  Calls
 *          whose kernels can run at the same time (different streams) need
 *          different queues.  A queue that does not start at zero leaves
 *          the results undefined (tiles skipped, or computed twice by
 *          workgroups that race on their output rows); the launch still
 *          ends and stays within the buffers.
 *          NULL or misaligned: BA_ERR_WORKSPACE.
 * Other arguments, checks and errors as in ba_att_forward. */
int ba_att_forward_queued(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                          const void* q, const void* k, const void* v, const int32_t* block_idx,
                          const int32_t* block_cnt, int32_t max_keep, void* o, int32_t o_dtype,
                          float* lse, uint32_t* queue, void* stream);

/* Split key lists (split-KV).  Every row's list of kept key blocks is cut
 * into n_split contiguous parts (1 <= n_split <= 64); each part is attended
 * by its own workgroup into fp32 partial results in the workspace, and the
 * parts are then recombined exactly in log space (see ba_att_merge).  For
 * shapes whose B*H*n workgroups cannot fill the device (few heads, short
 * sequences); the result equals ba_att_forward's up to fp32 rounding.
 * Workspace: ba_att_forward_split_workspace_bytes(...) bytes, 16-byte
 * aligned: n_split partial outputs fp32 [B,H,N,D] then n_split partial LSEs
 * fp32 [B,H,N].  Other arguments as in ba_att_forward. */
size_t ba_att_forward_split_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t n_split);

/* Suggested n_split for ba_att_forward_split on the current device: the
 * largest P whose B*H*T*P workgroups still fit in one round of the device
 * (its compute units times 3 resident four-wave attention tiles), with T the
 * tiles per head (n at block 128, one per pair of query blocks, ceil(n/2),
 * at block 64), at most the chunks of a full list (max_keep*block/64) and
 * 64.  1 means the unsplit launch already fills the device.  Host only (one
 * device query); returns 0 on invalid arguments or when the device cannot
 * be queried.  (A helper of this interface, not an operation of the pages.) */
int32_t ba_att_forward_split_parts(int32_t B, int32_t H, int32_t N, int32_t block, int32_t max_keep);
int ba_att_forward_split(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                         const void* q, const void* k, const void* v, const int32_t* block_idx,
                         const int32_t* block_cnt, int32_t max_keep, int32_t n_split, void* o,
                         int32_t o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Exact recombination of attention results over disjoint key sets
 * (FlashBlock review, "Core claim" / "What carries the argument": a softmax
 * row over a union of key sets assembled from each set's output and
 * log-normaliser):
 *   LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p.
 * A part with LSE_p = -inf is empty and weighs 0; if every part is empty the
 * row gets O = 0 and LSE = -inf.
 *   o_parts    fp32 [n_parts,B,H,N,D], 16-byte aligned       (in)
 *   lse_parts  fp32 [n_parts,B,H,N], natural log             (in)
 *   o          [B,H,N,D] of o_dtype; lse fp32 [B,H,N] or NULL (out)
 * 1 <= n_parts <= 64. */
int ba_att_merge(int32_t B, int32_t H, int32_t N, int32_t D, int32_t n_parts, const float* o_parts,
                 const float* lse_parts, void* o, int32_t o_dtype, float* lse, void* stream);

/* Block-sparse attention merged with an external contribution: the caller's
 * attention result (o_ext fp32 [B,H,N,D], lse_ext fp32 [B,H,N], natural log)
 * over a key set disjoint from the kept blocks -- for instance a cached
 * estimate of the dropped blocks, as in FlashBlock's sparse-plus-residual
 * combination (FlashBlock review, "What carries the argument") -- is folded
 * into the result as by ba_att_merge with two parts.  With o_ext/lse_ext the
 * attention over the complementary blocks the result is dense attention.
 * Other arguments as in ba_att_forward. */
int ba_att_forward_ext(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                       const void* q, const void* k, const void* v, const int32_t* block_idx,
                       const int32_t* block_cnt, int32_t max_keep, const float* o_ext,
                       const float* lse_ext, void* o, int32_t o_dtype, float* lse, void* stream);

/* Dense bidirectional attention softmax(scale*Q K^T) V with its LSE; the
 * comparator of the sparse pass.  Arguments as in ba_att_forward. */
int ba_att_dense(int32_t B, int32_t H, int32_t N, int32_t D, float scale, const void* q,
                 const void* k, const void* v, void* o, int32_t o_dtype, float* lse, void* stream);

/* ---- selection-quality diagnostics -------------------------------------
 * The review's "Core claim" and abstract have the diagonal-variance score
 * stand in for the full covariance, and the pre-downsampled scores stand in
 * for the post-downsample attention map; its referee report notes that
 * neither approximation is quantified.  These calls measure both.  They are
 * not on the attention path. */

/* Exact post-downsample maps of full attention (the review's "oracle"
 * post-downsample map), for x = scale*<q_s, k_t> over all tokens:
 *   m_lme[b,h,I,J]  = ln( mean_{s in I, t in J} exp(x_st) )
 *   m_prob[b,h,I,J] = mean_{s in I, t in J} exp(x_st - LSE_s)
 * with LSE_s the natural-log normaliser of row s over all keys, passed in as
 * `lse` (fp32 [B,H,N], e.g. ba_att_dense's).  lse and m_prob are both NULL
 * (M_prob not computed) or both set.  m_lme, m_prob fp32 [B,H,n,n] (out).
 * Cost: the score half of dense attention.  Supported: n*block/32 <= 4096
 * (N <= 131072). */
int ba_att_block_map(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                     const void* q, const void* k, const float* lse, float* m_lme, float* m_prob,
                     void* stream);

/* Block scores without the diagonal restriction and without any correction:
 *   s_full[b,h,I,J] = scale*<qm_I, km_J>
 *                     + scale^2/2 * ( <Cq_I, Ck_J>_F + km_J' Cq_I km_J + qm_I' Ck_J qm_I )
 *   s_mean[b,h,I,J] = scale*<qm_I, km_J>            (optional, may be NULL)
 * qm, km are block means and Cq, Ck the population (1/|I|) covariance
 * matrices of the block's tokens.  s_full is the same second-cumulant score
 * as ba_att_select's with the covariances kept whole.  Computed as one fp32
 * product of augmented rows of D + D(D+1) entries (means, packed upper
 * triangles of the second moments).  Workspace:
 * ba_att_score_full_workspace_bytes(...) bytes, 16-byte aligned.  That is
 * 2*B*H*n*(D + D(D+1))*4 bytes for the augmented rows (545 MB at
 * B1 H32 N8192 D128 b64) plus the split-product parts.  Supported: n <= 512.
 * Returns 0 bytes for an unsupported shape. */
size_t ba_att_score_full_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block);
int ba_att_score_full(int32_t B, int32_t H, int32_t N, int32_t D, int32_t block, float scale,
                      const void* q, const void* k, float* s_full, float* s_mean, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Row-by-row agreement of a block score map x with a reference map r (both
 * fp32 [B,H,n,n]):
 *   recall[b,h,I] = |kept(x row) & kept(r row)| / keep, where kept() is the
 *                   norm-sort rule of ba_att_select (value descending, ties
 *                   to the lower index, first `keep`);
 *   rho[b,h,I]    = Spearman's rank correlation, the Pearson correlation of
 *                   tie-averaged ranks, or 0 when either row is constant.
 * Both comparisons are made on the fp32 values as given.  recall, rho fp32
 * [B,H,n] (out).  Supported: 1 <= keep <= n <= 512. */
int ba_att_rank_agreement(int32_t B, int32_t H, int32_t n_blocks, int32_t keep, const float* x,
                          const float* r, float* recall, float* rho, void* stream);

/* Static description of a status code.  (A helper of this interface; not an
 * operation of the pages.) */
const char* ba_att_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BA_ATT_H */
