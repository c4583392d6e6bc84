"""Plain fp64 CPU oracle for Block Approximate Sparse Attention (BA-Att).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark use it.  It shares no code,
tables or constants with the HIP path and imports nothing from it.

Sources (cited by page title and section; no page prints an equation, an
algorithm box or a worked example, so every formula below is a reading):

* [BA-Att review] -- pith.science review of "Efficient Long-Context Modeling
  in Diffusion Language Models via Block Approximate Sparse Attention"
  (arXiv 2605.19726): sections "The pith", "Core claim", "What carries the
  argument", "Load-bearing premise", the abstract, and the referee report.
* [BA-Att listing] -- sota2.com listing of the same paper (abstract).
* [FlashBlock review] -- pith.science review of FlashBlock (arXiv
  2602.05305), sections "Core claim" / "What carries the argument": the
  exact split of a softmax row into two key sets and their recombination in
  log space (used here only as a test identity).

Readings taken where the pages are silent (each is also listed in the
design notes of the repository):

R1  blocks: n = ceil(N / b); block I holds tokens [I*b, min((I+1)*b, N)).
R2  "pre-downsampling" pools each block by the mean over its valid tokens.
R3  "diagonal QK variances" are per-channel population variances (1/|I|).
R4  the "covariance-compensated correction" is the second-cumulant term of
    ln E[exp(X)] ~ E[X] + Var[X]/2 for X = scale*<q_s, k_t>, (s, t) uniform
    on I x J, with the covariances cut to their diagonals:
      S[I,J] = scale*<qm_I, km_J>
             + 0.5*scale^2 * sum_c (vq_Ic*vk_Jc + vq_Ic*km_Jc^2 + qm_Ic^2*vk_Jc)
R5  "norm sorting" orders each query-block row of S descending (lower J
    first on exact ties) and keeps the first keep = n - floor(sp*n + 1e-9)
    blocks, clamped to [1, n].  Normalising a row by its softmax (the
    "norm") is monotone, so it changes no order; it defines the relative cut
    margin 1 - exp(-(s_keep - s_keep+1)).
R6  the attention is exact bidirectional softmax attention restricted to the
    tokens of the kept key blocks (keys >= N do not exist), natural-log LSE
    that includes the softmax scale.
R7  the "oracle post-downsample attention map" is the full N x N attention
    pooled per block pair after the nonlinearity: the block log-mean-exp of
    the logits (the quantity R4 approximates) and, secondarily, the block
    mean of the row-softmax probabilities.
R8  attention results over disjoint key sets (the parts of a split key
    list, or a caller's external contribution such as a cached estimate of
    the dropped blocks) recombine exactly in log space:
      LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p;
    an empty part has LSE_p = -inf and weight 0.
R9  the selection-quality diagnostics (full covariance vs diagonal vs no
    correction, against the post-downsample maps of R7) compare maps row by
    row: block recall = |top_keep(x) & top_keep(r)| / keep with both sets
    taken by the norm-sort rule of R5, and Spearman's rho = the Pearson
    correlation of tie-averaged ranks (0 when a row is constant, where rho
    is undefined).  The uncorrected score is the first-order term of R4
    alone, scale*<qm_I, km_J>.

Parity status: the oracle is pinned by closed forms, exact special cases and
brute force (see the tests); parity with the paper's own equations is
unpinned because the pages print none.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "num_blocks",
    "block_sizes",
    "keep_count",
    "block_stats",
    "compact_score",
    "compact_score_full_cov",
    "uncorrected_score",
    "average_ranks",
    "rank_agreement",
    "norm_sort_row",
    "norm_sort",
    "cut_margins",
    "select_head",
    "select_oracle",
    "postdownsample_map",
    "postdownsample_map_rows",
    "block_attention",
    "block_attention_rows",
    "dense_attention",
    "attention_oracle",
    "merge_attention",
]


# --------------------------------------------------------------------------
# O0: input representation and block partition
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float64.

    A bf16 number is the upper half of an IEEE binary32 word, so shifting
    the 16 bits up and reinterpreting gives the float32 value exactly; the
    float64 conversion is exact as well.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def num_blocks(N: int, b: int) -> int:
    """n = ceil(N/b): the block-wise partition of [BA-Att review, "The pith"]
    (reading R1)."""
    if N < 1 or b < 1:
        raise ValueError("N and b must be positive")
    return -(-N // b)


def block_sizes(N: int, b: int) -> list[int]:
    """|I| for every block; only the last block may be partial (R1)."""
    n = num_blocks(N, b)
    return [min(b, N - I * b) for I in range(n)]


def keep_count(n: int, sparsity: float) -> int:
    """Kept key blocks per query-block row at a block-sparsity ratio.

    [BA-Att review, "The pith" / "Core claim"]: the operator drops a fraction
    of blocks ("half the blocks" at 50 percent sparsity).  Reading R5: a fixed
    count per row, keep = n - floor(sp*n + 1e-9), clamped to [1, n].
    """
    if not (0.0 <= sparsity < 1.0):
        raise ValueError("sparsity must lie in [0, 1)")
    drop = int(math.floor(sparsity * n + 1e-9))
    return max(1, min(n, n - drop))


# --------------------------------------------------------------------------
# O2: block-wise pre-downsampling (mean and diagonal variance per block)
# --------------------------------------------------------------------------

def block_stats(X: np.ndarray, b: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-block channel means and population variances of X [N, D] (fp64).

    [BA-Att review, "What carries the argument"]: a block-wise
    pre-downsampled operation; [abstract]: only the diagonal QK variances are
    used.  Readings R2 (mean over the |I| valid tokens) and R3 (population
    variance).  Two passes: the mean first, then the centred sum of squares.
    """
    X = np.asarray(X, dtype=np.float64)
    N, D = X.shape
    n = num_blocks(N, b)
    mean = np.empty((n, D))
    var = np.empty((n, D))
    for I in range(n):
        rows = X[I * b: min((I + 1) * b, N)]
        m = rows.sum(axis=0) / rows.shape[0]
        mean[I] = m
        var[I] = ((rows - m) ** 2).sum(axis=0) / rows.shape[0]
    return mean, var


# --------------------------------------------------------------------------
# O3: covariance-compensated compact score
# --------------------------------------------------------------------------

def compact_score(qm: np.ndarray, qv: np.ndarray, km: np.ndarray, kv: np.ndarray,
                  scale: float) -> np.ndarray:
    """Corrected compact score S [n_q, n_k] from pooled block statistics.

    [BA-Att review, "Core claim" and abstract]: a correction that stands in
    for the full covariance using only diagonal QK variances.  Reading R4:
    the first-order term scale*<qm_I, km_J> plus half the variance of
    scale*<q, k> over the block pair, keeping only diagonal covariances, which
    leaves three per-channel products.  Each sum over channels is one matrix
    product.
    """
    mean_term = scale * (qm @ km.T)
    var_qk = qv @ kv.T              # sum_c vq_c * vk_c
    var_q_meank = qv @ (km ** 2).T  # sum_c vq_c * km_c^2
    meanq_var_k = (qm ** 2) @ kv.T  # sum_c qm_c^2 * vk_c
    return mean_term + 0.5 * scale * scale * (var_qk + var_q_meank + meanq_var_k)


def compact_score_full_cov(Qb: list[np.ndarray], Kb: list[np.ndarray], scale: float) -> np.ndarray:
    """Diagnostic: the same second-cumulant score with FULL covariances.

    This is what the diagonal correction approximates ([BA-Att review,
    abstract]: the diagonal variances approximate the full covariance).  For
    (s, t) uniform on I x J, q and k are independent, so
    Var[<q,k>] = tr(Cq Ck) + km^T Cq km + qm^T Ck qm.  Qb/Kb are lists of the
    per-block token matrices.  O(D^2) per block pair; diagnostics only.
    """
    stats_q = []
    for X in Qb:
        m = X.mean(axis=0)
        C = (X - m).T @ (X - m) / X.shape[0]
        stats_q.append((m, C))
    stats_k = []
    for X in Kb:
        m = X.mean(axis=0)
        C = (X - m).T @ (X - m) / X.shape[0]
        stats_k.append((m, C))
    S = np.empty((len(Qb), len(Kb)))
    for I, (qm, Cq) in enumerate(stats_q):
        for J, (km, Ck) in enumerate(stats_k):
            var = np.sum(Cq * Ck.T) + km @ Cq @ km + qm @ Ck @ qm
            S[I, J] = scale * (qm @ km) + 0.5 * scale * scale * var
    return S


def uncorrected_score(qm: np.ndarray, km: np.ndarray, scale: float) -> np.ndarray:
    """Diagnostic: the compact score without the covariance correction,
    scale*<qm_I, km_J> -- the first-order term of reading R4 alone, i.e.
    ranking blocks by the logits of their pooled queries and keys."""
    return scale * (qm @ km.T)


# --------------------------------------------------------------------------
# O4: norm sorting into a block mask
# --------------------------------------------------------------------------

def norm_sort_row(s_row: np.ndarray, keep: int) -> list[int]:
    """Kept key blocks of one query-block row, ascending.

    [BA-Att review, "Core claim" / "Load-bearing premise"]: blocks are sorted
    by their score in the downsampled space and the leading ones are kept.
    Reading R5: order by (score descending, block index ascending), keep the
    first `keep`.
    """
    order = sorted(range(len(s_row)), key=lambda J: (-float(s_row[J]), J))
    return sorted(order[:keep])


def norm_sort(S: np.ndarray, keep: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Mask uint8 [n_q, n_k] (1 = kept), idx int32 [n_q, keep] ascending,
    cnt int32 [n_q] for one head."""
    nq, nk = S.shape
    mask = np.zeros((nq, nk), dtype=np.uint8)
    idx = np.zeros((nq, keep), dtype=np.int32)
    for I in range(nq):
        kept = norm_sort_row(S[I], keep)
        mask[I, kept] = 1
        idx[I] = kept
    cnt = np.full(nq, keep, dtype=np.int32)
    return mask, idx, cnt


def average_ranks(x: np.ndarray) -> np.ndarray:
    """1-based ranks of the entries of x, tied entries sharing the mean of
    the ranks they span: rank_i = #{j: x_j < x_i} + (#{j: x_j = x_i} + 1)/2."""
    x = np.asarray(x, dtype=np.float64)
    less = (x[None, :] < x[:, None]).sum(axis=1)
    equal = (x[None, :] == x[:, None]).sum(axis=1)
    return less + (equal + 1) / 2.0


def rank_agreement(x_row: np.ndarray, r_row: np.ndarray, keep: int) -> tuple[float, float]:
    """Selection-quality diagnostic of one query-block row (reading R9).

    [BA-Att review, "Core claim": the pre-downsampled scores stand in for the
    post-downsample map; referee report: how well the diagonal approximation
    ranks blocks is not measured].  Returns (recall, rho):
      recall = |kept(x) & kept(r)| / keep, kept by the norm-sort rule;
      rho    = Pearson correlation of average_ranks(x) and average_ranks(r),
               0 when either row is constant.
    """
    kx = set(norm_sort_row(x_row, keep))
    kr = set(norm_sort_row(r_row, keep))
    recall = len(kx & kr) / keep
    a = average_ranks(x_row)
    b = average_ranks(r_row)
    a = a - a.mean()
    b = b - b.mean()
    den = math.sqrt(float(np.sum(a * a)) * float(np.sum(b * b)))
    rho = float(np.sum(a * b)) / den if den > 0 else 0.0
    return recall, rho


def cut_margins(S: np.ndarray, keep: int) -> np.ndarray:
    """Relative margin of each row's cut on the row-normalised scores.

    With p = softmax(S[I, :]) (the "norm" of reading R5), the relative gap
    between the last kept and the first dropped block is
    (p_keep - p_keep+1) / p_keep = 1 - exp(-(s_keep - s_keep+1)).  Rows with
    keep == n have no cut and report +inf.
    """
    nq, nk = S.shape
    out = np.full(nq, np.inf)
    if keep >= nk:
        return out
    for I in range(nq):
        srt = sorted((float(x) for x in S[I]), reverse=True)
        out[I] = -math.expm1(-(srt[keep - 1] - srt[keep]))
    return out


def select_head(q: np.ndarray, k: np.ndarray, b: int, sparsity: float, scale: float):
    """Selection pass for one head: q, k fp64 [N, D].

    Returns (mask, idx, cnt, S, stats) with stats = (qm, qv, km, kv).
    """
    n = num_blocks(q.shape[0], b)
    keep = keep_count(n, sparsity)
    qm, qv = block_stats(q, b)
    km, kv = block_stats(k, b)
    S = compact_score(qm, qv, km, kv, scale)
    mask, idx, cnt = norm_sort(S, keep)
    return mask, idx, cnt, S, (qm, qv, km, kv)


def select_oracle(q_bits: np.ndarray, k_bits: np.ndarray, b: int, sparsity: float,
                  scale: float | None = None, heads=None):
    """Selection pass over [B, H, N, D] bf16 bit arrays.

    `heads` optionally restricts the work to a list of (batch, head) pairs.
    Returns dict with mask [B,H,n,n], idx [B,H,n,keep], cnt [B,H,n],
    S [B,H,n,n] (fp64) and the pooled statistics; unselected heads are zero.
    """
    B, H, N, D = q_bits.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    n = num_blocks(N, b)
    keep = keep_count(n, sparsity)
    out = {
        "mask": np.zeros((B, H, n, n), dtype=np.uint8),
        "idx": np.zeros((B, H, n, keep), dtype=np.int32),
        "cnt": np.zeros((B, H, n), dtype=np.int32),
        "S": np.zeros((B, H, n, n)),
        "qm": np.zeros((B, H, n, D)), "qv": np.zeros((B, H, n, D)),
        "km": np.zeros((B, H, n, D)), "kv": np.zeros((B, H, n, D)),
        "keep": keep, "n": n, "scale": scale,
    }
    if heads is None:
        heads = [(bi, hi) for bi in range(B) for hi in range(H)]
    for bi, hi in heads:
        q = bf16_bits_to_f64(q_bits[bi, hi])
        k = bf16_bits_to_f64(k_bits[bi, hi])
        mask, idx, cnt, S, (qm, qv, km, kv) = select_head(q, k, b, sparsity, scale)
        out["mask"][bi, hi] = mask
        out["idx"][bi, hi] = idx
        out["cnt"][bi, hi] = cnt
        out["S"][bi, hi] = S
        out["qm"][bi, hi], out["qv"][bi, hi] = qm, qv
        out["km"][bi, hi], out["kv"][bi, hi] = km, kv
    return out


# --------------------------------------------------------------------------
# O1: brute-force post-downsample attention map
# --------------------------------------------------------------------------

def postdownsample_map(q: np.ndarray, k: np.ndarray, b: int, scale: float):
    """The oracle post-downsample map of [BA-Att review, "Core claim"] (R7).

    Full logits X = scale*q k^T, then per block pair:
      M_lme[I,J]  = ln( mean_{s in I, t in J} exp(X[s,t]) )
      M_prob[I,J] = mean_{s in I, t in J} softmax_row(X)[s,t]
    Quadratic in N: small inputs only.
    """
    N = q.shape[0]
    n = num_blocks(N, b)
    X = scale * (q @ k.T)
    rowmax = X.max(axis=1, keepdims=True)
    E = np.exp(X - rowmax)
    P = E / E.sum(axis=1, keepdims=True)
    M_lme = np.empty((n, n))
    M_prob = np.empty((n, n))
    for I in range(n):
        rs = slice(I * b, min((I + 1) * b, N))
        for J in range(n):
            cs = slice(J * b, min((J + 1) * b, N))
            blk = X[rs, cs]
            m = blk.max()
            M_lme[I, J] = m + math.log(np.exp(blk - m).mean())
            M_prob[I, J] = P[rs, cs].mean()
    return M_lme, M_prob


def postdownsample_map_rows(q: np.ndarray, k: np.ndarray, b: int, scale: float, blocks):
    """Rows `blocks` (query-block indices) of both maps of postdownsample_map,
    from the logits of those blocks' queries only: X_I = scale * q_I k^T,
    row-softmax normalised over all N keys, pooled per key block."""
    N = q.shape[0]
    n = num_blocks(N, b)
    M_lme = np.empty((len(blocks), n))
    M_prob = np.empty((len(blocks), n))
    for a, I in enumerate(blocks):
        rs = slice(I * b, min((I + 1) * b, N))
        X = scale * (q[rs] @ k.T)
        rowmax = X.max(axis=1, keepdims=True)
        E = np.exp(X - rowmax)
        P = E / E.sum(axis=1, keepdims=True)
        for J in range(n):
            cs = slice(J * b, min((J + 1) * b, N))
            blk = X[:, cs]
            m = blk.max()
            M_lme[a, J] = m + math.log(np.exp(blk - m).mean())
            M_prob[a, J] = P[:, cs].mean()
    return M_lme, M_prob


# --------------------------------------------------------------------------
# O5 / O6: block-sparse and dense attention
# --------------------------------------------------------------------------

def _softmax_attention(x_logits: np.ndarray, v: np.ndarray):
    """Rows of exact softmax attention from fp64 logits [r, T] and values
    [T, D]: LSE = m + ln sum exp(x - m), O = sum exp(x - LSE) v."""
    m = x_logits.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(x_logits - m).sum(axis=1, keepdims=True))
    O = np.exp(x_logits - lse) @ v
    return O, lse[:, 0]


def _kept_keys(mask_row: np.ndarray, b: int, N: int) -> np.ndarray:
    """Token indices t < N of the key blocks kept in one mask row."""
    parts = [np.arange(J * b, min((J + 1) * b, N)) for J in range(len(mask_row)) if mask_row[J]]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def block_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                    b: int, scale: float):
    """Block-sparse attention for one head (reading R6).

    [BA-Att review, "The pith"]: attention is computed only over the kept
    blocks.  For every valid query s of block I the logits scale*<q_s, k_t>
    run over the tokens t < N of the key blocks J with mask[I, J] == 1.
    Returns O [N, D] and LSE [N] (natural log, scale included).  A row whose
    mask keeps no block has an empty key set: the empty sum gives O = 0 and
    LSE = ln 0 = -inf.
    """
    N = q.shape[0]
    n = num_blocks(N, b)
    O = np.zeros_like(v, dtype=np.float64)
    lse = np.zeros(N)
    for I in range(n):
        rows = np.arange(I * b, min((I + 1) * b, N))
        keys = _kept_keys(mask[I], b, N)
        if keys.size == 0:
            O[rows], lse[rows] = 0.0, -np.inf
            continue
        X = scale * (q[rows] @ k[keys].T)
        O[rows], lse[rows] = _softmax_attention(X, v[keys])
    return O, lse


def block_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                         b: int, scale: float, rows):
    """Block-sparse attention for a chosen subset of query rows only (same
    definition as `block_attention`); used for sampled parity at full size."""
    N = q.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, v.shape[1]))
    lse = np.zeros(rows.size)
    for i, s in enumerate(rows):
        I = int(s) // b
        keys = _kept_keys(mask[I], b, N)
        if keys.size == 0:
            O[i], lse[i] = 0.0, -np.inf
            continue
        X = scale * (q[s:s + 1] @ k[keys].T)
        O[i:i + 1], lse[i:i + 1] = _softmax_attention(X, v[keys])
    return O, lse


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows=None):
    """Textbook full bidirectional attention softmax(scale*q k^T) v with its
    natural-log LSE; the comparator that the pages quote their speedup
    against ([BA-Att review, "If this is right"]).  `rows` restricts the
    queries."""
    qs = q if rows is None else q[np.asarray(rows)]
    return _softmax_attention(scale * (qs @ k.T), v)


def attention_oracle(q_bits, k_bits, v_bits, mask, b: int, scale: float | None = None,
                     heads=None, rows=None):
    """Block-sparse attention over [B,H,N,D] bf16 bit arrays and a mask
    [B,H,n,n].  `heads` restricts to (batch, head) pairs; `rows` (an array of
    query indices) restricts the queries of every selected head.
    Returns {(bi, hi): (O, LSE)}."""
    B, H, N, D = q_bits.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if heads is None:
        heads = [(bi, hi) for bi in range(B) for hi in range(H)]
    res = {}
    for bi, hi in heads:
        q = bf16_bits_to_f64(q_bits[bi, hi])
        k = bf16_bits_to_f64(k_bits[bi, hi])
        v = bf16_bits_to_f64(v_bits[bi, hi])
        if rows is None:
            res[(bi, hi)] = block_attention(q, k, v, mask[bi, hi], b, scale)
        else:
            res[(bi, hi)] = block_attention_rows(q, k, v, mask[bi, hi], b, scale, rows)
    return res


# --------------------------------------------------------------------------
# O7: recombination of attention over disjoint key sets
# --------------------------------------------------------------------------

def merge_attention(o_parts, lse_parts):
    """Exact recombination of attention over disjoint key sets (reading R8).

    [FlashBlock review, "Core claim" / "What carries the argument"]: the
    softmax of a row over the union of disjoint key sets is assembled from
    each set's normalised output and log-normaliser.  With LSE_p = ln Z_p and
    O_p = (1/Z_p) sum_{t in T_p} e^{x_t} v_t, the union has Z = sum_p Z_p, so
    LSE = ln sum_p e^{LSE_p} and O = sum_p (Z_p/Z) O_p.

    o_parts [P, ..., D], lse_parts [P, ...].  Parts with LSE_p = -inf are
    empty (weight 0); when every part is empty, O = 0 and LSE = -inf.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    nonempty = np.isfinite(m)
    m0 = np.where(nonempty, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m0), 0.0)  # Z_p / e^m
    z = w.sum(axis=0)
    z1 = np.where(nonempty, z, 1.0)
    lse = np.where(nonempty, m0 + np.log(z1), -np.inf)
    O = (w[..., None] * o_parts).sum(axis=0) / z1[..., None]
    O = np.where(nonempty[..., None], O, 0.0)
    return O, lse
