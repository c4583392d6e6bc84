"""Pins of the fp64 CPU oracle against closed forms, exact special cases,
library routines and brute force (CPU only).

No page prints an equation or a worked example for BA-Att, so every pin
here is mathematical: the oracle's reading of the selection score is the
second-order cumulant expansion of the block log-mean-exp, and blocks built
from all sign patterns give that log-mean-exp in closed form.  The
mutation tests at the end plant plausible mistakes in copies of the oracle's
steps and check that some pin rejects each of them.
"""

import itertools
import math

import numpy as np
import pytest
import scipy.special

from oracle import ba_att_oracle as orc


# ---------------------------------------------------------------- helpers

def sign_block(mean, sigma):
    """All 2^D sign patterns around `mean` with per-channel amplitude
    `sigma`: token s has channel c equal to mean_c + sigma_c * (+1 if bit c of
    s is set else -1).  Channel means are exactly `mean`, population
    variances exactly sigma^2, and distinct channels are uncorrelated."""
    D = len(mean)
    s = np.arange(2 ** D)[:, None]
    h = np.where((s >> np.arange(D)[None, :]) & 1, 1.0, -1.0)
    return np.asarray(mean)[None, :] + h * np.asarray(sigma)[None, :]


def closed_form_lme(qm, qs, km, ks, scale):
    """ln mean exp(scale <q, k>) over all (q, k) pairs of two sign blocks.
    Every (h, g) in {+-1}^D x {+-1}^D appears once, so the channels are
    independent and the mean of the exponential factorises over channels
    into the average of the four sign combinations of each channel."""
    tot = 0.0
    for c in range(len(qm)):
        e = 0.0
        for h, g in itertools.product((-1.0, 1.0), repeat=2):
            e += math.exp(scale * (qm[c] + qs[c] * h) * (km[c] + ks[c] * g))
        tot += math.log(e / 4.0)
    return tot


def oracle_pair_score(Xq, Xk, scale, stats=orc.block_stats, score=orc.compact_score):
    """Oracle S for one query block and one key block given their tokens."""
    b = Xq.shape[0]
    qm, qv = stats(Xq, b)
    km, kv = stats(Xk, b)
    return float(score(qm, qv, km, kv, scale)[0, 0])


def order_ratio(qm, qs0, km, ks0, scale, stats=orc.block_stats, score=orc.compact_score,
                eps=(0.2, 0.1)):
    """err(eps)/err(eps/2) of |S - M_lme| when the within-block amplitudes
    shrink with eps (ratio 16 = fourth order, 4 = second order)."""
    errs = []
    for e in eps:
        qs, ks = e * np.asarray(qs0), e * np.asarray(ks0)
        S = oracle_pair_score(sign_block(qm, qs), sign_block(km, ks), scale, stats, score)
        errs.append(abs(S - closed_form_lme(qm, qs, km, ks, scale)))
    return errs[0] / errs[1], errs


def topk_valid(values, kept, keep):
    """Brute force: `kept` has `keep` elements and every kept index precedes
    every dropped one in the order (value desc, index asc)."""
    kept = set(int(j) for j in kept)
    if len(kept) != keep:
        return False
    for a in kept:
        for d in set(range(len(values))) - kept:
            if (values[a], -a) < (values[d], -d):
                return False
    return True


RNG = np.random.default_rng(7)
D4_QM = RNG.normal(size=4)
D4_KM = RNG.normal(size=4)
D4_QS = RNG.uniform(0.5, 1.5, size=4)
D4_KS = RNG.uniform(0.5, 1.5, size=4)


# ---------------------------------------------------------------- O0

def test_bf16_upcast_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    got = orc.bf16_bits_to_f64(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, 0.0, -0.0]
    assert list(got) == want


def test_partition_and_tail():
    assert orc.num_blocks(1024, 64) == 16
    assert orc.num_blocks(8192, 64) == 128
    assert orc.num_blocks(32760, 128) == 256
    assert orc.block_sizes(32760, 128)[-1] == 120
    assert orc.block_sizes(32760, 128)[:-1] == [128] * 255
    assert orc.num_blocks(1, 64) == 1 and orc.block_sizes(1, 64) == [1]


@pytest.mark.parametrize("n,sp,keep", [
    (16, 0.5, 8), (128, 0.5, 64), (256, 0.5, 128), (256, 0.75, 64), (256, 0.0, 256),
    (128, 0.999, 1), (1, 0.5, 1), (3, 1 / 3, 2), (10, 0.3, 7), (10, 0.7, 3),
    (100, 0.29, 71),  # 0.29*100 is 28.999999999999996 in binary64
])
def test_keep_count(n, sp, keep):
    assert orc.keep_count(n, sp) == keep


def test_keep_count_rejects_out_of_range():
    for sp in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            orc.keep_count(16, sp)


# ---------------------------------------------------------------- O2

def test_block_stats_closed_forms():
    # sign blocks: exact means and population variances
    X = sign_block(D4_QM, D4_QS)
    m, v = orc.block_stats(X, X.shape[0])
    assert np.allclose(m[0], D4_QM, rtol=0, atol=1e-15)
    assert np.allclose(v[0], D4_QS ** 2, rtol=1e-14, atol=0)
    # partial tail block: tokens 0..L-1 give mean (L-1)/2, population var (L^2-1)/12
    N, b = 37, 16
    X = np.repeat(np.arange(N, dtype=np.float64)[:, None] % b, 3, axis=1)
    m, v = orc.block_stats(X, b)
    for I, L in enumerate(orc.block_sizes(N, b)):
        assert np.allclose(m[I], (L - 1) / 2)
        assert np.allclose(v[I], (L * L - 1) / 12)


def test_block_stats_two_pass_under_large_offset():
    # a large common offset must not destroy the variance (no E[x^2]-E[x]^2)
    X = sign_block(np.full(4, 1e8), np.full(4, 1e-3))
    _, v = orc.block_stats(X, X.shape[0])
    assert np.allclose(v[0], 1e-6, rtol=1e-6)


# ---------------------------------------------------------------- O3 pins

def test_p1_block_size_one_is_exact_logit_map():
    rng = np.random.default_rng(1)
    N, D = 48, 8
    q, k = rng.normal(size=(N, D)), rng.normal(size=(N, D))
    scale = 1 / math.sqrt(D)
    mask, idx, cnt, S, _ = orc.select_head(q, k, 1, 0.5, scale)
    X = np.array([[scale * sum(q[s, c] * k[t, c] for c in range(D)) for t in range(N)]
                  for s in range(N)])
    assert np.allclose(S, X, rtol=1e-13, atol=1e-14)
    keep = orc.keep_count(N, 0.5)
    for s in range(N):
        assert topk_valid(S[s], np.flatnonzero(mask[s]), keep)
        assert topk_valid(X[s], np.flatnonzero(mask[s]), keep)


@pytest.mark.parametrize("N,b", [(64, 8), (60, 8), (45, 16)])
def test_p2_block_constant_correction_vanishes(N, b):
    rng = np.random.default_rng(N + b)
    n = orc.num_blocks(N, b)
    D = 6
    scale = 0.7
    qb, kb = rng.normal(size=(n, D)), rng.normal(size=(n, D))
    q = np.repeat(qb, b, axis=0)[:N]
    k = np.repeat(kb, b, axis=0)[:N]
    for sp in (0.25, 0.5, 0.75):
        mask, idx, cnt, S, (qm, qv, km, kv) = orc.select_head(q, k, b, sp, scale)
        assert np.abs(qv).max() < 1e-28 and np.abs(kv).max() < 1e-28  # zero up to rounding
        M_lme, M_prob = orc.postdownsample_map(q, k, b, scale)
        assert np.allclose(S, M_lme, rtol=0, atol=1e-12)
        keep = orc.keep_count(n, sp)
        m2, _, _ = orc.norm_sort(M_lme, keep)
        m3, _, _ = orc.norm_sort(M_prob, keep)
        assert np.array_equal(mask, m2)
        assert np.array_equal(mask, m3)


def test_sign_blocks_bruteforce_map_matches_closed_form():
    scale = 0.6
    Xq, Xk = sign_block(D4_QM, D4_QS), sign_block(D4_KM, D4_KS)
    M_lme, M_prob = orc.postdownsample_map(np.vstack([Xq, Xk]), np.vstack([Xk, Xq]), 16, scale)
    assert abs(M_lme[0, 0] - closed_form_lme(D4_QM, D4_QS, D4_KM, D4_KS, scale)) < 1e-12
    assert abs(M_lme[1, 1] - closed_form_lme(D4_KM, D4_KS, D4_QM, D4_QS, scale)) < 1e-12
    # every softmax row sums to one; with |J| = 16 keys per block that makes
    # 16 * sum_J M_prob[I, J] = 1 for every query block I
    assert np.allclose(M_prob.sum(axis=1) * 16, 1.0)


def test_correction_is_fourth_order_with_all_terms():
    ratio, errs = order_ratio(D4_QM, D4_QS, D4_KM, D4_KS, 0.6)
    assert errs[1] < 1e-3
    assert 12.0 < ratio < 20.0, ratio


@pytest.mark.parametrize("which", ["q_const", "k_const"])
def test_single_side_variance_terms(which):
    # one side constant: only q^2*vk (or vq*k^2) survives; exact MGF expansion
    qs = np.zeros(4) if which == "q_const" else D4_QS
    ks = D4_KS if which == "q_const" else np.zeros(4)
    ratio, _ = order_ratio(D4_QM, qs, D4_KM, ks, 0.6)
    assert 12.0 < ratio < 20.0, ratio


def test_zero_mean_blocks_leading_constant():
    # zero means: M_lme = sum ln cosh(a_c), S = sum a_c^2/2, a = scale*sq*sk,
    # so S - M_lme = sum a^4/12 + O(a^6)
    scale = 0.5
    sq, sk = np.array([1.0, 0.7, 1.3, 0.9]), np.array([0.8, 1.1, 1.0, 1.2])
    for e in (0.05, 0.025):
        qs, ks = math.sqrt(e) * sq, math.sqrt(e) * sk
        S = oracle_pair_score(sign_block(np.zeros(4), qs), sign_block(np.zeros(4), ks), scale)
        a = scale * qs * ks
        exact = float(np.sum(np.log(np.cosh(a))))
        assert abs(exact - closed_form_lme(np.zeros(4), qs, np.zeros(4), ks, scale)) < 1e-14
        lead = float(np.sum(a ** 4) / 12)
        assert abs((S - exact) / lead - 1.0) < 0.02


def test_full_cov_equals_diagonal_on_diagonal_covariance():
    scale = 0.6
    Xq, Xk = sign_block(D4_QM, D4_QS), sign_block(D4_KM, D4_KS)
    full = orc.compact_score_full_cov([Xq], [Xk], scale)[0, 0]
    assert abs(full - oracle_pair_score(Xq, Xk, scale)) < 1e-12


def test_full_cov_third_order_on_correlated_perturbations():
    # random (correlated) within-block perturbations: the full-covariance
    # score converges one order faster than the diagonal one
    rng = np.random.default_rng(3)
    D, b, scale = 8, 32, 0.5
    qm, km = rng.normal(size=D), rng.normal(size=D)
    A, Bm = rng.normal(size=(b, D)), rng.normal(size=(b, D))
    A -= A.mean(axis=0)
    Bm -= Bm.mean(axis=0)
    full, diag = [], []
    for e in (0.1, 0.05):
        Xq, Xk = qm + e * A, km + e * Bm
        M, _ = orc.postdownsample_map(np.vstack([Xq]), np.vstack([Xk]), b, scale)
        full.append(abs(orc.compact_score_full_cov([Xq], [Xk], scale)[0, 0] - M[0, 0]))
        diag.append(abs(oracle_pair_score(Xq, Xk, scale) - M[0, 0]))
    assert full[0] / full[1] > 6.5
    assert diag[0] / diag[1] < 5.0
    assert diag[1] > full[1]


# ---------------------------------------------------------------- O4 pins

def test_norm_sort_ties_go_to_lower_index():
    S = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]])
    assert orc.norm_sort_row(S[0], 2) == [1, 2]
    assert orc.norm_sort_row(S[0], 3) == [1, 2, 4]
    assert orc.norm_sort_row(S[0], 4) == [1, 2, 3, 4]
    mask, idx, cnt = orc.norm_sort(S, 3)
    assert mask.tolist() == [[0, 1, 1, 0, 1]] and idx.tolist() == [[1, 2, 4]] and cnt.tolist() == [3]


def test_norm_sort_bruteforce_random_rows():
    rng = np.random.default_rng(11)
    for n in (1, 2, 7, 16):
        S = np.round(rng.normal(size=(20, n)), 1)  # rounding forces ties
        for keep in range(1, n + 1):
            mask, idx, cnt = orc.norm_sort(S, keep)
            for I in range(20):
                assert topk_valid(S[I], idx[I], keep)
                assert list(idx[I]) == sorted(idx[I])
                assert mask[I].sum() == keep == cnt[I]
                assert set(np.flatnonzero(mask[I])) == set(idx[I])


def test_cut_margin_closed_form():
    S = np.array([[0.0, 1.0, 2.0], [5.0, 5.0, 1.0]])
    m = orc.cut_margins(S, 1)
    assert abs(m[0] - (1 - math.exp(-1))) < 1e-15 and m[1] == 0.0
    assert np.all(np.isinf(orc.cut_margins(S, 3)))


def test_p4_selection_matches_postdownsample_bruteforce():
    # sign-pattern blocks with random means and small amplitudes: S differs
    # from the exact block log-mean-exp by O(eps^4); wherever that is below
    # half a row's cut gap the two selections must agree exactly
    rng = np.random.default_rng(5)
    D, b, n = 4, 16, 8
    scale = 0.5
    qmeans, kmeans = rng.normal(size=(n, D)), rng.normal(size=(n, D))
    checked = 0
    for eps in (0.05, 0.1):
        qs, ks = eps * rng.uniform(0.5, 1.5, (n, D)), eps * rng.uniform(0.5, 1.5, (n, D))
        q = np.vstack([sign_block(qmeans[i], qs[i]) for i in range(n)])
        k = np.vstack([sign_block(kmeans[i], ks[i]) for i in range(n)])
        M_lme, _ = orc.postdownsample_map(q, k, b, scale)
        for sp in (0.25, 0.5, 0.75):
            mask, idx, cnt, S, _ = orc.select_head(q, k, b, sp, scale)
            keep = orc.keep_count(n, sp)
            err = np.abs(S - M_lme).max()
            ref, _, _ = orc.norm_sort(M_lme, keep)
            for I in range(n):
                srt = np.sort(M_lme[I])[::-1]
                if srt[keep - 1] - srt[keep] > 2 * err:
                    assert np.array_equal(mask[I], ref[I])
                    checked += 1
    assert checked >= 30


# ---------------------------------------------------------------- O5/O6 pins

def _rand_head(N, D, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(N, D)), rng.normal(size=(N, D)), rng.normal(size=(N, D))


@pytest.mark.parametrize("N,b", [(128, 16), (100, 16)])
def test_p3_zero_sparsity_is_textbook_attention(N, b):
    q, k, v = _rand_head(N, 8, N)
    scale = 1 / math.sqrt(8)
    mask, idx, cnt, S, _ = orc.select_head(q, k, b, 0.0, scale)
    assert mask.all() and np.all(cnt == orc.num_blocks(N, b))
    O, lse = orc.block_attention(q, k, v, mask, b, scale)
    X = scale * q @ k.T
    P = scipy.special.softmax(X, axis=1)
    assert np.allclose(O, P @ v, rtol=0, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(X, axis=1), rtol=0, atol=1e-12)
    Od, lsed = orc.dense_attention(q, k, v, scale)
    assert np.allclose(O, Od, rtol=0, atol=1e-12) and np.allclose(lse, lsed, rtol=0, atol=1e-12)


def test_sparse_attention_equals_masked_library_softmax():
    N, b, D = 100, 16, 8
    q, k, v = _rand_head(N, D, 2)
    scale = 0.4
    n = orc.num_blocks(N, b)
    rng = np.random.default_rng(9)
    mask = (rng.random((n, n)) < 0.5).astype(np.uint8)
    mask[np.arange(n), rng.integers(0, n, n)] = 1
    O, lse = orc.block_attention(q, k, v, mask, b, scale)
    tok_mask = np.kron(mask, np.ones((b, b)))[:N, :N].astype(bool)
    X = np.where(tok_mask, scale * q @ k.T, -np.inf)
    assert np.allclose(O, scipy.special.softmax(X, axis=1) @ v, rtol=0, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(X, axis=1), rtol=0, atol=1e-12)
    rows = [0, 17, 63, 99]
    Or, lr = orc.block_attention_rows(q, k, v, mask, b, scale, rows)
    assert np.allclose(Or, O[rows], atol=1e-13) and np.allclose(lr, lse[rows], atol=1e-13)


def test_p9_log_space_merge_identity():
    # two disjoint key sets recombine exactly in log space (the split used by
    # block-external caching): LSE = logaddexp(LSE1, LSE2) and
    # O = exp(LSE1-LSE) O1 + exp(LSE2-LSE) O2
    N, b, D = 96, 16, 8
    q, k, v = _rand_head(N, D, 4)
    scale = 0.35
    n = orc.num_blocks(N, b)
    m1 = np.zeros((n, n), np.uint8)
    m1[:, ::2] = 1
    m2 = 1 - m1
    O1, l1 = orc.block_attention(q, k, v, m1, b, scale)
    O2, l2 = orc.block_attention(q, k, v, m2, b, scale)
    O, l = orc.block_attention(q, k, v, np.ones((n, n), np.uint8), b, scale)
    lm = np.logaddexp(l1, l2)
    assert np.allclose(l, lm, atol=1e-12)
    assert np.allclose(O, np.exp(l1 - lm)[:, None] * O1 + np.exp(l2 - lm)[:, None] * O2, atol=1e-12)


def test_merge_over_random_partition_is_textbook_attention():
    # the keys of every row cut into three random disjoint sets; each set's
    # attention is the textbook softmax over it, and the merge must give the
    # textbook softmax over all keys
    rng = np.random.default_rng(11)
    N, D, scale = 40, 8, 0.4
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    part = rng.integers(0, 3, size=N)
    rows = np.arange(0, N, 3)
    Os, ls = [], []
    for p in range(3):
        keys = np.flatnonzero(part == p)
        O, lse = orc.dense_attention(q, k[keys], v[keys], scale, rows=rows)
        Os.append(O)
        ls.append(lse)
    Om, lm = orc.merge_attention(Os, ls)
    Od, ld = orc.dense_attention(q, k, v, scale, rows=rows)
    assert np.allclose(Om, Od, atol=1e-12) and np.allclose(lm, ld, atol=1e-12)


def test_merge_sparse_plus_dropped_blocks_is_dense():
    N, b, D = 80, 16, 8
    q, k, v = _rand_head(N, D, 9)
    scale = 0.3
    mask, _, _, _, _ = orc.select_head(q, k, b, 0.5, scale)
    O1, l1 = orc.block_attention(q, k, v, mask, b, scale)
    O2, l2 = orc.block_attention(q, k, v, 1 - mask, b, scale)
    Om, lm = orc.merge_attention([O1, O2], [l1, l2])
    Od, ld = orc.dense_attention(q, k, v, scale)
    assert np.allclose(Om, Od, atol=1e-12) and np.allclose(lm, ld, atol=1e-12)


def test_merge_closed_forms_and_empty_parts():
    rng = np.random.default_rng(12)
    O1, O2 = rng.standard_normal((2, 5, 4))
    a = rng.standard_normal(5)
    # equal normalisers: the average, and ln 2 more
    Om, lm = orc.merge_attention([O1, O2], [a, a])
    assert np.allclose(Om, 0.5 * (O1 + O2), atol=1e-15) and np.allclose(lm, a + math.log(2), atol=1e-15)
    # normalisers in ratio 3:1
    Om, lm = orc.merge_attention([O1, O2], [a + math.log(3), a])
    assert np.allclose(Om, 0.75 * O1 + 0.25 * O2, atol=1e-14) and np.allclose(lm, a + math.log(4), atol=1e-14)
    # an empty part is the identity; a single part is the identity
    ninf = np.full(5, -np.inf)
    Om, lm = orc.merge_attention([O1, np.zeros((5, 4))], [a, ninf])
    assert np.array_equal(Om, O1) and np.array_equal(lm, a)
    Om, lm = orc.merge_attention([O1], [a])
    assert np.allclose(Om, O1, atol=0) and np.array_equal(lm, a)
    # every part empty: the empty sum
    Om, lm = orc.merge_attention([O1, O2], [ninf, ninf])
    assert np.all(Om == 0) and np.all(np.isneginf(lm))


def test_p10_invariances():
    N, b, D = 64, 8, 8
    q, k, v = _rand_head(N, D, 6)
    scale = 0.5
    n = orc.num_blocks(N, b)
    mask, idx, cnt, S, _ = orc.select_head(q, k, b, 0.5, scale)
    O, l = orc.block_attention(q, k, v, mask, b, scale)
    O3, l3 = orc.block_attention(q, k, 3.0 * v, mask, b, scale)
    assert np.allclose(O3, 3.0 * O, atol=1e-12) and np.allclose(l3, l, atol=1e-13)
    Oc, _ = orc.block_attention(q, k, np.full_like(v, 2.5), mask, b, scale)
    assert np.allclose(Oc, 2.5, atol=1e-12)
    # permuting key blocks permutes the mask columns on rows with a clear cut
    perm = np.random.default_rng(0).permutation(n)
    tok = np.concatenate([np.arange(J * b, (J + 1) * b) for J in perm])
    maskp, _, _, Sp, _ = orc.select_head(q, k[tok], b, 0.5, scale)
    assert np.allclose(Sp, S[:, perm], atol=1e-13)
    margins = orc.cut_margins(S, orc.keep_count(n, 0.5))
    clear = margins > 1e-6
    assert clear.sum() >= n // 2
    assert np.array_equal(maskp[clear], mask[:, perm][clear])


def test_attention_oracle_wrapper_on_bits():
    from block_sparse_attention_ba_amd.workloads import make_inputs
    x = make_inputs("tiny")
    sel = orc.select_oracle(x["q"], x["k"], 64, 0.5)
    assert sel["n"] == 16 and sel["keep"] == 8
    assert np.all(sel["mask"].sum(axis=-1) == 8)
    res = orc.attention_oracle(x["q"], x["k"], x["v"], sel["mask"], 64)
    O, lse = res[(0, 0)]
    assert O.shape == (1024, 64) and np.all(np.isfinite(lse))
    # a row subset reproduces the full computation
    rows = np.array([0, 511, 1023])
    sub = orc.attention_oracle(x["q"], x["k"], x["v"], sel["mask"], 64, rows=rows)[(0, 0)]
    assert np.allclose(sub[0], O[rows], atol=1e-13) and np.allclose(sub[1], lse[rows], atol=1e-13)


# ---------------------------------------------------------------- planted mistakes

def _sample_var_stats(X, b):
    m, v = orc.block_stats(X, b)
    L = X.shape[0]
    return m, v * L / (L - 1)


def _score_without_half(qm, qv, km, kv, scale):
    return scale * qm @ km.T + scale ** 2 * (qv @ kv.T + qv @ (km ** 2).T + (qm ** 2) @ kv.T)


def _score_without_vv(qm, qv, km, kv, scale):
    return scale * qm @ km.T + 0.5 * scale ** 2 * (qv @ (km ** 2).T + (qm ** 2) @ kv.T)


def _score_without_qk2(qm, qv, km, kv, scale):
    return scale * qm @ km.T + 0.5 * scale ** 2 * (qv @ kv.T + qv @ (km ** 2).T)


def _score_wrong_scale(qm, qv, km, kv, scale):
    return orc.compact_score(qm, qv, km, kv, scale * scale)


@pytest.mark.parametrize("stats,score", [
    (_sample_var_stats, orc.compact_score),
    (orc.block_stats, _score_without_half),
    (orc.block_stats, _score_without_qk2),
    (orc.block_stats, _score_wrong_scale),
])
def test_planted_mistakes_fail_the_order_pin(stats, score):
    qs = np.zeros(4) if score is _score_without_qk2 else D4_QS
    ratio, _ = order_ratio(D4_QM, qs, D4_KM, D4_KS, 0.6, stats=stats, score=score)
    assert not (12.0 < ratio < 20.0)


def test_planted_dropped_variance_product_fails_zero_mean_pin():
    scale = 0.5
    qs, ks = math.sqrt(0.05) * np.ones(4), math.sqrt(0.05) * np.ones(4)
    Xq, Xk = sign_block(np.zeros(4), qs), sign_block(np.zeros(4), ks)
    exact = closed_form_lme(np.zeros(4), qs, np.zeros(4), ks, scale)
    lead = float(np.sum((scale * qs * ks) ** 4) / 12)
    good = oracle_pair_score(Xq, Xk, scale)
    bad = oracle_pair_score(Xq, Xk, scale, score=_score_without_vv)
    assert abs((good - exact) / lead - 1) < 0.02
    assert abs((bad - exact) / lead - 1) > 10


def _merge_plain_average(o_parts, lse_parts):
    return np.mean(o_parts, axis=0), np.log(np.sum(np.exp(lse_parts), axis=0))


def _merge_unnormalised(o_parts, lse_parts):
    lse = np.log(np.sum(np.exp(lse_parts), axis=0))
    return np.sum(np.exp(np.asarray(lse_parts))[..., None] * np.asarray(o_parts), axis=0), lse


@pytest.mark.parametrize("merge", [_merge_plain_average, _merge_unnormalised])
def test_planted_merge_mistakes_fail_the_partition_pin(merge):
    N, b, D = 80, 16, 8
    q, k, v = _rand_head(N, D, 9)
    mask, _, _, _, _ = orc.select_head(q, k, b, 0.5, 0.3)
    O1, l1 = orc.block_attention(q, k, v, mask, b, 0.3)
    O2, l2 = orc.block_attention(q, k, v, 1 - mask, b, 0.3)
    Om, _ = merge([O1, O2], [l1, l2])
    Od, _ = orc.dense_attention(q, k, v, 0.3)
    assert not np.allclose(Om, Od, atol=1e-6)


def test_empty_mask_row_is_the_empty_sum():
    N, b, D = 48, 16, 4
    q, k, v = _rand_head(N, D, 8)
    mask = np.ones((3, 3), np.uint8)
    mask[1] = 0
    O, lse = orc.block_attention(q, k, v, mask, b, 0.5)
    assert np.all(O[16:32] == 0) and np.all(np.isneginf(lse[16:32]))
    assert np.all(np.isfinite(lse[:16])) and np.all(np.isfinite(lse[32:]))
    Or, lr = orc.block_attention_rows(q, k, v, mask, b, 0.5, [3, 20])
    assert np.all(Or[1] == 0) and np.isneginf(lr[1]) and np.allclose(Or[0], O[3])


# ------------------------------------------------ selection-quality diagnostics

def test_uncorrected_score_is_the_pooled_logit():
    rng = np.random.default_rng(21)
    N, b, D, scale = 70, 16, 5, 0.4
    q, k = rng.normal(size=(N, D)), rng.normal(size=(N, D))
    qm, qv = orc.block_stats(q, b)
    km, kv = orc.block_stats(k, b)
    S0 = orc.uncorrected_score(qm, km, scale)
    n = orc.num_blocks(N, b)
    for I in range(n):
        for J in range(n):
            mq = q[I * b:(I + 1) * b].mean(axis=0)
            mk = k[J * b:(J + 1) * b].mean(axis=0)
            assert abs(S0[I, J] - scale * sum(mq[c] * mk[c] for c in range(D))) < 1e-13
    # the corrected score minus its three variance products is this score
    assert np.allclose(orc.compact_score(qm, np.zeros_like(qv), km, np.zeros_like(kv), scale), S0,
                       rtol=0, atol=1e-14)
    assert np.all(orc.compact_score(qm, qv, km, kv, scale) > S0)  # the correction is a variance: >= 0


def test_average_ranks_and_rank_agreement_closed_forms():
    x = np.array([3.0, 1.0, 3.0, 2.0])
    r = np.array([1.0, 2.0, 3.0, 4.0])
    assert orc.average_ranks(x).tolist() == [3.5, 1.0, 3.5, 2.0]
    # hand computation: centred ranks a = (1, -1.5, 1, -0.5), b = (-1.5, -0.5, 0.5, 1.5):
    # sum ab = -1, sum a^2 = 4.5, sum b^2 = 5; kept(x, 2) = {0, 2}, kept(r, 2) = {2, 3}
    rec, rho = orc.rank_agreement(x, r, 2)
    assert rec == 0.5
    assert abs(rho - (-1.0 / math.sqrt(22.5))) < 1e-15
    rng = np.random.default_rng(22)
    y = rng.normal(size=33)
    assert orc.rank_agreement(y, y, 7) == (1.0, 1.0)
    assert orc.rank_agreement(y, 3.0 * y + 1.0, 7) == (1.0, 1.0)  # monotone maps keep ranks
    rec, rho = orc.rank_agreement(y, -y, 16)
    assert rec == 0.0 and abs(rho + 1.0) < 1e-14
    # a constant row has no ranking: rho is defined as 0, recall follows the tie rule
    c = np.full(10, 2.5)
    rec, rho = orc.rank_agreement(c, np.arange(10.0), 3)
    assert rho == 0.0 and rec == 0.0  # kept(c) = {0, 1, 2} (ties to the lower index), kept(r) = {7, 8, 9}
    rec, rho = orc.rank_agreement(c, -np.arange(10.0), 3)
    assert rho == 0.0 and rec == 1.0  # kept(r) = {0, 1, 2}


def test_spearman_matches_library_on_tied_rows():
    import scipy.stats
    rng = np.random.default_rng(23)
    for trial in range(40):
        n = int(rng.integers(5, 70))
        x = np.round(rng.normal(size=n), 1)  # many ties
        r = np.round(x + rng.normal(size=n), 1) if trial % 2 else np.round(rng.normal(size=n), 1)
        _, rho = orc.rank_agreement(x, r, max(1, n // 3))
        ref = scipy.stats.spearmanr(x, r).statistic
        assert abs(rho - ref) < 1e-12, (trial, rho, ref)


def test_recall_matches_bruteforce_sort():
    rng = np.random.default_rng(24)
    for trial in range(60):
        n = int(rng.integers(2, 80))
        keep = int(rng.integers(1, n + 1))
        x = np.round(rng.normal(size=n), 1)
        r = np.round(rng.normal(size=n), 1)
        top = lambda v: set(np.lexsort((np.arange(n), -v))[:keep].tolist())  # value desc, index asc
        rec, _ = orc.rank_agreement(x, r, keep)
        assert rec == len(top(x) & top(r)) / keep


def _ordinal_ranks(x):
    out = np.empty(len(x))
    out[np.argsort(x, kind="stable")] = np.arange(1, len(x) + 1)
    return out


def test_planted_ordinal_ranks_fail_the_library_pin(monkeypatch):
    import scipy.stats
    monkeypatch.setattr(orc, "average_ranks", _ordinal_ranks)
    rng = np.random.default_rng(25)
    x = np.round(rng.normal(size=40), 0)
    r = np.round(x + rng.normal(size=40), 0)
    _, rho = orc.rank_agreement(x, r, 10)
    assert abs(rho - scipy.stats.spearmanr(x, r).statistic) > 1e-3


def test_postdownsample_map_rows_are_rows_of_the_map():
    rng = np.random.default_rng(26)
    N, b, D, scale = 150, 32, 6, 0.5
    q, k = rng.normal(size=(N, D)), rng.normal(size=(N, D))
    M_lme, M_prob = orc.postdownsample_map(q, k, b, scale)
    rows = [4, 0, 2]
    R_lme, R_prob = orc.postdownsample_map_rows(q, k, b, scale, rows)
    assert np.allclose(R_lme, M_lme[rows], rtol=0, atol=1e-13)
    assert np.allclose(R_prob, M_prob[rows], rtol=0, atol=1e-15)


def test_oracle_matches_its_stored_golden_results():
    """Regression fixture of the oracle itself (tests/golden/oracle_tiny.json,
    written by tests/golden/make_oracle_golden.py from the oracle alone: the
    pages print no worked example)."""
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    try:
        import make_oracle_golden as mk
    finally:
        sys.path.remove(here)
    with open(os.path.join(here, "oracle_tiny.json")) as f:
        gold = json.load(f)
    now = mk.compute()
    assert now["keep"] == gold["keep"]
    assert now["mask"] == gold["mask"] and now["idx"] == gold["idx"]
    assert np.allclose(now["S"], gold["S"], rtol=1e-12, atol=1e-14)
    assert np.allclose(now["lse"], gold["lse"], rtol=1e-12, atol=1e-12)
    for r, row in gold["o_rows"].items():
        assert np.allclose(now["o_rows"][r], row, rtol=1e-11, atol=1e-12), r


def test_p7_gaussian_log_mgf():
    """Q block-constant, K ~ N(km, diag sigma^2): the block log-mean-exp is the
    log-MGF of a Gaussian, scale<q,km> + scale^2/2 sum q^2 sigma^2, which is
    exactly the q^2*vk term of the corrected score (the other two vanish)."""
    import scipy.special
    scale = 0.5
    qv = np.array([0.8, -0.5, 1.2, 0.3])
    km = np.array([0.3, 0.9, -0.4, 0.2])
    sd = np.array([0.5, 0.7, 0.4, 0.9])
    # for a block-constant query block, M_lme[I, J] = ln mean_{t in J} e^{scale <q, k_t>}
    rng = np.random.default_rng(27)
    ks = km + sd * rng.standard_normal((64, 4))
    qs = np.tile(qv, (64, 1))
    M, _ = orc.postdownsample_map(np.vstack([qs]), np.vstack([ks]), 64, scale)
    assert abs(M[0, 0] - (scipy.special.logsumexp(scale * ks @ qv) - math.log(64))) < 1e-13
    # large key block: S (sample statistics) against the brute-force map and the closed form
    J = 200_000
    k = km + sd * rng.standard_normal((J, 4))
    brute = scipy.special.logsumexp(scale * k @ qv) - math.log(J)
    qm, qvar = orc.block_stats(np.tile(qv, (8, 1)), 8)
    kmean, kvar = orc.block_stats(k, J)
    S = orc.compact_score(qm, qvar, kmean, kvar, scale)[0, 0]
    closed = scale * qv @ km + 0.5 * scale ** 2 * np.sum(qv ** 2 * sd ** 2)
    assert abs(S - brute) < 1e-3, (S, brute)
    assert abs(S - closed) < 3e-3, (S, closed)
    # a planted missing 1/2 on the correction misses by about scale^2/2 * sum q^2 sd^2 = 0.073
    wrong = scale * (qm @ kmean.T)[0, 0] + scale ** 2 * np.sum(qm[0] ** 2 * kvar[0])
    assert abs(wrong - brute) > 0.05
