"""HIP path vs the fp64 oracle on seeded inputs small enough for the oracle
to finish in seconds, spanning several tiles and ragged tails, plus the edge
cases of the operator.  Everything runs through the C ABI.

Bars: masks bit-exact except rows whose oracle cut margin is below 1e-4
relative (counted); O max abs error <= 1e-2 and LSE within 1e-3 (fp32
output); index work bit-exact."""

import math
import sys

import numpy as np
import pytest

from block_sparse_attention_ba_amd import workloads as wl
from oracle import ba_att_oracle as orc
from tests.helpers import LSE_TOL, O_TOL, compare_masks, max_abs, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_bits(shape, seed, scale=1.0, mean=0.0):
    rng = np.random.default_rng(seed)
    x = (mean + scale * rng.standard_normal(shape)).astype(np.float32)
    return wl.f32_to_bf16_bits(x)


def clustered_bits(B, H, N, D, seed):
    """Block-structured inputs (means shared by runs of tokens) so that
    scores have clear winners as well as ties-free cuts."""
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((B, H, 8, D)).astype(np.float32)
    lab = rng.integers(0, 8, size=(B, H, (N + 31) // 32)).repeat(32, axis=-1)[..., :N]
    base = np.take_along_axis(mu, lab[..., None].repeat(D, -1), axis=2)
    q = base + 0.5 * rng.standard_normal((B, H, N, D)).astype(np.float32)
    k = base + 0.5 * rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    return wl.f32_to_bf16_bits(q), wl.f32_to_bf16_bits(k), wl.f32_to_bf16_bits(v)


SELECT_CASES = [
    # (B, H, N, D, block, sparsity, kind)
    (1, 1, 1024, 64, 64, 0.5, "normal"),
    (1, 2, 1000, 64, 64, 0.5, "clustered"),     # ragged tail of 40 tokens
    (2, 2, 2048, 128, 64, 0.75, "clustered"),
    (1, 3, 2000, 128, 128, 0.5, "clustered"),   # tail of 80 tokens
    (1, 2, 4096, 128, 128, 0.0, "normal"),
    (1, 1, 200, 128, 128, 0.5, "normal"),       # 2 blocks, tail of 72
    (1, 1, 50, 64, 64, 0.5, "normal"),          # a single partial block
    (1, 2, 8192, 128, 64, 0.9, "clustered"),    # 128 blocks per row
    (1, 1, 16384, 64, 64, 0.5, "normal"),       # 256 blocks per row
    (1, 1, 20000, 128, 64, 0.5, "clustered"),   # 313 blocks: 5 elements per lane
    (1, 2, 1024, 128, 64, 0.95, "clustered"),   # keep = 1 of 16: the row maximum alone
    # many heads: score grids that cover the device twice (two workgroups per CU)
    (1, 256, 2000, 64, 64, 0.5, "clustered"),   # n = 32: 14 of 16 waves without a column tile
    (1, 40, 12790, 128, 64, 0.5, "normal"),     # n = 200, ragged last block and row tile
    (1, 27, 19193, 64, 64, 0.75, "clustered"),  # n = 300: column tiles past n
    (1, 128, 16384, 64, 64, 0.5, "normal"),     # 64-row score tiles: four rows per radix search
    (1, 128, 16384, 128, 64, 0.5, "normal"),
]


def make_case(B, H, N, D, kind, seed):
    if kind == "normal":
        return (rand_bits((B, H, N, D), seed), rand_bits((B, H, N, D), seed + 1),
                rand_bits((B, H, N, D), seed + 2))
    return clustered_bits(B, H, N, D, seed)


@pytest.mark.parametrize("case", SELECT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_select_matches_oracle(gpu_lib, case):
    import torch
    B, H, N, D, block, sp, kind = case
    _log("select case", case)
    q, k, _ = make_case(B, H, N, D, kind, seed=N + D + block)
    ref = orc.select_oracle(q, k, block, sp)
    n, keep = ref["n"], ref["keep"]
    ws = torch.empty(gpu_lib.select_workspace_bytes(B, H, N, D, block), dtype=torch.uint8, device="cuda")
    mask, idx, cnt, score = gpu_lib.select(to_dev(q), to_dev(k), block, sp, return_score=True, workspace=ws)
    torch.cuda.synchronize()
    mask, idx, cnt, score = (t.cpu().numpy() for t in (mask, idx, cnt, score))

    # pooled statistics in the caller's workspace: [aq | ak], 3D fp32 per block
    aw = ws.view(torch.float32).cpu().numpy().astype(np.float64)
    # stored statistics: aq = [scale * mean_q, scale^2 / 2 * var_q], ak = [mean_k, var_k]
    aq = aw[: B * H * n * 2 * D].reshape(B, H, n, 2 * D)
    ak = aw[B * H * n * 2 * D: 2 * B * H * n * 2 * D].reshape(B, H, n, 2 * D)
    sc = 1 / math.sqrt(D)
    assert np.allclose(aq[..., :D], sc * ref["qm"], rtol=1e-5, atol=1e-6)
    assert np.allclose(aq[..., D:], 0.5 * sc * sc * ref["qv"], rtol=1e-4, atol=1e-7)
    assert np.allclose(ak[..., :D], ref["km"], rtol=1e-5, atol=1e-6)
    assert np.allclose(ak[..., D:], ref["kv"], rtol=1e-4, atol=1e-6)

    # score map: fp32 dot of the augmented 3D terms [aq0, aq1, aq0^2/2] .
    # [ak0, ak1 + ak0^2, ak1]; bound by a few ulps of the sum of |terms|
    S = ref["S"]
    aq3 = np.concatenate([aq[..., :D], aq[..., D:], 0.5 * aq[..., :D] ** 2], axis=-1)
    ak3 = np.concatenate([ak[..., :D], ak[..., D:] + ak[..., :D] ** 2, ak[..., D:]], axis=-1)
    mag = np.einsum("bhic,bhjc->bhij", np.abs(aq3), np.abs(ak3))
    err = np.abs(score - S)
    assert np.all(err <= 4e-5 * mag + 1e-7), float((err / (mag + 1e-30)).max())

    assert np.all(cnt == keep)
    res = compare_masks(mask, S, ref["mask"], keep)
    _log("  rows", res["rows"], "exact", res["exact"], "near-tie rows", res["near_tie_rows"],
         "near-tie mismatches", res["near_tie_mismatch"], "bad", len(res["bad"]))
    assert not res["bad"], res["bad"][:10]
    # idx is the ascending list of the mask's ones
    for r, row in enumerate(mask.reshape(-1, n)):
        assert np.array_equal(idx.reshape(-1, keep)[r], np.flatnonzero(row))


ATTN_CASES = [
    # (B, H, N, D, block, sparsity)
    (1, 1, 1024, 64, 64, 0.5),
    (1, 2, 1000, 64, 64, 0.5),
    (1, 2, 1100, 128, 64, 0.5),
    (2, 1, 1500, 128, 128, 0.5),
    (1, 2, 2048, 128, 128, 0.75),
    (1, 1, 200, 128, 128, 0.0),
    (1, 1, 50, 64, 64, 0.0),
    (1, 2, 1000, 64, 128, 0.5),
    (1, 1, 4096, 128, 64, 0.9),
    # 128-key tail blocks of at most 64 rows: the second 64-key half starts
    # past N and must copy nothing (in the last batch it is the tensor's end)
    (2, 1, 777, 64, 128, 0.5),
    (1, 2, 800, 128, 128, 0.0),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_forward_with_oracle_mask(gpu_lib, case):
    import torch
    B, H, N, D, block, sp = case
    _log("forward case", case)
    q, k, v = make_case(B, H, N, D, "clustered", seed=3 * N + D)
    ref = orc.select_oracle(q, k, block, sp)
    idx = torch.from_numpy(ref["idx"]).cuda()
    cnt = torch.from_numpy(ref["cnt"]).cuda()
    o, lse = gpu_lib.forward(to_dev(q), to_dev(k), to_dev(v), idx, cnt, block, out_dtype=torch.float32)
    o16, lse16 = gpu_lib.forward(to_dev(q), to_dev(k), to_dev(v), idx, cnt, block, out_dtype=torch.bfloat16)
    oq, lseq = gpu_lib.forward_queued(to_dev(q), to_dev(k), to_dev(v), idx, cnt, block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the work-queue launch: same tiles, same code, same bits
    assert torch.equal(oq, o) and torch.equal(lseq, lse)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    o16 = o16.float().cpu().numpy()
    att = orc.attention_oracle(q, k, v, ref["mask"], block)
    for (bi, hi), (Oo, Lo) in att.items():
        eo, el = max_abs(o[bi, hi], Oo), max_abs(lse[bi, hi], Lo)
        _log(f"  head {bi},{hi}: max|dO| {eo:.2e} max|dLSE| {el:.2e}")
        assert eo <= O_TOL and el <= LSE_TOL
    # bf16 output is the fp32 result rounded once
    assert np.all(np.abs(o16 - o) <= np.abs(o) * 2.0 ** -8 + 1e-6)
    assert np.array_equal(lse16.cpu().numpy(), lse)


@pytest.mark.parametrize("case", [(1, 1, 1024, 64), (1, 2, 1000, 128), (2, 1, 777, 64), (1, 1, 64, 128)],
                         ids=lambda c: "x".join(map(str, c)))
def test_dense_matches_oracle(gpu_lib, case):
    import torch
    B, H, N, D = case
    _log("dense case", case)
    q, k, v = (rand_bits((B, H, N, D), 10 + i, scale=1.5) for i in range(3))
    o, lse = gpu_lib.dense(to_dev(q), to_dev(k), to_dev(v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    sc = 1 / math.sqrt(D)
    for bi in range(B):
        for hi in range(H):
            Oo, Lo = orc.dense_attention(orc.bf16_bits_to_f64(q[bi, hi]), orc.bf16_bits_to_f64(k[bi, hi]),
                                         orc.bf16_bits_to_f64(v[bi, hi]), sc)
            assert max_abs(o[bi, hi], Oo) <= O_TOL
            assert max_abs(lse[bi, hi], Lo) <= LSE_TOL


@pytest.mark.parametrize("block", [64, 128])
def test_zero_sparsity_equals_dense_bitwise(gpu_lib, block):
    import torch
    B, H, N, D = 1, 2, 1000, 128
    q, k, v = (to_dev(rand_bits((B, H, N, D), 20 + i)) for i in range(3))
    mask, idx, cnt = gpu_lib.select(q, k, block, 0.0)
    o_s, l_s = gpu_lib.forward(q, k, v, idx, cnt, block)
    o_d, l_d = gpu_lib.dense(q, k, v)
    torch.cuda.synchronize()
    assert bool((mask == 1).all())
    assert torch.equal(l_s, l_d)
    assert torch.equal(o_s, o_d)


def test_mask_to_index_bit_exact_and_edge_rows(gpu_lib):
    import torch
    rng = np.random.default_rng(0)
    for n in (1, 5, 64, 65, 200, 512, 1024):
        m = (rng.random((2, 1, n, n)) < 0.4).astype(np.uint8)
        m[0, 0, 0] = 0          # an empty row
        m[0, 0, -1] = 1         # a full row
        max_keep = n
        idx, cnt = gpu_lib.mask_to_index(torch.from_numpy(m).cuda(), max_keep)
        torch.cuda.synchronize()
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for r, row in enumerate(m.reshape(-1, n)):
            ones = np.flatnonzero(row)
            assert cnt.reshape(-1)[r] == ones.size
            assert np.array_equal(idx.reshape(-1, max_keep)[r][: ones.size], ones)
    # truncation: cnt reports the full count, idx holds the lowest max_keep
    m = np.ones((1, 1, 8, 8), np.uint8)
    idx, cnt = gpu_lib.mask_to_index(torch.from_numpy(m).cuda(), 3)
    torch.cuda.synchronize()
    assert np.all(cnt.cpu().numpy() == 8) and np.all(idx.cpu().numpy() == np.arange(3))


def test_empty_rows_and_invalid_entries(gpu_lib):
    import torch
    B, H, N, D, block = 1, 1, 700, 64, 64
    q, k, v = make_case(B, H, N, D, "clustered", seed=99)
    n = orc.num_blocks(N, block)
    rng = np.random.default_rng(1)
    mask = (rng.random((B, H, n, n)) < 0.5).astype(np.uint8)
    mask[0, 0, 3] = 0  # empty row -> O = 0, LSE = -inf
    idx, cnt = gpu_lib.mask_to_index(torch.from_numpy(mask).cuda())
    # invalid entries are skipped: append an out-of-range index to row 5
    idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
    c5 = cnt_np[0, 0, 5]
    if c5 < n:
        idx_np[0, 0, 5, c5] = n + 7
        cnt_np[0, 0, 5] = c5 + 1
    o, lse = gpu_lib.forward(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(idx_np).cuda(),
                             torch.from_numpy(cnt_np).cuda(), block)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy()[0, 0], lse.cpu().numpy()[0, 0]
    Oo, Lo = orc.attention_oracle(q, k, v, mask, block)[(0, 0)]
    assert np.all(o[3 * 64:4 * 64] == 0) and np.all(np.isneginf(lse[3 * 64:4 * 64]))
    assert max_abs(o, Oo) <= O_TOL and max_abs(lse, Lo) <= LSE_TOL


def test_runs_are_deterministic(gpu_lib):
    import torch
    q, k, v = (to_dev(x) for x in make_case(1, 4, 4096, 128, "clustered", seed=5))
    outs = []
    for _ in range(2):
        mask, idx, cnt, score = gpu_lib.select(q, k, 64, 0.5, return_score=True)
        o, lse = gpu_lib.forward(q, k, v, idx, cnt, 64, out_dtype=torch.bfloat16)
        od, ld = gpu_lib.dense(q, k, v, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (mask, idx, cnt, score, o, lse, od, ld)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_custom_scale_and_end_to_end_tiny(gpu_lib):
    """The tiny workload end to end (select on the GPU, then forward with the
    GPU's own mask) against the oracle, with a non-default softmax scale."""
    import torch
    x = wl.make_inputs("tiny")
    scale = 0.2
    q, k, v = (to_dev(x[t]) for t in ("q", "k", "v"))
    mask, idx, cnt = gpu_lib.select(q, k, 64, 0.5, scale=scale)
    o, lse = gpu_lib.forward(q, k, v, idx, cnt, 64, scale=scale)
    torch.cuda.synchronize()
    ref = orc.select_oracle(x["q"], x["k"], 64, 0.5, scale=scale)
    res = compare_masks(mask.cpu().numpy(), ref["S"], ref["mask"], ref["keep"])
    assert not res["bad"]
    Oo, Lo = orc.attention_oracle(x["q"], x["k"], x["v"], mask.cpu().numpy(), 64, scale=scale)[(0, 0)]
    assert max_abs(o.cpu().numpy()[0, 0], Oo) <= O_TOL
    assert max_abs(lse.cpu().numpy()[0, 0], Lo) <= LSE_TOL


@pytest.mark.parametrize("block", [64, 128])
def test_forward_list_contract_edge_cases(gpu_lib, block):
    """The index-list contract of ba_att_forward (include/ba_att.h): a count
    above max_keep is clamped, a negative count is an empty row, entries
    outside [0, n) are skipped wherever they stand, any order is accepted,
    and a repeated entry is counted twice -- also when the lists are cut into
    parts (ba_att_forward_split).  Each row is checked against textbook
    attention over exactly the multiset of keys its list names."""
    import torch
    B, H, N, D = 1, 1, 1000, 64
    q, k, v = make_case(B, H, N, D, "clustered", seed=123)
    n = orc.num_blocks(N, block)
    max_keep = 6
    rng = np.random.default_rng(block)
    idx = np.full((B, H, n, max_keep), -1, np.int32)
    cnt = np.zeros((B, H, n), np.int32)
    lists = {}
    for I in range(n):
        picks = rng.choice(n, size=min(4, n), replace=False)
        lists[I] = list(picks)
    lists[0] = [n - 1, 0, 2][: min(3, n)]           # descending-first order, tail block included
    lists[1] = [1, -1, n + 3, 0][: 4]                # invalid entries in the middle
    lists[2] = [2, 2, 0] if n > 2 else [0, 0]        # a repeated entry
    for I, lst in lists.items():
        idx[0, 0, I, :len(lst)] = lst
        cnt[0, 0, I] = len(lst)
    cnt[0, 0, n - 1] = max_keep + 5                  # clamped to max_keep
    idx[0, 0, n - 1] = rng.permutation(n)[:max_keep] if n >= max_keep else np.resize(np.arange(n), max_keep)
    if n > 3:
        cnt[0, 0, 3] = -3                            # empty row
    args = (to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), block)
    results = {"forward": gpu_lib.forward(*args), "forward_split(3)": gpu_lib.forward_split(*args, 3)}
    torch.cuda.synchronize()
    check_rows_against_lists(q, k, v, idx, cnt, block, max_keep, results)


def check_rows_against_lists(q, k, v, idx, cnt, block, max_keep, results, blocks=None):
    """Every row of the query blocks `blocks` (default: all) of every batch,
    head and result against textbook attention over exactly the multiset of
    keys its clamped list names (entries outside [0, n) skipped).  fp32
    output to O_TOL; bf16 output adds its own rounding, half an ulp of the
    largest |O|."""
    B, H, N, D = q.shape
    n = orc.num_blocks(N, block)
    scale = 1.0 / math.sqrt(D)
    outs = {path: (o.float().cpu().numpy(), lse.cpu().numpy(), str(o.dtype) == "torch.bfloat16")
            for path, (o, lse) in results.items()}
    for b in range(B):
        for h in range(H):
            qq, kk, vv = (orc.bf16_bits_to_f64(x[b, h]) for x in (q, k, v))
            for path, (o_all, lse_all, bf16) in outs.items():
                o, lse = o_all[b, h], lse_all[b, h]
                for I in (range(n) if blocks is None else blocks):
                    rows = np.arange(I * block, min((I + 1) * block, N))
                    c = min(max(int(cnt[b, h, I]), 0), max_keep)
                    keys = [t for J in idx[b, h, I, :c] if 0 <= J < n
                            for t in range(J * block, min((J + 1) * block, N))]
                    if not keys:
                        assert np.all(o[rows] == 0) and np.all(np.isneginf(lse[rows])), (path, b, h, I)
                        continue
                    keys = np.asarray(keys)
                    Oe, Le = orc.dense_attention(qq[rows], kk[keys], vv[keys], scale)
                    tol = O_TOL + (float(np.abs(Oe).max()) * 2.0 ** -9 if bf16 else 0.0)
                    assert max_abs(o[rows], Oe) <= tol, (path, b, h, I, max_abs(o[rows], Oe))
                    assert max_abs(lse[rows], Le) <= LSE_TOL, (path, b, h, I, max_abs(lse[rows], Le))


def _forward_case(gpu_lib, q, k, v, idx, cnt, block, paths):
    import torch
    args = (to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), block)
    out = {}
    for name in paths:
        dt = torch.bfloat16 if name.endswith("bf16") else torch.float32
        if name.startswith("forward_split"):
            out[name] = gpu_lib.forward_split(*args, int(name.split("(")[1].split(")")[0]), out_dtype=dt)
        elif name.startswith("forward_queued"):
            out[name] = gpu_lib.forward_queued(*args, out_dtype=dt)
        else:
            out[name] = gpu_lib.forward(*args, out_dtype=dt)
    torch.cuda.synchronize()
    return out


def test_forward_pair_walks_keep_each_rows_multiset(gpu_lib):
    """At block 64 one tile serves two neighbouring query blocks and walks
    the union of their lists once, in the golden-ratio order, with a block
    both rows keep copied once.  A block repeated within and across the two
    lists must still count as often as each row names it (2 and 1 copies,
    1 and 2, 2 and 2); rows may share no block, or every block in a
    different order (both lists full: the walk is then ascending); an odd n
    leaves the last tile one row, here a full-length list with repeats."""
    B, H, N, D, block = 1, 1, 64 * 9 - 5, 64, 64     # n = 9: four pairs and a single row
    q, k, v = make_case(B, H, N, D, "clustered", seed=321)
    n = orc.num_blocks(N, block)
    max_keep = n
    lists = {0: [5, 5, 3], 1: [5, 3, 3, 7],           # 5: 2 and 1 copies; 3: 1 and 2
             2: [1, 1, 4, 4], 3: [4, 4, 1, 8],        # 2 and 2 copies of two blocks
             4: [0, 2, 6, -1], 5: [1, 3, 7, 12],      # nothing shared; an invalid entry in each
             6: [8, 0, 4, 2, 6, 1, 3, 7, 5],          # both full, in different orders
             7: [2, 4, 0, 8, 1, 3, 5, 7, 6],
             8: [8, 8, 8, 0, 7, 1, 2, 2, 5]}          # the single row: n entries, with repeats
    idx = np.full((B, H, n, max_keep), -1, np.int32)
    cnt = np.zeros((B, H, n), np.int32)
    for I, lst in lists.items():
        idx[0, 0, I, :len(lst)] = lst
        cnt[0, 0, I] = len(lst)
    res = _forward_case(gpu_lib, q, k, v, idx, cnt, block,
                        ["forward f32", "forward bf16", "forward_split(2) f32", "forward_split(4) bf16",
                         "forward_queued f32"])
    check_rows_against_lists(q, k, v, idx, cnt, block, max_keep, res)


@pytest.mark.parametrize("block", [64, 128])
def test_forward_lists_too_long_to_reorder(gpu_lib, block):
    """A tile reorders at most 2048 walk entries (the union of two rows'
    lists at block 64, one row's at block 128); longer lists are walked as
    given.  Rows of 2100 entries, mostly repeats with some invalid ones,
    beside rows short enough to be reordered."""
    B, H, D = 1, 1, 64
    N = 4 * block - 17
    q, k, v = make_case(B, H, N, D, "normal", seed=block + 7)
    n = orc.num_blocks(N, block)
    max_keep = 2100
    rng = np.random.default_rng(block + 1)
    idx = rng.integers(0, n, size=(B, H, n, max_keep)).astype(np.int32)
    idx[0, 0, 1, ::97] = -1
    idx[0, 0, 3, 5::89] = n
    cnt = np.array([[[2100, 2100, 700, 1000]]], np.int32)   # tiles of 4200 and 1700 entries at block 64
    res = _forward_case(gpu_lib, q, k, v, idx, cnt, block, ["forward f32", "forward_split(3) f32",
                                                            "forward_queued f32"])
    check_rows_against_lists(q, k, v, idx, cnt, block, max_keep, res)


@pytest.mark.parametrize("keep", [32, 33, 64, 65])
@pytest.mark.parametrize("block", [64, 128])
def test_forward_tail_tile_too_short_for_its_walk(gpu_lib, block, keep):
    """A tile builds its walk in its own output rows, so a last tile of one
    token (D = 64: room for 32 walk entries in bf16, 64 in fp32) reorders a
    list of up to that many entries and walks a longer one as given; both
    sides of both limits, in both output types."""
    B, H, D = 1, 1, 64
    n = 71                                                  # odd: at block 64 the last tile is one block
    N = block * (n - 1) + 1                                 # of one token
    q, k, v = make_case(B, H, N, D, "clustered", seed=block + keep)
    rng = np.random.default_rng(block * keep)
    idx = np.stack([rng.choice(n, size=keep, replace=False) for _ in range(n)])[None, None].astype(np.int32)
    cnt = np.full((B, H, n), keep, np.int32)
    res = _forward_case(gpu_lib, q, k, v, idx, cnt, block, ["forward f32", "forward bf16", "forward_queued bf16"])
    check_rows_against_lists(q, k, v, idx, cnt, block, keep, res, blocks=[0, 1, n - 3, n - 2, n - 1])


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65])
@pytest.mark.parametrize("D,block", [(64, 64), (128, 128)])
def test_degenerate_sequence_lengths(gpu_lib, N, D, block):
    """Sequences of one token, of less than one block, of exactly one block
    and of one block plus one token, through selection, forward, split
    forward, work-queue forward and dense, against the oracle."""
    import torch
    B, H = 1, 2
    q, k, v = make_case(B, H, N, D, "normal", seed=N + D)
    ref = orc.select_oracle(q, k, block, 0.5)
    mask, idx, cnt = gpu_lib.select(to_dev(q), to_dev(k), block, 0.5)
    torch.cuda.synchronize()
    res = compare_masks(mask.cpu().numpy(), ref["S"], ref["mask"], ref["keep"])
    assert not res["bad"], res["bad"][:5]
    assert np.all(cnt.cpu().numpy() == ref["keep"])
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    oidx, ocnt = torch.from_numpy(ref["idx"]).cuda(), torch.from_numpy(ref["cnt"]).cuda()
    o, lse = gpu_lib.forward(Q, K, V, oidx, ocnt, block)
    os_, ls_ = gpu_lib.forward_split(Q, K, V, oidx, ocnt, block, 3)
    oq, lq = gpu_lib.forward_queued(Q, K, V, oidx, ocnt, block)
    od, ld = gpu_lib.dense(Q, K, V)
    torch.cuda.synchronize()
    att = orc.attention_oracle(q, k, v, ref["mask"], block)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        Oo, Lo = att[(0, h)]
        for name, (go, gl) in {"forward": (o, lse), "split": (os_, ls_), "queued": (oq, lq)}.items():
            assert max_abs(go[0, h].cpu().numpy(), Oo) <= O_TOL, (name, h)
            assert max_abs(gl[0, h].cpu().numpy(), Lo) <= LSE_TOL, (name, h)
        qq, kk, vv = (orc.bf16_bits_to_f64(x[0, h]) for x in (q, k, v))
        Od, Ldn = orc.dense_attention(qq, kk, vv, scale)
        assert max_abs(od[0, h].cpu().numpy(), Od) <= O_TOL
        assert max_abs(ld[0, h].cpu().numpy(), Ldn) <= LSE_TOL

