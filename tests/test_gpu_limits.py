"""The operator at the edges of its supported sizes, against the fp64 oracle
through the C ABI:

* selection at long rows up to the longest supported (n = 512, 1024 and
  2048 key blocks, one head, and with enough heads that the score pass
  takes 32 query-block rows per workgroup), masks bit-exact except near-tie
  rows, index lists the ascending ones of the mask, and the score map
  within an fp32 bound of the oracle's;
* the block-sparse forward at N = 2^18 with a ragged tail block, and at the
  ABI's largest sequence N = 2^20, each from a host-built block list (a few
  random blocks per row, the partial tail block, an empty row), on sampled
  query rows;
* the dense kernel at N = 2^20 on sampled rows.
"""

import math
import sys

import numpy as np
import pytest

from block_sparse_attention_ba_amd import workloads as wl
from oracle import ba_att_oracle as orc
from tests.helpers import LSE_TOL, O_TOL, compare_masks, index_matches_mask, max_abs, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_bits(shape, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return wl.f32_to_bf16_bits(x)


SELECT_CASES = [(1, 32768, 64, 64), (1, 65536, 128, 128), (16, 65536, 128, 128),
                (1, 131072, 128, 128), (8, 131072, 128, 128), (1, 131072, 128, 64), (1, 131071, 64, 64)]


@pytest.mark.parametrize("H,N,D,block", SELECT_CASES, ids=[f"H{c[0]}-N{c[1]}-D{c[2]}-b{c[3]}" for c in SELECT_CASES])
def test_select_at_long_rows(gpu_lib, H, N, D, block):
    import torch
    n = orc.num_blocks(N, block)
    assert n in (512, 1024, 2048)
    _log("select limits case", (H, N, D, block), "n", n)
    rng = np.random.default_rng(N + H)
    # clustered rows so that the kept half of a row has clear winners
    q = np.empty((1, H, N, D), np.uint16)
    k = np.empty((1, H, N, D), np.uint16)
    for h in range(H):
        mu = rng.standard_normal((16, D)).astype(np.float32)
        lab = rng.integers(0, 16, size=N // 64 + 1).repeat(64)[:N]
        q[0, h] = wl.f32_to_bf16_bits(mu[lab] + 0.5 * rng.standard_normal((N, D)).astype(np.float32))
        k[0, h] = wl.f32_to_bf16_bits(mu[lab] + 0.5 * rng.standard_normal((N, D)).astype(np.float32))
    mask, idx, cnt, score = gpu_lib.select(to_dev(q), to_dev(k), block, 0.5, return_score=True)
    torch.cuda.synchronize()
    ref = orc.select_oracle(q, k, block, 0.5)
    gm = mask.cpu().numpy()
    res = compare_masks(gm, ref["S"], ref["mask"], ref["keep"])
    _log("select limits", {k2: v2 for k2, v2 in res.items() if k2 != "bad"})
    assert not res["bad"], res["bad"][:5]
    assert np.all(cnt.cpu().numpy() == ref["keep"])
    assert index_matches_mask(gm, idx.cpu().numpy(), cnt.cpu().numpy())
    # |dS| within a few fp32 ulps of the sum of the absolute terms
    s = ref["scale"]
    hs2 = 0.5 * s * s
    terms = (s * np.abs(ref["qm"]) @ np.abs(ref["km"]).transpose(0, 1, 3, 2)
             + hs2 * (ref["qv"] @ (ref["kv"] + ref["km"] ** 2).transpose(0, 1, 3, 2)
                      + ref["qm"] ** 2 @ ref["kv"].transpose(0, 1, 3, 2)))
    assert np.all(np.abs(score.cpu().numpy() - ref["S"]) <= 4e-5 * terms + 1e-7)


def host_lists(n, keep, rng):
    """Each row keeps `keep` distinct random blocks including the tail block;
    row 1 is empty (cnt 0)."""
    idx = np.zeros((1, 1, n, keep), np.int32)
    cnt = np.full((1, 1, n), keep, np.int32)
    for I in range(n):
        pick = rng.choice(n - 1, size=keep - 1, replace=False)
        idx[0, 0, I] = np.sort(np.concatenate([pick, [n - 1]]))
    cnt[0, 0, 1] = 0
    return idx, cnt


@pytest.mark.parametrize("N,D,block", [((1 << 18) - 37, 64, 128), (1 << 20, 128, 128)])
def test_forward_at_long_sequences(gpu_lib, N, D, block):
    import torch
    _log("forward limits case", (N, D, block))
    q, k, v = (rand_bits((1, 1, N, D), 900 + i) for i in range(3))
    n = orc.num_blocks(N, block)
    keep = 5
    rng = np.random.default_rng(N)
    idx, cnt = host_lists(n, keep, rng)
    o, lse = gpu_lib.forward(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(cnt).cuda(), block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = o[0, 0].cpu().numpy(), lse[0, 0].cpu().numpy()
    rows = sorted({0, block, block + 7, N - 1, (n - 1) * block, *(int(r) for r in rng.integers(0, N, 6))})
    qq, kk, vv = orc.bf16_bits_to_f64(q[0, 0]), orc.bf16_bits_to_f64(k[0, 0]), orc.bf16_bits_to_f64(v[0, 0])
    mask = np.zeros((n, n), np.uint8)
    for I in {r // block for r in rows}:
        mask[I, idx[0, 0, I, :cnt[0, 0, I]]] = 1
    Or, Lr = orc.block_attention_rows(qq, kk, vv, mask, block, 1.0 / math.sqrt(D), rows)
    assert max_abs(o[rows], Or) <= O_TOL
    assert max_abs(lse[rows], Lr) <= LSE_TOL
    # the empty row (query block 1) is the empty sum
    assert np.all(o[block:2 * block] == 0) and np.all(np.isneginf(lse[block:2 * block]))


def test_dense_at_the_longest_sequence(gpu_lib):
    import torch
    N, D = 1 << 20, 128
    _log("dense limits case", (N, D))
    q, k, v = (rand_bits((1, 1, N, D), 950 + i) for i in range(3))
    o, lse = gpu_lib.dense(to_dev(q), to_dev(k), to_dev(v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = o[0, 0].cpu().numpy(), lse[0, 0].cpu().numpy()
    rows = [0, 12345, N // 2, N - 1]
    qq, kk, vv = orc.bf16_bits_to_f64(q[0, 0]), orc.bf16_bits_to_f64(k[0, 0]), orc.bf16_bits_to_f64(v[0, 0])
    Od, Ld = orc.dense_attention(qq, kk, vv, 1.0 / math.sqrt(D), rows=rows)
    assert max_abs(o[rows], Od) <= O_TOL
    assert max_abs(lse[rows], Ld) <= LSE_TOL
