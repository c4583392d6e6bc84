"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same C-ABI calls, same shapes).

* Masks: every row of every head against the fp64 oracle, bit-exact except
  rows whose oracle cut margin is below 1e-4 relative (counted and printed).
* Attention: the GPU forward fed the oracle's block lists, on a seeded sample
  of query rows per head (first and last rows of the sequence, rows of the
  partial tail block, random rows) against the oracle computed row by row;
  and the GPU's own mask end to end on a smaller sample.
* Dense: sampled rows of the dense kernel against textbook attention.
"""

import math
import sys
import zlib

import numpy as np
import pytest

from block_sparse_attention_ba_amd import workloads as wl
from oracle import ba_att_oracle as orc
from tests.helpers import LSE_TOL, O_TOL, compare_masks, max_abs, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CASES = [("tiny", 0.5), ("llada8b", 0.5), ("long_b64", 0.0), ("long_b64", 0.5), ("long_b64", 0.75),
         ("long_b128", 0.5), ("long_b128", 0.75), ("shift", 0.5), ("video", 0.5)]

_CACHE = {}


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def inputs(name):
    key = "long" if name.startswith("long") else name
    if key not in _CACHE:
        _CACHE.clear()  # keep one workload resident
        _log(f"generating {name} ...")
        _CACHE[key] = wl.make_inputs(name)
    x = dict(_CACHE[key])
    x["workload"] = wl.WORKLOADS[name]
    return x


def sample_rows(N, b, rng, count):
    n = orc.num_blocks(N, b)
    tail = np.arange((n - 1) * b, N)
    picks = {0, N - 1, int(tail[0]), int(tail[len(tail) // 2])}
    picks.update(int(r) for r in rng.integers(0, N, size=count))
    return np.array(sorted(picks))


@pytest.mark.parametrize("name,sp", CASES, ids=[f"{n}-{s}" for n, s in CASES])
def test_fullsize_select_and_forward(gpu_lib, name, sp):
    import torch
    x = inputs(name)
    w = x["workload"]
    B, H, N, D, blk = w.B, w.H, w.N, w.D, w.block
    _log(f"case {name} sparsity {sp}: B{B} H{H} N{N} D{D} block {blk}")
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])

    mask, idx, cnt = gpu_lib.select(q, k, blk, sp)
    torch.cuda.synchronize()
    gmask = mask.cpu().numpy()
    ref = orc.select_oracle(x["q"], x["k"], blk, sp)
    res = compare_masks(gmask, ref["S"], ref["mask"], ref["keep"])
    _log(f"  mask rows {res['rows']}: exact {res['exact']}, near-tie rows {res['near_tie_rows']}, "
         f"near-tie mismatches {res['near_tie_mismatch']}, bad {len(res['bad'])}")
    assert not res["bad"], res["bad"][:10]
    assert np.all(cnt.cpu().numpy() == ref["keep"])

    # forward on the oracle's block lists, fp32 output
    oidx = torch.from_numpy(ref["idx"]).cuda()
    ocnt = torch.from_numpy(ref["cnt"]).cuda()
    o, lse = gpu_lib.forward(q, k, v, oidx, ocnt, blk, out_dtype=torch.float32)
    o16, _ = gpu_lib.forward(q, k, v, oidx, ocnt, blk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(zlib.crc32(f"{name}-{sp}".encode()))
    heads = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(4)]
    rows = sample_rows(N, blk, rng, 12)
    worst_o = worst_l = 0.0
    for bi, hi in heads:
        Oo, Lo = orc.attention_oracle(x["q"], x["k"], x["v"], ref["mask"], blk, heads=[(bi, hi)],
                                      rows=rows)[(bi, hi)]
        go = o[bi, hi, rows].cpu().numpy()
        gl = lse[bi, hi, rows].cpu().numpy()
        worst_o = max(worst_o, max_abs(go, Oo))
        worst_l = max(worst_l, max_abs(gl, Lo))
        g16 = o16[bi, hi, rows].float().cpu().numpy()
        assert np.all(np.abs(g16 - go) <= np.abs(go) * 2.0 ** -8 + 1e-6)
    _log(f"  forward (oracle mask), {len(heads)} heads x {len(rows)} rows: max|dO| {worst_o:.2e}, "
         f"max|dLSE| {worst_l:.2e}")
    assert worst_o <= O_TOL and worst_l <= LSE_TOL

    # end to end: the GPU's own mask
    o2, lse2 = gpu_lib.forward(q, k, v, idx, cnt, blk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bi, hi = heads[-1]
    rows2 = rows[:6]
    Oo, Lo = orc.attention_oracle(x["q"], x["k"], x["v"], gmask, blk, heads=[(bi, hi)], rows=rows2)[(bi, hi)]
    assert max_abs(o2[bi, hi, rows2].cpu().numpy(), Oo) <= O_TOL
    assert max_abs(lse2[bi, hi, rows2].cpu().numpy(), Lo) <= LSE_TOL


@pytest.mark.parametrize("name", ["llada8b", "video"])
def test_fullsize_dense(gpu_lib, name):
    import torch
    x = inputs(name)
    w = x["workload"]
    _log(f"dense {name}")
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    o, lse = gpu_lib.dense(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = sample_rows(w.N, w.block, rng, 6)
    sc = 1 / math.sqrt(w.D)
    for bi, hi in [(0, 0), (w.B - 1, w.H - 1)]:
        Oo, Lo = orc.dense_attention(orc.bf16_bits_to_f64(x["q"][bi, hi]), orc.bf16_bits_to_f64(x["k"][bi, hi]),
                                     orc.bf16_bits_to_f64(x["v"][bi, hi]), sc, rows=rows)
        assert max_abs(o[bi, hi, rows].cpu().numpy(), Oo) <= O_TOL
        assert max_abs(lse[bi, hi, rows].cpu().numpy(), Lo) <= LSE_TOL
