"""Seeded sweep of random block lists through the sparse forward: random
shapes, lengths up to and past max_keep, repeated and out-of-range entries
in any order, empty rows and negative counts, through the forward, the split
forward and the work-queue forward.  At block 64 neighbouring rows
are walked as one tile (their lists merged with owner bits), so this sweep
exercises the walk construction on lists the selection pass never emits.
Every row is checked against textbook attention over exactly the multiset
of keys its clamped list names, for the forward and the split forward, in
fp32 and bf16 output.

BA_RANDOM_LISTS=<count> widens the sweep (24 seeds by default)."""

import os

import numpy as np
import pytest

from oracle import ba_att_oracle as orc
from tests.test_gpu_parity import _forward_case, check_rows_against_lists, make_case

pytestmark = pytest.mark.gpu


def random_lists(seed):
    """(B, H, N, D, block, max_keep, idx, cnt) of one seeded case."""
    rng = np.random.default_rng(9100 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    block = int(rng.choice([64, 128]))
    N = int(rng.integers(1, 1400))
    n = orc.num_blocks(N, block)
    max_keep = int(rng.integers(1, 2 * n + 3))
    idx = np.full((B, H, n, max_keep), -1, np.int32)
    cnt = np.zeros((B, H, n), np.int32)
    for b in range(B):
        for h in range(H):
            for I in range(n):
                kind = int(rng.integers(0, 6))
                if kind == 0:                                   # empty, or a negative count
                    cnt[b, h, I] = int(rng.integers(-3, 1))
                    continue
                length = int(rng.integers(1, max_keep + 1))
                if kind == 1:                                   # a distinct set, ascending
                    lst = np.sort(rng.choice(n, size=min(length, n), replace=False))
                elif kind == 2 and I > 0 and cnt[b, h, I - 1] > 0:   # the neighbour's list, shuffled
                    prev = idx[b, h, I - 1, :min(int(cnt[b, h, I - 1]), max_keep)]
                    lst = rng.permutation(prev)
                else:                                           # repeats, out-of-range entries, any order
                    lst = rng.integers(-2, n + 2, size=length)
                lst = np.asarray(lst, np.int32)[:max_keep]
                idx[b, h, I, :len(lst)] = lst
                # now and then a count past max_keep, which the forward clamps
                cnt[b, h, I] = len(lst) if rng.integers(0, 4) else max_keep + int(rng.integers(1, 4))
    return B, H, N, D, block, max_keep, idx, cnt


@pytest.mark.parametrize("seed", range(int(os.environ.get("BA_RANDOM_LISTS", "24"))))
def test_random_lists_through_the_forward(gpu_lib, seed):
    B, H, N, D, block, max_keep, idx, cnt = random_lists(seed)
    q, k, v = make_case(B, H, N, D, "clustered", seed=seed + 50)
    parts = 2 + seed % 4
    print(f"seed {seed}: B{B} H{H} N{N} D{D} block {block} max_keep {max_keep} split {parts}", flush=True)
    res = _forward_case(gpu_lib, q, k, v, idx, cnt, block,
                        ["forward f32", "forward bf16", f"forward_split({parts}) f32", f"forward_split({parts}) bf16",
                         "forward_queued f32", "forward_queued bf16"])
    # the queued launch runs the forward's own code on every tile
    for dt in ("f32", "bf16"):
        import torch
        assert torch.equal(res[f"forward_queued {dt}"][0], res[f"forward {dt}"][0]), (seed, dt)
        assert torch.equal(res[f"forward_queued {dt}"][1], res[f"forward {dt}"][1]), (seed, dt)
    check_rows_against_lists(q, k, v, idx, cnt, block, max_keep, res)
