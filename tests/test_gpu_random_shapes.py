"""Seeded sweep of random shapes through every path of the operator
(selection, block-sparse forward, split key lists, dense) against the fp64
oracle, through the C ABI.  The shapes mix batch and head counts, head
dimensions, block sizes, sparsities and sequence lengths with ragged tails,
so that the parity cases of the other files are not the only shapes seen.

Bars as in test_gpu_parity: masks bit-exact except near-tie rows (counted),
O within 1e-2 and LSE within 1e-3 with fp32 output; the split result also
within 2^-8 max|v| of the unsplit one."""

import math
import os
import sys

import numpy as np
import pytest

from block_sparse_attention_ba_amd import workloads as wl
from oracle import ba_att_oracle as orc
from tests.helpers import LSE_TOL, O_TOL, compare_masks, max_abs, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def random_case(seed):
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    block = int(rng.choice([64, 128]))
    N = int(rng.integers(1, 2600))
    sp = float(rng.choice([0.0, 0.25, 0.5, 0.75, 0.9]))
    n_split = int(rng.integers(1, 9))
    return B, H, N, D, block, sp, n_split


def make_inputs(B, H, N, D, seed):
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((B, H, 6, D)).astype(np.float32)
    lab = rng.integers(0, 6, size=(B, H, (N + 47) // 48)).repeat(48, axis=-1)[..., :N]
    base = np.take_along_axis(mu, lab[..., None].repeat(D, -1), axis=2)
    q = base + 0.6 * rng.standard_normal((B, H, N, D)).astype(np.float32)
    k = base + 0.6 * rng.standard_normal((B, H, N, D)).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    return wl.f32_to_bf16_bits(q), wl.f32_to_bf16_bits(k), wl.f32_to_bf16_bits(v)


# 16 seeds by default; BA_RANDOM_SHAPES=<count> widens the sweep
@pytest.mark.parametrize("seed", range(int(os.environ.get("BA_RANDOM_SHAPES", "16"))))
def test_random_shape_all_paths(gpu_lib, seed):
    import torch
    B, H, N, D, block, sp, ns = random_case(seed)
    _log("random shape", dict(seed=seed, B=B, H=H, N=N, D=D, block=block, sp=sp, n_split=ns))
    q, k, v = make_inputs(B, H, N, D, 100 + seed)
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    ref = orc.select_oracle(q, k, block, sp)

    mask, idx_g, cnt_g = gpu_lib.select(Q, K, block, sp)
    torch.cuda.synchronize()
    res = compare_masks(mask.cpu().numpy(), ref["S"], ref["mask"], ref["keep"])
    assert not res["bad"], (seed, res["bad"][:5])
    assert np.all(cnt_g.cpu().numpy() == ref["keep"])

    idx = torch.from_numpy(ref["idx"]).cuda()
    cnt = torch.from_numpy(ref["cnt"]).cuda()
    o, lse = gpu_lib.forward(Q, K, V, idx, cnt, block, out_dtype=torch.float32)
    os_, ls_ = gpu_lib.forward_split(Q, K, V, idx, cnt, block, ns, out_dtype=torch.float32)
    od, ld = gpu_lib.dense(Q, K, V, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse, os_, ls_ = o.cpu().numpy(), lse.cpu().numpy(), os_.cpu().numpy(), ls_.cpu().numpy()
    od, ld = od.cpu().numpy(), ld.cpu().numpy()
    att = orc.attention_oracle(q, k, v, ref["mask"], block)
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            O_ref, L_ref = att[(b, h)]
            assert max_abs(o[b, h], O_ref) <= O_TOL, (seed, b, h)
            assert max_abs(lse[b, h], L_ref) <= LSE_TOL, (seed, b, h)
            assert max_abs(os_[b, h], O_ref) <= O_TOL, (seed, b, h)
            assert max_abs(ls_[b, h], L_ref) <= LSE_TOL, (seed, b, h)
            vmax = float(np.abs(orc.bf16_bits_to_f64(v[b, h])).max())
            assert max_abs(os_[b, h], o[b, h]) <= 2.0 ** -8 * vmax, (seed, b, h)
            qq, kk, vv = (orc.bf16_bits_to_f64(x[b, h]) for x in (q, k, v))
            Od, Ld = orc.dense_attention(qq, kk, vv, scale)
            assert max_abs(od[b, h], Od) <= O_TOL, (seed, b, h)
            assert max_abs(ld[b, h], Ld) <= LSE_TOL, (seed, b, h)
