"""Split key lists, log-space merge and external contributions on the GPU,
against the fp64 oracle (same seeded inputs, element by element).

* ba_att_forward_split: the kept blocks of every row cut into n_split parts
  and merged must reproduce the oracle's attention over the whole kept set,
  including parts that are empty.  The merge is exact, but every part
  rounds its probabilities to bf16 relative to its own running max, so O
  differs from the unsplit GPU result within that rounding (each side is
  within 2^-9 relative of exact per probability: |dO| <= 2^-8 max|v|),
  while the LSE, summed in fp32, agrees to 1e-5.
* ba_att_merge: random partial results with empty parts and empty rows
  against oracle.merge_attention.
* ba_att_forward_ext: with the external input set to the oracle's attention
  over the dropped blocks, sparse + external must be dense attention.
"""

import math
import sys

import numpy as np
import pytest

from oracle import ba_att_oracle as orc
from tests.helpers import LSE_TOL, O_TOL, max_abs, to_dev

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def rand_bits(shape, seed):
    from block_sparse_attention_ba_amd.workloads import f32_to_bf16_bits
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


SPLIT_CASES = [
    # (B, H, N, D, block, sparsity, n_split)
    (1, 1, 1024, 64, 64, 0.5, 1),
    (1, 1, 1024, 64, 64, 0.5, 3),
    (1, 2, 1000, 128, 64, 0.5, 2),      # ragged tail
    (1, 2, 2000, 128, 128, 0.75, 4),    # two chunks per block, ragged tail
    (2, 1, 777, 64, 128, 0.5, 7),       # more parts than some rows have chunks
    (1, 1, 512, 128, 64, 0.0, 64),      # 8 chunks, 64 parts: most parts empty
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_forward_split_matches_oracle(gpu_lib, case):
    import torch
    B, H, N, D, block, sp, ns = case
    _log("split case", case)
    q, k, v = (rand_bits((B, H, N, D), 100 + N + i) for i in range(3))
    ref = orc.select_oracle(q, k, block, sp)
    idx = torch.from_numpy(ref["idx"]).cuda()
    cnt = torch.from_numpy(ref["cnt"]).cuda()
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    o, lse = gpu_lib.forward_split(Q, K, V, idx, cnt, block, ns, out_dtype=torch.float32)
    o1, l1 = gpu_lib.forward(Q, K, V, idx, cnt, block, out_dtype=torch.float32)
    o16, _ = gpu_lib.forward_split(Q, K, V, idx, cnt, block, ns, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for name, t in (("split O", o), ("split LSE", lse), ("forward O", o1), ("forward LSE", l1)):
        bad = torch.isnan(t)
        if bool(bad.any()):
            where = torch.nonzero(bad)[:8].tolist()
            _log(f"  NaN in {name}: {int(bad.sum())} values, first at {where}")
    res = orc.attention_oracle(q, k, v, ref["mask"], block)
    for bi in range(B):
        for hi in range(H):
            Oo, Lo = res[(bi, hi)]
            assert max_abs(o[bi, hi].cpu().numpy(), Oo) <= O_TOL
            assert max_abs(lse[bi, hi].cpu().numpy(), Lo) <= LSE_TOL
    # split and unsplit differ only by where the probabilities are rounded
    vmax = float(V.float().abs().max())
    assert float((o - o1).abs().max()) <= 2.0 ** -8 * vmax
    assert float((lse - l1).abs().max()) <= 1e-5
    # bf16 output is the rounded fp32 output
    assert torch.all((o16.float() - o).abs() <= o.abs() * 2.0 ** -8 + 1e-6)


def test_forward_split_empty_rows(gpu_lib):
    import torch
    B, H, N, D, block = 1, 1, 640, 64, 64
    n = orc.num_blocks(N, block)
    q, k, v = (rand_bits((B, H, N, D), 300 + i) for i in range(3))
    m = (np.random.default_rng(5).random((B, H, n, n)) < 0.5).astype(np.uint8)
    m[0, 0, 2] = 0   # an empty row
    m[0, 0, 7] = 1   # a full row
    idx, cnt = gpu_lib.mask_to_index(torch.from_numpy(m).cuda(), n)
    o, lse = gpu_lib.forward_split(to_dev(q), to_dev(k), to_dev(v), idx, cnt, block, 5)
    torch.cuda.synchronize()
    Oo, Lo = orc.attention_oracle(q, k, v, m, block)[(0, 0)]
    o, lse = o[0, 0].cpu().numpy(), lse[0, 0].cpu().numpy()
    rows = slice(2 * block, 3 * block)
    assert np.all(o[rows] == 0) and np.all(np.isneginf(lse[rows]))
    fin = np.isfinite(Lo)
    assert max_abs(o[fin], Oo[fin]) <= O_TOL and max_abs(lse[fin], Lo[fin]) <= LSE_TOL


@pytest.mark.parametrize("P,D,out", [(1, 64, "f32"), (2, 128, "f32"), (5, 128, "bf16"), (3, 64, "bf16")])
def test_merge_matches_oracle(gpu_lib, P, D, out):
    import torch
    B, H, N = 2, 3, 77
    rng = np.random.default_rng(P * 1000 + D)
    o_parts = rng.standard_normal((P, B, H, N, D)).astype(np.float32)
    lse_parts = (3.0 * rng.standard_normal((P, B, H, N))).astype(np.float32)
    lse_parts[rng.random((P, B, H, N)) < 0.2] = -np.inf   # empty parts
    lse_parts[:, 0, 0, 5] = -np.inf                        # a row empty in every part
    odt = torch.float32 if out == "f32" else torch.bfloat16
    o, lse = gpu_lib.merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(), out_dtype=odt)
    torch.cuda.synchronize()
    Oo, Lo = orc.merge_attention(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    go, gl = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(np.isneginf(gl), np.isneginf(Lo))
    fin = np.isfinite(Lo)
    assert np.max(np.abs(gl[fin] - Lo[fin])) <= 1e-5
    tol = 1e-5 if out == "f32" else 2.0 ** -8
    assert np.all(np.abs(go - Oo) <= tol * (1 + np.abs(Oo)))
    assert np.all(go[0, 0, 5] == 0)


@pytest.mark.parametrize("case", [(1, 2, 1000, 64, 64, 0.5), (1, 1, 1500, 128, 128, 0.75)],
                         ids=lambda c: "x".join(map(str, c)))
def test_forward_ext_sparse_plus_dropped_is_dense(gpu_lib, case):
    import torch
    B, H, N, D, block, sp = case
    q, k, v = (rand_bits((B, H, N, D), 500 + N + i) for i in range(3))
    ref = orc.select_oracle(q, k, block, sp)
    dropped = orc.attention_oracle(q, k, v, 1 - ref["mask"], block)
    o_ext = np.stack([np.stack([dropped[(bi, hi)][0] for hi in range(H)]) for bi in range(B)]).astype(np.float32)
    l_ext = np.stack([np.stack([dropped[(bi, hi)][1] for hi in range(H)]) for bi in range(B)]).astype(np.float32)
    idx = torch.from_numpy(ref["idx"]).cuda()
    cnt = torch.from_numpy(ref["cnt"]).cuda()
    o, lse = gpu_lib.forward_ext(to_dev(q), to_dev(k), to_dev(v), idx, cnt, block,
                                 torch.from_numpy(o_ext).cuda(), torch.from_numpy(l_ext).cuda())
    torch.cuda.synchronize()
    sc = 1 / math.sqrt(D)
    for bi in range(B):
        for hi in range(H):
            Od, Ld = orc.dense_attention(orc.bf16_bits_to_f64(q[bi, hi]), orc.bf16_bits_to_f64(k[bi, hi]),
                                         orc.bf16_bits_to_f64(v[bi, hi]), sc)
            assert max_abs(o[bi, hi].cpu().numpy(), Od) <= O_TOL
            assert max_abs(lse[bi, hi].cpu().numpy(), Ld) <= LSE_TOL


def test_forward_ext_empty_external_is_plain_forward(gpu_lib):
    import torch
    B, H, N, D, block = 1, 2, 1100, 128, 64
    q, k, v = (rand_bits((B, H, N, D), 700 + i) for i in range(3))
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    mask, idx, cnt = gpu_lib.select(Q, K, block, 0.5)
    o_ext = torch.zeros((B, H, N, D), dtype=torch.float32, device="cuda")
    l_ext = torch.full((B, H, N), -math.inf, dtype=torch.float32, device="cuda")
    o, lse = gpu_lib.forward_ext(Q, K, V, idx, cnt, block, o_ext, l_ext)
    o1, l1 = gpu_lib.forward(Q, K, V, idx, cnt, block)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)


def test_suggested_split_fills_the_device_once(gpu_lib):
    """ba_att_forward_split_parts: the largest part count whose workgroups
    fit one round of this GPU, and forward_auto equal to the unsplit forward
    within the split tolerance."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (B, H, N, block, max_keep) in [(1, 1, 32768, 64, 256), (1, 32, 8192, 64, 64), (1, 1, 8192, 64, 64),
                                       (1, 1, 8192, 128, 32), (1, 1, 1000, 64, 2), (2, 4, 4096, 128, 16)]:
        n = orc.num_blocks(N, block)
        tiles = B * H * ((n + 1) // 2 if block == 64 else n)  # block 64: a tile per pair of query blocks
        resident = cus * 3
        parts = gpu_lib.forward_split_parts(B, H, N, block, max_keep)
        assert 1 <= parts <= min(64, max_keep * block // 64)
        assert parts == 1 or parts * tiles <= resident        # one round
        assert parts == min(64, max_keep * block // 64) or (parts + 1) * tiles > resident  # the largest such
    B, H, N, D, block = 1, 2, 3000, 128, 64
    q, k, v = (to_dev(rand_bits((B, H, N, D), 500 + i)) for i in range(3))
    mask, idx, cnt = gpu_lib.select(q, k, block, 0.5)
    assert gpu_lib.forward_split_parts(B, H, N, block, int(idx.shape[3])) > 1
    o_ref, l_ref = gpu_lib.forward(q, k, v, idx, cnt, block)
    o, l = gpu_lib.forward_auto(q, k, v, idx, cnt, block)
    torch.cuda.synchronize()
    vmax = float(v.float().abs().max())
    assert float((o - o_ref).abs().max()) <= 2.0 ** -8 * vmax
    assert float((l - l_ref).abs().max()) <= 1e-5
