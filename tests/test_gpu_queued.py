"""The work-queue sparse forward (ba_att_forward_queued) on the GPU.

Its kernel runs the forward's own tile code, so every output must equal
ba_att_forward's bit for bit; rows are also checked against the oracle
where the case is small.  The queue protocol is checked directly: the
caller's queue holds zeros again after every call, so consecutive calls on
one stream (the second smaller than the first), grids larger than the tile
count (fewer tiles than XCDs), a caller-owned queue on a second stream and
replays of a captured HIP graph all see every tile exactly once."""

import numpy as np
import pytest

from oracle import ba_att_oracle as orc
from tests.helpers import LSE_TOL, O_TOL, max_abs, to_dev
from tests.test_gpu_parity import check_rows_against_lists, make_case

pytestmark = pytest.mark.gpu


def _log(*a):
    import sys
    print(*a, file=sys.stderr, flush=True)


def _normal_qkv(B, H, N, D, seed):
    """Seeded bf16 Q, K, V ~ N(0, 1) drawn on the GPU."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    return tuple(torch.randn((B, H, N, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))


def _lists(B, H, N, block, sp, seed):
    """Seeded random kept-block lists of the selection's shape (keep per row)."""
    n = orc.num_blocks(N, block)
    keep = orc.keep_count(n, sp)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(n)[:keep] for _ in range(B * H * n)]).reshape(B, H, n, keep)
    return np.sort(idx, axis=-1).astype(np.int32), np.full((B, H, n), keep, np.int32)


def _run(gpu_lib, q, k, v, idx, cnt, block, queue=None, out_dtype=None):
    import torch
    dt = out_dtype or torch.float32
    I, C = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    o, lse = gpu_lib.forward(q, k, v, I, C, block, out_dtype=dt)
    oq, lq = gpu_lib.forward_queued(q, k, v, I, C, block, out_dtype=dt, queue=queue)
    return (o, lse), (oq, lq)


def _zero(queue):
    import torch
    torch.cuda.synchronize()
    return bool(torch.all(queue == 0))


def test_consecutive_calls_on_one_queue(gpu_lib):
    """A large call (more tiles than the resident grid, paired block-64
    tiles), then a smaller one on the same queue: both equal the forward,
    the small one is checked against the oracle, the queue is zero after
    each."""
    import torch
    queue = torch.zeros(gpu_lib.QUEUE_WORDS, dtype=torch.int32, device="cuda")
    B, H, N, D, block = 1, 32, 8192 - 40, 128, 64
    _log(f"large: B{B} H{H} N{N} D{D} block {block}")
    q, k, v = _normal_qkv(B, H, N, D, seed=101)
    idx, cnt = _lists(B, H, N, block, 0.5, seed=1)
    (o, lse), (oq, lq) = _run(gpu_lib, q, k, v, idx, cnt, block, queue=queue)
    assert _zero(queue)
    assert torch.equal(oq, o) and torch.equal(lq, lse)

    B, H, N, D, block = 2, 1, 1000, 64, 128
    _log(f"small: B{B} H{H} N{N} D{D} block {block}")
    qb, kb, vb = make_case(B, H, N, D, "clustered", seed=77)
    idx, cnt = _lists(B, H, N, block, 0.5, seed=2)
    (o, lse), (oq, lq) = _run(gpu_lib, to_dev(qb), to_dev(kb), to_dev(vb), idx, cnt, block, queue=queue)
    assert _zero(queue)
    assert torch.equal(oq, o) and torch.equal(lq, lse)
    check_rows_against_lists(qb, kb, vb, idx, cnt, block, idx.shape[-1], {"queued": (oq, lq)})


@pytest.mark.parametrize("B,H,N,D,block", [(1, 1, 64, 64, 64), (1, 1, 300, 128, 128),
                                           (1, 1, 64 * 9, 64, 64), (1, 3, 1500, 128, 64),
                                           (2, 2, 777, 64, 128)],
                         ids=lambda x: str(x))
def test_fewer_tiles_than_the_grid(gpu_lib, B, H, N, D, block):
    """1 to a few dozen tiles: most workgroups of the resident grid find
    every queue empty and leave at once."""
    import torch
    q, k, v = make_case(B, H, N, D, "normal", seed=N + D + block)
    idx, cnt = _lists(B, H, N, block, 0.5, seed=N)
    (o, lse), (oq, lq) = _run(gpu_lib, to_dev(q), to_dev(k), to_dev(v), idx, cnt, block)
    torch.cuda.synchronize()
    assert torch.equal(oq, o) and torch.equal(lq, lse)
    check_rows_against_lists(q, k, v, idx, cnt, block, idx.shape[-1], {"queued": (oq, lq)})
    stream = torch.cuda.current_stream().cuda_stream
    assert bool(torch.all(gpu_lib.queue_for(torch.device("cuda", torch.cuda.current_device()), stream) == 0))


def test_caller_queue_on_a_second_stream(gpu_lib):
    """A caller-owned queue on a stream of its own (default priority),
    beside the library's queue of the default stream."""
    import torch
    B, H, N, D, block = 1, 8, 4096, 128, 128
    q, k, v = _normal_qkv(B, H, N, D, seed=102)
    idx, cnt = _lists(B, H, N, block, 0.75, seed=3)
    ref, _ = _run(gpu_lib, q, k, v, idx, cnt, block)
    side = torch.cuda.Stream()
    queue = torch.zeros(gpu_lib.QUEUE_WORDS, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        oq, lq = gpu_lib.forward_queued(q, k, v, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                                        block, queue=queue)
    side.synchronize()
    assert _zero(queue)
    assert torch.equal(oq, ref[0]) and torch.equal(lq, ref[1])


def test_graph_replays(gpu_lib):
    """The queue needs no clearing between launches, so a captured launch
    replays correctly: four replays, with eager calls between them, each
    equal to the eager result bit for bit."""
    import torch
    B, H, N, D, block = 1, 4, 2048 + 33, 64, 64
    q, k, v = _normal_qkv(B, H, N, D, seed=103)
    idx, cnt = _lists(B, H, N, block, 0.5, seed=4)
    I, C = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    queue = torch.zeros(gpu_lib.QUEUE_WORDS, dtype=torch.int32, device="cuda")
    o = torch.empty(B, H, N, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    eager_o, eager_l = gpu_lib.forward(q, k, v, I, C, block)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        gpu_lib.forward_queued(q, k, v, I, C, block, out=o, lse=lse, queue=queue)  # warm-up, eager
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            gpu_lib.forward_queued(q, k, v, I, C, block, out=o, lse=lse, queue=queue)
    torch.cuda.synchronize()
    for rep in range(4):
        o.zero_()
        lse.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager_o) and torch.equal(lse, eager_l), rep
        assert _zero(queue), rep
        gpu_lib.forward(q, k, v, I, C, block)  # eager work between replays
        torch.cuda.synchronize()


def test_selection_then_queued_forward_matches_oracle(gpu_lib):
    """End to end on the tiny workload's shape: the GPU's selection, then
    the queued forward, against the oracle's attention on the GPU's mask."""
    import torch
    B, H, N, D, block = 1, 2, 1024 + 17, 64, 64
    q, k, v = make_case(B, H, N, D, "clustered", seed=5)
    mask, idx, cnt = gpu_lib.select(to_dev(q), to_dev(k), block, 0.5)
    o, lse = gpu_lib.forward_queued(to_dev(q), to_dev(k), to_dev(v), idx, cnt, block)
    torch.cuda.synchronize()
    att = orc.attention_oracle(q, k, v, mask.cpu().numpy(), block)
    for (bi, hi), (Oo, Lo) in att.items():
        assert max_abs(o[bi, hi].cpu().numpy(), Oo) <= O_TOL
        assert max_abs(lse[bi, hi].cpu().numpy(), Lo) <= LSE_TOL
