"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: the library allocates nothing and issues no memset, so select +
forward (and dense) can be captured whole.  Every replay, with eager work and
host synchronisations between replays, must equal the eager result bit for
bit."""

import numpy as np
import pytest

from block_sparse_attention_ba_amd import workloads as wl

pytestmark = pytest.mark.gpu


# the second shape gives the score pass 64 rows per workgroup and 96 KB of
# LDS, so its launch also sets the kernel's dynamic-LDS attribute under capture
SHAPES = [(1, 4, 3000, 128, 64, 0.5), (1, 128, 16384, 128, 64, 0.5)]


@pytest.mark.parametrize("shape", SHAPES, ids=["small", "wide-score-tiles"])
def test_select_forward_graph_replays_match_eager(gpu_lib, shape):
    import torch
    from block_sparse_attention_ba_amd import _lib

    lib = _lib.load()
    B, H, N, D, blk, sp = shape
    print("graph capture case", shape, flush=True)
    dev = torch.device("cuda:0")

    def bits(seed):
        x = np.random.default_rng(seed).standard_normal((B, H, N, D)).astype(np.float32)
        return torch.from_numpy(wl.f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = bits(1), bits(2), bits(3)
    n = lib.ba_att_num_blocks(N, blk)
    keep = lib.ba_att_keep_count(n, sp)
    ws = torch.empty(lib.ba_att_select_workspace_bytes(B, H, N, D, blk), dtype=torch.uint8, device=dev)
    mask = torch.empty((B, H, n, n), dtype=torch.uint8, device=dev)
    idx = torch.empty((B, H, n, keep), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    o = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    od = torch.empty_like(o)
    ld = torch.empty_like(lse)

    def step(stream):
        s = stream.cuda_stream
        assert lib.ba_att_select(B, H, N, D, blk, 0.0, sp, q.data_ptr(), k.data_ptr(), mask.data_ptr(),
                                 idx.data_ptr(), cnt.data_ptr(), None, ws.data_ptr(), ws.numel(), s) == 0
        assert lib.ba_att_forward(B, H, N, D, blk, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                  cnt.data_ptr(), keep, o.data_ptr(), 1, lse.data_ptr(), s) == 0
        assert lib.ba_att_dense(B, H, N, D, 0.0, q.data_ptr(), k.data_ptr(), v.data_ptr(), od.data_ptr(), 1,
                                ld.data_ptr(), s) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)  # eager reference
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (mask, idx, cnt, o, lse, od, ld)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        for t in (mask, idx, cnt, o, lse, od, ld):  # stale contents the replay must overwrite
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((mask, idx, cnt, o, lse, od, ld), ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
        # eager work between replays
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(o, ref[3])
