"""ba_att_select_noalloc, the selection pass on the library's fixed device
scratch, through the C ABI against ba_att_select with a caller's workspace:
mask, index lists, counts and the score map must be identical bit for bit.
Two calls in a row, the second on a smaller input, then the first input
again (the scratch keeps the previous call's contents, which must not leak
into a result)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CASES = [  # (B, H, N, D, block, sparsity)
    (1, 8, 8192, 128, 64, 0.5),
    (2, 3, 1000, 64, 128, 0.3),
]


def _inputs(case, seed):
    import torch
    B, H, N, D, block, sp = case
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, H, N, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, N, D), generator=g, device="cuda").to(torch.bfloat16)
    # a few strong keys so that rows have clear winners
    k[:, :, ::97] *= 4
    return q, k


def _outputs(case):
    import torch
    B, H, N, D, block, sp = case
    n = (N + block - 1) // block
    keep = max(1, min(n, n - int(np.floor(sp * n + 1e-9))))
    return (torch.full((B, H, n, n), 7, dtype=torch.uint8, device="cuda"),
            torch.full((B, H, n, keep), -5, dtype=torch.int32, device="cuda"),
            torch.full((B, H, n), -5, dtype=torch.int32, device="cuda"),
            torch.full((B, H, n, n), float("nan"), dtype=torch.float32, device="cuda"))


def _noalloc(lib, case, q, k):
    import torch
    B, H, N, D, block, sp = case
    mask, idx, cnt, score = _outputs(case)
    st = lib.ba_att_select_noalloc(B, H, N, D, block, 0.0, sp, q.data_ptr(), k.data_ptr(), mask.data_ptr(),
                                   idx.data_ptr(), cnt.data_ptr(), score.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.ba_att_status_string(st)
    return mask, idx, cnt, score


def _with_workspace(lib, case, q, k):
    import torch
    B, H, N, D, block, sp = case
    mask, idx, cnt, score = _outputs(case)
    ws = torch.empty(lib.ba_att_select_workspace_bytes(B, H, N, D, block), dtype=torch.uint8, device="cuda")
    st = lib.ba_att_select(B, H, N, D, block, 0.0, sp, q.data_ptr(), k.data_ptr(), mask.data_ptr(),
                           idx.data_ptr(), cnt.data_ptr(), score.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.ba_att_status_string(st)
    return mask, idx, cnt, score


def _same(a, b):
    import torch
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.float32 else x,
                           y.view(torch.uint8) if y.dtype == torch.float32 else y)


def test_noalloc_equals_select_on_consecutive_calls():
    import torch
    from block_sparse_attention_ba_amd import _lib
    lib = _lib.load()
    inputs = [_inputs(c, 100 + i) for i, c in enumerate(CASES)]
    first = None
    for case, (q, k) in zip(CASES, inputs):
        print("noalloc case", case, flush=True)
        got = _noalloc(lib, case, q, k)
        want = _with_workspace(lib, case, q, k)
        torch.cuda.synchronize()
        _same(got, want)
        cnt = got[2].cpu().numpy()
        assert np.all(cnt == got[1].shape[-1])
        if first is None:
            first = got
    # the first (larger) input again, after the smaller call left its data
    print("noalloc case", CASES[0], "again", flush=True)
    again = _noalloc(lib, CASES[0], *inputs[0])
    torch.cuda.synchronize()
    _same(again, first)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    """A shape whose statistics need more than 64 MiB is refused before any
    launch (the outputs stay untouched)."""
    import torch
    from block_sparse_attention_ba_amd import _lib
    lib = _lib.load()
    q = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    out = torch.full((16,), 3, dtype=torch.int32, device="cuda")
    st = lib.ba_att_select_noalloc(2, 32, 65536, 128, 64, 0.0, 0.5, q.data_ptr(), q.data_ptr(), out.data_ptr(),
                                   out.data_ptr(), out.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 5
    assert torch.all(out == 3)
