"""The machine-peak microbenchmarks (libba_peaks.so) compute what they claim,
so that the rates the benchmark reports from them are rates of real work:
the copy reproduces its source, the read kernel's per-thread XOR digests
combine to the XOR of every word of the buffer (each 16-byte vector read
exactly once), the constant-operand MFMA loop gives its closed form, and the
random-operand loop is deterministic, finite and linear in its iteration
count."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def peaks(gpu_lib):
    import torch
    from block_sparse_attention_ba_amd import _lib
    return _lib.load_peaks(), torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("nbytes,groups,nt", [(16, 1, 0), (4096, 2, 1), ((1 << 20) + 48, 5, 0), ((1 << 20) + 48, 7, 1)])
def test_read_digest_and_copy(peaks, nbytes, groups, nt):
    import torch
    pk, s = peaks
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(groups * 256, dtype=torch.int32, device="cuda")
    assert pk.ba_peak_read(src.data_ptr(), nbytes, sink.data_ptr(), groups, nt, s) == 0
    dst = torch.zeros_like(src)
    assert pk.ba_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, groups, s) == 0
    torch.cuda.synchronize()
    digest = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert digest == np.bitwise_xor.reduce(host)
    assert torch.equal(dst, src)


def test_mfma_loop_on_constant_operands_closed_form(peaks):
    """Every element of a 32x32x16 product of all-x operands is 16 x^2; four
    accumulators of 16 elements per lane over `iters` rounds: 1024 x^2 iters
    per thread, exact for x = 2^-10."""
    import torch
    pk, s = peaks
    groups, iters, x = 3, 5, 2.0 ** -10
    sink = torch.zeros(groups * 256, dtype=torch.float32, device="cuda")
    assert pk.ba_peak_mfma_bf16(sink.data_ptr(), groups, iters, x, s) == 0
    torch.cuda.synchronize()
    assert torch.all(sink == 1024 * x * x * iters)


def test_mfma_loop_on_random_operands_is_linear_in_iterations(peaks):
    import torch
    pk, s = peaks
    groups = 4
    out = {}
    for iters in (1, 1, 3):
        sink = torch.zeros(groups * 256, dtype=torch.float32, device="cuda")
        assert pk.ba_peak_mfma_bf16_random(sink.data_ptr(), groups, iters, 77, s) == 0
        torch.cuda.synchronize()
        out.setdefault(iters, []).append(sink.cpu().numpy().astype(np.float64))
    one, again, three = out[1][0], out[1][1], out[3][0]
    assert np.all(np.isfinite(one)) and np.any(one != 0)
    assert np.array_equal(one, again)
    assert np.max(np.abs(three - 3 * one)) <= 1e-4 * max(1.0, float(np.max(np.abs(three))))
    other = torch.zeros(groups * 256, dtype=torch.float32, device="cuda")
    assert pk.ba_peak_mfma_bf16_random(other.data_ptr(), groups, 1, 78, s) == 0
    torch.cuda.synchronize()
    assert not np.array_equal(other.cpu().numpy(), one)   # the seed changes the operands
