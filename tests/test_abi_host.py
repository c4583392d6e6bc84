"""C-ABI contract checks that run without a GPU: the library loads, exports
every symbol the header declares, its host-only helpers agree with the
oracle's integer rules, and invalid arguments are rejected before anything is
launched (these calls never reach the HIP runtime)."""

import os
import re

import pytest

from oracle import ba_att_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ba_att.h")


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_ba_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_ba_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ba_att_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("ba_att_select", "ba_att_forward", "ba_att_dense", "ba_att_mask_to_index",
                 "ba_att_num_blocks", "ba_att_keep_count", "ba_att_select_workspace_bytes",
                 "ba_att_status_string"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    from block_sparse_attention_ba_amd import _lib
    bound = {name for name, _, _ in _lib.SIGNATURES}
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in bound, f"{name} has no binding signature"


def test_num_blocks_matches_oracle(lib):
    for N in (1, 63, 64, 65, 1000, 1024, 8192, 16384, 32760, 32768):
        for b in (64, 128):
            assert lib.ba_att_num_blocks(N, b) == orc.num_blocks(N, b)
    assert lib.ba_att_num_blocks(0, 64) == -1


def test_keep_count_matches_oracle_bit_exactly(lib):
    sps = [0.0, 0.1, 0.25, 0.29, 1 / 3, 0.3, 0.5, 0.7, 0.75, 0.9, 0.99, 0.999]
    for n in list(range(1, 80)) + [128, 255, 256, 512, 1024]:
        for sp in sps:
            assert lib.ba_att_keep_count(n, sp) == orc.keep_count(n, sp), (n, sp)
    assert lib.ba_att_keep_count(16, 1.0) == -1
    assert lib.ba_att_keep_count(16, -0.5) == -1
    assert lib.ba_att_keep_count(0, 0.5) == -1


def test_workspace_bytes(lib):
    assert lib.ba_att_select_workspace_bytes(1, 32, 8192, 128, 64) == 2 * 32 * 128 * 256 * 4
    assert lib.ba_att_select_workspace_bytes(1, 40, 32760, 128, 128) == 2 * 40 * 256 * 256 * 4
    assert lib.ba_att_select_workspace_bytes(1, 1, 1024, 96, 64) == 0


def test_status_strings(lib):
    for code, text in ((0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape or size"),
                       (3, b"workspace or work queue missing, misaligned or too small"), (4, b"HIP launch failed")):
        assert lib.ba_att_status_string(code) == text


FAKE = 0x10000  # an aligned non-null value: every call below fails validation first


def test_select_rejects_before_launch(lib):
    ok = dict(B=1, H=1, N=1024, D=64, block=64, scale=0.0, sp=0.5)

    def call(**kw):
        a = dict(ok, q=FAKE, k=FAKE, mask=FAKE, idx=FAKE, cnt=FAKE, score=None, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.ba_att_select(a["B"], a["H"], a["N"], a["D"], a["block"], a["scale"], a["sp"],
                                 a["q"], a["k"], a["mask"], a["idx"], a["cnt"], a["score"], a["ws"],
                                 a["wsb"], None)

    assert call(q=None) == 1
    assert call(idx=None) == 1
    assert call(sp=1.0) == 1 and call(sp=-0.1) == 1 and call(sp=float("nan")) == 1
    assert call(N=0) == 1 and call(B=0) == 1
    assert call(D=96) == 2
    assert call(block=32) == 2
    assert call(N=2049 * 64) == 2            # more than 2048 blocks per row
    assert call(N=4097 * 128, block=128) == 2
    assert call(q=FAKE + 2) == 1             # misaligned
    assert call(ws=None) == 3
    assert call(wsb=16) == 3


def test_forward_and_dense_reject_before_launch(lib):
    def fwd(**kw):
        a = dict(B=1, H=1, N=1024, D=128, block=64, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE,
                 mk=8, o=FAKE, od=1, lse=None)
        a.update(kw)
        return lib.ba_att_forward(a["B"], a["H"], a["N"], a["D"], a["block"], 0.0, a["q"], a["k"],
                                  a["v"], a["idx"], a["cnt"], a["mk"], a["o"], a["od"], a["lse"], None)

    assert fwd(v=None) == 1 and fwd(o=None) == 1 and fwd(cnt=None) == 1
    assert fwd(od=7) == 1
    assert fwd(mk=0) == 1
    assert fwd(D=80) == 2 and fwd(block=256) == 2
    assert fwd(o=FAKE + 8) == 1
    assert fwd(lse=FAKE + 2) == 1

    def dense(**kw):
        a = dict(B=1, H=1, N=1024, D=128, q=FAKE, k=FAKE, v=FAKE, o=FAKE, od=0, lse=None)
        a.update(kw)
        return lib.ba_att_dense(a["B"], a["H"], a["N"], a["D"], 0.0, a["q"], a["k"], a["v"],
                                a["o"], a["od"], a["lse"], None)

    assert dense(q=None) == 1 and dense(D=32) == 2 and dense(N=-1) == 1 and dense(od=2) == 1
    assert dense(N=(1 << 20) + 1) == 2
    assert dense(B=1 << 16, H=1 << 8) == 2  # too many elements


def test_forward_queued_rejects_before_launch(lib):
    def fwd(**kw):
        a = dict(B=1, H=1, N=1024, D=128, block=64, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE,
                 mk=8, o=FAKE, od=1, lse=None, queue=FAKE)
        a.update(kw)
        return lib.ba_att_forward_queued(a["B"], a["H"], a["N"], a["D"], a["block"], 0.0, a["q"], a["k"],
                                         a["v"], a["idx"], a["cnt"], a["mk"], a["o"], a["od"], a["lse"],
                                         a["queue"], None)

    # the forward's own checks come first, then the queue's
    assert fwd(v=None) == 1 and fwd(o=None) == 1 and fwd(od=7) == 1 and fwd(mk=0) == 1
    assert fwd(D=80) == 2 and fwd(block=256) == 2
    assert fwd(queue=None) == 3
    assert fwd(queue=FAKE + 16) == 3  # not 64-byte aligned
    assert fwd(queue=None, q=None) == 1


def test_queue_words_agree_between_header_and_binding():
    from block_sparse_attention_ba_amd import api
    text = open(HEADER).read()
    m = re.search(r"#define BA_ATT_QUEUE_WORDS (\d+)", text)
    assert m and int(m.group(1)) == api.QUEUE_WORDS


def test_split_merge_ext_reject_before_launch(lib):
    assert lib.ba_att_forward_split_workspace_bytes(1, 2, 100, 64, 3) == 3 * 2 * 100 * 65 * 4
    assert lib.ba_att_forward_split_workspace_bytes(1, 2, 100, 64, 0) == 0
    assert lib.ba_att_forward_split_workspace_bytes(1, 2, 100, 64, 65) == 0
    assert lib.ba_att_forward_split_workspace_bytes(1, 2, 100, 96, 2) == 0

    def split(**kw):
        a = dict(B=1, H=1, N=1024, D=128, block=64, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE, mk=8,
                 ns=2, o=FAKE, od=1, lse=None, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.ba_att_forward_split(a["B"], a["H"], a["N"], a["D"], a["block"], 0.0, a["q"], a["k"],
                                        a["v"], a["idx"], a["cnt"], a["mk"], a["ns"], a["o"], a["od"],
                                        a["lse"], a["ws"], a["wsb"], None)

    assert split(ns=0) == 1 and split(ns=65) == 1
    assert split(ws=None) == 3 and split(wsb=1024) == 3
    assert split(v=None) == 1 and split(block=32) == 2 and split(o=FAKE + 4) == 1

    def merge(**kw):
        a = dict(B=1, H=2, N=64, D=64, P=2, op=FAKE, lp=FAKE, o=FAKE, od=0, lse=None)
        a.update(kw)
        return lib.ba_att_merge(a["B"], a["H"], a["N"], a["D"], a["P"], a["op"], a["lp"], a["o"], a["od"],
                                a["lse"], None)

    assert merge(P=0) == 1 and merge(P=65) == 1 and merge(op=None) == 1 and merge(lp=None) == 1
    assert merge(D=96) == 2 and merge(od=3) == 1 and merge(op=FAKE + 8) == 1

    def ext(**kw):
        a = dict(B=1, H=1, N=1024, D=64, block=64, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE, mk=8,
                 oe=FAKE, le=FAKE, o=FAKE, od=1, lse=None)
        a.update(kw)
        return lib.ba_att_forward_ext(a["B"], a["H"], a["N"], a["D"], a["block"], 0.0, a["q"], a["k"], a["v"],
                                      a["idx"], a["cnt"], a["mk"], a["oe"], a["le"], a["o"], a["od"], a["lse"],
                                      None)

    assert ext(oe=None) == 1 and ext(le=None) == 1 and ext(oe=FAKE + 4) == 1 and ext(D=80) == 2


def test_mask_to_index_rejects_before_launch(lib):
    def m2i(**kw):
        a = dict(B=1, H=1, n=16, mask=FAKE, mk=16, idx=FAKE, cnt=FAKE)
        a.update(kw)
        return lib.ba_att_mask_to_index(a["B"], a["H"], a["n"], a["mask"], a["mk"], a["idx"],
                                        a["cnt"], None)

    assert m2i(mask=None) == 1 and m2i(mk=0) == 1 and m2i(n=0) == 1
    assert m2i(n=2049) == 2
    assert m2i(idx=FAKE + 1) == 1


def test_python_binding_fails_loudly_without_library(tmp_path):
    from block_sparse_attention_ba_amd import _lib
    saved = _lib._lib
    try:
        _lib._lib = None
        with pytest.raises(ImportError):
            _lib.load(str(tmp_path / "missing.so"))
    finally:
        _lib._lib = saved


def test_diagnostics_reject_before_launch(lib):
    kf = 128 + 128 * 129
    ws = lib.ba_att_score_full_workspace_bytes(1, 32, 8192, 128, 64)
    assert ws >= 2 * 32 * 128 * kf * 4 and ws % 4 == 0
    assert lib.ba_att_score_full_workspace_bytes(1, 1, 1024, 96, 64) == 0
    assert lib.ba_att_score_full_workspace_bytes(1, 1, 1024, 64, 32) == 0
    assert lib.ba_att_score_full_workspace_bytes(1, 1, 64 * 513, 64, 64) == 0  # n > 512

    def bmap(**kw):
        a = dict(B=1, H=1, N=1024, D=64, block=64, q=FAKE, k=FAKE, lse=FAKE, ml=FAKE, mp=FAKE)
        a.update(kw)
        return lib.ba_att_block_map(a["B"], a["H"], a["N"], a["D"], a["block"], 0.0, a["q"], a["k"], a["lse"],
                                    a["ml"], a["mp"], None)

    assert bmap(q=None) == 1 and bmap(ml=None) == 1
    assert bmap(lse=None) == 1 and bmap(mp=None) == 1  # lse and m_prob go together
    assert bmap(D=96) == 2 and bmap(block=256) == 2 and bmap(q=FAKE + 2) == 1
    assert bmap(N=64 * 2049) == 2  # LDS partials of more than 4096 (block, wave) pairs

    def full(**kw):
        a = dict(B=1, H=1, N=1024, D=64, block=64, q=FAKE, k=FAKE, sf=FAKE, sm=None, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.ba_att_score_full(a["B"], a["H"], a["N"], a["D"], a["block"], 0.0, a["q"], a["k"], a["sf"],
                                     a["sm"], a["ws"], a["wsb"], None)

    assert full(sf=None) == 1 and full(k=None) == 1 and full(D=80) == 2 and full(block=16) == 2
    assert full(ws=None) == 3 and full(wsb=4096) == 3 and full(ws=FAKE + 4) == 3

    def agree(**kw):
        a = dict(B=1, H=1, n=16, keep=8, x=FAKE, r=FAKE, rec=FAKE, rho=FAKE)
        a.update(kw)
        return lib.ba_att_rank_agreement(a["B"], a["H"], a["n"], a["keep"], a["x"], a["r"], a["rec"], a["rho"],
                                         None)

    assert agree(keep=0) == 1 and agree(keep=17) == 1 and agree(x=None) == 1 and agree(rho=None) == 1
    assert agree(n=513, keep=8) == 2 and agree(x=FAKE + 2) == 1


def test_python_binding_rejects_host_tensors_before_any_call():
    import torch
    from block_sparse_attention_ba_amd import api
    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.dense(x, x, x)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.select(x, x, 64, 0.5)


def test_peaks_library_exports_its_header_and_rejects_bad_arguments():
    import ctypes
    from block_sparse_attention_ba_amd import _lib
    if not os.path.exists(_lib.PEAKS_PATH):
        from block_sparse_attention_ba_amd import build
        build.build()
    peaks = _lib.load_peaks()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ba_peaks.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(ba_peak_\w+)\s*\(", text)))
    assert declared == sorted(name for name, _, _ in _lib.PEAK_SIGNATURES)
    for name in declared:
        assert hasattr(peaks, name), name
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below is rejected on the host
    assert peaks.ba_peak_read(None, 16, fake, 1, 0, None) == 1
    assert peaks.ba_peak_read(fake, 15, fake, 1, 1, None) == 1
    assert peaks.ba_peak_read(fake, 16, fake, 0, 0, None) == 1
    assert peaks.ba_peak_copy(fake, fake, 64, 1, None) == 1  # overlapping
    assert peaks.ba_peak_copy(ctypes.c_void_p((1 << 20) + 8), ctypes.c_void_p(1 << 30), 64, 1, None) == 1
    assert peaks.ba_peak_mfma_bf16(None, 1, 1, 0.0, None) == 1
    assert peaks.ba_peak_mfma_bf16(fake, 1, 0, 0.0, None) == 1
    assert peaks.ba_peak_mfma_bf16_random(None, 1, 1, 0, None) == 1
    assert peaks.ba_peak_mfma_bf16_random(fake, 0, 1, 0, None) == 1
    assert peaks.ba_peak_mfma_bf16_random(fake, 1, 0, 0, None) == 1


def test_split_parts_rejects_invalid_shapes_before_any_device_query(lib):
    assert lib.ba_att_forward_split_parts(0, 1, 1024, 64, 4) == 0
    assert lib.ba_att_forward_split_parts(1, 1, 0, 64, 4) == 0
    assert lib.ba_att_forward_split_parts(1, 1, 1024, 96, 4) == 0
    assert lib.ba_att_forward_split_parts(1, 1, 1024, 64, 0) == 0
    assert lib.ba_att_forward_split_parts(1, 1, (1 << 20) + 1, 64, 4) == 0


def test_select_noalloc_rejects_before_launch(lib):
    """The allocation-free selection call checks its arguments like
    ba_att_select and refuses, before touching the GPU, a shape whose pooled
    statistics exceed its fixed 64 MiB scratch."""
    ok = dict(B=1, H=1, N=1024, D=64, block=64, scale=0.0, sp=0.5)

    def call(**kw):
        a = dict(ok, q=FAKE, k=FAKE, mask=FAKE, idx=FAKE, cnt=FAKE, score=None)
        a.update(kw)
        return lib.ba_att_select_noalloc(a["B"], a["H"], a["N"], a["D"], a["block"], a["scale"], a["sp"],
                                         a["q"], a["k"], a["mask"], a["idx"], a["cnt"], a["score"], None)

    assert call(q=None) == 1 and call(sp=1.0) == 1 and call(q=FAKE + 2) == 1
    assert call(D=96) == 2 and call(block=32) == 2 and call(N=2049 * 64) == 2
    # 2*64*1024*256*4 bytes of statistics: beyond the scratch
    assert lib.ba_att_select_workspace_bytes(2, 32, 65536, 128, 64) > (64 << 20)
    assert call(B=2, H=32, N=65536, D=128, block=64) == 5
    # the distribution-shift shape (B2 H32 N32768 D128 b128) fits: 32 MiB
    assert lib.ba_att_select_workspace_bytes(2, 32, 32768, 128, 128) == 32 << 20
    assert b"scratch" in lib.ba_att_status_string(5)
