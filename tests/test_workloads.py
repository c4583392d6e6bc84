"""Seeded workload generators (CPU): reproducibility, bf16 rounding against
its definition, and the structure each recipe promises."""

import numpy as np
import pytest

from block_sparse_attention_ba_amd import workloads as wl


def test_bf16_round_to_nearest_even():
    vals = np.array([
        1.0,
        1.0 + 2.0 ** -8,            # halfway, low neighbour even -> 1.0
        1.0 + 3 * 2.0 ** -8,        # halfway, high neighbour even -> 1 + 2^-6
        1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above halfway -> up
        -2.5, 3.0e38, 1e-40,
    ], dtype=np.float32)
    got = wl.f32_to_bf16_bits(vals)
    assert got[0] == 0x3F80
    assert got[1] == 0x3F80
    assert got[2] == 0x3F82
    assert got[3] == 0x3F81
    assert wl.bf16_bits_to_f32(got[4:5])[0] == -2.5
    # every result is one of the two bf16 neighbours and the nearer one
    x = np.random.default_rng(0).normal(size=20000).astype(np.float32) * 7
    r = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x)).astype(np.float64)
    u = x.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    hi = ((u & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    assert np.all((r == lo) | (r == hi))
    assert np.all(np.abs(r - x) <= np.minimum(np.abs(lo - x), np.abs(hi - x)) + 0.0)


def test_tiny_is_reproducible_and_shaped():
    a = wl.make_inputs("tiny")
    b = wl.make_inputs("tiny")
    for t in ("q", "k", "v"):
        assert a[t].shape == (1, 1, 1024, 64) and a[t].dtype == np.uint16
        assert np.array_equal(a[t], b[t])
    q = wl.bf16_bits_to_f32(a["q"])
    assert abs(q.mean()) < 0.02 and abs(q.std() - 1.0) < 0.02
    assert not np.array_equal(a["q"], a["k"])


def test_workload_table_matches_stated_shapes():
    w = wl.WORKLOADS
    assert (w["llada8b"].B, w["llada8b"].H, w["llada8b"].N, w["llada8b"].D, w["llada8b"].block) == (1, 32, 8192, 128, 64)
    assert w["long_b64"].block == 64 and w["long_b128"].block == 128 and w["long_b64"].sparsities == (0.0, 0.5, 0.75)
    assert (w["shift"].B, w["shift"].H, w["shift"].N) == (2, 32, 32768)
    v = w["video"]
    assert v.grid[0] * v.grid[1] * v.grid[2] == v.N == 32760 and v.H == 40
    assert v.N % v.block == 120


def test_runs_have_stated_lengths():
    rng = np.random.default_rng(3)
    lab = wl._runs(16384, rng)
    change = np.flatnonzero(np.diff(lab) != 0) + 1
    bounds = np.concatenate([[0], change, [16384]])
    lengths = np.diff(bounds)
    # adjacent runs may draw the same component and merge; all but the last
    # run are at least 32 long and labels lie in 0..15
    assert lengths[:-1].min() >= 32
    assert lab.min() >= 0 and lab.max() <= 15


def test_planted_keys_are_aligned_and_scaled():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((512, 16)).astype(np.float32)
    k = rng.standard_normal((512, 16)).astype(np.float32)
    k0 = k.copy()
    wl._plant_keys(k, q, 10, np.random.default_rng(5))
    changed = np.flatnonzero(np.any(k != k0, axis=1))
    assert changed.size == 10
    ratio = np.linalg.norm(k[changed], axis=1) / np.linalg.norm(k0[changed], axis=1)
    assert np.allclose(ratio, 4.0, rtol=1e-5)
    cos = (k[changed] @ q.T) / np.linalg.norm(k[changed], axis=1)[:, None] / np.linalg.norm(q, axis=1)[None, :]
    assert np.all(cos.max(axis=1) > 0.9999)


@pytest.mark.slow
def test_llada_salient_count():
    x = wl.make_inputs("llada8b")
    k = wl.bf16_bits_to_f32(x["k"][0, 0]).astype(np.float64)
    nrm = np.linalg.norm(k, axis=1)
    # planted keys have about 4x the typical norm (sqrt(128) ~ 11.3)
    assert abs(int((nrm > 30).sum()) - 164) <= 3
