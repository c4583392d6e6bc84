"""The comparison rules of GPU results against the oracle (oracle/parity.py),
on the CPU: the near-tie rule of the mask comparison, the index-list check
and the error measure, each with cases that must pass and planted mistakes
that must fail."""

import math

import numpy as np

from oracle.parity import ABS_BAND, compare_masks, index_matches_mask, map_heads, max_abs


def _masks(S, keep):
    order = np.lexsort((np.arange(S.shape[-1])[None, :].repeat(S.shape[0], 0), -S), axis=-1)
    m = np.zeros(S.shape, dtype=np.uint8)
    np.put_along_axis(m, order[:, :keep], 1, axis=-1)
    return m


def test_band_is_the_relative_margin():
    assert math.isclose(1 - math.exp(-ABS_BAND), 1e-4, rel_tol=1e-12)


def test_equal_masks_are_exact_and_gaps_are_counted():
    rng = np.random.default_rng(0)
    S = rng.standard_normal((40, 16))
    S[3, 5] = S[3, np.argsort(-S[3])[3]] - ABS_BAND / 4   # near tie at the cut for keep = 4
    keep = 4
    m = _masks(S, keep)
    res = compare_masks(m, S, m, keep)
    assert res["exact"] == 40 and not res["bad"] and res["near_tie_mismatch"] == 0
    assert res["near_tie_rows"] >= 1


def test_swap_inside_the_band_is_counted_not_failed():
    S = np.array([[3.0, 2.0, 1.0 + ABS_BAND / 3, 1.0, 0.0]])
    keep = 3
    ref = _masks(S, keep)
    gpu = ref.copy()
    gpu[0, 2], gpu[0, 3] = 0, 1  # takes the near-tied block instead
    res = compare_masks(gpu, S, ref, keep)
    assert res["near_tie_rows"] == 1 and res["near_tie_mismatch"] == 1 and not res["bad"]


def test_swap_outside_the_band_fails():
    S = np.array([[3.0, 2.0, 1.5, 1.0, 0.0]])
    ref = _masks(S, 3)
    gpu = ref.copy()
    gpu[0, 2], gpu[0, 3] = 0, 1
    assert compare_masks(gpu, S, ref, 3)["bad"] == [0]


def test_wrong_count_fails_even_in_a_near_tie():
    S = np.array([[3.0, 2.0, 1.0 + ABS_BAND / 3, 1.0, 0.0]])
    ref = _masks(S, 3)
    gpu = ref.copy()
    gpu[0, 3] = 1  # four kept
    assert compare_masks(gpu, S, ref, 3)["bad"] == [0]


def test_index_lists_must_hold_the_ascending_ones():
    m = np.array([[[[1, 0, 1, 1], [0, 1, 1, 0]]]], dtype=np.uint8)
    idx = np.array([[[[0, 2, 3], [1, 2, 0]]]], dtype=np.int32)
    cnt = np.array([[[3, 2]]], dtype=np.int32)
    assert index_matches_mask(m, idx, cnt)
    bad = idx.copy()
    bad[0, 0, 0, :3] = [0, 3, 2]          # not ascending
    assert not index_matches_mask(m, bad, cnt)
    bad = idx.copy()
    bad[0, 0, 1, 1] = 3                   # names a dropped block
    assert not index_matches_mask(m, bad, cnt)
    assert not index_matches_mask(m, idx, np.array([[[3, 1]]], dtype=np.int32))  # wrong count


def test_max_abs_treats_nan_as_failure_and_equal_infinities_as_equal():
    assert max_abs([1.0, -np.inf], [1.5, -np.inf]) == 0.5
    assert max_abs([np.nan], [0.0]) == math.inf
    assert max_abs([np.inf], [-np.inf]) == math.inf


def test_map_heads_keeps_the_order():
    assert map_heads(lambda h: h * h, list(range(20)), threads=4) == [h * h for h in range(20)]
