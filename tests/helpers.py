"""Shared helpers of the GPU parity tests (no test functions here)."""

from __future__ import annotations

import math

import numpy as np

# relative cut margin below which a row's cut counts as ambiguous:
# (p_keep - p_keep+1)/p_keep < 1e-4  <=>  s_keep - s_keep+1 < -ln(1 - 1e-4)
REL_MARGIN = 1e-4
ABS_BAND = -math.log1p(-REL_MARGIN)

O_TOL = 1e-2      # max |O - O_oracle|
LSE_TOL = 1e-3    # max |LSE - LSE_oracle|


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def compare_masks(gpu_mask: np.ndarray, S: np.ndarray, oracle_mask: np.ndarray, keep: int) -> dict:
    """Row-by-row mask comparison against the oracle with the near-tie rule.

    A row must equal the oracle's unless its oracle cut margin is ambiguous
    (s_keep - s_keep+1 < ABS_BAND); such rows are counted, and the GPU's row
    must still be a valid top-`keep` up to that band.  Returns counts and
    the list of failing rows."""
    rows = S.reshape(-1, S.shape[-1])
    g = gpu_mask.reshape(rows.shape).astype(bool)
    o = oracle_mask.reshape(rows.shape).astype(bool)
    n = rows.shape[1]
    res = {"rows": rows.shape[0], "exact": 0, "near_tie_rows": 0, "near_tie_mismatch": 0, "bad": []}
    for r in range(rows.shape[0]):
        s = rows[r]
        srt = np.sort(s)[::-1]
        ambiguous = keep < n and (srt[keep - 1] - srt[keep]) < ABS_BAND
        res["near_tie_rows"] += int(ambiguous)
        if np.array_equal(g[r], o[r]):
            res["exact"] += 1
            continue
        if ambiguous and g[r].sum() == keep:
            worst_kept = s[g[r]].min()
            best_dropped = s[~g[r]].max() if keep < n else -np.inf
            if best_dropped - worst_kept <= 2 * ABS_BAND:
                res["near_tie_mismatch"] += 1
                continue
        res["bad"].append(r)
    return res


def max_abs(a, b) -> float:
    """max |a - b|, where equal infinities count as equal and a NaN on
    either side counts as an infinite error."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if np.isnan(a).any() or np.isnan(b).any():
        return math.inf
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0
