"""Comparison rules of GPU results against the fp64 oracle.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
smoke check and the benchmark's CPU-baseline leg use it; the product path
never imports it.  It holds no arithmetic of the method, only the bars that a
result must meet and a helper that runs the oracle head by head on several
host threads.

Bars:
  * block masks are bit-exact, except rows whose oracle cut is ambiguous:
    the relative margin (p_keep - p_keep+1)/p_keep of the row-normalised
    scores is below 1e-4, i.e. s_keep - s_keep+1 < -ln(1 - 1e-4).  Such rows
    are counted; a differing row must still be a valid top-keep within that
    band;
  * max |O - O_oracle| <= 1e-2 and max |LSE - LSE_oracle| <= 1e-3.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

REL_MARGIN = 1e-4
ABS_BAND = -math.log1p(-REL_MARGIN)

O_TOL = 1e-2      # max |O - O_oracle|
LSE_TOL = 1e-3    # max |LSE - LSE_oracle|


def compare_masks(gpu_mask: np.ndarray, S: np.ndarray, oracle_mask: np.ndarray, keep: int) -> dict:
    """Row-by-row mask comparison against the oracle with the near-tie rule.

    Returns the row count, exact rows, near-tie rows (ambiguous cuts),
    near-tie mismatches (rows that differ inside the band) and the list of
    failing rows (flat row indices)."""
    rows = S.reshape(-1, S.shape[-1])
    g = gpu_mask.reshape(rows.shape).astype(bool)
    o = oracle_mask.reshape(rows.shape).astype(bool)
    n = rows.shape[1]
    res = {"rows": rows.shape[0], "exact": 0, "near_tie_rows": 0, "near_tie_mismatch": 0, "bad": []}
    if keep < n:
        part = -np.partition(-rows, (keep - 1, keep), axis=1)  # the keep-th and (keep+1)-th largest
        gaps = part[:, keep - 1] - part[:, keep]
        ambiguous = gaps < ABS_BAND
    else:
        ambiguous = np.zeros(rows.shape[0], dtype=bool)
    res["near_tie_rows"] = int(ambiguous.sum())
    equal = np.all(g == o, axis=1)
    res["exact"] = int(equal.sum())
    for r in np.nonzero(~equal)[0]:
        s = rows[r]
        if ambiguous[r] and g[r].sum() == keep:
            worst_kept = s[g[r]].min()
            best_dropped = s[~g[r]].max() if keep < n else -np.inf
            if best_dropped - worst_kept <= 2 * ABS_BAND:
                res["near_tie_mismatch"] += 1
                continue
        res["bad"].append(int(r))
    return res


def index_matches_mask(mask: np.ndarray, idx: np.ndarray, cnt: np.ndarray) -> bool:
    """True when every row's list holds exactly the ones of its mask row, in
    ascending order: cnt = number of ones, the first cnt entries strictly
    increasing, and each names a kept block."""
    n = mask.shape[-1]
    m = mask.reshape(-1, n).astype(bool)
    ix = idx.reshape(m.shape[0], -1).astype(np.int64)
    c = cnt.reshape(-1).astype(np.int64)
    if not np.array_equal(c, m.sum(axis=1)):
        return False
    width = ix.shape[1]
    if c.max(initial=0) > width:
        return False
    used = np.arange(width)[None, :] < c[:, None]
    if np.any(used & ((ix < 0) | (ix >= n))):
        return False
    inc = np.diff(ix, axis=1) > 0
    if np.any(used[:, 1:] & ~inc):
        return False
    hit = np.take_along_axis(m, np.clip(ix, 0, n - 1), axis=1)
    return bool(np.all(hit | ~used))


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


def host_threads(cap: int = 16) -> int:
    """Threads for the oracle on this host: the cores this process may run
    on, at most `cap`."""
    return max(1, min(cap, len(os.sched_getaffinity(0))))


def map_heads(fn, heads, threads: int | None = None) -> list:
    """fn(head) for every head, on a pool of host threads with one BLAS
    thread each (numpy releases the interpreter lock inside its array
    loops and BLAS calls, so heads run in parallel).  Results in the order of
    `heads`."""
    from threadpoolctl import threadpool_limits
    threads = threads or host_threads()
    with threadpool_limits(limits=1):
        if threads == 1:
            return [fn(h) for h in heads]
        with ThreadPoolExecutor(max_workers=threads) as ex:
            return list(ex.map(fn, heads))
