"""Seeded synthetic workloads for the BA-Att operator.

This module builds inputs only: it holds none of the operator's arithmetic
and serves both the HIP path and the CPU oracle.  Every tensor is returned as
bf16 bit patterns (numpy uint16, layout [B, H, N, D], D fastest), produced by
round-to-nearest-even from float32 draws.

The five workloads stand in, by shape only, for the public suites on which
the BA-Att paper reports quality (long-context LM suites at 4K-32K tokens with
LLaDA-family models, and video models): no item of any suite is used.

Seeding: numpy PCG64 with seed 20260519 + workload index (1..5).  The root
SeedSequence spawns four children (Q noise, K noise, V noise, structure) and
each child spawns one grandchild per (batch, head), so every head draws its
own structure and heads can be generated in any order.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "f32_to_bf16_bits", "bf16_bits_to_f32", "make_inputs"]

SEED_BASE = 20260519


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed offset and position in the workload list (1-based)
    B: int
    H: int
    N: int
    D: int
    block: int
    sparsities: tuple
    kind: str
    grid: tuple | None = None
    description: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 1024, 64, 64, (0.5,), "normal",
                     description="B1 H1 N1024 D64 b64, Q/K/V ~ N(0,1)"),
    "llada8b": Workload("llada8b", 2, 1, 32, 8192, 128, 64, (0.5,), "salient",
                        description="LLaDA-8B-shaped layer: B1 H32 N8192 D128 b64, "
                                    "Q/K/V ~ N(0,1) + 2% planted salient keys"),
    "long_b64": Workload("long_b64", 3, 1, 32, 16384, 128, 64, (0.0, 0.5, 0.75), "mixture",
                         description="long-context: B1 H32 N16384 D128 b64, 16-cluster mixture"),
    "long_b128": Workload("long_b128", 3, 1, 32, 16384, 128, 128, (0.0, 0.5, 0.75), "mixture",
                          description="long-context: B1 H32 N16384 D128 b128, 16-cluster mixture"),
    "shift": Workload("shift", 4, 2, 32, 32768, 128, 128, (0.5,), "shift",
                      description="distribution shift: B2 H32 N32768 D128 b128, drifting "
                                  "mixture + local band + needles"),
    "video": Workload("video", 5, 1, 40, 32760, 128, 128, (0.5,), "video", grid=(21, 30, 52),
                      description="video-DiT-shaped: B1 H40 21x30x52=32760 tokens D128 b128, "
                                  "smooth 3D field + N(0,0.3^2) noise"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite
    inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _plant_keys(k: np.ndarray, q: np.ndarray, count: int, rng: np.random.Generator) -> None:
    """Overwrite `count` keys at distinct uniform positions with a key of four
    times its own norm pointing along a uniformly chosen query."""
    N = k.shape[0]
    pos = rng.choice(N, size=count, replace=False)
    src = rng.integers(0, N, size=count)
    kn = np.linalg.norm(k[pos], axis=1, keepdims=True)
    qd = q[src] / np.linalg.norm(q[src], axis=1, keepdims=True)
    k[pos] = (4.0 * kn * qd).astype(np.float32)


def _runs(N: int, rng: np.random.Generator, lo: int = 32, hi: int = 512, comps: int = 16) -> np.ndarray:
    """Component label per position: contiguous runs of length U{lo..hi}
    (the last run truncated), each run given a uniform component."""
    labels = np.empty(N, dtype=np.int64)
    t = 0
    while t < N:
        L = int(rng.integers(lo, hi + 1))
        labels[t:t + L] = int(rng.integers(0, comps))
        t += L
    return labels


def _head(w: Workload, rq, rk, rv, rs):
    N, D = w.N, w.D
    f32 = np.float32
    if w.kind in ("normal", "salient"):
        q = rq.standard_normal((N, D), dtype=f32)
        k = rk.standard_normal((N, D), dtype=f32)
        v = rv.standard_normal((N, D), dtype=f32)
        if w.kind == "salient":
            _plant_keys(k, q, int(round(0.02 * N)), rs)
        return q, k, v
    if w.kind == "mixture":
        mu = rs.standard_normal((16, D), dtype=f32)
        lab = _runs(N, rs)
        base = mu[lab]
        q = base + f32(0.5) * rq.standard_normal((N, D), dtype=f32)
        k = base + f32(0.5) * rk.standard_normal((N, D), dtype=f32)
        v = rv.standard_normal((N, D), dtype=f32)
        return q, k, v
    if w.kind == "shift":
        mu0 = rs.standard_normal((16, D), dtype=f32)
        mu1 = rs.standard_normal((16, D), dtype=f32)
        lab = _runs(N, rs)
        tau = (np.arange(N, dtype=np.float64) / (N - 1)).astype(f32)[:, None]
        base = (f32(1) - tau) * mu0[lab] + tau * mu1[lab]
        # local band: anchors every 256 tokens, linearly interpolated between
        n_anchor = (N - 1) // 256 + 2
        anchors = rs.standard_normal((n_anchor, D), dtype=f32)
        pos = np.arange(N)
        a0 = pos // 256
        frac = ((pos % 256) / 256.0).astype(f32)[:, None]
        band = (f32(1) - frac) * anchors[a0] + frac * anchors[a0 + 1]
        base = base + band
        q = base + f32(0.5) * rq.standard_normal((N, D), dtype=f32)
        k = base + f32(0.5) * rk.standard_normal((N, D), dtype=f32)
        v = rv.standard_normal((N, D), dtype=f32)
        _plant_keys(k, q, 32, rs)
        return q, k, v
    if w.kind == "video":
        from scipy.ndimage import gaussian_filter1d
        T, Hh, Ww = w.grid
        F = rs.standard_normal((T, Hh, Ww, D), dtype=f32)
        for ax in range(3):
            F = gaussian_filter1d(F, sigma=2.0, axis=ax, mode="reflect", truncate=4.0)
        F = F.reshape(N, D)
        F = (F / F.std(axis=0, keepdims=True)).astype(f32)
        q = F + f32(0.3) * rq.standard_normal((N, D), dtype=f32)
        k = F + f32(0.3) * rk.standard_normal((N, D), dtype=f32)
        v = rv.standard_normal((N, D), dtype=f32)
        return q, k, v
    raise ValueError(f"unknown workload kind {w.kind!r}")


def make_inputs(name: str) -> dict:
    """Seeded bf16 Q, K, V bit arrays [B, H, N, D] for a named workload."""
    w = WORKLOADS[name]
    B, H, N, D = w.B, w.H, w.N, w.D
    root = np.random.SeedSequence(SEED_BASE + w.index)
    cq, ck, cv, cs = root.spawn(4)
    sq, sk, sv, ss = (c.spawn(B * H) for c in (cq, ck, cv, cs))
    out = {x: np.empty((B, H, N, D), dtype=np.uint16) for x in ("q", "k", "v")}
    for i in range(B * H):
        gens = [np.random.Generator(np.random.PCG64(s[i])) for s in (sq, sk, sv, ss)]
        q, k, v = _head(w, *gens)
        bi, hi = divmod(i, H)
        out["q"][bi, hi] = f32_to_bf16_bits(q)
        out["k"][bi, hi] = f32_to_bf16_bits(k)
        out["v"][bi, hi] = f32_to_bf16_bits(v)
    out["workload"] = w
    return out
