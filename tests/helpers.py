"""Shared helpers of the GPU parity tests (no test functions here)."""

from __future__ import annotations

import math

import numpy as np

from oracle.parity import (  # noqa: F401  (the shared bars)
    ABS_BAND, LSE_TOL, O_TOL, REL_MARGIN, compare_masks, index_matches_mask, map_heads, max_abs)


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
