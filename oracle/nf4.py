"""NF4 codebook built from normal quantiles (oracle; test infrastructure only).

"INT4 and Low-Bit Inference", section 5 (The formats) describes NF4 only as 16
levels placed at the quantiles of a normal distribution, normalised absmax-style
(its further-reading list points to QLoRA). The construction below follows that
description and QLoRA's published recipe: one exact zero, eight positive and seven
negative levels at equally spaced probabilities of the standard normal between 1/2
and an end probability ``p_end``, each side divided by its extreme so the codebook
runs from -1 to +1. The pages give no end probability; the reading taken here is
``p_end = 1 - 1/32`` (the centre of the last of 16 equal-mass bins).

The result is frozen in ``tests/golden/nf4_codebook.txt``. Agreement with any
third-party NF4 table is unpinned; the kernels take the codebook as an argument.
"""
from __future__ import annotations

import math

import numpy as np


def _normal_cdf(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def inverse_normal_cdf(p: float) -> float:
    """Phi^{-1}(p) by bisection on the normal CDF (plain and slow; 0 < p < 1)."""
    if not 0.0 < p < 1.0:
        raise ValueError("p must lie strictly between 0 and 1")
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _normal_cdf(mid) < p:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 1e-300:
            break
    return 0.5 * (lo + hi)


def nf4_levels_f64(p_end: float = 1.0 - 1.0 / 32.0) -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending."""
    top = inverse_normal_cdf(p_end)
    pos = [inverse_normal_cdf(p) / top for p in np.linspace(0.5, p_end, 9)[1:]]
    neg = [-inverse_normal_cdf(p) / top for p in np.linspace(0.5, p_end, 8)[1:]]
    return np.array(sorted(neg + [0.0] + pos), dtype=np.float64)


def nf4_codebook(p_end: float = 1.0 - 1.0 / 32.0) -> np.ndarray:
    """The 16 NF4 levels rounded to fp16 (nearest-even), ascending."""
    return nf4_levels_f64(p_end).astype(np.float16)
