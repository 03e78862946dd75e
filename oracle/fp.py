"""Rounding of fp64 values to the 16-bit storage types (oracle; test infrastructure only).

fp16 values are returned as ``np.float16``; bf16 values as ``np.uint16`` bit patterns
(NumPy has no bf16 type). bf16 is the top half of an IEEE binary32, so it has fp32's
exponent range and an 8-bit significand.
"""
from __future__ import annotations

import numpy as np


def round_nearest_f16(v) -> np.ndarray:
    """Round fp64 values to fp16, nearest with ties to even (NumPy's own cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def round_up_f16(v) -> np.ndarray:
    """Smallest fp16 value >= v (rounding toward +infinity)."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    low = h.astype(np.float64) < v
    if np.any(low):
        h = np.where(low, np.nextafter(h, np.float16(np.inf)), h)
    return h


def _bf16_from_f64(v: np.ndarray, mode: str) -> np.ndarray:
    """Round fp64 -> bf16 by splitting into significand and exponent (normal range)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
    scaled = m * 256.0                      # 8 significant bits before the point
    if mode == "nearest":
        r = np.rint(scaled)                 # ties to even
    elif mode == "up":
        r = np.ceil(scaled)
    else:
        raise ValueError(mode)
    out = np.ldexp(r / 256.0, e).astype(np.float32)   # exact: <= 9 significant bits
    return (out.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_nearest_bf16_bits(v) -> np.ndarray:
    """Round fp64 values to bf16, nearest with ties to even; uint16 bit patterns."""
    return _bf16_from_f64(v, "nearest")


def round_up_bf16_bits(v) -> np.ndarray:
    """Smallest bf16 value >= v (v > 0 in every use here); uint16 bit patterns."""
    return _bf16_from_f64(v, "up")


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def scale_values(scales, dtype: str) -> np.ndarray:
    """fp64 values of a stored scale tensor (``np.float16`` or bf16 uint16 bits)."""
    if dtype == "f16":
        return np.asarray(scales, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(scales)
    raise ValueError(dtype)
