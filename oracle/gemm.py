"""The W4A16 GEMM reference: dequantize, then multiply (oracle; test infrastructure only).

"4.3 Weight-only INT4", section 1 (W4A16 storage and compute) and section 4 (Marlin):
the fused kernel computes the same product as the naive path that expands the INT4
weight to FP16 and then runs an ordinary GEMM; fusion only moves where the expanded
weight lives. So the result is ``y[M, N] = x[M, K] @ W_hat[K, N]`` with W_hat from
:mod:`oracle.dequant`. The reference carries the product and the sum in fp64; the
kernels accumulate in fp32, and parity allows ``max|y - y_ref| <= 1e-3 * max|y_ref|``.
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_bits_to_f64


def _as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


def gemm_ref(x: np.ndarray, w_hat: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """``x[M,K] @ W_hat[K,N]`` in fp64; both operands stored in ``dtype``."""
    return _as_f64(x, dtype) @ _as_f64(w_hat, dtype)


def gemm_ref_columns(x: np.ndarray, w_hat_cols: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """Same as :func:`gemm_ref` for a subset of columns (``w_hat_cols[K, n_sample]``)."""
    return gemm_ref(x, w_hat_cols, dtype)


def gemm_bruteforce(x_vals, qweight, scale_vals, zero_vals, group_size: int, round16) -> list:
    """Triple loop over Python ints and floats, for tiny shapes only.

    ``x_vals[M][K]`` and ``scale_vals[G][N]`` are Python floats (exact values of the
    16-bit inputs), ``zero_vals[G][N]`` ints, ``qweight`` the packed int32 words and
    ``round16`` the rounding of one exact product to the weight type. Codes are pulled
    out of the words with shifts on Python ints, independently of :mod:`oracle.packing`.
    """
    M = len(x_vals)
    K = len(x_vals[0]) if M else 8 * len(qweight)
    N = len(scale_vals[0])
    y = [[0.0] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            word = int(qweight[k // 8][n]) & 0xFFFFFFFF
            code = (word >> (4 * (k % 8))) & 0xF
            g = k // group_size
            w = round16((code - zero_vals[g][n]) * scale_vals[g][n])
            for m in range(M):
                y[m][n] += x_vals[m][k] * w
    return y
