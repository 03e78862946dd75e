"""AWQ: activation-aware per-channel scaling before quantization (oracle; test
infrastructure only).

"4.3 Weight-only INT4", section 3 (AWQ). A weight error dw_j reaches the output as
x_j * dw_j (section 3.1), so the input channels whose activations run large are the ones
to protect. Rather than keep them in 16 bits, section 3.2 scales each input channel j: row
j of the weight W[K, N] is multiplied by s_j before quantization and activation column j is
divided by s_j, so with S = diag(s)

    Y = (X S^-1)(S W)   exactly,   and   Y_hat = (X S^-1) D(Q(S W)).

What is deployed is the regular INT4 format of S W together with the vector S^-1; the
product is the plain W4A16 GEMM of the scaled activations.

Readings taken where the section leaves a step open (listed in the design notes):
* S^-1 is stored in the activation type (fp16, or bf16 as uint16 bits) and the activation
  the GEMM multiplies is x'[m, j] = RN(x[m, j] * s_inv[j]) in that type: one rounding of the
  exact product (two 16-bit significands multiply exactly in fp64). The weight is scaled by
  1 / s_inv[j] of the stored value, so (X S^-1)(S W) = X W up to fp64 rounding;
* the search space: the section says the scale factors are searched on calibration data
  and does not give the family. The AWQ paper's one-parameter family is used:
  s_j = a_j ** alpha with a_j = mean_n |X[n, j]| (floored at 1e-8 of the largest, so a
  channel that never fires keeps a finite scale), normalised so that max(s) * min(s) = 1,
  alpha on the grid 0, 1/n, ..., (n-1)/n, and the alpha with the least output error
  ||X W - X' D(Q(S W))||_F^2 wins (alpha = 0 gives s = 1, plain RTN);
* the clipping search the section pairs with the scale search is not done: its form is
  not given.
"""
from __future__ import annotations

import numpy as np

from .dequant import dequant_affine
from .fp import bf16_bits_to_f64, round_nearest_bf16_bits, round_nearest_f16
from .packing import pack_codes, pack_zeros
from .quant import quantize_rtn_asym, quantize_rtn_sym, to_offset_binary


def _values(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(dtype)


def _store(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return round_nearest_f16(v)
    if dtype == "bf16":
        return round_nearest_bf16_bits(v)
    raise ValueError(dtype)


def scale_activations(x: np.ndarray, s_inv: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """X S^-1 as the GEMM sees it: ``RN(x[m, j] * s_inv[j])`` in ``dtype``.

    ``x[M, K]`` and ``s_inv[K]`` are stored in ``dtype`` (np.float16 or bf16 bits); the
    result is stored the same way."""
    xv, sv = _values(x, dtype), _values(s_inv, dtype)
    if xv.ndim != 2 or sv.shape != (xv.shape[1],):
        raise ValueError("x must be (M, K) and s_inv (K,)")
    return _store(xv * sv[None, :], dtype)


def scale_weight(W: np.ndarray, s_inv: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """S W with s_j = 1 / s_inv[j] (stored value): row j of ``W[K, N]`` times s_j, fp64."""
    s = 1.0 / _values(s_inv, dtype)
    return np.asarray(W, dtype=np.float64) * s[:, None]


def candidate_scales(X: np.ndarray, alpha: float, dtype: str = "f16") -> np.ndarray:
    """The stored S^-1 of one point of the search: s = a ** alpha, a_j = mean |X[:, j]|,
    normalised to max(s) * min(s) = 1, stored as RN(1 / s) in ``dtype``."""
    a = np.mean(np.abs(np.asarray(X, dtype=np.float64)), axis=0)
    top = float(a.max()) if a.size else 0.0
    a = np.maximum(a, 1e-8 * top if top > 0 else 1.0)
    s = a ** float(alpha)
    s = s / np.sqrt(s.max() * s.min())
    return _store(1.0 / s, dtype)


def _quantize(Ws: np.ndarray, group_size: int, dtype: str, symmetric: bool):
    """RTN of S W in the stored format, and its dequantized 16-bit value D(Q(S W))."""
    if symmetric:
        q, scales = quantize_rtn_sym(Ws, group_size, dtype)
        w_hat = dequant_affine(pack_codes(to_offset_binary(q)), scales, None, group_size, dtype)
        return (q, scales), w_hat
    q, scales, zeros = quantize_rtn_asym(Ws, group_size, dtype)
    w_hat = dequant_affine(pack_codes(q), scales, pack_zeros(zeros), group_size, dtype)
    return (q, scales, zeros), w_hat


def output_error(W: np.ndarray, X: np.ndarray, s_inv: np.ndarray, w_hat: np.ndarray,
                 dtype: str = "f16") -> float:
    """||X W - X' D(Q(S W))||_F^2 with X taken in ``dtype`` on both sides."""
    Xq = _store(np.asarray(X, dtype=np.float64), dtype)
    Y = _values(Xq, dtype) @ np.asarray(W, dtype=np.float64)
    Y_hat = _values(scale_activations(Xq, s_inv, dtype), dtype) @ _values(w_hat, dtype)
    return float(np.sum((Y - Y_hat) ** 2))


def awq_quantize(W: np.ndarray, X: np.ndarray, group_size: int, dtype: str = "f16",
                 symmetric: bool = False, n_grid: int = 20):
    """Search alpha, then quantize S W. Returns ``(quant, s_inv, alpha, errors)``:
    ``quant`` is the RTN tuple of S W (``(q, scales, zeros)`` affine, ``(q, scales)``
    symmetric, as :mod:`oracle.quant` returns them), ``s_inv[K]`` the stored S^-1,
    ``alpha`` the chosen grid point and ``errors`` the output error of every grid point."""
    W = np.asarray(W, dtype=np.float64)
    best = None
    errors = []
    for i in range(n_grid):
        alpha = i / n_grid
        s_inv = candidate_scales(X, alpha, dtype)
        quant, w_hat = _quantize(scale_weight(W, s_inv, dtype), group_size, dtype, symmetric)
        err = output_error(W, X, s_inv, w_hat, dtype)
        errors.append(err)
        if best is None or err < best[0]:
            best = (err, quant, s_inv, alpha)
    return best[1], best[2], best[3], errors
