"""GPTQ: quantize and compensate as you go (oracle; test infrastructure only).

"4.3 Weight-only INT4", section 2 (GPTQ). The objective is the layer-output
reconstruction error ||X W - X W_hat||_F^2 over calibration inputs X[n, K] (section 2.1),
which for one output column w has the Hessian H = 2 X^T X. Weights are fixed one input
channel at a time (one row of W[K, N], every output column at once); after row i is fixed
to its dequantized value w_hat_i, the rows still free (the index set F) move by

    dw_F = -(w_i - w_hat_i) / [H_F^-1]_ii * [H_F^-1]_{:, i}        (section 2.2)

which turns row i into w_hat_i exactly and compensates the rest. w_hat_i is the
dequantized value on the weight's own scale (here the 16-bit W_hat the GEMM multiplies).

Readings taken where the section leaves a step open (listed in the design notes):
* damping: the section says the reference implementation adds damping for numerical
  stability without a value; 1% of the mean of diag(H) is added to the diagonal;
* rows are fixed in index order 0..K-1 (no activation reordering);
* a group's scale and zero-point come from the group's rows as they stand when its first
  row is reached (earlier groups' compensation included), with the same RTN rules as
  :func:`oracle.quant.quantize_rtn_asym` / ``quantize_rtn_sym``; the codes of later rows in
  the group use those fixed parameters;
* after fixing row i, H_F^-1 for the smaller set is obtained from the current one by the
  block-inverse (Schur complement) identity, which equals inverting H restricted to the
  remaining rows (``exact_inverse=True`` does the latter, for checking).
"""
from __future__ import annotations

import numpy as np

from .dequant import _round_to
from .fp import scale_values
from .quant import quantize_rtn_asym, quantize_rtn_sym


def hessian(X: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """``H = 2 X^T X`` (fp64) plus ``damp * mean(diag H)`` on the diagonal."""
    X = np.asarray(X, dtype=np.float64)
    H = 2.0 * X.T @ X
    d = float(np.mean(np.diag(H))) if H.size else 0.0
    if damp and d > 0:
        H = H + damp * d * np.eye(H.shape[0])
    return H


def compensate(W_F: np.ndarray, w_hat_i: np.ndarray, Hinv_F: np.ndarray):
    """One step of section 2.2. ``W_F[|F|, N]`` holds the free rows with row i first,
    ``Hinv_F`` is ``[H_F^-1]`` for the same index order. Returns the rows after the update
    (row i equal to ``w_hat_i``) and ``[H_F'^-1]`` for F' = F without i."""
    err = (W_F[0] - w_hat_i) / Hinv_F[0, 0]
    W_new = W_F - np.outer(Hinv_F[:, 0], err)
    Hinv_next = Hinv_F[1:, 1:] - np.outer(Hinv_F[1:, 0], Hinv_F[0, 1:]) / Hinv_F[0, 0]
    return W_new, Hinv_next


def gptq_quantize(W: np.ndarray, X: np.ndarray, group_size: int, scale_dtype: str = "f16",
                  symmetric: bool = False, damp: float = 0.01, exact_inverse: bool = False):
    """GPTQ with groups along K. Returns the same tuple as the RTN quantizers:
    ``(q[K,N] uint8 0..15, scales[K/g,N] stored, zeros[K/g,N] uint8)`` for the affine
    format, ``(q[K,N] int8 -8..7, scales[K/g,N] stored)`` for the symmetric one."""
    W = np.array(W, dtype=np.float64)
    K, N = W.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    H = hessian(X, damp)
    if H.shape != (K, K):
        raise ValueError("X must have K columns")
    Hinv = np.linalg.inv(H)
    q = np.zeros((K, N), dtype=np.int16)
    G = K // group_size
    s_rows, z_rows = [], []
    for i in range(K):
        if i % group_size == 0:
            if symmetric:
                _, s_store = quantize_rtn_sym(W[i:i + group_size], group_size, scale_dtype)
                z = np.zeros(N)
            else:
                _, s_store, zq = quantize_rtn_asym(W[i:i + group_size], group_size, scale_dtype)
                z = zq[0].astype(np.float64)
                z_rows.append(zq[0])
            s_rows.append(s_store[0])
            s = scale_values(s_store, scale_dtype)[0]
        lo, hi = (-8, 7) if symmetric else (0, 15)
        qi = np.clip(np.rint(W[i] / s) + z, lo, hi)
        w_hat = _round_to((qi - z) * s, scale_dtype)
        w_hat = w_hat.astype(np.float64) if scale_dtype == "f16" else scale_values(w_hat, "bf16")
        Hinv_F = np.linalg.inv(H[i:, i:]) if exact_inverse else Hinv
        W[i:], Hinv = compensate(W[i:], w_hat, Hinv_F)
        q[i] = qi
    scales = np.stack(s_rows)
    if symmetric:
        return q.astype(np.int8), scales
    return q.astype(np.uint8), scales, np.stack(z_rows).astype(np.uint8)
