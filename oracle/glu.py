"""SwiGLU epilogue of a fused gate+up projection (oracle; test infrastructure only).

The pages stop at the linear layer and name operator fusion as the next step ("4.3
Weight-only INT4", closing section, "Next: 07 - Kernel and operator fusion"); they do not
define the MLP. The reading taken here is the Llama MLP whose shapes the pages' decode
examples use (the 4096x28672 gate+up projection is two 4096x14336 halves): the two
projections are stored side by side in one (K, 2N) weight, gate columns first, and the
epilogue forms ``h = SiLU(x W_gate) * (x W_up)`` with ``SiLU(a) = a * sigmoid(a) =
a / (1 + exp(-a))``. Everything is fp64 on the fp64 GEMM reference.

Parity bound (derived, not printed by the pages): the kernels form g = x W_gate and
u = x W_up in fp32 within ``eps * Y`` of the reference (the GEMM bound, eps = 1e-3,
Y = max|y| over both halves). To first order ``|dh| <= |SiLU'| |u| |dg| + |SiLU(g)| |du|``
with ``max |SiLU'| < 1.1`` and ``|SiLU(g)| <= |g|``, so
``|h - h_ref| <= eps * Y * (1.1 * max|u| + max|g|)``.
"""
from __future__ import annotations

import numpy as np

from .gemm import gemm_ref


def silu(a) -> np.ndarray:
    """``a * sigmoid(a)`` in fp64, written as ``a / (1 + exp(-a))``."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_split(y: np.ndarray):
    """The gate and up halves of a fused projection's output ``y[M, 2N]``."""
    n = y.shape[1] // 2
    if y.shape[1] != 2 * n:
        raise ValueError("the fused projection has an even number of columns")
    return y[:, :n], y[:, n:]


def swiglu_ref(x: np.ndarray, w_hat: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """``SiLU(x W_gate) * (x W_up)`` for ``W_hat[K, 2N]`` = [W_gate | W_up], fp64."""
    g, u = swiglu_split(gemm_ref(x, w_hat, dtype))
    return silu(g) * u


def swiglu_bound(y_ref: np.ndarray, eps: float = 1e-3) -> float:
    """The elementwise parity bound above, from the fused projection's reference output."""
    g, u = swiglu_split(y_ref)
    Y = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    return eps * Y * (1.1 * float(np.max(np.abs(u), initial=0.0)) + float(np.max(np.abs(g), initial=0.0)))
