"""W4A8: INT4 weights, per-token INT8 activations, an integer matrix product (oracle; test
infrastructure only).

"INT4 LLMs: What 4-Bit Quantization Means…", section on weight-only quantization: one
implementation keeps the weights in [-8, 7], unpacks them to INT8, runs an INT8 x INT8 matrix
multiply and dequantizes the result with the input and per-channel scales; section "Weights
and activations (W4A4 and W4A8)": W4A8 pairs 4-bit weights with 8-bit activations. "INT8 vs
INT4 Quantization, in depth", section "Two regimes": past the crossover batch only the math
rate matters, and the INT8 path doubles it. So, per output element,

    y[m, n] = sx[m] * sw[n] * sum_k xq[m, k] * q[k, n]

Readings taken where the pages leave a step open (listed in the design notes):
* activations are quantized symmetrically per token (row): sx = RN_f32(max_k |x[m, k]| / 127)
  and xq = clip(rint(RN_f32(x / sx)), -127, 127), the scale and the quotient in fp32 (each one
  correctly rounded), rint half-to-even, so the integer code is a reproducible decision; a
  row of zeros has sx = 0 and xq = 0;
* weights are the symmetric INT4 format with one scale per output channel: the format of
  :func:`oracle.quant.quantize_rtn_sym` with a single group spanning K (codes -8..7 stored
  offset-binary, the scale stored in the activation type);
* the sum of products is an exact integer (each term at most 127 * 8 in magnitude); the
  result is that integer times the two scales, in fp64.
"""
from __future__ import annotations

import numpy as np

from .fp import bf16_bits_to_f64
from .packing import unpack_codes


def _values(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(dtype)


def quantize_act_int8(x: np.ndarray, dtype: str = "f16"):
    """Per-token symmetric INT8: returns ``(xq[M, K] int8, sx[M] float32)``.

    ``x[M, K]`` is stored in ``dtype`` (np.float16, or bf16 uint16 bits)."""
    xv = _values(x, dtype).astype(np.float32)              # exact: 16-bit values fit fp32
    if xv.ndim != 2:
        raise ValueError("x must be (M, K)")
    amax = np.max(np.abs(xv), axis=1) if xv.shape[1] else np.zeros(xv.shape[0], np.float32)
    sx = (amax / np.float32(127.0)).astype(np.float32)     # one fp32 rounding
    safe = np.where(sx > 0, sx, np.float32(1.0)).astype(np.float32)   # zero rows stay 0
    quo = (xv / safe[:, None]).astype(np.float32)          # one fp32 rounding per element
    xq = np.clip(np.rint(quo), -127, 127)
    return xq.astype(np.int8), sx


def signed_codes(qweight: np.ndarray) -> np.ndarray:
    """Canonical packed offset-binary codes ``qweight[K/8, N]`` -> signed int8 ``q[K, N]``
    (stored nibble u, value u - 8)."""
    return (unpack_codes(qweight).astype(np.int16) - 8).astype(np.int8)


def int_gemm(xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """The exact integer product ``xq[M, K] @ q[K, N]`` (int64). Every term is an integer of
    magnitude at most 127 * 8, so every partial sum, in any order, is an integer below 2**53
    (for K < 2**43) and the fp64 matrix product is exact."""
    K = np.shape(xq)[1]
    if K * 127 * 8 >= 2 ** 53:
        raise ValueError("K too large for an exact fp64 product")
    p = np.asarray(xq, dtype=np.float64) @ np.asarray(q, dtype=np.float64)
    return p.astype(np.int64)


def gemm_w4a8_ref(x: np.ndarray, qweight: np.ndarray, wscale: np.ndarray,
                  dtype: str = "f16") -> np.ndarray:
    """``y[M, N]`` (fp64) of the W4A8 path: per-token INT8 x, INT4 codes from the canonical
    ``qweight[K/8, N]`` (offset-binary), one scale per output channel ``wscale[N]`` (or
    ``[1, N]``) stored in ``dtype``."""
    xq, sx = quantize_act_int8(x, dtype)
    acc = int_gemm(xq, signed_codes(qweight)).astype(np.float64)   # exact: below 2**53
    sw = _values(np.asarray(wscale).reshape(-1), dtype)
    return acc * sx.astype(np.float64)[:, None] * sw[None, :]
