"""Dequantization: codes + group metadata -> 16-bit weight matrix (oracle; test only).

"4.3 Weight-only INT4", section 1 (W4A16 storage and compute): the kernel reads the
codes and dequantizes them to FP16/BF16 before the multiply; section 3.2 (equation for
Y-hat) names D as dequantization "with Scale and zero-point". The plain reading taken
here is one rounding of the exact affine value:

    W_hat[k, n] = RN_t((q[k, n] - z[k // g, n]) * s[k // g, n])

with t the activation type (fp16, or bf16 for bf16 activations), RN nearest-even. The
product of a 5-bit integer and an fp16/bf16 significand is exact in fp64, so the only
rounding is the final one. Symmetric weights are the same with z = 8 (offset binary).

NF4: W_hat = RN_t(c[code] * a) with ``c`` the 16-entry codebook and ``a`` the fp16
absmax of the code's block; the product of two fp16 values is exact in fp64.

fp16 results are ``np.float16``; bf16 results are uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

from .fp import round_nearest_f16, round_nearest_bf16_bits, scale_values
from .packing import unpack_codes, unpack_zeros


def _round_to(v: np.ndarray, wdtype: str) -> np.ndarray:
    if wdtype == "f16":
        return round_nearest_f16(v)
    if wdtype == "bf16":
        return round_nearest_bf16_bits(v)
    raise ValueError(wdtype)


def dequant_affine(qweight: np.ndarray, scales: np.ndarray, qzeros, group_size: int,
                   wdtype: str = "f16") -> np.ndarray:
    """Asymmetric dequantization; ``qzeros=None`` means the symmetric zero 8.

    ``scales`` are stored in ``wdtype`` (np.float16, or bf16 uint16 bits).
    """
    q = unpack_codes(qweight).astype(np.float64)            # (K, N)
    K, N = q.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    s = scale_values(scales, wdtype)                        # (K/g, N)
    if s.shape != (K // group_size, N):
        raise ValueError("scales must be (K/group_size, N)")
    if qzeros is None:
        z = np.full_like(s, 8.0)
    else:
        z = unpack_zeros(qzeros).astype(np.float64)
        if z.shape != s.shape:
            raise ValueError("qzeros must be (K/group_size, N/8)")
    rows = np.arange(K) // group_size
    return _round_to((q - z[rows]) * s[rows], wdtype)


def dequant_sym(qweight: np.ndarray, scales: np.ndarray, group_size: int,
                wdtype: str = "f16") -> np.ndarray:
    """Symmetric dequantization: stored nibble u = code + 8, so W_hat = RN((u - 8) * s)."""
    return dequant_affine(qweight, scales, None, group_size, wdtype)


def dequant_nf4(qweight: np.ndarray, absmax: np.ndarray, codebook: np.ndarray,
                block_size: int = 64, wdtype: str = "f16") -> np.ndarray:
    """NF4 dequantization with an fp16 codebook and fp16 absmax per block of K."""
    codes = unpack_codes(qweight)                            # (K, N)
    K, N = codes.shape
    a = np.asarray(absmax, dtype=np.float16).astype(np.float64)
    if a.shape != (K // block_size, N) or K % block_size:
        raise ValueError("absmax must be (K/block_size, N)")
    c = np.asarray(codebook, dtype=np.float16).astype(np.float64)
    if c.shape != (16,):
        raise ValueError("codebook must hold 16 values")
    rows = np.arange(K) // block_size
    return _round_to(c[codes] * a[rows], wdtype)
