"""Round-to-nearest group quantization (oracle; test infrastructure only).

These functions make the GEMM's inputs from full-precision weights ``W[K, N]``
(K = input features, the reduction axis; N = output features). Groups run along K:
"INT4 and Low-Bit Inference", section 6-9 (packed layout) counts 4096/128 = 32 scale
rows for a 4096-row weight, so one scale row per group of K.

Readings taken where the pages leave a step open (each is listed in the design notes):
* affine grid: the 16 levels span the group's own range ("INT4 LLMs", section "Why
  mapping to 16 values still works"; affine schemes add an offset), so the step is
  range / (2**bits - 1); this is what makes the 4-bit tick gap 17 times the 8-bit one
  ("4.3 Weight-only INT4", introduction);
* the range always includes 0, so the zero-point lands on a code in 0..15 and w = 0
  dequantizes to exactly 0;
* scales are rounded *up* to the storage type, so every weight stays within half a
  step of its dequantized value;
* symmetric codes are the signed values -8..7 ("INT4 LLMs", section "What INT4 means
  in an LLM") with step max|w| / 7, stored offset-binary (code + 8);
* round-half-to-even wherever a real number is rounded to an integer.
"""
from __future__ import annotations

import numpy as np

from .fp import round_up_f16, round_up_bf16_bits, bf16_bits_to_f64


def _round_up_scale(s: np.ndarray, scale_dtype):
    """Return (fp64 values, stored array) of scales rounded up to the storage type."""
    if scale_dtype is None:
        return s, s
    if scale_dtype == "f16":
        h = round_up_f16(s)
        return h.astype(np.float64), h
    if scale_dtype == "bf16":
        b = round_up_bf16_bits(s)
        return bf16_bits_to_f64(b), b
    raise ValueError(scale_dtype)


def _groups(W: np.ndarray, group_size: int) -> np.ndarray:
    K, N = W.shape
    if group_size <= 0 or K % group_size:
        raise ValueError("K must be a multiple of group_size")
    return np.asarray(W, dtype=np.float64).reshape(K // group_size, group_size, N)


def quantize_rtn_asym(W: np.ndarray, group_size: int, scale_dtype="f16", bits: int = 4):
    """Asymmetric (affine) RTN per (group of K, column).

    Returns ``(q[K,N] uint8 in 0..2**bits-1, scales[K/g,N] stored, zeros[K/g,N] uint8)``
    where stored scales are ``np.float16`` ("f16"), bf16 uint16 bits ("bf16") or fp64
    (``None``, used only to check the grid arithmetic without storage rounding).

    Per group G of column n: mn = min(min G, 0), mx = max(max G, 0),
    s = RU((mx - mn) / (2**bits - 1)), z = rint(-mn / s), q = clip(rint(w / s) + z).
    An all-zero group gets s = 1, z = 0.
    """
    Wg = _groups(W, group_size)
    qmax = (1 << bits) - 1
    mn = np.minimum(Wg.min(axis=1), 0.0)
    mx = np.maximum(Wg.max(axis=1), 0.0)
    rng = mx - mn
    s_val, s_store = _round_up_scale(np.where(rng == 0, 1.0, rng / qmax), scale_dtype)
    z = np.rint(-mn / s_val)
    q = np.clip(np.rint(Wg / s_val[:, None, :]) + z[:, None, :], 0, qmax)
    K, N = W.shape
    return q.reshape(K, N).astype(np.uint8), s_store, z.astype(np.uint8)


def quantize_rtn_sym(W: np.ndarray, group_size: int, scale_dtype="f16"):
    """Symmetric RTN: signed codes in -8..7 with s = RU(max|G| / 7).

    Returns ``(q[K,N] int8 signed, scales[K/g,N] stored)``. An all-zero group gets s = 1.
    Use :func:`to_offset_binary` for the stored 4-bit form.
    """
    Wg = _groups(W, group_size)
    amax = np.abs(Wg).max(axis=1)
    s_val, s_store = _round_up_scale(np.where(amax == 0, 1.0, amax / 7.0), scale_dtype)
    q = np.clip(np.rint(Wg / s_val[:, None, :]), -8, 7)
    K, N = W.shape
    return q.reshape(K, N).astype(np.int8), s_store


def to_offset_binary(q_signed: np.ndarray) -> np.ndarray:
    """Signed code -8..7 -> stored nibble 0..15 (code + 8); dequantized with zero 8."""
    q = np.asarray(q_signed, dtype=np.int16)
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("signed 4-bit codes must lie in -8..7")
    return (q + 8).astype(np.uint8)


def quantize_nf4(W: np.ndarray, codebook: np.ndarray, block_size: int = 64):
    """NF4: per block of K (one column), absmax scale a = RU_fp16(max|block|) and
    code = the codebook level nearest to w / a (ties to the lower index).

    "INT4 and Low-Bit Inference", section 5 (The formats): the 16 levels sit at normal
    quantiles instead of uniformly. Returns ``(codes[K,N] uint8, absmax[K/b,N] fp16)``.
    """
    Wg = _groups(W, block_size)
    amax = np.abs(Wg).max(axis=1)
    a_store = round_up_f16(np.where(amax == 0, 1.0, amax))
    a = a_store.astype(np.float64)
    c = np.asarray(codebook, dtype=np.float16).astype(np.float64)
    r = Wg / a[:, None, :]
    codes = np.zeros(r.shape, dtype=np.uint8)
    best = np.abs(r - c[0])
    for i in range(1, c.size):                   # strict '<' keeps the lower index on ties
        d = np.abs(r - c[i])
        better = d < best
        codes[better] = i
        best = np.where(better, d, best)
    K, N = W.shape
    return codes.reshape(K, N).astype(np.uint8), a_store
