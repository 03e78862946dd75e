"""Seeded synthetic inputs for the W4A16 GEMM, shared by tests, benchmark and smoke check.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no quantization, packing, dequantization or matrix product), so both the
CPU oracle's callers and the GPU path's callers may use it.

Recipe (the workloads named on the pages are Llama-3-shaped linears with Gaussian
weights; no dataset or trained checkpoint is involved):

* full-precision weights ``W[K, N]`` ~ N(0, 0.02) in fp32, drawn in blocks of 256
  columns so that any column slice of a large matrix can be regenerated alone;
* activations ``x[M, K]`` ~ N(0, 1) drawn in fp32 and stored as fp16 (numpy cast) or
  bf16 (round-to-nearest-even on the fp32 bit pattern, returned as uint16 bits);
* timing-only quantized weights: uniformly random 32-bit words for ``qweight`` and
  ``qzeros`` (every 4-bit code value equally likely) and fp16/bf16 scales drawn
  uniformly from a band that RTN of N(0, 0.02) weights produces.

Seeds are ``1000*config + 10*shape + role + 100000*layer``.
"""
from __future__ import annotations

import numpy as np

ROLE_W = 0
ROLE_X = 1
ROLE_CODES = 2
ROLE_SCALES = 3
ROLE_ZEROS = 4
ROLE_XSCALE = 5

COL_BLOCK = 256


def seed_for(config: int, shape: int = 0, role: int = 0, layer: int = 0) -> int:
    return 1000 * config + 10 * shape + role + 100000 * layer


def generator(seed: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(block)]))


def gaussian_weight(K: int, N: int, seed: int, sigma: float = 0.02,
                    col0: int = 0, ncols: int | None = None) -> np.ndarray:
    """Columns ``[col0, col0+ncols)`` of a ``K x N`` fp32 matrix ~ N(0, sigma)."""
    if ncols is None:
        ncols = N - col0
    if col0 < 0 or ncols < 0 or col0 + ncols > N:
        raise ValueError("column slice out of range")
    out = np.empty((K, ncols), dtype=np.float32)
    b0 = col0 // COL_BLOCK
    b1 = (col0 + ncols + COL_BLOCK - 1) // COL_BLOCK
    for b in range(b0, b1):
        blk = generator(seed, b).standard_normal((K, COL_BLOCK), dtype=np.float32)
        blk *= np.float32(sigma)
        lo = max(col0, b * COL_BLOCK)
        hi = min(col0 + ncols, (b + 1) * COL_BLOCK)
        out[:, lo - col0:hi - col0] = blk[:, lo - b * COL_BLOCK:hi - b * COL_BLOCK]
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store fp32 values as bf16 (round to nearest, ties to even), as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activations(M: int, K: int, seed: int, dtype: str = "f16") -> np.ndarray:
    """``x[M, K]`` ~ N(0, 1): np.float16 for ``"f16"``, uint16 bf16 bits for ``"bf16"``."""
    x = generator(seed).standard_normal((M, K), dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def random_words(rows: int, cols: int, seed: int) -> np.ndarray:
    """Uniformly random int32 words (each 4-bit field uniform on 0..15)."""
    return generator(seed).integers(0, 2**32, size=(rows, cols), dtype=np.uint32).view(np.int32)


def random_scales(rows: int, cols: int, seed: int, dtype: str = "f16",
                  lo: float = 0.004, hi: float = 0.009) -> np.ndarray:
    """Positive scales ~ U(lo, hi): np.float16, or uint16 bf16 bits."""
    s = generator(seed).uniform(lo, hi, size=(rows, cols)).astype(np.float32)
    if dtype == "f16":
        return s.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(s)
    raise ValueError(dtype)


def channel_scales(K: int, seed: int, dtype: str = "f16", spread: float = 4.0) -> np.ndarray:
    """Per-input-channel factors for scaled activations: ``2**u`` with u ~ U(-log2 spread,
    log2 spread), stored as np.float16 or uint16 bf16 bits (a positive ``(K,)`` vector)."""
    u = generator(seed).uniform(-np.log2(spread), np.log2(spread), size=K)
    s = np.exp2(u).astype(np.float32)
    if dtype == "f16":
        return s.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(s)
    raise ValueError(dtype)


def timing_weights(K: int, N: int, group_size: int, seed: int, symmetric: bool = False,
                   scale_dtype: str = "f16"):
    """Random canonical ``(qweight[K/8,N], scales[K/g,N], qzeros[K/g,N/8] or None)``.

    Kernel time does not depend on code values, so timing runs use these directly.
    """
    G = K // group_size
    qweight = random_words(K // 8, N, seed + ROLE_CODES)
    scales = random_scales(G, N, seed + ROLE_SCALES, scale_dtype)
    qzeros = None if symmetric else random_words(G, N // 8, seed + ROLE_ZEROS)
    return qweight, scales, qzeros
