"""Packing of 4-bit codes into 32-bit words (oracle; test infrastructure only).

"4.3 Weight-only INT4", section 1 (W4A16 storage and compute): one 32-bit word holds
eight 4-bit codes. "INT4 and Low-Bit Inference", section 6-9 (packed layout) fixes the
orientation through its shapes for a (4096, 11008) weight: ``qweight`` is
(4096/8, 11008), so codes are packed along K; ``qzeros`` is (32, 11008/8), so
zero-points are packed along N.

Reading for the nibble order (the pages are silent): least-significant nibble first,
code j of a word in bits 4j..4j+3. On a little-endian machine byte b of the word then
holds codes 2b (low nibble) and 2b+1 (high nibble): two codes per byte, as "INT4 LLMs"
(TL;DR) states.
"""
from __future__ import annotations

import numpy as np


def _pack8(codes: np.ndarray, axis: int) -> np.ndarray:
    c = np.asarray(codes)
    if c.size and (c.min() < 0 or c.max() > 15):
        raise ValueError("codes must lie in 0..15")
    c = np.moveaxis(c.astype(np.uint32), axis, 0)
    if c.shape[0] % 8:
        raise ValueError("packed axis must be a multiple of 8")
    c = c.reshape(c.shape[0] // 8, 8, *c.shape[1:])
    word = np.zeros((c.shape[0], *c.shape[2:]), dtype=np.uint32)
    for j in range(8):
        word |= c[:, j] << np.uint32(4 * j)
    return np.ascontiguousarray(np.moveaxis(word, 0, axis)).view(np.int32)


def _unpack8(words: np.ndarray, axis: int) -> np.ndarray:
    w = np.moveaxis(np.asarray(words).view(np.uint32), axis, 0)
    out = np.empty((w.shape[0], 8, *w.shape[1:]), dtype=np.uint8)
    for j in range(8):
        out[:, j] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    out = out.reshape(w.shape[0] * 8, *w.shape[1:])
    return np.ascontiguousarray(np.moveaxis(out, 0, axis))


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Codes ``q[K, N]`` (0..15) -> ``qweight[K/8, N]`` int32."""
    return _pack8(q, 0)


def unpack_codes(qweight: np.ndarray) -> np.ndarray:
    """``qweight[K/8, N]`` int32 -> codes ``q[K, N]`` uint8."""
    return _unpack8(qweight, 0)


def pack_zeros(z: np.ndarray) -> np.ndarray:
    """Zero-points ``z[G, N]`` (0..15) -> ``qzeros[G, N/8]`` int32."""
    return _pack8(z, 1)


def unpack_zeros(qzeros: np.ndarray) -> np.ndarray:
    """``qzeros[G, N/8]`` int32 -> zero-points ``z[G, N]`` uint8."""
    return _unpack8(qzeros, 1)
