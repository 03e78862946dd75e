"""Storage arithmetic of the packed INT4 format (oracle; test infrastructure only).

Per weight: 4 bits of code, one 16-bit scale per group of g, and (asymmetric only) one
4-bit zero-point per group. "INT4 and Low-Bit Inference", section 5 (The formats):
4 + 16/128 + 4/128 bits for g128 with a zero, 4 + 16/32 + 4/32 for g32.
"4.3 Weight-only INT4", section 1 (equation): 4/8 + 2/128 bytes for g128 scale-only.
Section 6-9 (packed layout) of the first page totals the three tensors in bytes.
"""
from __future__ import annotations


def storage_bytes(K: int, N: int, group_size: int, zeros: bool = True,
                  scale_bytes: int = 2) -> dict:
    """Bytes of ``qweight`` (K/8 x N int32), ``scales`` (K/g x N) and ``qzeros``
    (K/g x N/8 int32, or none for the symmetric format)."""
    if K % 8 or K % group_size or (zeros and N % 8):
        raise ValueError("shape does not pack")
    qweight = (K // 8) * N * 4
    scales = (K // group_size) * N * scale_bytes
    qzeros = (K // group_size) * (N // 8) * 4 if zeros else 0
    return {"qweight": qweight, "scales": scales, "qzeros": qzeros,
            "total": qweight + scales + qzeros, "fp16": K * N * 2}


def bits_per_weight(group_size: int, zeros: bool = True, scale_bits: int = 16,
                    code_bits: int = 4) -> float:
    return code_bits + scale_bits / group_size + (code_bits / group_size if zeros else 0.0)


def bytes_per_weight(group_size: int, zeros: bool = True, scale_bits: int = 16) -> float:
    return bits_per_weight(group_size, zeros, scale_bits) / 8.0
