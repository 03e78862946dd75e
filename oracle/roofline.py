"""Roofline arithmetic for weight-only INT4 (oracle; test infrastructure only).

"INT8 vs INT4 Quantization, in depth", sections "Two regimes" and "Worked example":
a decode step reads every weight once and does two flops per weight per sequence, so
its time is about max(weight bytes / bandwidth, 2 * params * batch / peak); the batch
where the two terms meet is where the step turns compute-bound.
"4.3 Weight-only INT4", section 4 (figure): the naive path writes the expanded FP16
weight back and reads it again.
"""
from __future__ import annotations


def algo_bytes(M: int, K: int, N: int, group_size: int, zeros: bool = True,
               act_bytes: int = 2, out_bytes: int = 2, scale_bytes: int = 2) -> int:
    """Bytes one W4A16 GEMM must move: codes, scales, zeros, activations and output."""
    G = K // group_size
    return (K * N // 2 + G * N * scale_bytes + (G * N // 2 if zeros else 0)
            + act_bytes * M * K + out_bytes * M * N)


def algo_bytes_nf4(M: int, K: int, N: int, block_size: int = 64, act_bytes: int = 2,
                   out_bytes: int = 2) -> int:
    """NF4: codes, one fp16 absmax per block, activations and output (codebook ~0)."""
    return K * N // 2 + (K // block_size) * N * 2 + act_bytes * M * K + out_bytes * M * N


def flops(M: int, K: int, N: int) -> int:
    return 2 * M * N * K


def t_memory(nbytes: float, bandwidth: float) -> float:
    return nbytes / bandwidth


def t_compute(nflops: float, peak: float) -> float:
    return nflops / peak


def t_roof(nbytes: float, nflops: float, bandwidth: float, peak: float) -> float:
    return max(t_memory(nbytes, bandwidth), t_compute(nflops, peak))


def decode_floor(params: float, bytes_per_param: float, bandwidth: float) -> float:
    """Seconds per decode step when weight reads dominate."""
    return params * bytes_per_param / bandwidth


def step_compute(params: float, batch: float, peak: float) -> float:
    """Seconds of arithmetic per decode step: 2 flops per weight per sequence."""
    return 2.0 * params * batch / peak


def crossover_batch(bytes_per_param: float, bandwidth: float, peak: float) -> float:
    """Batch where 2*P*B/peak equals P*bytes_per_param/bandwidth."""
    return bytes_per_param * peak / (2.0 * bandwidth)


def naive_bytes_per_weight(code_bytes: float = 0.5, expanded_bytes: float = 2.0) -> float:
    """Naive path: read codes, write the FP16 weight, read it again in the GEMM."""
    return code_bytes + expanded_bytes + expanded_bytes
