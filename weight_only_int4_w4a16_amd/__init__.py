"""W4A16 fused dequantize-GEMM for MI355X (gfx950).

``y[M, N] = x[M, K] @ W_hat[K, N]`` with W_hat rebuilt on-chip from packed INT4 codes,
per-group scales and optional zero-points (or an NF4 codebook), 16-bit activations and
fp32 accumulation. The compute runs in hand-written HIP kernels behind the C ABI of
``include/w4a16.h``; :mod:`.binding` only marshals tensors into it. Importing this package
does not load the library; the first call does, and raises if it was not built.
"""
from .binding import (W4A16Error, F16, BF16, F32, lib, packed_bytes, workspace_bytes,
                      awq_workspace_bytes, w4a8_workspace_bytes, pack, gemm, gemm_static, gemm_nf4, gemm_awq,
                      gemm_w4a8, w4a8_kernel_name, quantize_act_int8, gemm_swiglu, gemm_nf4_swiglu, dequant,
                      dequant_nf4, kernel_name, read_probe, version)

__all__ = ["W4A16Error", "F16", "BF16", "F32", "lib", "packed_bytes", "workspace_bytes",
           "awq_workspace_bytes", "w4a8_workspace_bytes", "pack", "gemm", "gemm_static", "gemm_nf4", "gemm_awq",
           "gemm_w4a8", "w4a8_kernel_name", "quantize_act_int8", "gemm_swiglu", "gemm_nf4_swiglu", "dequant", "dequant_nf4", "kernel_name",
           "read_probe", "version"]
