"""CPU oracle for the W4A16 fused dequantize-GEMM.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct NumPy
implementation of what the W4A16 path computes, written from the pages and pinned
against what they print (see ``tests/test_oracle_*.py``). Only the test-suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product library
never does and shares no code with it.

Floating point is carried in fp64 except where the pages fix a precision: scales are
stored as FP16 (BF16 for bf16 activations) and the dequantized weight is rounded to
the 16-bit activation type before the multiply, because the kernel "dequantizes them
on-chip to FP16/BF16, then multiplies with 16-bit activations" ("4.3 Weight-only
INT4", section 1, W4A16 storage and compute). All bit work uses unsigned integers.

Modules
  fp        rounding of fp64 values to fp16/bf16 (nearest-even and upward)
  quant     RTN group quantization: asymmetric uint4, symmetric int4, NF4
  packing   eight 4-bit codes per int32 along K; zero-points eight per int32 along N
  dequant   codes + scales (+ zeros | codebook) -> 16-bit weight matrix
  gemm      dequantize-then-matmul reference (fp64) and a brute-force loop version
  glu       SwiGLU epilogue of a fused gate+up projection, and its parity bound
  gptq      GPTQ: row-by-row quantization with inverse-Hessian error compensation
  awq       AWQ: per-input-channel scale search, S W quantized, activations times S^-1
  w4a8      W4A8: per-token INT8 activations, per-channel INT4 weights, integer product
  storage   bytes and bits per weight of the packed format
  roofline  memory/compute floors and the batch crossover

Parity status: every function above is pinned by a ``-m "not gpu"`` test; the NF4
codebook's agreement with any third-party table is unpinned (the kernel takes the
codebook as an argument, so GEMM parity does not depend on it).
"""
from .fp import (round_nearest_f16, round_up_f16, round_nearest_bf16_bits, round_up_bf16_bits,
                 bf16_bits_to_f64, scale_values)
from .quant import quantize_rtn_asym, quantize_rtn_sym, quantize_nf4, to_offset_binary
from .nf4 import nf4_codebook, inverse_normal_cdf
from .packing import pack_codes, unpack_codes, pack_zeros, unpack_zeros
from .dequant import dequant_affine, dequant_sym, dequant_nf4
from .gemm import gemm_ref, gemm_ref_columns, gemm_bruteforce
from .glu import silu, swiglu_split, swiglu_ref, swiglu_bound
from .gptq import hessian, compensate, gptq_quantize
from . import awq
from . import w4a8
from .storage import storage_bytes, bits_per_weight, bytes_per_weight
from . import roofline

__all__ = [
    "round_nearest_f16", "round_up_f16", "round_nearest_bf16_bits", "round_up_bf16_bits",
    "bf16_bits_to_f64", "scale_values",
    "quantize_rtn_asym", "quantize_rtn_sym", "quantize_nf4", "to_offset_binary",
    "nf4_codebook", "inverse_normal_cdf",
    "pack_codes", "unpack_codes", "pack_zeros", "unpack_zeros",
    "dequant_affine", "dequant_sym", "dequant_nf4",
    "gemm_ref", "gemm_ref_columns", "gemm_bruteforce",
    "silu", "swiglu_split", "swiglu_ref", "swiglu_bound",
    "hessian", "compensate", "gptq_quantize", "awq", "w4a8",
    "storage_bytes", "bits_per_weight", "bytes_per_weight", "roofline",
]
