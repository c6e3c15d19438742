"""CPU oracle for the fused-dequantization decode GEMV (test infrastructure).

This package is the plain, slow, obviously correct definition of what the
GPU path computes. It exists only to check that path: the tests, the smoke
check and the CPU-baseline leg of the bench may import it; the product (the
C-ABI library and its Python binding) never does, and this package imports
nothing from the product.

Everything is NumPy, in float64. Weights are dequantized exactly per the
format definitions (every dequantized weight q*d is exact in float64) and
the dot products are taken in float64, so the oracle's own rounding is many
orders of magnitude below the tolerance it checks against.

Modules
  formats   bit-level decoders (bf16, binary16, int8, 4-bit nibble blocks)
            and dequantization of each weight format
  gemv      y = W x in float64, plus the per-output magnitude sum |W||x|
            the tolerance is scaled by, and the parity check itself
  quantize  the bf16 -> int8-g32 / 4-bit quantizers (largest-magnitude
            value maps to code -8)
  argmax    the first index of the maximum, with NaN handling
  attention grouped-query decode attention over a bf16 KV cache
  fused     the operations fused on either side of a GEMV: RMSNorm of the
            float32 residual stream into the bf16 GEMV input, the residual
            add, SwiGLU of paired gate/up rows, and their tolerances

Parity status: every function here is pinned by tests that do not re-use it
(library conversions, hand-built blocks with closed-form dot products,
exact rational brute force, quantizer error bounds, torch's rms_norm and
silu, closed-form normalizations and activations, torch's
scaled_dot_product_attention and closed-form attention cases); there is no
unpinned
function.
"""
from .formats import (BF16, INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64, GROUP, K_ALIGN,
                      scales_per_row, bf16_to_f64, f16_to_f64,
                      f64_to_f16_bits, dequantize)
from .gemv import gemv_ref, check_parity, parity_report
from .quantize import quantize_from_bf16
from .argmax import argmax_ref

__all__ = ["BF16", "INT8_G32", "Q4_0_G32", "INT4_G128", "INT8_ROW", "INT4_G64", "GROUP", "K_ALIGN",
           "scales_per_row", "bf16_to_f64", "f16_to_f64",
           "f64_to_f16_bits", "dequantize", "gemv_ref", "check_parity", "parity_report",
           "quantize_from_bf16", "argmax_ref"]
