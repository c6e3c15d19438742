"""Weight quantizers from bf16 (test infrastructure).

Only the tests, the smoke check and the bench's CPU baseline use this module.

4-bit formats (Q4_0-g32, int4-g128): per group, take the element of largest
magnitude with its sign, m, and set the scale d = m / -8 so that m maps
exactly to code 0, i.e. to the value -8 * d ("Writing an LLM inference engine
from scratch in Rust", "Is the 4-bit model still good?": the llama.cpp-style
scale that replaced largest-absolute-value / 8; "infer", design notes on
weight-only quantization, where the largest-magnitude value also maps to -8).
Readings where the pages are silent:
  * a tie in |w| between elements goes to the first in index order;
  * d is rounded to binary16 (nearest, ties to even) before the codes are
    computed, and the codes use that rounded d;
  * code = round_half_even(w / d) + 8, clamped to [0, 15], the division
    taken in float64;
  * a group whose rounded d is 0 (all zero, or too small for binary16)
    gets d = +0 (bit pattern 0x0000) and every code 8.
int8-g32 and int8-row: symmetric, d = binary16(amax / 127) with amax the
largest |w| of the group (of the row for int8-row: "infer" quantizes int8
per row); code = round_half_even(w / d) clamped to [-127, 127]; a group
whose rounded d is 0 gets d = +0 and code 0. int4-g64 follows the 4-bit rule
with groups of 64.
Both: a non-finite weight or a scale that overflows binary16 (|d| > 65504
after rounding) is an error (ValueError), as in the C-ABI packer.

Codes are packed per formats.py: 4-bit element j of a group in the low
nibble of byte j, element j + G/2 in the high nibble.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .formats import (GROUP, INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64, bf16_to_f64, f16_to_f64,
                      f64_to_f16_bits)


def _rne(t: np.ndarray) -> np.ndarray:
    return np.rint(t)  # IEEE round to nearest, ties to even


def quantize_from_bf16(fmt: int, w_bits: np.ndarray, M: int, K: int
                       ) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 weights [M][K] -> (codes, f16 scale bits [M][K/G], or [M] for int8-row) in the
    planar layout."""
    if fmt not in (INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64):
        raise ValueError("quantize_from_bf16: not a quantized format")
    G = K if GROUP[fmt] == 0 else GROUP[fmt]
    w = bf16_to_f64(np.asarray(w_bits).reshape(M, K))
    if not np.isfinite(w).all():
        raise ValueError("non-finite weight")
    wg = w.reshape(M, K // G, G)
    aw = np.abs(wg)
    int8 = fmt in (INT8_G32, INT8_ROW)
    if int8:
        d_exact = aw.max(axis=2) / 127.0
    else:
        first_max = np.argmax(aw, axis=2)                       # first index of max |w|
        m = np.take_along_axis(wg, first_max[..., None], axis=2)[..., 0]
        d_exact = m / -8.0
    d_bits = f64_to_f16_bits(d_exact)
    d_bits = np.where((d_bits & 0x7FFF) == 0, 0, d_bits).astype(np.uint16)  # zero scale is +0
    d = f16_to_f64(d_bits)
    if not np.isfinite(d).all():
        raise ValueError("scale overflows binary16")
    zero = (d == 0)[..., None]
    safe_d = np.where(zero, 1.0, d[..., None])
    if int8:
        q = np.clip(_rne(wg / safe_d), -127, 127)
        q = np.where(zero, 0, q).astype(np.int8).reshape(M, K)
        return q, (d_bits.reshape(M) if fmt == INT8_ROW else d_bits)
    q = np.clip(_rne(wg / safe_d) + 8, 0, 15)
    q = np.where(zero, 8, q).astype(np.uint8)                  # [M][K/G][G]
    half = G // 2
    packed = (q[..., :half] | (q[..., half:] << 4)).astype(np.uint8)
    return packed, d_bits
