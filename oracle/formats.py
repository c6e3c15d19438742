"""Bit-level decoders and exact float64 dequantization of the weight formats.

Test infrastructure: only the tests, the smoke check and the bench's CPU
baseline use this module.

Formats (all planar: codes in one array, scales in another, row-major):

* bf16: the upper 16 bits of an IEEE binary32 number. Inferno's bf16 path
  ("Writing an LLM inference engine from scratch in Rust", Lesson 1) and the
  infer engine's bf16 weights ("infer", design notes) store weights this way.
* int8-g32: one signed 8-bit code per weight and one binary16 scale per 32
  consecutive weights of a row; weight = code * scale. This is the 32-value
  int8 block with one scale that inferno quantizes activations into
  (Lesson 6) and llama.cpp's Q8_0 block the infer page compares against
  (perplexity table notes), applied here to weights.
* Q4_0-g32: per 32 consecutive weights of a row, 16 bytes of 4-bit codes and
  one binary16 scale, 4.5 bits per weight (Rust page, Lesson 1). A code q in
  [0, 15] stands for the weight (q - 8) * scale: the stored value is the
  weight plus 8 (Lesson 6, the bias-removal identity). Element j of the
  block sits in the low nibble of byte j and element j + 16 in the high
  nibble of the same byte (the Lesson 6 kernel pairs the low nibbles with
  activations 0..15 and the high nibbles with 16..31).
* int4-g128: the same value rule with one scale per 128 weights, 64 code
  bytes per block ("infer", g128 rows of the decode and perplexity tables).
  The pages do not give its nibble order; this oracle takes the same
  half-split as Q4_0: element j in the low nibble of byte j, element j + 64
  in the high nibble.
* int4-g64: the same value rule with one scale per 64 weights, 32 code bytes
  per block ("infer", the g64 row of the perplexity table), the same
  half-split: element j in the low nibble of byte j, element j + 32 in the
  high nibble.
* int8-row: one signed 8-bit code per weight and one binary16 scale per row;
  weight = code * scale ("infer": its int8 weights carry one scale per row,
  perplexity table and its notes). The pages do not give the scale's type;
  binary16, like every other scale here.
"""
from __future__ import annotations

import numpy as np

BF16, INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64 = 0, 1, 2, 3, 4, 5
# weights per scale; 0: one scale per row (int8-row)
GROUP = {BF16: 1, INT8_G32: 32, Q4_0_G32: 32, INT4_G128: 128, INT8_ROW: 0, INT4_G64: 64}
# K must be a multiple of this
K_ALIGN = {BF16: 32, INT8_G32: 32, Q4_0_G32: 32, INT4_G128: 128, INT8_ROW: 32, INT4_G64: 64}
NIBBLE_FORMATS = (Q4_0_G32, INT4_G128, INT4_G64)


def scales_per_row(fmt: int, K: int) -> int:
    """Number of scales of one row (0 for bf16)."""
    if fmt == BF16:
        return 0
    return 1 if GROUP[fmt] == 0 else K // GROUP[fmt]


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact): a bf16 is the high half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact, subnormals included).

    sign: bit 15; biased exponent e: bits 14..10 (bias 15); fraction f: bits 9..0.
    e == 0: (f / 2^10) * 2^-14; 0 < e < 31: (1 + f / 2^10) * 2^(e - 15); e == 31: inf / NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    neg = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    mag = np.where(e == 0, f * 2.0 ** -24, np.ldexp(1024.0 + f, (e - 25).astype(np.int32)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(neg == 1, -mag, mag)


def f64_to_f16_bits(v) -> np.ndarray:
    """float64 -> binary16 bits, round to nearest, ties to even; overflow -> inf.

    Written from the binary16 definition: write |v| = s * 2^E with s in [1, 2);
    the kept significand is s * 2^10 (normal range) or |v| * 2^24 (subnormal
    range, E < -14); scale by that power of two (exact), round the result to
    the nearest integer with ties to even, and rebuild the bit pattern. A
    carry out of the significand bumps the exponent, a carry past the largest
    finite value (65504) gives infinity, and a subnormal that rounds up to
    2^10 becomes the smallest normal. NaN maps to the quiet NaN 0x7E00.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x8000, 0).astype(np.int64)
    finite_nz = np.isfinite(a) & (a > 0)
    safe = np.where(finite_nz, a, 1.0)
    _, e = np.frexp(safe)                  # safe = m * 2^e, m in [0.5, 1)
    E = e.astype(np.int64) - 1             # safe = s * 2^E, s in [1, 2)
    sub = E < -14
    shift = np.where(sub, 24, 10 - E)
    n = _rne(np.ldexp(safe, shift.astype(np.int32)))
    # normal range: n in [1024, 2048]; a carry to 2048 moves to the next binade
    carry = (~sub) & (n == 2048)
    n = np.where(carry, 1024, n)
    E = np.where(carry, E + 1, E)
    normal_bits = ((E + 15) << 10) | (n - 1024)
    bits = np.where(sub, n, normal_bits)   # subnormal n == 1024 is the smallest normal
    bits = np.where((~sub) & (E > 15), 0x7C00, bits)
    bits = np.where(a == 0, 0, bits)
    bits = np.where(np.isinf(a), 0x7C00, bits)
    bits = bits | sign
    bits = np.where(np.isnan(v), 0x7E00, bits)
    return bits.astype(np.uint16)


def _rne(t: np.ndarray) -> np.ndarray:
    """Round non-negative float64 values to the nearest integer, ties to even."""
    fl = np.floor(t)
    r = t - fl                             # exact
    n = fl.astype(np.int64)
    up = (r > 0.5) | ((r == 0.5) & ((n & 1) == 1))
    return n + up.astype(np.int64)


def decode_nibble_blocks(codes: np.ndarray, group: int) -> np.ndarray:
    """uint8[M][K/G][G/2] -> int64 codes [M][K] in element order.

    Element j < G/2 of a block is the low nibble of byte j; element j + G/2 is
    the high nibble of byte j.
    """
    c = np.asarray(codes, dtype=np.uint8)
    M, nb, half = c.shape
    assert half * 2 == group
    lo = (c & 0x0F).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    return np.concatenate([lo, hi], axis=2).reshape(M, nb * group)


def dequantize(fmt: int, w: np.ndarray, s, K: int) -> np.ndarray:
    """Exact float64 weights W_hat[M][K] for one weight format.

    bf16: W_hat = value of the bf16 bits.
    int8-g32: W_hat[m, k] = q[m, k] * d[m, k // 32].
    int8-row: W_hat[m, k] = q[m, k] * d[m].
    Q4_0-g32 / int4-g128 / int4-g64: W_hat[m, k] = (q[m, k] - 8) * d[m, k // G].
    Every product is exact in float64 (at most 8 + 11 significant bits).
    """
    if fmt == BF16:
        return bf16_to_f64(w).reshape(-1, K)
    d = f16_to_f64(s)
    M = d.shape[0]
    if fmt == INT8_ROW:
        q = np.asarray(w, dtype=np.int8).astype(np.int64).reshape(M, K)
        return q.astype(np.float64) * d.reshape(M, 1)
    G = GROUP[fmt]
    if fmt == INT8_G32:
        q = np.asarray(w, dtype=np.int8).astype(np.int64).reshape(M, K)
    else:
        q = decode_nibble_blocks(np.asarray(w).reshape(M, K // G, G // 2), G) - 8
    d_per_elem = np.repeat(d.reshape(M, K // G), G, axis=1)
    return q.astype(np.float64) * d_per_elem
