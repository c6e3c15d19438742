"""float64 reference for the GEMV's fused prologue and epilogues.

Test infrastructure: only the tests, the smoke check and the bench's CPU
baseline use this module.

The infer page's decode step (its pipeline figure and design notes) keeps the
residual stream in float32 and fuses the operations on either side of each
GEMV into it:

* RMSNorm of the residual stream, applied while the GEMV stages its input:
  x = h / sqrt(mean(h^2) + eps) * g (the "normalize the vector" step of the
  Rust page's layer walk-through; g is the per-channel norm weight).
* A residual add in the GEMV's epilogue: y = residual + W x (the o and down
  projections write the residual stream in place).
* SwiGLU from paired gate/up rows: act = silu(gate) * up with
  silu(t) = t / (1 + exp(-t)), the feed-forward activation of the Rust
  page's layer walk-through.

Readings taken where the pages are silent:
* The GEMV consumes bf16 activations, so the normalized vector is rounded to
  bf16 (round to nearest, ties to even) before the product; the rounding is
  applied once, to the exact value.
* "Paired" rows are adjacent rows: row 2i of the gate|up matrix is gate row
  i and row 2i+1 is up row i, so the fused matrix has M = 2F rows and the
  activation has F = M/2 entries per batch row.
* The activation is written as bf16 (the next GEMV's input type), rounded
  once from the exact value.

Every function here works in float64 on exactly decoded inputs.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64


def f64_to_bf16_bits(v) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest with ties to even, in one rounding.

    Written from the bf16 definition (binary32's sign, 8-bit exponent and the
    top 7 fraction bits): write |v| = s * 2^E with s in [1, 2); keep
    s * 2^7 (normal range, E >= -126) or |v| * 2^133 (subnormal range); the
    power-of-two scaling is exact, the result is rounded to the nearest
    integer with ties to even. A carry out of the significand bumps the
    exponent; past the largest finite bf16 the result is infinity. NaN maps
    to the quiet NaN 0x7FC0.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x8000, 0).astype(np.int64)
    finite_nz = np.isfinite(a) & (a > 0)
    safe = np.where(finite_nz, a, 1.0)
    _, e = np.frexp(safe)                  # safe = m * 2^e, m in [0.5, 1)
    E = e.astype(np.int64) - 1             # safe = s * 2^E, s in [1, 2)
    sub = E < -126
    shift = np.where(sub, 133, 7 - E)
    t = np.ldexp(safe, shift.astype(np.int32))
    fl = np.floor(t)
    n = fl.astype(np.int64)
    r = t - fl                             # exact
    n = n + ((r > 0.5) | ((r == 0.5) & ((n & 1) == 1))).astype(np.int64)
    carry = (~sub) & (n == 256)
    n = np.where(carry, 128, n)
    E = np.where(carry, E + 1, E)
    normal_bits = ((E + 127) << 7) | (n - 128)
    bits = np.where(sub, n, normal_bits)   # a subnormal that rounds to 128 is the smallest normal
    bits = np.where((~sub) & (E > 127), 0x7F80, bits)
    bits = np.where(a == 0, 0, bits)
    bits = np.where(np.isinf(a), 0x7F80, bits)
    bits = bits | sign
    bits = np.where(np.isnan(v), 0x7FC0, bits)
    return bits.astype(np.uint16)


def rmsnorm_ref(h: np.ndarray, g_bits: np.ndarray, eps: float) -> np.ndarray:
    """Exact-as-float64 RMSNorm of each row of h [B][K] (float32 values).

    x[b, k] = h[b, k] / sqrt(mean_k(h[b, :]^2) + eps) * g[k]
    """
    hf = np.asarray(h, dtype=np.float64)
    hf = hf.reshape(-1, hf.shape[-1])
    g = bf16_to_f64(g_bits).reshape(-1)
    ms = np.mean(hf * hf, axis=1, keepdims=True)
    return hf / np.sqrt(ms + float(eps)) * g[None, :]


def rmsnorm_bf16(h: np.ndarray, g_bits: np.ndarray, eps: float) -> np.ndarray:
    """The GEMV input the fused prologue produces: bf16 bits of rmsnorm_ref."""
    return f64_to_bf16_bits(rmsnorm_ref(h, g_bits, eps))


def silu(t: np.ndarray) -> np.ndarray:
    """t * sigmoid(t) = t / (1 + exp(-t)) in float64 (exp overflow gives -0 or 0)."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def swiglu_ref(y_pairs: np.ndarray) -> np.ndarray:
    """act[b, i] = silu(y[b, 2i]) * y[b, 2i+1] for a [B][2F] GEMV output."""
    y = np.asarray(y_pairs, dtype=np.float64)
    return silu(y[:, 0::2]) * y[:, 1::2]


def swiglu_bound(y_ref: np.ndarray, y_tol: np.ndarray) -> np.ndarray:
    """Largest |act_gpu - act_ref| allowed when the paired GEMV outputs are
    within y_tol of y_ref and the activation is rounded to bf16 once.

    With gate g, up u, |silu'| <= 1.1 (its maximum is about 1.0998, at
    t ~ 2.4) and |silu(g) - silu(g_ref)| <= 1.1 * tol_g:
      |silu(g) u - silu(g_ref) u_ref|
        <= 1.1 tol_g (|u_ref| + tol_u) + |silu(g_ref)| tol_u,
    plus float32 evaluation (a few units in the last place of float32,
    bounded by 2^-20 of the value) and the final bf16 rounding (at most 2^-8
    relative, half a bf16 unit rounded up to a power of two), plus 1e-30 so
    that zero results compare.
    """
    y = np.asarray(y_ref, dtype=np.float64)
    t = np.asarray(y_tol, dtype=np.float64)
    g, u = y[:, 0::2], y[:, 1::2]
    tg, tu = t[:, 0::2], t[:, 1::2]
    act = silu(g) * u
    prop = 1.1 * tg * (np.abs(u) + tu) + np.abs(silu(g)) * tu
    mag = np.abs(act) + prop
    return prop + (2.0 ** -8 + 2.0 ** -20) * mag + 1e-30


def residual_bound(y_ref: np.ndarray, y_tol: np.ndarray) -> np.ndarray:
    """Largest |y_gpu - (residual + W x)| allowed: the GEMV's own bound plus
    one float32 rounding of the add (2^-24 relative, doubled for margin)."""
    y = np.asarray(y_ref, dtype=np.float64)
    return np.asarray(y_tol, dtype=np.float64) + 2.0 ** -23 * (np.abs(y) + y_tol)
