"""float64 reference for y = W x and the parity check against it.

Test infrastructure: only the tests, the smoke check and the bench's CPU
baseline use this module.

The method computes an ordinary matrix-vector product over the dequantized
weights: decode reads every weight once and does one multiply-add with it
("infer", the roofline discussion; "Writing an LLM inference engine from
scratch in Rust", the recap and Lesson 1). So the reference is that
definition: dequantize exactly (formats.dequantize) and take the dot
products in float64. Rows are processed in chunks only to bound memory.

Tolerance: a GPU output passes iff it is finite and
|y - y_ref| <= 1e-3 * sum_k |W_hat[m,k] * x[b,k]| + 1e-5.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .formats import GROUP, BF16, INT8_G32, INT8_ROW, bf16_to_f64, dequantize, scales_per_row

REL_TOL = 1e-3
ABS_TOL = 1e-5


def _row_slice(fmt: int, w: np.ndarray, s, M: int, K: int, rows: np.ndarray):
    """Select whole rows of the planar code and scale arrays."""
    if fmt == BF16:
        return np.asarray(w).reshape(M, K)[rows], None
    if fmt in (INT8_G32, INT8_ROW):  # one code per weight
        wr = np.asarray(w).reshape(M, K)[rows]
    else:
        G = GROUP[fmt]
        wr = np.asarray(w).reshape(M, K // G, G // 2)[rows]
    sr = np.asarray(s).reshape(M, scales_per_row(fmt, K))[rows]
    return wr, sr


def gemv_ref(fmt: int, w: np.ndarray, s, x_bits: np.ndarray, M: int, K: int,
             rows: Optional[Sequence[int]] = None, chunk_rows: int = 1024
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Return (y_ref, a_ref), both float64 [B][len(rows)].

    y_ref[b, m] = sum_k W_hat[m, k] * x[b, k]
    a_ref[b, m] = sum_k |W_hat[m, k] * x[b, k]|   (the tolerance scale)
    x_bits: bf16 bit patterns [B][K]. rows: subset of output rows (default all).
    """
    x = bf16_to_f64(np.asarray(x_bits).reshape(-1, K))            # [B][K]
    ax = np.abs(x)
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    B = x.shape[0]
    y = np.empty((B, rows.size), dtype=np.float64)
    a = np.empty((B, rows.size), dtype=np.float64)
    for c0 in range(0, rows.size, chunk_rows):
        r = rows[c0:c0 + chunk_rows]
        wr, sr = _row_slice(fmt, w, s, M, K, r)
        W_hat = dequantize(fmt, wr, sr, K)                         # [r][K] exact
        y[:, c0:c0 + r.size] = (W_hat @ x.T).T
        a[:, c0:c0 + r.size] = (np.abs(W_hat) @ ax.T).T
    return y, a


def parity_report(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray) -> dict:
    """Per-output check |y - y_ref| <= 1e-3 * a_ref + 1e-5 and y finite."""
    yg = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(yg - y_ref)
    bound = REL_TOL * a_ref + ABS_TOL
    finite = np.isfinite(yg)
    ok = finite & (err <= bound)
    ratio = np.where(finite, err / bound, np.inf)
    worst = int(np.argmax(ratio)) if ratio.size else 0
    return {
        "ok": bool(ok.all()),
        "n": int(ok.size),
        "n_bad": int((~ok).sum()),
        "max_err_over_bound": float(ratio.max()) if ratio.size else 0.0,
        "max_abs_err": float(err[finite].max()) if finite.any() else float("nan"),
        "worst_flat_index": worst,
    }


def check_parity(y_gpu, y_ref, a_ref) -> bool:
    return parity_report(y_gpu, y_ref, a_ref)["ok"]
