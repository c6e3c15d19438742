"""float64 reference for grouped-query decode attention (test infrastructure).

Only the tests, the smoke check and the bench's CPU baseline use this module.

Decode attention compares one new query per head against the keys of every
earlier position stored in the KV cache and takes the softmax-weighted
average of their values (the Rust page's layer walk-through, "Attention").
With grouped-query attention, groups of query heads share one key/value
head: query head h reads key/value head h // (n_q / n_kv) (the same page:
32 query heads, 4 key/value heads, groups of 8; "infer": 32 and 8 for
Llama-3.2-1B, one block per key/value head serving its query heads). The KV
cache holds bf16 values ("infer": bf16 KV cache; the Rust page stores f16).

The reference is that definition, in float64 on exactly decoded inputs:
    s_t = scale * sum_j q[h, j] k[t, j],  t < L
    p_t = exp(s_t - max_t s_t)
    out[h, j] = sum_t p_t v[t, j] / sum_t p_t
The maximum is subtracted for range only (it cancels in the ratio).

Readings where the pages are silent:
* q is float32 (the GEMV's output), the output float32; the scale is a
  parameter (1 / sqrt(head_dim) for Llama models);
* cache layout [batch][n_kv][max_ctx][head_dim], positions 0..L_b - 1 of
  sequence b valid, L_b >= 1 given per sequence (a batch mixes lengths).

Tolerance (parity_report): per output, |out - ref| <= 1e-3 * A + 1e-5 with
A = sum_t p_t |v[t, j]| / sum_t p_t, the GEMV's relative bound applied to
the weighted average of |v| (float32 scores and sums err by ~1e-6 of that at
these lengths).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64

REL_TOL = 1e-3
ABS_TOL = 1e-5


def attention_decode_ref(q: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, ctx_lens, scale: float):
    """q float32 [B][n_q][d]; k, v bf16 bits [B][n_kv][max_ctx][d]; ctx_lens [B].

    Returns (out, A), float64 [B][n_q][d]."""
    q = np.asarray(q, dtype=np.float64)
    B, n_q, d = q.shape
    n_kv = k_bits.shape[1]
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    group = n_q // n_kv
    out = np.empty((B, n_q, d))
    A = np.empty((B, n_q, d))
    for b in range(B):
        L = int(ctx_lens[b])
        for kvh in range(n_kv):
            K = bf16_to_f64(k_bits[b, kvh, :L])           # [L][d]
            V = bf16_to_f64(v_bits[b, kvh, :L])
            for h in range(kvh * group, (kvh + 1) * group):
                s = scale * (K @ q[b, h])
                p = np.exp(s - s.max())
                den = p.sum()
                out[b, h] = (p @ V) / den
                A[b, h] = (p @ np.abs(V)) / den
    return out, A


def parity_report(out_gpu: np.ndarray, out_ref: np.ndarray, A: np.ndarray) -> dict:
    og = np.asarray(out_gpu, dtype=np.float64)
    err = np.abs(og - out_ref)
    bound = REL_TOL * A + ABS_TOL
    finite = np.isfinite(og)
    ok = finite & (err <= bound)
    ratio = np.where(finite, err / bound, np.inf)
    return {"ok": bool(ok.all()), "n": int(ok.size), "n_bad": int((~ok).sum()),
            "max_err_over_bound": float(ratio.max()) if ratio.size else 0.0}
