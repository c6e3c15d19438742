"""Greedy token choice over LM-head logits (test infrastructure).

Only the tests, the smoke check and the bench's CPU baseline use this module.

The decode step ends with an argmax over the vocabulary logits ("infer", the
decode pipeline figure and the per-kernel table's argmax row); its kernel
tests cover ties ("infer", test-suite notes). Reading taken where the pages
are silent: NumPy's argmax semantics, i.e.
  * the result is the first index of the maximum (ties -> lowest index);
  * -0.0 and +0.0 compare equal (a tie);
  * if any value is NaN, the result is the index of the first NaN;
  * all -inf gives index 0.
"""
from __future__ import annotations

import numpy as np


def argmax_ref(logits: np.ndarray) -> np.ndarray:
    """float32 logits [B][V] -> int32 [B], written from the definition above."""
    a = np.asarray(logits, dtype=np.float32)
    if a.ndim == 1:
        a = a[None, :]
    out = np.empty(a.shape[0], dtype=np.int32)
    for b in range(a.shape[0]):
        row = a[b]
        nan_at = np.flatnonzero(np.isnan(row))
        if nan_at.size:
            out[b] = nan_at[0]
            continue
        best = row.max()
        out[b] = np.flatnonzero(row == best)[0]
    return out
