"""Pins of the decode-attention oracle (oracle/attention.py) against things
other than itself: closed forms worked out by hand, torch's
scaled_dot_product_attention in float64 (with its grouped-query option), and
planted mistakes that must make a pin fail."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.attention as oatt
import synth


def _bf16(a):
    return synth.round_f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _case(B, n_q, n_kv, d, T, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n_q, d)).astype(np.float32)
    k = _bf16(rng.standard_normal((B, n_kv, T, d)))
    v = _bf16(rng.standard_normal((B, n_kv, T, d)))
    return q, k, v


def _pins_ok() -> bool:
    d = 8
    # one position: the output is that position's value row, exactly
    q, k, v = _case(1, 4, 2, d, 5, 1)
    out, _ = oatt.attention_decode_ref(q, k, v, [1], 0.125)
    vv = oatt.bf16_to_f64(v[0, :, 0])
    if not (out[0, :2] == vv[0]).all() or not (out[0, 2:] == vv[1]).all():
        return False
    # q = 0: equal weights, the plain mean of the first L value rows
    out, _ = oatt.attention_decode_ref(np.zeros_like(q), k, v, [4], 0.125)
    if not np.allclose(out[0, 0], oatt.bf16_to_f64(v[0, 0, :4]).mean(axis=0), rtol=1e-14, atol=1e-15):
        return False
    # two positions, score difference 0.5 * (1 * 2) = 1: weights 1/(1+e), e/(1+e)
    q1 = np.zeros((1, 1, d), np.float32); q1[0, 0, 0] = 1.0
    k1 = np.zeros((1, 1, 2, d), np.float32); k1[0, 0, 1, 0] = 2.0
    v1 = np.zeros((1, 1, 2, d), np.float32); v1[0, 0, 0] = 3.0; v1[0, 0, 1] = -1.0
    out, A = oatt.attention_decode_ref(q1, _bf16(k1), _bf16(v1), [2], 0.5)
    want = (3.0 - math.e) / (1.0 + math.e)
    wantA = (3.0 + math.e) / (1.0 + math.e)
    if not (np.allclose(out, want, rtol=1e-14, atol=0) and np.allclose(A, wantA, rtol=1e-14, atol=0)):
        return False
    # grouped heads: query head h reads key/value head h // (n_q / n_kv)
    vg = np.zeros((1, 2, 3, d), np.float32); vg[0, 0] = 1.0; vg[0, 1] = -2.0
    qg, kg, _ = _case(1, 4, 2, d, 3, 2)
    out, _ = oatt.attention_decode_ref(qg, kg, _bf16(vg), [3], 0.3)
    if not (np.allclose(out[0, :2], 1.0, rtol=1e-14) and np.allclose(out[0, 2:], -2.0, rtol=1e-14)):
        return False
    # scores near 800: finite, the larger one takes weight 1 / (1 + e^-10)
    qb = np.zeros((1, 1, d), np.float32); qb[0, 0, 0] = 100.0
    kb = np.zeros((1, 1, 2, d), np.float32); kb[0, 0, 0, 0] = 8.0; kb[0, 0, 1, 0] = 7.875
    vb = np.zeros((1, 1, 2, d), np.float32); vb[0, 0, 0] = 1.0
    out, _ = oatt.attention_decode_ref(qb, _bf16(kb), _bf16(vb), [2], 1.0)   # s = 800, 787.5
    if not np.allclose(out, 1.0 / (1.0 + math.exp(-12.5)), rtol=1e-14):
        return False
    # positions past the sequence's length are never read (NaN there)
    q, k, v = _case(2, 4, 1, d, 6, 3)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 3:] = 0x7FC0
    v2[0, :, 3:] = 0x7FC0
    o1, _ = oatt.attention_decode_ref(q, k, v, [3, 6], 0.25)
    o2, _ = oatt.attention_decode_ref(q, k2, v2, [3, 6], 0.25)
    if not (o1 == o2).all():
        return False
    # torch's scaled_dot_product_attention in float64 (grouped-query option)
    q, k, v = _case(3, 8, 2, 64, 40, 4)
    lens = [40, 1, 17]
    out, _ = oatt.attention_decode_ref(q, k, v, lens, 0.125)
    for b, L in enumerate(lens):
        tq = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]
        tk = torch.from_numpy(oatt.bf16_to_f64(k[b, :, :L]))[None]
        tv = torch.from_numpy(oatt.bf16_to_f64(v[b, :, :L]))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.125, enable_gqa=True)
        if not np.allclose(out[b], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-14):
            return False
    return True


def test_attention_oracle_pins():
    assert _pins_ok()


_orig = oatt.attention_decode_ref


def _mut_gqa_modulo(q, k, v, lens, scale):
    # query head h reads key/value head h % n_kv instead of h // group
    n_q, n_kv = q.shape[1], k.shape[1]
    g = n_q // n_kv
    perm = np.array([(h % n_kv) * g + (h // n_kv) for h in range(n_q)])
    out, A = _orig(q[:, perm], k, v, lens, scale)
    inv = np.argsort(perm)
    return out[:, inv], A[:, inv]


def _mut_no_scale(q, k, v, lens, scale):
    return _orig(q, k, v, lens, 1.0)


def _mut_no_max(q, k, v, lens, scale):
    qf = np.asarray(q, dtype=np.float64)
    B, n_q, d = qf.shape
    n_kv = k.shape[1]
    g = n_q // n_kv
    out = np.empty((B, n_q, d)); A = np.empty((B, n_q, d))
    with np.errstate(over="ignore", invalid="ignore"):
        for b in range(B):
            L = int(lens[b])
            for h in range(n_q):
                K = oatt.bf16_to_f64(k[b, h // g, :L]); V = oatt.bf16_to_f64(v[b, h // g, :L])
                p = np.exp(scale * (K @ qf[b, h]))
                out[b, h] = p @ V / p.sum(); A[b, h] = p @ np.abs(V) / p.sum()
    return out, A


def _mut_full_cache(q, k, v, lens, scale):
    return _orig(q, k, v, [k.shape[2]] * len(lens), scale)


def _mut_abs_dropped(q, k, v, lens, scale):
    out, A = _orig(q, k, v, lens, scale)
    return out, np.abs(out)


MUTANTS = {"gqa_modulo": _mut_gqa_modulo, "scale_dropped": _mut_no_scale, "no_max_subtraction": _mut_no_max,
           "length_ignored": _mut_full_cache, "abs_dropped": _mut_abs_dropped}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_planted_mistakes_are_caught(monkeypatch, name):
    assert _pins_ok()
    monkeypatch.setattr(oatt, "attention_decode_ref", MUTANTS[name])
    try:
        caught = not _pins_ok()
    except Exception:
        caught = True
    assert caught, f"planted mistake {name} went unnoticed"


# ------------------------------------------------ the parity check itself
# parity_report is the pass/fail rule every GPU attention test applies:
# pass iff the output is finite and |out - ref| <= 1e-3 * A + 1e-5. These
# pins drive it with hand-picked outputs on both sides of that bound.
def _report_pins_ok() -> bool:
    ref = np.array([[[1.0, -2.0, 0.0, 5.0]]])
    A = np.array([[[10.0, 4.0, 0.0, 1000.0]]])          # bounds 0.01001, 0.00401, 1e-5, 1.00001
    r = oatt.parity_report(ref.copy(), ref, A)
    if not (r["ok"] and r["n"] == 4 and r["n_bad"] == 0 and r["max_err_over_bound"] == 0.0):
        return False
    inside = ref + np.array([[[0.010009, -0.004009, 0.0000099, -1.0000099]]])
    r = oatt.parity_report(inside, ref, A)
    if not r["ok"] or not (0.99 < r["max_err_over_bound"] <= 1.0):
        return False
    # each output pushed just outside its own bound, one at a time, either sign
    for i, e in enumerate((0.010011, 0.004011, 0.0000101, 1.0000101)):
        for sgn in (1.0, -1.0):
            out = ref.copy()
            out[0, 0, i] += sgn * e
            r = oatt.parity_report(out, ref, A)
            if r["ok"] or r["n_bad"] != 1 or not (1.0 < r["max_err_over_bound"] < 1.02):
                return False
    # values far off in the negative direction fail (all four bounds are below 3)
    r = oatt.parity_report(ref - 3.0, ref, A)
    if r["ok"] or r["n_bad"] != 4:
        return False
    # non-finite outputs fail and count as infinitely far, even where the bound is huge
    bigA = np.full_like(A, 1e300)
    for bad in (np.nan, np.inf, -np.inf):
        out = ref.copy()
        out[0, 0, 2] = bad
        r = oatt.parity_report(out, ref, bigA)
        if r["ok"] or r["n_bad"] != 1 or r["max_err_over_bound"] != np.inf:
            return False
    return True


def test_attention_parity_report_definition():
    assert _report_pins_ok()


_orig_report = oatt.parity_report


def _mut_report_abs_tol(scale):
    def f(out_gpu, out_ref, A):
        old = oatt.ABS_TOL
        oatt.ABS_TOL = old * scale
        try:
            return _orig_report(out_gpu, out_ref, A)
        finally:
            oatt.ABS_TOL = old
    return f


def _mut_report_rel_tol(out_gpu, out_ref, A):
    old = oatt.REL_TOL
    oatt.REL_TOL = 1e-2
    try:
        return _orig_report(out_gpu, out_ref, A)
    finally:
        oatt.REL_TOL = old


def _mut_report_no_finite(out_gpu, out_ref, A):
    og = np.asarray(out_gpu, dtype=np.float64)
    err = np.abs(og - out_ref)
    bound = oatt.REL_TOL * A + oatt.ABS_TOL
    with np.errstate(invalid="ignore"):
        ok = ~(err > bound)
        ratio = err / bound
    return {"ok": bool(ok.all()), "n": int(ok.size), "n_bad": int((~ok).sum()),
            "max_err_over_bound": float(np.nanmax(ratio))}


def _mut_report_signed(out_gpu, out_ref, A):
    og = np.asarray(out_gpu, dtype=np.float64)
    err = og - out_ref
    bound = oatt.REL_TOL * A + oatt.ABS_TOL
    finite = np.isfinite(og)
    ok = finite & (err <= bound)
    ratio = np.where(finite, np.abs(err) / bound, np.inf)
    return {"ok": bool(ok.all()), "n": int(ok.size), "n_bad": int((~ok).sum()),
            "max_err_over_bound": float(ratio.max())}


REPORT_MUTANTS = {"abs_tol_x10": _mut_report_abs_tol(10.0), "abs_tol_zero": _mut_report_abs_tol(0.0),
                  "rel_tol_1e-2": _mut_report_rel_tol, "finite_check_dropped": _mut_report_no_finite,
                  "signed_error": _mut_report_signed}


@pytest.mark.parametrize("name", sorted(REPORT_MUTANTS))
def test_attention_report_planted_mistakes_are_caught(monkeypatch, name):
    assert _report_pins_ok()
    monkeypatch.setattr(oatt, "parity_report", REPORT_MUTANTS[name])
    try:
        caught = not _report_pins_ok()
    except Exception:
        caught = True
    assert caught, f"planted mistake {name} went unnoticed"
