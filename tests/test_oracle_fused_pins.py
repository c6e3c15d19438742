"""Pins of the fused prologue/epilogue oracle (oracle/fused.py) against things
other than itself: the bf16 definition and torch's float32 -> bfloat16 cast,
torch's rms_norm and silu in float64, closed forms worked out by hand, and
planted mistakes that must make a pin fail.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle.formats as oformats
import oracle.fused as ofused


# ------------------------------------------------------------ bf16 rounding
def _bf16_pins_ok() -> bool:
    # every bf16 value (NaNs aside) rounds to itself
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oformats.bf16_to_f64(bits)
    back = ofused.f64_to_bf16_bits(v)
    fin = ~np.isnan(v)
    if not (back[fin] == bits[fin]).all() or not (back[~fin] == 0x7FC0).all():
        return False
    # values representable in float32: one rounding, so torch's float32 ->
    # bfloat16 cast (round to nearest even) is the reference
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(200_000) * np.exp2(rng.integers(-140, 120, 200_000))).astype(np.float32)
    # exact midpoints between neighbouring bf16 values, and one float32 ulp either side
    mids = ((rng.integers(0, 1 << 16, 20_000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    mids = mids[np.isfinite(mids)]
    up = (mids.view(np.uint32) + 1).view(np.float32)
    dn = (mids.view(np.uint32) - 1).view(np.float32)
    allf = np.concatenate([f, mids, up, dn])
    ref = torch.from_numpy(allf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = ofused.f64_to_bf16_bits(allf.astype(np.float64))
    if not (got == ref).all():
        return False
    # a float64 value just above a midpoint rounds up even when rounding it to
    # float32 first would land on the midpoint (a double rounding to even)
    one_mid = 1.0 + 2.0 ** -8                      # midpoint of 1.0 (even) and 1.0078125
    if ofused.f64_to_bf16_bits(one_mid + 2.0 ** -40) != 0x3F81:
        return False
    if ofused.f64_to_bf16_bits(one_mid) != 0x3F80 or ofused.f64_to_bf16_bits(-one_mid) != 0xBF80:
        return False
    # overflow: the midpoint between the largest finite bf16 and 2^128 ties to even = inf
    mx = oformats.bf16_to_f64(np.uint16(0x7F7F))
    if ofused.f64_to_bf16_bits(float(mx) + 2.0 ** 119) != 0x7F80:
        return False
    if ofused.f64_to_bf16_bits(2.0 ** -133) != 0x0001 or ofused.f64_to_bf16_bits(2.0 ** -135) != 0x0000:
        return False
    return True


def test_bf16_rounding_definition():
    assert _bf16_pins_ok()


# ------------------------------------------------------------------ RMSNorm
def _bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rmsnorm_pins_ok() -> bool:
    # constant rows with eps = 0 normalize to sign(c) exactly: bits of +-g
    h = np.array([[0.75] * 8, [-3.0] * 8], dtype=np.float32)
    g = _bf16([1.0, 2.0, 0.5, -1.0, 1.0, 1.0, 1.0, 1.0])
    x = ofused.rmsnorm_ref(h, g, 0.0)
    want = np.array([[1.0, 2.0, 0.5, -1.0, 1, 1, 1, 1], [-1.0, -2.0, -0.5, 1.0, -1, -1, -1, -1]])
    if not (x == want).all():
        return False
    # eps enters under the root: c = 0.5, eps = 0.25 -> 0.5 / sqrt(0.5) = sqrt(0.5)
    x = ofused.rmsnorm_ref(np.full((1, 4), 0.5, np.float32), _bf16([1.0] * 4), 0.25)
    if not np.allclose(x, math.sqrt(0.5), rtol=1e-15, atol=0):
        return False
    # the mean is over K, not a sum: h = (3, 4, 0, 0) -> mean of squares 25/4,
    # rms 2.5 -> (1.2, 1.6, 0, 0)
    x = ofused.rmsnorm_ref(np.array([[3.0, 4.0, 0.0, 0.0]], np.float32), _bf16([1.0] * 4), 0.0)
    if not np.allclose(x, [[1.2, 1.6, 0.0, 0.0]], rtol=1e-15, atol=0):
        return False
    # torch's rms_norm in float64 on random rows
    rng = np.random.default_rng(2)
    h = rng.standard_normal((3, 2048)).astype(np.float32)
    gb = _bf16(rng.uniform(0.5, 1.5, 2048).astype(np.float32))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h.astype(np.float64)), (2048,),
                                       weight=torch.from_numpy(oformats.bf16_to_f64(gb)), eps=1e-5).numpy()
    if not np.allclose(ofused.rmsnorm_ref(h, gb, 1e-5), ref, rtol=1e-13, atol=0):
        return False
    # scale invariance with eps = 0: h * 2^k normalizes to the same vector
    if not (ofused.rmsnorm_ref(h * np.float32(8.0), gb, 0.0) == ofused.rmsnorm_ref(h, gb, 0.0)).all():
        return False
    # rmsnorm_bf16 is the one rounding of rmsnorm_ref
    xb = ofused.rmsnorm_bf16(h, gb, 1e-5)
    return bool((xb == ofused.f64_to_bf16_bits(ofused.rmsnorm_ref(h, gb, 1e-5))).all())


def test_rmsnorm_closed_forms_and_library():
    assert _rmsnorm_pins_ok()


# ------------------------------------------------------------------- SwiGLU
def _swiglu_pins_ok() -> bool:
    t = np.linspace(-60.0, 60.0, 4001)
    ref = torch.nn.functional.silu(torch.from_numpy(t)).numpy()
    if not np.allclose(ofused.silu(t), ref, rtol=1e-14, atol=1e-300):
        return False
    if ofused.silu(np.array([0.0]))[0] != 0.0 or ofused.silu(np.array([-1000.0]))[0] != 0.0:
        return False
    # pairing: y = (gate0, up0, gate1, up1, gate2, up2) = (0, 5, 2, 3, -1, 0.5)
    # act0 = silu(0) * 5 = 0; act1 = 2 / (1 + e^-2) * 3; act2 = -1 / (1 + e) * 0.5
    y = np.array([[0.0, 5.0, 2.0, 3.0, -1.0, 0.5]])
    want = [0.0, 6.0 / (1.0 + math.exp(-2.0)), -0.5 / (1.0 + math.e)]
    if not np.allclose(ofused.swiglu_ref(y), [want], rtol=1e-15, atol=0):
        return False
    # the derivative bound the tolerance uses: max |silu'| < 1.1
    tt = np.linspace(-20, 20, 400_001)
    s = 1.0 / (1.0 + np.exp(-tt))
    if np.abs(s * (1.0 + tt * (1.0 - s))).max() >= 1.1:
        return False
    # a float32 evaluation rounded once to bf16 lies inside the bound
    rng = np.random.default_rng(3)
    yp = rng.standard_normal((4, 4096)) * 4.0
    g32 = yp[:, 0::2].astype(np.float32)
    u32 = yp[:, 1::2].astype(np.float32)
    act32 = (g32 / (np.float32(1) + np.exp(-g32))) * u32
    actb = oformats.bf16_to_f64(torch.from_numpy(act32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    yref = yp.astype(np.float32).astype(np.float64)
    err = np.abs(actb - ofused.swiglu_ref(yref))
    return bool((err <= ofused.swiglu_bound(yref, np.zeros_like(yref))).all())


def test_swiglu_pairing_and_library():
    assert _swiglu_pins_ok()


# The upper side of swiglu_bound: the bound must hold when the paired GEMV
# outputs sit anywhere within their own tolerances (the propagation terms),
# and it must not be loose - on inputs where one term dominates, the worst
# achievable error comes within 15 % of it.
def _bf16_of_f32(a32):
    return oformats.bf16_to_f64(torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
                                .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def _act_f32(g, u):
    """silu(g) * u evaluated in float32 and rounded once to bf16."""
    g32 = np.asarray(g, dtype=np.float32)
    u32 = np.asarray(u, dtype=np.float32)
    with np.errstate(over="ignore"):
        return _bf16_of_f32((g32 / (np.float32(1) + np.exp(-g32))) * u32)


def _swiglu_bound_pins_ok() -> bool:
    # hand-worked values. Gate 0, up 2, tolerances 0.01 / 0.02: silu(0) = 0, so
    # the bound is 1.1 * 0.01 * (2 + 0.02) = 0.02222 times (1 + 2^-8 + 2^-20).
    # Gate 1, up -3, tolerances 0 / 0.5: silu(1) = 1 / (1 + 1/e) = 0.73105857863,
    # propagation 0.5 * 0.73105857863 = 0.36552928932, magnitude 3 * 0.73105857863
    # + 0.36552928932 = 2.55870502521, bound 0.36552928932 + 2.55870502521 *
    # (2^-8 + 2^-20) = 0.37552667099.
    y = np.array([[0.0, 2.0, 1.0, -3.0]])
    t = np.array([[0.01, 0.02, 0.0, 0.5]])
    b = ofused.swiglu_bound(y, t)
    if b.shape != (1, 2) or abs(b[0, 0] - 0.0223068180656) > 1e-12 or abs(b[0, 1] - 0.37552667099) > 1e-10:
        return False
    # containment: random outputs and tolerances, the pair moved to every corner
    # of its tolerance box and to random interior points
    rng = np.random.default_rng(11)
    n = 20_000
    g = rng.uniform(-8, 8, n)
    u = rng.uniform(-8, 8, n)
    tg = rng.uniform(0, 0.3, n) * rng.choice([0.0, 0.01, 1.0], n)
    tu = rng.uniform(0, 0.3, n) * rng.choice([0.0, 0.01, 1.0], n)
    yref = np.stack([g, u], axis=1).reshape(1, -1)
    tol = np.stack([tg, tu], axis=1).reshape(1, -1)
    bound = ofused.swiglu_bound(yref, tol)[0]
    exact = ofused.swiglu_ref(yref)[0]
    moves = [(sg, su) for sg in (-1.0, 1.0) for su in (-1.0, 1.0)]
    moves += [tuple(rng.uniform(-1, 1, 2)) for _ in range(4)]
    for sg, su in moves:
        err = np.abs(_act_f32(g + sg * tg, u + su * tu) - exact)
        if not (err <= bound).all():
            return False
    # tightness: each case is dominated by one term of the bound
    #   gate at silu's steepest point (t ~ 2.4, slope 1.0998) moved by its tolerance,
    #   up moved by its tolerance next to a large silu(gate),
    #   zero tolerances (the bf16 rounding alone, at a value just below a midpoint)
    cases = [(2.4, 10.0, 0.1, 0.0, +1, 0), (8.0, 0.0, 0.0, 1.0, 0, +1), (-8.0, 0.0, 0.0, 1.0, 0, -1)]
    for gg, uu, tgg, tuu, sg, su in cases:
        yy = np.array([[gg, uu]])
        bb = ofused.swiglu_bound(yy, np.array([[tgg, tuu]]))[0, 0]
        err = abs(_act_f32(gg + sg * tgg, uu + su * tuu)[0] - ofused.swiglu_ref(yy)[0, 0])
        if not (0.85 * bb <= err <= bb):
            return False
    # the rounding term alone: an activation halfway up a bf16 interval
    # (1 + 2^-8 - 2^-12) rounds down by nearly half a unit = 2^-8 relative
    gg = 30.0                                   # silu(30) = 30 to float32 precision
    uu = (1.0 + 2.0 ** -8 - 2.0 ** -12) / 30.0
    yy = np.array([[gg, uu]])
    bb = ofused.swiglu_bound(yy, np.zeros_like(yy))[0, 0]
    err = abs(_act_f32(gg, uu)[0] - ofused.swiglu_ref(yy)[0, 0])
    return bool(0.85 * bb <= err <= bb)


def test_swiglu_bound_value_containment_and_tightness():
    assert _swiglu_bound_pins_ok()


def test_residual_bound_covers_one_float32_add():
    rng = np.random.default_rng(4)
    r = rng.standard_normal(100_000).astype(np.float32) * 30
    a = rng.standard_normal(100_000).astype(np.float32)
    got = (r + a).astype(np.float64)
    exact = r.astype(np.float64) + a.astype(np.float64)
    assert (np.abs(got - exact) <= ofused.residual_bound(exact, np.zeros_like(exact))).all()
    assert ofused.residual_bound(np.array([1.0]), np.array([0.0]))[0] < 2.0 ** -22


# -------------------------------------------------------- planted mistakes
_orig_rms = ofused.rmsnorm_ref
_orig_bf16 = ofused.f64_to_bf16_bits
_orig_swiglu = ofused.swiglu_ref


def _mut_rms_no_eps(h, g, eps):
    return _orig_rms(h, g, 0.0)


def _mut_rms_sum(h, g, eps):
    hf = np.asarray(h, dtype=np.float64).reshape(-1, np.asarray(h).shape[-1])
    return _orig_rms(h, g, eps) * np.sqrt(np.mean(hf * hf, axis=1, keepdims=True) + eps) / \
        np.sqrt(np.sum(hf * hf, axis=1, keepdims=True) + eps)


def _mut_rms_no_weight(h, g, eps):
    return _orig_rms(h, np.full_like(np.asarray(g), 0x3F80), eps)


def _mut_bf16_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _mut_swiglu_swapped(y):
    y = np.asarray(y, dtype=np.float64)
    return ofused.silu(y[:, 1::2]) * y[:, 0::2]


def _mut_swiglu_halves(y):
    y = np.asarray(y, dtype=np.float64)
    F = y.shape[1] // 2
    return ofused.silu(y[:, :F]) * y[:, F:]


def _mut_silu_sigmoid(t):
    t = np.asarray(t, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-t))


_orig_swiglu_bound = ofused.swiglu_bound


def _mut_bound_times(k):
    return lambda y, t: k * _orig_swiglu_bound(y, t)


def _mut_bound_no_prop(y, t):
    return _orig_swiglu_bound(y, np.zeros_like(np.asarray(y, dtype=np.float64)))


def _mut_bound_no_up_term(y, t):
    """The |silu(g)| * tol_u term dropped (only the gate's error propagated)."""
    t = np.array(t, dtype=np.float64)
    t[:, 1::2] = 0.0
    return _orig_swiglu_bound(y, t)


def _mut_bound_no_gate_term(y, t):
    """The silu-slope * tol_g term dropped (only the up value's error propagated)."""
    t = np.array(t, dtype=np.float64)
    t[:, 0::2] = 0.0
    return _orig_swiglu_bound(y, t)


def _mut_bound_no_rounding(y, t):
    """The final bf16 rounding left out of the bound."""
    y = np.asarray(y, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    g, u = y[:, 0::2], y[:, 1::2]
    return 1.1 * t[:, 0::2] * (np.abs(u) + t[:, 1::2]) + np.abs(ofused.silu(g)) * t[:, 1::2] + 1e-30


FUSED_MUTANTS = {
    "rmsnorm_eps_dropped": [("rmsnorm_ref", _mut_rms_no_eps)],
    "rmsnorm_sum_not_mean": [("rmsnorm_ref", _mut_rms_sum)],
    "rmsnorm_weight_dropped": [("rmsnorm_ref", _mut_rms_no_weight)],
    "bf16_truncation": [("f64_to_bf16_bits", _mut_bf16_truncate)],
    "swiglu_gate_up_swapped": [("swiglu_ref", _mut_swiglu_swapped)],
    "swiglu_halves_not_pairs": [("swiglu_ref", _mut_swiglu_halves)],
    "silu_is_sigmoid": [("silu", _mut_silu_sigmoid)],
    "swiglu_bound_x4": [("swiglu_bound", _mut_bound_times(4.0))],
    "swiglu_bound_x8": [("swiglu_bound", _mut_bound_times(8.0))],
    "swiglu_bound_prop_dropped": [("swiglu_bound", _mut_bound_no_prop)],
    "swiglu_bound_up_term_dropped": [("swiglu_bound", _mut_bound_no_up_term)],
    "swiglu_bound_gate_term_dropped": [("swiglu_bound", _mut_bound_no_gate_term)],
    "swiglu_bound_rounding_dropped": [("swiglu_bound", _mut_bound_no_rounding)],
}


def _fused_pins_pass() -> bool:
    try:
        return (_bf16_pins_ok() and _rmsnorm_pins_ok() and _swiglu_pins_ok()
                and _swiglu_bound_pins_ok())
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(FUSED_MUTANTS))
def test_fused_planted_mistakes_are_caught(monkeypatch, name):
    assert _fused_pins_pass()
    for attr, repl in FUSED_MUTANTS[name]:
        monkeypatch.setattr(ofused, attr, repl)
    assert not _fused_pins_pass(), f"planted mistake {name} went unnoticed"
