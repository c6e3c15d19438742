"""Pins of the CPU oracle against things other than itself.

* decoders against library conversions (NumPy binary16, torch bfloat16);
* the binary16 rounding against NumPy's float64 -> float16 cast, including
  exact ties;
* hand-built blocks whose dot products were worked out by hand from the
  format definitions (tests/golden/hand_blocks.json);
* exact rational brute force on tiny random inputs;
* quantizer error bounds and the largest-magnitude -> code 0 rule;
* argmax against numpy.argmax on ties, NaN, signed zeros and -inf;
* mutation checks: plausible mistakes planted in the oracle (on the CPU)
  must make at least one of these pins fail.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.argmax as oargmax
import oracle.formats as oformats
import oracle.gemv as ogemv
import oracle.quantize as oquant
import synth
from helpers import build_case, load_json

FMTS_Q = [synth.INT8_G32, synth.Q4_0_G32, synth.INT4_G128, synth.INT8_ROW, synth.INT4_G64]
ALL_FMTS = [synth.BF16] + FMTS_Q


# ------------------------------------------------------------------ decoders
def test_f16_decode_matches_numpy_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    # signed zeros keep their sign
    assert np.signbit(oracle.f16_to_f64(np.array([0x8000], np.uint16)))[0]


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_f64_to_f16_matches_numpy_including_ties():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(200_000) * 10.0 ** rng.integers(-9, 6, 200_000)
    fin = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    fin = np.unique(fin[np.isfinite(fin)])
    mids = (fin[:-1] + fin[1:]) / 2                      # exact ties (dyadic)
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25,
                     2.0 ** -25 * 1.0000001, 2.0 ** -14 * (1 - 2 ** -11), 3.0 * 2 ** -26])
    for arr in (v, fin, mids, edge):
        got = oracle.f64_to_f16_bits(arr)
        ref = arr.astype(np.float16).view(np.uint16)
        assert (got == ref).all()


# ---------------------------------------------------------- hand-built blocks
HAND = load_json("hand_blocks.json")["cases"]


def _check_hand_case(case) -> bool:
    fmt, M, K, w, s, x, y_exact = build_case(case)
    y, a = oracle.gemv_ref(fmt, w, s, x, M, K)
    want = np.array([[float(v) for v in row] for row in y_exact])
    return y.shape == want.shape and bool((y == want).all())


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
def test_hand_built_blocks(case):
    assert _check_hand_case(case), case.get("why", case["name"])


# ------------------------------------------------------- exact brute force
def _frac_f16(bits):
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def _frac_bf16(bits):
    t = torch.tensor([int(np.int16(np.uint16(bits).view(np.int16)))], dtype=torch.int16)
    return Fraction(float(t.view(torch.bfloat16).to(torch.float64)[0]))


def _brute_weight(fmt, w, s, m, k, K):
    """One weight as an exact rational, indexed element by element."""
    if fmt == synth.BF16:
        return _frac_bf16(w[m, k])
    if fmt == synth.INT8_ROW:
        return int(w[m, k]) * _frac_f16(s[m])
    G = synth.GROUP[fmt]
    d = _frac_f16(s[m, k // G])
    if fmt == synth.INT8_G32:
        return int(w[m, k]) * d
    j = k % G
    half = G // 2
    byte = int(w[m, k // G, j % half])
    q = (byte & 0xF) if j < half else (byte >> 4)
    return (q - 8) * d


def _brute_force_ok(fmt, M, K, B, seed) -> bool:
    g = synth.make_gemv("t", fmt, M, K, B, cfg=9, layer=seed, proj="o")
    y, a = oracle.gemv_ref(fmt, g.w, g.s, g.x, M, K)
    for b in range(B):
        xs = [_frac_bf16(g.x[b, k]) for k in range(K)]
        for m in range(M):
            terms = [_brute_weight(fmt, g.w, g.s, m, k, K) * xs[k] for k in range(K)]
            exact = sum(terms, Fraction(0))
            abs_sum = sum((abs(t) for t in terms), Fraction(0))
            if abs(Fraction(y[b, m]) - exact) > Fraction(K) * Fraction(2) ** -52 * abs_sum:
                return False
            if abs(Fraction(a[b, m]) - abs_sum) > Fraction(K) * Fraction(2) ** -52 * abs_sum:
                return False
    return True


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("K", [128, 256])
def test_brute_force_exact_rational(fmt, K):
    assert _brute_force_ok(fmt, M=3, K=K, B=2, seed=K + fmt)


def test_brute_force_q4_k32_batch3():
    assert _brute_force_ok(synth.Q4_0_G32, M=4, K=32, B=3, seed=1)
    assert _brute_force_ok(synth.INT8_G32, M=4, K=64, B=3, seed=2)


# -------------------------------------------------------------- quantizers
def _quant_bounds_ok(fmt, w_bits, M, K) -> bool:
    """Error bounds of the quantizers (binary16 unit roundoff u = 2^-11).

    int8: |w - w_hat| <= |d|/2.  4-bit: |w - w_hat| <= |d|/2 except the top code
    (clamped from 8 to 7): <= |d| (1 + 2^-8); the group's largest-magnitude
    element m gets code 0 and reconstructs within |m| 2^-11. Valid for normal d.
    """
    G = synth.GROUP[fmt] or K                    # int8-row: the whole row
    codes, d_bits = oracle.quantize_from_bf16(fmt, w_bits, M, K)
    w = oracle.bf16_to_f64(w_bits).reshape(M, K)
    w_hat = oracle.dequantize(fmt, codes, d_bits, K)
    d = np.repeat(np.abs(oracle.f16_to_f64(d_bits)).reshape(M, K // G), G, axis=1)
    err = np.abs(w - w_hat)
    if fmt in (synth.INT8_G32, synth.INT8_ROW):
        return bool((err <= d / 2).all())
    q = oformats.decode_nibble_blocks(codes.reshape(M, K // G, G // 2), G)
    ok_regular = (err <= d / 2) | ((q == 15) & (err <= d * (1 + 2 ** -8)))
    wg = w.reshape(M, K // G, G)
    idx = np.argmax(np.abs(wg), axis=2)
    qg = q.reshape(M, K // G, G)
    q_at_max = np.take_along_axis(qg, idx[..., None], axis=2)[..., 0]
    m_val = np.take_along_axis(wg, idx[..., None], axis=2)[..., 0]
    mh = np.take_along_axis(w_hat.reshape(M, K // G, G), idx[..., None], axis=2)[..., 0]
    nz = m_val != 0
    return bool(ok_regular.all() and (q_at_max[nz] == 0).all()
                and (np.abs(mh - m_val) <= np.abs(m_val) * 2 ** -11).all())


@pytest.mark.parametrize("fmt", FMTS_Q)
def test_quantize_roundtrip_within_format_error(fmt):
    """bf16 weights ~ N(0, 0.02^2) at the 2048x2048 shape, each quantized format."""
    rng = np.random.default_rng(123)
    w_bits = synth.bf16_normal(rng, (2048, 2048), 0.02)
    assert _quant_bounds_ok(fmt, w_bits, 2048, 2048)


def test_quantize_positive_max_maps_to_minus8():
    """Largest magnitude positive: signed rule maps it to code 0 exactly, where the
    largest-|w|/8 rule would have clipped it to +7 (a 12.5 % error)."""
    K = 32
    vals = np.zeros(K, dtype=np.float32)
    vals[:8] = [0.5, -0.25, 0.125, 0.0, 0.75, -0.5, 0.25, 0.375]
    w_bits = synth.round_f32_to_bf16_bits(vals[None, :])
    codes, d_bits = oracle.quantize_from_bf16(synth.Q4_0_G32, w_bits, 1, K)
    d = oracle.f16_to_f64(d_bits)[0, 0]
    assert d == -0.09375                           # 0.75 / -8, exact in binary16
    lo = codes[0, 0] & 0xF
    assert lo[4] == 0                              # 0.75 -> code 0 -> -8 * d = 0.75
    w_hat = oracle.dequantize(synth.Q4_0_G32, codes, d_bits, K)[0]
    assert w_hat[4] == 0.75
    # every element of this group is an exact multiple of d/... within d/2
    assert (np.abs(w_hat - vals.astype(np.float64)) <= abs(d) / 2 + 1e-12).all()


def test_quantize_special_groups():
    K = 32
    z = np.zeros((1, K), dtype=np.uint16)
    for fmt, zero_code in ((synth.Q4_0_G32, 0x88), (synth.INT8_G32, 0), (synth.INT4_G64, 0x88),
                           (synth.INT8_ROW, 0)):
        codes, d_bits = oracle.quantize_from_bf16(fmt, np.zeros((1, 64), dtype=np.uint16), 1, 64)
        assert (d_bits == 0).all()
        assert (codes.view(np.uint8) == np.uint8(zero_code)).all()
    # tie in |w| between +a and -a: the first in index order sets the sign of d
    vals = np.zeros((1, K), dtype=np.float32)
    vals[0, 3], vals[0, 9] = -0.5, 0.5
    codes, d_bits = oracle.quantize_from_bf16(synth.Q4_0_G32, synth.round_f32_to_bf16_bits(vals), 1, K)
    assert oracle.f16_to_f64(d_bits)[0, 0] == 0.0625   # -0.5 / -8
    assert (codes[0, 0, 3] & 0xF) == 0                  # -0.5 -> code 0
    assert (codes[0, 0, 9] & 0xF) == 15                 # +0.5 / 0.0625 = 8 -> clamped to 15
    # overflow of the binary16 scale is an error
    big = synth.round_f32_to_bf16_bits(np.full((1, K), 1e6, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_from_bf16(synth.Q4_0_G32, big, 1, K)
    inf = np.full((1, K), 0x7F80, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.quantize_from_bf16(synth.INT8_G32, inf, 1, K)


# ------------------------------------------------------------------ argmax
def _argmax_ok() -> bool:
    rng = np.random.default_rng(5)
    cases = [rng.standard_normal((4, 1000)).astype(np.float32),
             synth.f32_logits_with_ties(rng, 3, 4097)]
    t = np.zeros((1, 10), np.float32); t[0, 4] = -0.0; t[0, 2] = 0.0
    t[0, :] = -1.0; t[0, 2] = 0.0; t[0, 4] = -0.0; cases.append(t)      # -0.0 ties +0.0
    cases.append(np.full((1, 7), -np.inf, np.float32))                  # all -inf -> 0
    n = rng.standard_normal((2, 50)).astype(np.float32); n[0, 17] = np.nan; n[0, 30] = np.nan
    n[1, 3] = np.inf; cases.append(n)
    for c in cases:
        if not (oracle.argmax_ref(c) == np.argmax(c, axis=1)).all():
            return False
    return True


def test_argmax_matches_numpy_semantics():
    assert _argmax_ok()
    a = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    assert oracle.argmax_ref(a)[0] == 1
    a = np.array([[-0.0, 0.0]], np.float32)
    assert oracle.argmax_ref(a)[0] == 0


# -------------------------------------------------------------- tolerance
def test_parity_check_definition():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    a_ref = np.array([[10.0, 4.0, 0.0]])
    assert oracle.check_parity(y_ref.copy(), y_ref, a_ref)
    # bound = 1e-3 * a + 1e-5
    ok = y_ref + np.array([[0.010009, -0.004009, 0.0000099]])
    assert oracle.check_parity(ok, y_ref, a_ref)
    bad = y_ref + np.array([[0.010011, 0.0, 0.0]])
    assert not oracle.check_parity(bad, y_ref, a_ref)
    assert not oracle.check_parity(np.array([[np.nan, -2.0, 0.0]]), y_ref, a_ref)
    assert not oracle.check_parity(np.array([[np.inf, -2.0, 0.0]]), y_ref, a_ref)


# ------------------------------------------------------------ generators
def test_generators_deterministic():
    a = synth.make_gemv("o", synth.Q4_0_G32, 64, 2048, 2, 2, 0, "o")
    b = synth.make_gemv("o", synth.Q4_0_G32, 64, 2048, 2, 2, 0, "o")
    c = synth.make_gemv("o", synth.Q4_0_G32, 64, 2048, 2, 2, 1, "o")
    assert (a.w == b.w).all() and (a.s == b.s).all() and (a.x == b.x).all()
    assert not (a.w == c.w).all()
    assert a.seeds == (2_000_010, 2_000_011, 2_000_012)
    d = oracle.f16_to_f64(a.s)
    assert d.min() >= 0.000999 and d.max() <= 0.005
    i8 = synth.make_gemv("o", synth.INT8_G32, 8, 2048, 1, 3, 0, "o")
    assert i8.w.min() >= -127 and i8.w.max() <= 127


# ------------------------------------------------------- planted mistakes
def _all_pins_pass() -> bool:
    try:
        if not all(_check_hand_case(c) for c in HAND):
            return False
        if not _brute_force_ok(synth.INT4_G128, 2, 256, 2, 3):
            return False
        if not _brute_force_ok(synth.BF16, 2, 64, 2, 4):
            return False
        for fmt in FMTS_Q:
            rng = np.random.default_rng(fmt)
            if not _quant_bounds_ok(fmt, synth.bf16_normal(rng, (16, 256), 0.02), 16, 256):
                return False
        return _argmax_ok()
    except Exception:
        return False


def _mut_swap_nibbles(codes, group):
    c = np.asarray(codes, dtype=np.uint8)
    M, nb, half = c.shape
    lo = (c & 0x0F).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    return np.concatenate([hi, lo], axis=2).reshape(M, nb * group)


def _mut_interleave_nibbles(codes, group):
    c = np.asarray(codes, dtype=np.uint8)
    M, nb, half = c.shape
    lo = (c & 0x0F).astype(np.int64)
    hi = (c >> 4).astype(np.int64)
    return np.stack([lo, hi], axis=3).reshape(M, nb * group)


def _wrap_dequant(offset=0, roll_scales=False, neg=False):
    orig = oformats.dequantize

    def f(fmt, w, s, K):
        if roll_scales and s is not None:
            s = np.roll(np.asarray(s), 1, axis=-1)
        out = orig(fmt, w, s, K)
        if fmt in (synth.Q4_0_G32, synth.INT4_G128, synth.INT4_G64) and offset:
            G = synth.GROUP[fmt]
            d = np.repeat(oformats.f16_to_f64(s).reshape(out.shape[0], K // G), G, axis=1)
            out = out + offset * d
        return -out if neg else out
    return f


_orig_gemv = ogemv.gemv_ref
_orig_f16 = oformats.f16_to_f64
_orig_quant = oquant.quantize_from_bf16


def _mut_gemv_x_reversed(fmt, w, s, x_bits, M, K, rows=None, chunk_rows=1024):
    x_bits = np.asarray(x_bits).reshape(-1, K)[:, ::-1]
    return _orig_gemv(fmt, w, s, x_bits, M, K, rows, chunk_rows)


def _mut_gemv_abs_dropped(*a, **k):
    y, _ = _orig_gemv(*a, **k)
    return y, np.abs(y)


def _mut_f16_double(bits):
    return _orig_f16(bits) * 2.0


def _mut_quant_amax8(fmt, w_bits, M, K):
    """The unsigned largest-|w|/8 scale, which clips positive maxima to +7."""
    G = synth.GROUP[fmt]
    if fmt in (synth.INT8_G32, synth.INT8_ROW):
        return _orig_quant(fmt, w_bits, M, K)
    w = oformats.bf16_to_f64(np.asarray(w_bits).reshape(M, K)).reshape(M, K // G, G)
    d_bits = oformats.f64_to_f16_bits(np.abs(w).max(axis=2) / 8.0)
    d = oformats.f16_to_f64(d_bits)[..., None]
    q = np.clip(np.rint(w / np.where(d == 0, 1, d)) + 8, 0, 15).astype(np.uint8)
    half = G // 2
    return (q[..., :half] | (q[..., half:] << 4)).astype(np.uint8), d_bits


def _mut_argmax_last_tie(a):
    a = np.asarray(a, dtype=np.float32)
    a = a[None, :] if a.ndim == 1 else a
    return (a.shape[1] - 1 - np.argmax(a[:, ::-1], axis=1)).astype(np.int32)


MUTANTS = {
    "swap_lo_hi_nibbles": [(oformats, "decode_nibble_blocks", _mut_swap_nibbles)],
    "interleaved_nibbles": [(oformats, "decode_nibble_blocks", _mut_interleave_nibbles)],
    "offset_minus7": [(ogemv, "dequantize", _wrap_dequant(offset=1)),
                      (oracle, "dequantize", _wrap_dequant(offset=1))],
    "wrong_group_scale": [(ogemv, "dequantize", _wrap_dequant(roll_scales=True))],
    "sign_flip": [(ogemv, "dequantize", _wrap_dequant(neg=True))],
    "x_reversed": [(oracle, "gemv_ref", _mut_gemv_x_reversed)],
    "abs_sum_dropped": [(oracle, "gemv_ref", _mut_gemv_abs_dropped)],
    "f16_scale_doubled": [(oformats, "f16_to_f64", _mut_f16_double),
                          (oracle, "f16_to_f64", _mut_f16_double),
                          (oquant, "f16_to_f64", _mut_f16_double)],
    "quant_unsigned_amax8": [(oracle, "quantize_from_bf16", _mut_quant_amax8)],
    "argmax_last_tie": [(oracle, "argmax_ref", _mut_argmax_last_tie)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(monkeypatch, name):
    assert _all_pins_pass()
    for mod, attr, repl in MUTANTS[name]:
        monkeypatch.setattr(mod, attr, repl)
    assert not _all_pins_pass(), f"planted mistake {name} went unnoticed"


# ------------------------------------------- chunked rows and row subsets
# gemv_ref walks the output rows in chunks of chunk_rows (1024 by default)
# and can be asked for any subset of rows; every GPU parity test on a matrix
# taller than one chunk goes through that slicing. These pins compare it,
# row by row, with the exact rational brute force above on matrices taller
# than one chunk and on scattered, unsorted, repeated row subsets.
def _brute_rows(fmt, g, K, rows):
    """Exact (y, a) as Fractions for the listed rows of a generated case."""
    B = g.x.shape[0]
    xs = [[_frac_bf16(g.x[b, k]) for k in range(K)] for b in range(B)]
    ys, As = [], []
    for m in rows:
        wts = [_brute_weight(fmt, g.w, g.s, int(m), k, K) for k in range(K)]
        ys.append([sum((wts[k] * xs[b][k] for k in range(K)), Fraction(0)) for b in range(B)])
        As.append([sum((abs(wts[k] * xs[b][k]) for k in range(K)), Fraction(0)) for b in range(B)])
    return ys, As


def _rows_agree(y, a, ys, As, K) -> bool:
    for i, (yr, ar) in enumerate(zip(ys, As)):
        for b in range(len(yr)):
            tol = Fraction(K) * Fraction(2) ** -52 * ar[b]
            if abs(Fraction(float(y[b, i])) - yr[b]) > tol or abs(Fraction(float(a[b, i])) - ar[b]) > tol:
                return False
    return True


def _chunk_pins_ok() -> bool:
    # 2100 rows: two full 1024-row chunks and a 52-row tail; every row checked
    for fmt, K in ((synth.Q4_0_G32, 32), (synth.INT8_G32, 32)):
        M = 2100
        g = synth.make_gemv("t", fmt, M, K, 2, cfg=9, layer=40 + fmt, proj="o")
        y, a = oracle.gemv_ref(fmt, g.w, g.s, g.x, M, K)
        if y.shape != (2, M) or not _rows_agree(y, a, *_brute_rows(fmt, g, K, range(M)), K):
            return False
    # small chunks with a ragged last chunk, and a scattered, unsorted row
    # subset with repeats that crosses chunk boundaries
    rng = np.random.default_rng(41)
    for fmt, K, M in ((synth.INT4_G128, 128, 50), (synth.INT8_ROW, 64, 50), (synth.BF16, 32, 50)):
        g = synth.make_gemv("t", fmt, M, K, 2, cfg=9, layer=50 + fmt, proj="o")
        y, a = oracle.gemv_ref(fmt, g.w, g.s, g.x, M, K, chunk_rows=7)
        if not _rows_agree(y, a, *_brute_rows(fmt, g, K, range(M)), K):
            return False
        rows = np.concatenate([rng.permutation(M)[:23], [0, M - 1, 7, 7]])
        y, a = oracle.gemv_ref(fmt, g.w, g.s, g.x, M, K, rows=rows, chunk_rows=5)
        if y.shape != (2, rows.size) or not _rows_agree(y, a, *_brute_rows(fmt, g, K, rows), K):
            return False
    # the chunking changes nothing: one chunk and many chunks give equal bits
    g = synth.make_gemv("t", synth.Q4_0_G32, 300, 256, 3, cfg=9, layer=60, proj="o")
    y1, a1 = oracle.gemv_ref(synth.Q4_0_G32, g.w, g.s, g.x, 300, 256, chunk_rows=300)
    y2, a2 = oracle.gemv_ref(synth.Q4_0_G32, g.w, g.s, g.x, 300, 256, chunk_rows=13)
    return bool((y1 == y2).all() and (a1 == a2).all())


def test_chunked_rows_and_row_subsets_brute_force():
    assert _chunk_pins_ok()


_orig_row_slice = ogemv._row_slice


def _mut_chunk_off_by_one(fmt, w, s, x_bits, M, K, rows=None, chunk_rows=1024):
    """Chunks that step one row too far: the first row of every later chunk
    is never computed (and the tail reads one row short)."""
    x = oformats.bf16_to_f64(np.asarray(x_bits).reshape(-1, K))
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    y = np.zeros((x.shape[0], rows.size)); a = np.zeros_like(y)
    for c0 in range(0, rows.size, chunk_rows + 1):
        r = rows[c0:c0 + chunk_rows]
        wr, sr = _orig_row_slice(fmt, w, s, M, K, r)
        Wh = oformats.dequantize(fmt, wr, sr, K)
        y[:, c0:c0 + r.size] = (Wh @ x.T).T
        a[:, c0:c0 + r.size] = (np.abs(Wh) @ np.abs(x).T).T
    return y, a


def _mut_scales_chunk_relative(fmt, w, s, M, K, rows):
    """Scale rows indexed relative to the chunk instead of the matrix."""
    wr, _ = _orig_row_slice(fmt, w, s, M, K, rows)
    if s is None:
        return wr, None
    sr = np.asarray(s).reshape(M, -1)[np.asarray(rows) - np.asarray(rows).min()]
    return wr, sr


def _mut_scales_sorted_rows(fmt, w, s, M, K, rows):
    """Scale rows taken in sorted order while the codes keep the requested order."""
    wr, _ = _orig_row_slice(fmt, w, s, M, K, rows)
    if s is None:
        return wr, None
    return wr, np.asarray(s).reshape(M, -1)[np.sort(np.asarray(rows))]


def _mut_rows_ignored(fmt, w, s, x_bits, M, K, rows=None, chunk_rows=1024):
    """A subset request answered with the first len(rows) rows."""
    n = M if rows is None else len(rows)
    return _orig_gemv(fmt, w, s, x_bits, M, K, None if rows is None else np.arange(n), chunk_rows)


CHUNK_MUTANTS = {
    "chunk_step_off_by_one": [(oracle, "gemv_ref", _mut_chunk_off_by_one)],
    "scale_rows_chunk_relative": [(ogemv, "_row_slice", _mut_scales_chunk_relative)],
    "scale_rows_sorted": [(ogemv, "_row_slice", _mut_scales_sorted_rows)],
    "row_subset_ignored": [(oracle, "gemv_ref", _mut_rows_ignored)],
}


@pytest.mark.parametrize("name", sorted(CHUNK_MUTANTS))
def test_chunk_planted_mistakes_are_caught(monkeypatch, name):
    assert _chunk_pins_ok()
    for mod, attr, repl in CHUNK_MUTANTS[name]:
        monkeypatch.setattr(mod, attr, repl)
    try:
        caught = not _chunk_pins_ok()
    except Exception:
        caught = True
    assert caught, f"planted mistake {name} went unnoticed"
