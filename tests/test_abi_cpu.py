"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

* the library loads and exports every function qgemv.h declares;
* qgemv_packed_size reproduces the byte accounting printed on the infer page;
* qgemv_pack: canonical copy round-trip, and the bf16 quantizer is
  bit-identical to the oracle's quantizer;
* every validation error is returned before any HIP call.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import bandwidth_bound_quantized_amd as qg
import oracle
import synth
from helpers import load_json

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 8
    lib = ctypes.CDLL(qg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in qgemv.h but not exported"
    assert set(names) == set(qg.EXPORTS)
    assert "gfx950" in qg.version()


def test_status_strings():
    for st in (qg.OK, qg.EINVAL, qg.ESHAPE, qg.EALIGN, qg.ERANGE, qg.EHIP):
        assert qg.lib().qgemv_status_str(st).decode().startswith("QGEMV")


# -------------------------------------------------------- byte accounting
ACC = load_json("page_byte_accounting.json")


def _bytes(fmt, M, K, scales=True):
    w, s = qg.packed_size(fmt, M, K)
    return w + (s if scales else 0)


def test_packed_sizes_basic():
    assert qg.packed_size(qg.BF16, 2048, 2048) == (8388608, 0)
    assert qg.packed_size(qg.Q4_0_G32, 2048, 2048) == (2097152, 262144)   # 4.5 bits/weight
    assert qg.packed_size(qg.INT8_G32, 3072, 2048) == (6291456, 393216)
    assert qg.packed_size(qg.INT4_G128, 16384, 2048) == (16777216, 524288)
    assert qg.packed_size(qg.INT8_ROW, 128256, 2048) == (262668288, 256512)   # one scale per row
    assert qg.packed_size(qg.INT4_G64, 2048, 2048) == (2097152, 131072)      # 4.25 bits/weight


def test_per_token_totals_match_infer_decode_table():
    L = ACC["llama32_1b"]
    layer = L["layer_gemvs"]
    head = L["lm_head"]
    n = L["layers"]

    def total(fmt, head_fmt=None, scales=True):
        t = n * sum(_bytes(fmt, M, K, scales) for _, M, K in layer)
        return t + _bytes(head_fmt if head_fmt is not None else fmt, *head, scales)

    want = ACC["weights_per_token_GB"]
    assert round(total(qg.BF16) / 1e9, 2) == want["bf16"]
    assert round(total(qg.INT8_G32, scales=False) / 1e9, 2) == want["int8_codes_only"]
    assert round(total(qg.INT8_ROW) / 1e9, 2) == want["int8_codes_only"]      # infer's int8: per-row scales
    assert round(total(qg.Q4_0_G32) / 1e9, 2) == want["int4_g32"]
    assert round(total(qg.INT4_G128) / 1e9, 2) == want["int4_g128"]
    mixed = n * sum(_bytes(qg.Q4_0_G32, M, K) for _, M, K in layer) + _bytes(qg.INT8_ROW, *head)
    assert round(mixed / 1e9, 2) == want["int4_g32_int8_head"]


def test_quantized_gemv_table_percentages_reproduce():
    peak = ACC["measured_peak_GBps"]
    for name, M, K, us4, pct4, us8, pct8 in ACC["quantized_gemv_table"]["rows"]:
        b4 = _bytes(qg.Q4_0_G32, M, K)                 # 18 bytes per 32 weights
        b8 = _bytes(qg.INT8_ROW, M, K)                 # per-row int8: 1 byte per weight + 2 per row
        assert abs(b4 / us4 / 1e3 / peak * 100 - pct4) <= 1.0, name
        assert abs(b8 / us8 / 1e3 / peak * 100 - pct8) <= 1.0, name
    for name, M, K, us, gbps, pct in ACC["bf16_gemv_table"]["rows"]:
        b = _bytes(qg.BF16, M, K)
        assert abs(b / us / 1e3 - gbps) / gbps <= 0.01, name
        assert abs(b / us / 1e3 / peak * 100 - pct) <= 1.0, name


# ------------------------------------------------------------------ pack
@pytest.mark.parametrize("fmt", [qg.BF16, qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64])
def test_pack_canonical_roundtrip(fmt):
    g = synth.make_gemv("t", fmt, 37, 256, 1, 9, 1, "o")
    w, s = qg.pack(fmt, qg.SRC_CANONICAL, g.w, g.s, 37, 256)
    assert (w == g.w.reshape(-1).view(np.uint8)).all()
    if fmt != qg.BF16:
        assert (s == g.s.reshape(-1)).all()


def _quant_inputs():
    rng = np.random.default_rng(99)
    w = synth.bf16_normal(rng, (64, 512), 0.02)
    # edge groups: all zero, exact ties of +-a, a positive maximum, tiny values,
    # values whose scale is an f16 subnormal, and a large-but-representable group
    w[0, :128] = 0
    w[1, :32] = synth.round_f32_to_bf16_bits(np.zeros(32, np.float32))
    t = np.zeros(32, np.float32); t[3] = -0.5; t[9] = 0.5
    w[2, :32] = synth.round_f32_to_bf16_bits(t)
    t = np.linspace(-0.3, 0.75, 32).astype(np.float32)
    w[3, 32:64] = synth.round_f32_to_bf16_bits(t)
    w[4, :32] = synth.round_f32_to_bf16_bits(np.full(32, 1e-9, np.float32))
    w[5, :32] = synth.round_f32_to_bf16_bits(np.linspace(-3e-5, 2e-5, 32).astype(np.float32))
    w[6, :128] = synth.round_f32_to_bf16_bits(np.linspace(-500000, 400000, 128).astype(np.float32))
    w[7, :64] = synth.round_f32_to_bf16_bits(np.arange(64).astype(np.float32) * 0.0625 - 2.0)
    return w


@pytest.mark.parametrize("fmt", [qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64])
def test_pack_bf16_quantizer_bit_exact_vs_oracle(fmt):
    w = _quant_inputs()
    M, K = w.shape
    codes, scales = qg.pack(fmt, qg.SRC_BF16, w, None, M, K)
    o_codes, o_scales = oracle.quantize_from_bf16(fmt, w, M, K)
    assert (scales == o_scales.reshape(-1)).all()
    assert (codes == o_codes.reshape(-1).view(np.uint8)).all()


@pytest.mark.parametrize("fmt", [qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64])
def test_pack_bf16_quantizer_bit_exact_config1_shape(fmt):
    rng = np.random.default_rng(fmt + 1000)
    w = synth.bf16_normal(rng, (2048, 2048), 0.02)
    codes, scales = qg.pack(fmt, qg.SRC_BF16, w, None, 2048, 2048)
    o_codes, o_scales = oracle.quantize_from_bf16(fmt, w, 2048, 2048)
    assert (scales == o_scales.reshape(-1)).all()
    assert (codes == o_codes.reshape(-1).view(np.uint8)).all()


def test_pack_range_errors():
    w = np.full((1, 32), 0x7F80, dtype=np.uint16)            # +inf
    with pytest.raises(qg.QgemvError) as e:
        qg.pack(qg.Q4_0_G32, qg.SRC_BF16, w, None, 1, 32)
    assert e.value.status == qg.ERANGE
    big = synth.round_f32_to_bf16_bits(np.full((1, 32), 1e7, np.float32))   # scale > 65504
    with pytest.raises(qg.QgemvError) as e:
        qg.pack(qg.INT8_G32, qg.SRC_BF16, big, None, 1, 32)
    assert e.value.status == qg.ERANGE


# ------------------------------------------------------------ validation
FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MIS = 0x10002


def _run(fmt=qg.Q4_0_G32, W=FAKE, S=FAKE, x=FAKE, y=FAKE, M=64, K=2048, batch=1):
    return qg.lib().qgemv_run(fmt, W, S, x, y, M, K, batch, None)


def _run_flags(flags, fmt=qg.Q4_0_G32, M=64, K=2048, batch=1):
    return qg.lib().qgemv_run_flags(fmt, FAKE, FAKE, FAKE, FAKE, M, K, batch, flags, None)


def test_run_flags_validation_errors_before_any_launch():
    assert _run_flags(2) == qg.EINVAL                        # unknown flag bit
    assert _run_flags(-1) == qg.EINVAL
    assert _run_flags(qg.FLAG_BATCH_INVARIANT, batch=0) == qg.ESHAPE
    assert _run_flags(qg.FLAG_BATCH_INVARIANT, batch=9) == qg.ESHAPE
    # the invariant mode stages x as 8 rows at every batch: K that batch 1
    # takes can be too long for it
    assert _run_flags(qg.FLAG_BATCH_INVARIANT, fmt=qg.BF16, K=10272, batch=1) == qg.ESHAPE
    assert _run_flags(qg.FLAG_BATCH_INVARIANT, fmt=qg.Q4_0_G32, K=9664, batch=1) == qg.ESHAPE


def _fused(fmt=qg.Q4_0_G32, x=FAKE, y=FAKE, M=64, K=2048, batch=1, **kw):
    f = qg.Fusion()
    for k, v in kw.items():
        setattr(f, k, v)
    return qg.lib().qgemv_run_fused(fmt, FAKE, FAKE, x, y, M, K, batch, ctypes.byref(f), None)


def test_run_fused_validation_errors_before_any_launch():
    assert qg.lib().qgemv_run_fused(qg.Q4_0_G32, FAKE, FAKE, FAKE, FAKE, 64, 2048, 1, None, None) == qg.EINVAL
    assert _fused(x=None) == qg.EINVAL                                  # no input at all
    assert _fused(norm_input=FAKE, norm_weight=FAKE) == qg.EINVAL       # x and norm_input
    assert _fused(x=None, norm_input=FAKE) == qg.EINVAL                 # no norm weight
    assert _fused(x=None, norm_input=FAKE, norm_weight=FAKE, norm_eps=-1.0) == qg.EINVAL
    assert _fused(x=None, norm_input=FAKE, norm_weight=FAKE, norm_eps=float("nan")) == qg.EINVAL
    assert _fused(swiglu_out=FAKE) == qg.EINVAL                         # swiglu with y
    assert _fused(y=None) == qg.EINVAL                                  # no output
    assert _fused(y=None, swiglu_out=FAKE, residual=FAKE) == qg.EINVAL
    assert _fused(y=None, swiglu_out=FAKE, argmax_idx=FAKE, argmax_ws=FAKE) == qg.EINVAL
    assert _fused(argmax_idx=FAKE) == qg.EINVAL                         # idx without ws
    assert _fused(y=None, swiglu_out=FAKE, M=63) == qg.ESHAPE           # odd M
    assert _fused(batch=9) == qg.ESHAPE
    assert _fused(K=48) == qg.ESHAPE
    # x plus the prologue's scratch must fit in LDS where x is staged there
    assert _fused(fmt=qg.BF16, batch=5, K=10240) == qg.ESHAPE
    assert _fused(x=None, norm_input=FAKE + 4, norm_weight=FAKE) == qg.EALIGN
    assert _fused(residual=FAKE + 4) == qg.EALIGN
    assert _fused(y=None, swiglu_out=FAKE + 2) == qg.EALIGN
    assert _fused(argmax_idx=FAKE, argmax_ws=FAKE + 4) == qg.EALIGN


def test_attention_workspace_and_validation():
    L = qg.lib()
    n = ctypes.c_size_t()
    # Llama-3.2-1B heads (G = 4, head dim 64). Batch 1 at context 2048 is a small call
    # (batch x KV heads x context <= 65536): blocks of 16 positions, 4 waves per split,
    # 2048 / 64 = 32 splits per key/value head, each record 2G + G*D floats
    assert L.qgemv_attention_workspace_size(1, 32, 8, 64, 2048, ctypes.byref(n)) == qg.OK
    assert n.value == 8 * 32 * (2 * 4 + 4 * 64) * 4
    # ... at context 1024: 16 splits
    assert L.qgemv_attention_workspace_size(1, 32, 8, 64, 1024, ctypes.byref(n)) == qg.OK
    assert n.value == 8 * 16 * (2 * 4 + 4 * 64) * 4
    # batch 8 at context 2048 is not small: blocks of 32 positions (128 per split), and
    # the splits stop at about 256 workgroups: 256 / (8 x 8) = 4 per key/value head
    assert L.qgemv_attention_workspace_size(8, 32, 8, 64, 2048, ctypes.byref(n)) == qg.OK
    assert n.value == 8 * 8 * 4 * (2 * 4 + 4 * 64) * 4
    # one split (a context within one split of 4 x 16 positions): no records, the
    # 256-byte minimum; 128 positions are two splits
    assert L.qgemv_attention_workspace_size(1, 32, 8, 64, 64, ctypes.byref(n)) == qg.OK
    assert n.value == 256
    assert L.qgemv_attention_workspace_size(1, 32, 8, 64, 128, ctypes.byref(n)) == qg.OK
    assert n.value == 8 * 2 * (2 * 4 + 4 * 64) * 4
    assert L.qgemv_attention_workspace_size(1, 32, 8, 64, 2048, None) == qg.EINVAL
    for args in ((1, 24, 8, 64, 2048), (1, 32, 8, 96, 2048), (1, 32, 8, 64, 0), (0, 32, 8, 64, 16),
                 (1, 32, 0, 64, 16), (1, 32, 8, 128, 1 << 24)):
        assert L.qgemv_attention_workspace_size(*args, ctypes.byref(n)) == qg.ESHAPE, args

    def call(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, scale=0.125, ws=FAKE, n_q=32, d=64):
        return L.qgemv_attention_decode(q, k, v, lens, out, 1, n_q, 8, d, 2048, scale, ws, None)
    assert call(q=None) == qg.EINVAL
    assert call(ws=None) == qg.EINVAL
    assert call(scale=0.0) == qg.EINVAL
    assert call(scale=float("inf")) == qg.EINVAL
    assert call(n_q=12) == qg.ESHAPE
    assert call(d=80) == qg.ESHAPE
    assert call(q=FAKE + 4) == qg.EALIGN
    assert call(lens=FAKE + 2) == qg.EALIGN


def test_run_validation_errors_before_any_launch():
    assert _run(fmt=7) == qg.EINVAL
    assert _run(W=None) == qg.EINVAL
    assert _run(x=None) == qg.EINVAL
    assert _run(y=None) == qg.EINVAL
    assert _run(S=None) == qg.EINVAL
    assert _run(M=0) == qg.ESHAPE
    assert _run(K=48) == qg.ESHAPE
    assert _run(fmt=6) == qg.EINVAL
    assert _run(fmt=qg.INT4_G64, K=2048 + 32) == qg.ESHAPE             # K a multiple of 64
    assert _run(fmt=qg.INT4_G128, K=2048 + 32) == qg.ESHAPE
    assert _run(batch=0) == qg.ESHAPE
    assert _run(batch=9) == qg.ESHAPE
    assert _run(K=1 << 20) == qg.ESHAPE                 # x does not fit in LDS
    assert _run(fmt=qg.Q4_0_G32, batch=8, K=9664) == qg.ESHAPE      # 8*9664*2.125 > 160 KiB
    assert _run(fmt=qg.BF16, batch=5, K=10272) == qg.ESHAPE         # rounds up to 8 rows
    assert _run(W=MIS) == qg.EALIGN
    assert _run(x=FAKE + 8) == qg.EALIGN
    assert _run(y=FAKE + 4) == qg.EALIGN
    assert _run(S=FAKE + 2) == qg.EALIGN


def test_argmax_and_stream_read_validation():
    L = qg.lib()
    assert L.qgemv_argmax(None, 10, 1, FAKE, FAKE, None) == qg.EINVAL
    assert L.qgemv_argmax(FAKE, 0, 1, FAKE, FAKE, None) == qg.ESHAPE
    assert L.qgemv_argmax(FAKE, 1 << 31, 1, FAKE, FAKE, None) == qg.ESHAPE
    assert L.qgemv_argmax(FAKE, 10, 9, FAKE, FAKE, None) == qg.ESHAPE
    assert L.qgemv_argmax(FAKE + 2, 10, 1, FAKE, FAKE, None) == qg.EALIGN
    assert L.qgemv_argmax(FAKE, 10, 1, FAKE + 4, FAKE, None) == qg.EALIGN
    # the no-allocation argmax rejects a batch beyond its static workspace before any HIP call
    assert L.qgemv_argmax_noalloc(None, 10, 1, FAKE, None) == qg.EINVAL
    assert L.qgemv_argmax_noalloc(FAKE, 10, 1, None, None) == qg.EINVAL
    assert L.qgemv_argmax_noalloc(FAKE, 0, 1, FAKE, None) == qg.ESHAPE
    assert L.qgemv_argmax_noalloc(FAKE, 10, 0, FAKE, None) == qg.ESHAPE
    assert L.qgemv_argmax_noalloc(FAKE, 10, 9, FAKE, None) == qg.ESHAPE
    assert L.qgemv_argmax_noalloc(FAKE + 2, 10, 1, FAKE, None) == qg.EALIGN
    assert L.qgemv_argmax_noalloc(FAKE, 10, 1, FAKE + 1, None) == qg.EALIGN
    assert L.qgemv_stream_read(FAKE, 0, FAKE, 0, 4, None) == qg.ESHAPE
    assert L.qgemv_stream_read(FAKE, 24, FAKE, 0, 4, None) == qg.ESHAPE
    assert L.qgemv_stream_read(FAKE, 32, FAKE, 0, 3, None) == qg.EINVAL
    assert L.qgemv_stream_read(FAKE + 8, 32, FAKE, 0, 4, None) == qg.EALIGN


def test_pack_validation():
    L = qg.lib()
    buf = np.zeros(1 << 16, np.uint8)
    p = buf.ctypes.data
    assert L.qgemv_pack(9, 0, p, p, 1, 32, p, p) == qg.EINVAL
    assert L.qgemv_pack(qg.Q4_0_G32, 5, p, p, 1, 32, p, p) == qg.EINVAL
    assert L.qgemv_pack(qg.Q4_0_G32, 0, p, None, 1, 32, p, p) == qg.EINVAL
    assert L.qgemv_pack(qg.Q4_0_G32, 0, p, p, 1, 32, p, None) == qg.EINVAL
    assert L.qgemv_pack(qg.Q4_0_G32, 0, p, p, 1, 40, p, p) == qg.ESHAPE
    assert L.qgemv_pack(qg.INT4_G128, 0, p, p, 1, 64, p, p) == qg.ESHAPE
    w = ctypes.c_size_t(); s = ctypes.c_size_t()
    assert L.qgemv_packed_size(qg.BF16, 0, 32, ctypes.byref(w), ctypes.byref(s)) == qg.ESHAPE
    assert L.qgemv_packed_size(qg.BF16, 1, 32, None, ctypes.byref(s)) == qg.EINVAL


def test_grouped_validation_errors_before_any_launch():
    L = qg.lib()
    good = dict(fmt=qg.Q4_0_G32, M=64, K=2048)

    def descs(*entries):
        arr = (qg.GemvDesc * len(entries))()
        for i, e in enumerate(entries):
            d = dict(W=FAKE, scales=FAKE, x=FAKE, y=FAKE, fmt=good["fmt"], M=good["M"], K=good["K"], reserved=0)
            d.update(e)
            arr[i] = qg.GemvDesc(**d)
        return arr

    assert L.qgemv_run_grouped(None, 1, 1, None) == qg.EINVAL
    a = descs({})
    assert L.qgemv_run_grouped(ctypes.cast(a, ctypes.c_void_p), 0, 1, None) == qg.EINVAL
    assert L.qgemv_run_grouped(ctypes.cast(a, ctypes.c_void_p), 1, 0, None) == qg.ESHAPE
    assert L.qgemv_run_grouped(ctypes.cast(a, ctypes.c_void_p), 1, 9, None) == qg.ESHAPE
    big = descs(*([{}] * 2))
    assert L.qgemv_run_grouped(ctypes.cast(big, ctypes.c_void_p), 1025, 1, None) == qg.ESHAPE
    # one bad entry anywhere in the list rejects the whole call
    for bad, want in [({"W": None}, qg.EINVAL), ({"fmt": 9}, qg.EINVAL), ({"K": 48}, qg.ESHAPE),
                      ({"y": FAKE + 4}, qg.EALIGN), ({"scales": None}, qg.EINVAL), ({"M": 0}, qg.ESHAPE)]:
        arr = descs({}, {}, bad, {})
        assert L.qgemv_run_grouped(ctypes.cast(arr, ctypes.c_void_p), 4, 1, None) == want, bad


def test_grouped_class_validation():
    """qgemv_grouped_class rejects what qgemv_run_grouped would reject, before it
    looks at the device."""
    L = qg.lib()
    assert L.qgemv_grouped_class(9, 2048, 1) == qg.EINVAL
    assert L.qgemv_grouped_class(-1, 2048, 1) == qg.EINVAL
    assert L.qgemv_grouped_class(qg.Q4_0_G32, 48, 1) == qg.ESHAPE
    assert L.qgemv_grouped_class(qg.INT4_G128, 64, 1) == qg.ESHAPE
    assert L.qgemv_grouped_class(qg.Q4_0_G32, 0, 1) == qg.ESHAPE
    assert L.qgemv_grouped_class(qg.Q4_0_G32, 2048, 0) == qg.ESHAPE
    assert L.qgemv_grouped_class(qg.Q4_0_G32, 2048, 9) == qg.ESHAPE
    with pytest.raises(qg.QgemvError):
        qg.grouped_class(qg.BF16, 2048, 10)


def test_grouped_argmax_validation_errors_before_any_launch():
    L = qg.lib()
    arr = (qg.GemvDesc * 2)()
    for i in range(2):
        arr[i] = qg.GemvDesc(W=FAKE, scales=FAKE, x=FAKE, y=FAKE, fmt=qg.Q4_0_G32, M=64, K=2048, reserved=0)
    a = ctypes.cast(arr, ctypes.c_void_p)
    ws, idx = FAKE, FAKE
    f = L.qgemv_run_grouped_argmax
    assert f(None, 1, 1, 0, ws, idx, None) == qg.EINVAL
    assert f(a, 2, 9, 0, ws, idx, None) == qg.ESHAPE
    assert f(a, 2, 1, 2, ws, idx, None) == qg.EINVAL          # entry out of range
    assert f(a, 2, 1, -1, ws, idx, None) == qg.EINVAL
    assert f(a, 2, 1, 1, None, idx, None) == qg.EINVAL
    assert f(a, 2, 1, 1, ws, None, None) == qg.EINVAL
    assert f(a, 2, 1, 1, ws + 4, idx, None) == qg.EALIGN
    assert f(a, 2, 1, 1, ws, idx + 2, None) == qg.EALIGN
    arr[1].K = 40                                              # a bad GEMV still fails first
    assert f(a, 2, 1, 1, ws, idx, None) == qg.ESHAPE


def test_quantize_validation_errors_before_any_launch():
    f = qg.lib().qgemv_quantize
    assert f(qg.BF16, FAKE, 4, 64, FAKE, FAKE, None, None) == qg.EINVAL
    assert f(7, FAKE, 4, 64, FAKE, FAKE, None, None) == qg.EINVAL
    assert f(qg.Q4_0_G32, None, 4, 64, FAKE, FAKE, None, None) == qg.EINVAL
    assert f(qg.Q4_0_G32, FAKE, 4, 64, None, FAKE, None, None) == qg.EINVAL
    assert f(qg.Q4_0_G32, FAKE, 4, 64, FAKE, None, None, None) == qg.EINVAL
    assert f(qg.Q4_0_G32, FAKE, 0, 64, FAKE, FAKE, None, None) == qg.ESHAPE
    assert f(qg.Q4_0_G32, FAKE, 4, 48, FAKE, FAKE, None, None) == qg.ESHAPE
    assert f(qg.INT4_G128, FAKE, 4, 64, FAKE, FAKE, None, None) == qg.ESHAPE
    assert f(qg.Q4_0_G32, FAKE + 8, 4, 64, FAKE, FAKE, None, None) == qg.EALIGN
    assert f(qg.Q4_0_G32, FAKE, 4, 64, FAKE + 4, FAKE, None, None) == qg.EALIGN
    assert f(qg.Q4_0_G32, FAKE, 4, 64, FAKE, FAKE + 2, None, None) == qg.EALIGN
    assert f(qg.Q4_0_G32, FAKE, 4, 64, FAKE, FAKE, FAKE + 2, None) == qg.EALIGN
