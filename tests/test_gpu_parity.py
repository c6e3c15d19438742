"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: every output finite and |y - y_ref| <= 1e-3 * sum|w x| + 1e-5; hand-built
blocks and one-hot probes bit-exact; argmax bit-exact against the oracle's
argmax of the GPU's own logits.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bandwidth_bound_quantized_amd as qg  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from helpers import build_case, load_json  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"
ALL_FMTS = [qg.BF16, qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64]
FMT_IDS = ["bf16", "int8", "q4_0", "int4", "int8_row", "int4_g64"]
NIBBLE_FMTS = (qg.Q4_0_G32, qg.INT4_G128, qg.INT4_G64)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def gpu_gemv(fmt, w, s, x, M, K, B, y_fill=float("nan")):
    Wd = dev(np.ascontiguousarray(w).reshape(-1).view(np.uint8))
    Sd = dev(s.reshape(-1)) if s is not None else None
    Xd = dev(np.ascontiguousarray(x).reshape(B, K))
    Yd = torch.full((B, M), y_fill, dtype=torch.float32, device=DEV)
    print(f"[gpu] qgemv_run fmt={qg.FMT_NAMES[fmt]} M={M} K={K} B={B}", flush=True)
    qg.run(fmt, Wd, Sd, Xd, Yd, M, K, B)
    torch.cuda.synchronize()
    return Yd.cpu().numpy()


def assert_parity(fmt, w, s, x, M, K, B, y, rows=None, what=""):
    y_ref, a_ref = oracle.gemv_ref(fmt, w, s, x, M, K, rows=rows)
    yg = y if rows is None else y[:, rows]
    rep = oracle.parity_report(yg, y_ref, a_ref)
    assert rep["ok"], f"{what} {rep}"
    return rep


# ------------------------------------------------------------ hand blocks
HAND = load_json("hand_blocks.json")["cases"]


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
def test_hand_built_blocks_exact(case):
    fmt, M, K, w, s, x, y_exact = build_case(case)
    B = x.shape[0]
    y = gpu_gemv(fmt, w, s, x, M, K, B)
    want = np.array([[float(v) for v in row] for row in y_exact], dtype=np.float64)
    assert (y.astype(np.float64) == want).all(), (case["name"], y, want)


# -------------------------------------------------------- workload configs
def _workload_cases():
    cases = []
    for cfg in (1, 2, 3, 5):
        for B in synth.WORKLOAD_BATCHES[cfg]:
            for sp in synth.workload_specs(cfg):
                cases.append((cfg, B, sp))
    return cases


@pytest.mark.parametrize("cfg,B,sp", _workload_cases(),
                         ids=[f"cfg{c}-B{b}-{s.name}" for c, b, s in _workload_cases()])
def test_workload_gemv_parity(cfg, B, sp):
    g = synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
    y = gpu_gemv(g.fmt, g.w, g.s, g.x, g.M, g.K, B)
    assert np.isfinite(y).all()
    assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=f"cfg{cfg} {sp.name}")


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_decode_step_stream_layers_parity(B):
    """The 89-GEMV TinyLlama decode-step stream: two full layers and the LM head."""
    specs = synth.workload_specs(4)
    pick = [s for s in specs if s.name.startswith("L0.") or s.name.startswith("L21.")] + [specs[-1]]
    for sp in pick:
        g = synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
        y = gpu_gemv(g.fmt, g.w, g.s, g.x, g.M, g.K, B)
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=sp.name)


# ------------------------------------------------------------ exactness
@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FMT_IDS)
def test_onehot_probes_bit_exact(fmt):
    """x = e_k: y[b, m] = W_hat[m, k_b] exactly (one product, every other term 0)."""
    M, K, B = 300, 1024, 8
    g = synth.make_gemv("t", fmt, M, K, B, 8, fmt, "o")
    rng = np.random.default_rng(fmt)
    ks = rng.choice(K, B, replace=False)
    ks[0], ks[1] = 0, K - 1
    x = np.zeros((B, K), np.uint16)
    x[np.arange(B), ks] = 0x3F80
    y = gpu_gemv(fmt, g.w, g.s, x, M, K, B)
    W_hat = oracle.dequantize(fmt, g.w, g.s, K)
    want = W_hat[:, ks].T.astype(np.float32)
    assert (y == want).all()


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("M,K", [(1, 128), (63, 256), (65, 384), (1000, 5632), (7, 9216)])
def test_ragged_shapes_all_batches(fmt, M, K):
    if K % synth.K_ALIGN[fmt]:
        K = (K // 128 + 1) * 128
    for B in range(1, 9):
        nb = 1 if B == 1 else 2 if B == 2 else 4 if B <= 4 else 8
        lds = nb * K * 2 + (nb * K // 8 if fmt in NIBBLE_FMTS else 0)
        if lds > 160 * 1024:
            continue
        g = synth.make_gemv("t", fmt, M, K, B, 7, M % 997, "down")
        y = gpu_gemv(fmt, g.w, g.s, g.x, M, K, B)
        assert_parity(fmt, g.w, g.s, g.x, M, K, B, y, what=f"M={M} K={K} B={B}")


@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FMT_IDS)
def test_zero_weights_random_x(fmt):
    """All weights zero (codes 8 for 4-bit): every output within 1e-5 of 0."""
    M, K, B = 256, 5632 if fmt != qg.INT4_G128 else 5632 - 5632 % 128, 2
    g = synth.make_gemv("t", fmt, M, K, B, 7, 5, "o")
    w = np.zeros_like(g.w)
    if fmt in NIBBLE_FMTS:
        w[:] = 0x88
    s = None if g.s is None else np.full_like(g.s, 0x1D1F)    # ~0.005, the largest generated scale
    y = gpu_gemv(fmt, w, s, g.x, M, K, B)
    assert (np.abs(y) <= 1e-5).all(), np.abs(y).max()


def test_output_fully_written_and_guards_intact():
    fmt, M, K, B = qg.Q4_0_G32, 1003, 2048, 3
    g = synth.make_gemv("t", fmt, M, K, B, 7, 11, "qkv")
    Wd = dev(g.w.reshape(-1).view(np.uint8))
    Sd = dev(g.s.reshape(-1))
    Xd = dev(g.x)
    guard = 256
    buf = torch.full((B * M + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
    buf[:guard] = 12345.0
    buf[-guard:] = -6789.0
    Yd = buf[guard:guard + B * M]
    assert Yd.data_ptr() % 16 == 0
    qg.run(fmt, Wd, Sd, Xd, Yd, M, K, B)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    assert (h[:guard] == 12345.0).all() and (h[-guard:] == -6789.0).all()
    y = h[guard:guard + B * M].reshape(B, M)
    assert np.isfinite(y).all()
    assert_parity(fmt, g.w, g.s, g.x, M, K, B, y)


def test_repeat_runs_bitwise_identical():
    fmt, M, K, B = qg.INT8_G32, 4096, 2048, 4
    g = synth.make_gemv("t", fmt, M, K, B, 7, 12, "o")
    a = gpu_gemv(fmt, g.w, g.s, g.x, M, K, B)
    b = gpu_gemv(fmt, g.w, g.s, g.x, M, K, B, y_fill=0.0)
    assert (a.view(np.uint32) == b.view(np.uint32)).all()


def test_pack_bf16_then_run():
    """qgemv_pack's quantizer output feeds qgemv_run; result within the GEMV tolerance of
    the oracle run on the same codes (and the codes equal the oracle quantizer's)."""
    rng = np.random.default_rng(4)
    M, K, B = 512, 2048, 2
    wbf = synth.bf16_normal(rng, (M, K), 0.02)
    x = synth.bf16_normal(rng, (B, K), 1.0)
    for fmt in ALL_FMTS[1:]:
        codes, scales = qg.pack(fmt, qg.SRC_BF16, wbf, None, M, K)
        y = gpu_gemv(fmt, codes, scales, x, M, K, B)
        o_codes, o_scales = oracle.quantize_from_bf16(fmt, wbf, M, K)
        assert_parity(fmt, o_codes, o_scales, x, M, K, B, y)


# ------------------------------------------------------------------ argmax
def gpu_argmax(logits: np.ndarray, ws=None):
    B, V = logits.shape
    L = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    ws = qg.argmax_workspace(B) if ws is None else ws
    idx = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    print(f"[gpu] qgemv_argmax V={V} B={B}", flush=True)
    qg.argmax(L, V, B, ws, idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), ws


def _argmax_cases():
    rng = np.random.default_rng(21)
    cases = {}
    cases["random_128256x8"] = rng.standard_normal((8, 128256)).astype(np.float32)
    cases["random_32000x1"] = rng.standard_normal((1, 32000)).astype(np.float32)
    cases["ties_planted"] = synth.f32_logits_with_ties(rng, 8, 128256)
    t = rng.standard_normal((6, 128256)).astype(np.float32)
    # equal maxima straddling the slice boundaries of a 128256-logit row
    # (4 slices of 32064), a wave boundary, and the first/last elements
    for b, pos in enumerate([(32063, 32064), (63, 64), (0, 128255), (4095, 6143, 100000),
                             (64127, 64128, 96191), (96192, 128255)]):
        t[b, list(pos)] = 10.0
    cases["ties_boundaries"] = t
    n = rng.standard_normal((3, 5000)).astype(np.float32)
    n[0, 4000] = np.nan; n[0, 17] = np.nan                 # first NaN wins
    n[1, 3] = np.inf; n[1, 4999] = np.inf
    n[2, 2500] = np.nan; n[2, 10] = np.inf
    cases["nan_inf"] = n
    z = np.full((2, 3000), -1.0, np.float32)
    z[0, 5] = -0.0; z[0, 9] = 0.0                          # -0.0 ties +0.0 -> 5
    z[1, 7] = 0.0; z[1, 2] = -0.0                          # -> 2
    cases["signed_zeros"] = z
    cases["all_neg_inf"] = np.full((2, 777), -np.inf, np.float32)
    cases["tiny_V"] = rng.standard_normal((8, 1)).astype(np.float32)
    cases["V7"] = np.array([[1, 5, 5, 2, 0, 5, 1]] * 2, np.float32)
    cases["large_V"] = rng.standard_normal((1, 300001)).astype(np.float32)
    lv = rng.standard_normal((3, 70001)).astype(np.float32)   # odd V: scalar loads, 3 slices
    lv[0, [23334, 23333]] = 9.0; lv[1, [46667, 70000]] = 9.0; lv[2, 70000] = 9.0
    cases["odd_V_multislice_ties"] = lv
    return cases


ARGMAX_CASES = _argmax_cases()


@pytest.mark.parametrize("name", sorted(ARGMAX_CASES))
def test_argmax_bit_exact(name):
    logits = ARGMAX_CASES[name]
    idx, ws = gpu_argmax(logits)
    assert (idx == oracle.argmax_ref(logits)).all(), (idx, oracle.argmax_ref(logits))
    assert (ws.cpu().numpy() == 0).all()     # workspace returned to zero


def test_argmax_workspace_reuse_many_calls():
    rng = np.random.default_rng(3)
    ws = qg.argmax_workspace(8)
    for i in range(20):
        V = int(rng.integers(1, 200000))
        B = int(rng.integers(1, 9))
        logits = rng.standard_normal((B, V)).astype(np.float32)
        idx, ws = gpu_argmax(logits, ws)
        assert (idx == oracle.argmax_ref(logits)).all()


def _random_argmax_case(seed):
    """Seeded logits: random V and batch, values on a coarse grid (many ties), and in some
    rows a planted maximum repeated at random places, a NaN, +inf or -inf, or signed zeros."""
    rng = np.random.default_rng(13000 + seed)
    B = int(rng.integers(1, 9))
    V = int(rng.choice([1, 2, 63, 64, 65, 4097, 32000, 128256, int(rng.integers(1, 300000))]))
    levels = int(rng.choice([3, 50, 1 << 20]))
    x = (rng.integers(0, levels, size=(B, V)) / levels - 0.5).astype(np.float32)
    for b in range(B):
        kind = int(rng.integers(0, 6))
        pos = rng.integers(0, V, size=min(V, 4))
        if kind == 1:
            x[b, pos] = x[b].max()                       # the maximum at several places
        elif kind == 2:
            x[b, pos[-1]] = np.nan
        elif kind == 3:
            x[b, pos] = np.inf
        elif kind == 4:
            x[b] = -np.inf
            x[b, pos[:1]] = -np.float32(3e38)
        elif kind == 5:
            x[b] = np.where(rng.random(V) < 0.5, np.float32(-0.0), np.float32(0.0))
    return x


@pytest.mark.parametrize("seed", range(16))
def test_random_argmax_bit_exact(seed):
    """Seeded random logits with ties, NaN, infinities and signed zeros: the index equals
    the oracle's (lowest index among equal maxima, the first NaN), and the workspace
    returns to zero."""
    logits = _random_argmax_case(seed)
    idx, ws = gpu_argmax(logits)
    assert (idx == oracle.argmax_ref(logits)).all(), (idx, oracle.argmax_ref(logits))
    assert (ws.cpu().numpy() == 0).all()


@pytest.mark.parametrize("B", [1, 8])
def test_lm_head_then_argmax_on_gpu_logits(B):
    """int8-g32 LM head 128256x2048 then argmax, all on the GPU; the argmax must equal the
    oracle's argmax of the GPU's own logits, and the logits pass the GEMV tolerance."""
    sp = synth.workload_specs(5)[-1]
    g = synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
    Wd = dev(g.w.reshape(-1).view(np.uint8)); Sd = dev(g.s.reshape(-1)); Xd = dev(g.x)
    Yd = torch.empty((B, sp.M), dtype=torch.float32, device=DEV)
    ws = qg.argmax_workspace(B)
    idx = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    qg.run(sp.fmt, Wd, Sd, Xd, Yd, sp.M, sp.K, B)
    qg.argmax(Yd, sp.M, B, ws, idx)
    torch.cuda.synchronize()
    logits = Yd.cpu().numpy()
    assert (idx.cpu().numpy() == oracle.argmax_ref(logits)).all()
    assert_parity(sp.fmt, g.w, g.s, g.x, sp.M, sp.K, B, logits)


# ------------------------------------------------------------ stream read
def test_stream_read_checksum():
    n = (64 << 20) + 48
    rng = np.random.default_rng(0)
    host = rng.integers(0, 2 ** 32, size=n // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    for unroll in (1, 4, 16):
        for grid in (1, 300, 2048):
            sink = torch.zeros(grid, dtype=torch.int32, device=DEV)
            qg.stream_read(buf, n, sink, grid=grid, unroll=unroll)
            torch.cuda.synchronize()
            x = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
            assert x == np.bitwise_xor.reduce(host)


# ------------------------------------------------------------ grouped GEMVs
def _grouped(gemvs, B):
    """Upload, run all gemvs in one qgemv_run_grouped call, return host outputs."""
    dev_items = []
    for g in gemvs:
        W = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
        S = dev(g.s.reshape(-1)) if g.s is not None else None
        X = dev(np.ascontiguousarray(g.x).reshape(B, g.K))
        Y = torch.full((B, g.M), float("nan"), dtype=torch.float32, device=DEV)
        dev_items.append((g.fmt, W, S, X, Y, g.M, g.K))
    descs = qg.grouped_descs(dev_items)
    print(f"[gpu] qgemv_run_grouped n={len(gemvs)} B={B}", flush=True)
    qg.run_grouped(descs, B)
    torch.cuda.synchronize()
    return [it[4].cpu().numpy() for it in dev_items]


@pytest.mark.parametrize("cfg,B", [(2, 1), (2, 2), (3, 1), (5, 1), (5, 2), (1, 2),
                                   (2, 4), (2, 8), (3, 4), (5, 8), (1, 8), (6, 1), (6, 8)])
def test_grouped_workload_parity(cfg, B):
    gemvs = [synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
             for sp in synth.workload_specs(cfg)]
    ys = _grouped(gemvs, B)
    for g, y in zip(gemvs, ys):
        assert np.isfinite(y).all(), g.name
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=f"grouped {g.name}")


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_grouped_decode_step_stream_89_gemvs(B):
    """All 89 GEMVs of the TinyLlama decode-step stream in one call, every output row of
    every GEMV against the oracle (B 1, 2: one register-x launch whose waves take
    contiguous ranges of row groups; B 4, 8: matrix-core launches of at most 64 entries,
    each entry's tiles shared out among several workgroups and their waves)."""
    gemvs = synth.make_workload(4, B)
    ys = _grouped(gemvs, B)
    for g, y in zip(gemvs, ys):
        assert np.isfinite(y).all(), g.name
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=f"grouped {g.name}")


@pytest.mark.parametrize("B", [1, 2, 3, 8])
def test_grouped_mixed_formats_ragged_and_fallback(B):
    """Formats and row lengths mixed in one call, ragged M, entries no grouped kernel
    takes launched one by one (int8 K=8192 at B = 2; K not a multiple of the
    matrix-core step at B >= 3). At B = 1 the int8 rows of 4608..8192 share the
    grouped launch with the short ones, one row per wave step, including rows whose
    unit count is not a multiple of 64 (K = 4608, 5632)."""
    shapes = [(synth.Q4_0_G32, 1, 2048), (synth.BF16, 65, 256), (synth.INT8_G32, 1000, 2048),
              (synth.Q4_0_G32, 63, 5632), (synth.INT4_G128, 300, 8192), (synth.INT8_G32, 70, 8192),
              (synth.Q4_0_G32, 4097, 2048), (synth.BF16, 7, 2048), (synth.INT4_G128, 129, 384),
              (synth.Q4_0_G32, 2, 96), (synth.INT8_ROW, 513, 2048), (synth.INT4_G64, 1029, 2048),
              (synth.INT8_ROW, 40, 8192), (synth.INT4_G64, 3, 192), (synth.INT8_G32, 33, 5632),
              (synth.INT8_ROW, 9, 4608)]
    gemvs = [synth.make_gemv(f"g{i}", f, M, K, B, 6, i, "o") for i, (f, M, K) in enumerate(shapes)]
    ys = _grouped(gemvs, B)
    for g, y in zip(gemvs, ys):
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=f"mixed {g.name}")


def test_grouped_class_of_the_workload_shapes():
    """The launches qgemv_grouped_class names for the shapes measured here."""
    XR, MF, AL = qg.GROUP_XREG, qg.GROUP_MFMA, qg.GROUP_ALONE
    cases = [(qg.Q4_0_G32, 2048, 1, XR), (qg.Q4_0_G32, 5632, 2, XR), (qg.INT4_G128, 8192, 1, XR),
             (qg.INT8_G32, 8192, 1, XR), (qg.INT8_ROW, 4608, 1, XR), (qg.INT8_G32, 8192, 2, AL),
             (qg.INT8_G32, 9216, 1, AL), (qg.BF16, 2048, 2, XR), (qg.BF16, 4096, 1, AL),
             (qg.Q4_0_G32, 2048, 8, MF), (qg.INT8_G32, 8192, 3, MF), (qg.Q4_0_G32, 2048 + 32, 4, AL)]
    for fmt, K, B, want in cases:
        assert qg.grouped_class(fmt, K, B) == want, (qg.FMT_NAMES[fmt], K, B)


def test_grouped_contiguous_ranges_at_four_rows():
    """40 Q4_0 GEMVs of 3000x2048 at B=1: about 10 row groups of four rows per wave, so
    the waves take contiguous ranges, but at eight rows per step they would get fewer than
    eight each, so the launch keeps four. Every row of every GEMV against the oracle."""
    B = 1
    gemvs = [synth.make_gemv(f"c{i}", synth.Q4_0_G32, 3000, 2048, B, 6, 200 + i, "gate_up") for i in range(40)]
    ys = _grouped(gemvs, B)
    for g, y in zip(gemvs, ys):
        assert np.isfinite(y).all(), g.name
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=g.name)


def test_grouped_more_than_one_launch_per_class():
    """130 small Q4_0 GEMVs: more than the 64 entries one launch's table holds."""
    B = 1
    gemvs = [synth.make_gemv(f"s{i}", synth.Q4_0_G32, 33 + i, 2048, B, 6, 100 + i, "qkv") for i in range(130)]
    ys = _grouped(gemvs, B)
    for g, y in zip(gemvs, ys):
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=g.name)


# ------------------------------------------------ matrix-core path (batch 3..8)
# Shapes chosen for the launch plans they produce: few tiles with the row's
# steps split over up to 16 waves whose partial tiles are added in LDS
# (2048x2048, 17x4096, 2048x8192), many tiles per workgroup and more than one
# pass of the grid over them (40000x1024), a ragged last tile (4100, 17), and
# the shortest rows each format takes on this path (16x512).
MFMA_SHAPES = [(2048, 2048), (17, 4096), (4100, 1024), (16, 512), (40000, 1024), (2048, 8192)]


@pytest.mark.parametrize("B", [3, 5, 8])
@pytest.mark.parametrize("M,K", MFMA_SHAPES, ids=[f"{m}x{k}" for m, k in MFMA_SHAPES])
@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FMT_IDS)
def test_mfma_path_shapes(fmt, M, K, B):
    g = synth.make_gemv("t", fmt, M, K, B, 9, (M + K) % 991, "gate_up")
    y = gpu_gemv(fmt, g.w, g.s, g.x, M, K, B)
    assert np.isfinite(y).all()
    assert_parity(fmt, g.w, g.s, g.x, M, K, B, y, what=f"M={M} K={K} B={B}")


@pytest.mark.parametrize("fmt", [qg.Q4_0_G32, qg.INT4_G128, qg.INT4_G64], ids=["q4_0", "int4", "int4_g64"])
def test_mfma_path_all_codes_extreme(fmt):
    """Every 4-bit code 0 or 15 with the largest generated scale and x of one sign:
    the largest partial sums and the largest offset-term cancellation the
    synthetic inputs can produce."""
    M, K, B = 512, 4096, 8
    g = synth.make_gemv("t", fmt, M, K, B, 9, 3, "down")
    rng = np.random.default_rng(11)
    w = np.where(rng.random(g.w.shape) < 0.5, 0x00, 0xFF).astype(np.uint8)
    s = np.full_like(g.s, 0x1D1F)
    x = synth.bf16_normal(rng, (B, K), 1.0) & np.uint16(0x7FFF)     # |x|: sign bit cleared
    y = gpu_gemv(fmt, w, s, x, M, K, B)
    assert_parity(fmt, w, s, x, M, K, B, y, what="extreme")


# ------------------------------------------------- grouped GEMVs + fused argmax
def _grouped_argmax(gemvs, B, am, ws=None):
    """Upload, run all gemvs + the argmax of entry am in one qgemv_run_grouped_argmax call."""
    dev_items = []
    for g in gemvs:
        W = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
        S = dev(g.s.reshape(-1)) if g.s is not None else None
        X = dev(np.ascontiguousarray(g.x).reshape(B, g.K))
        Y = torch.full((B, g.M), float("nan"), dtype=torch.float32, device=DEV)
        dev_items.append((g.fmt, W, S, X, Y, g.M, g.K))
    descs = qg.grouped_descs(dev_items)
    ws = qg.fused_argmax_workspace(B) if ws is None else ws
    idx = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    print(f"[gpu] qgemv_run_grouped_argmax n={len(gemvs)} B={B} am={am}", flush=True)
    qg.run_grouped_argmax(descs, B, am, ws, idx)
    torch.cuda.synchronize()
    return [it[4].cpu().numpy() for it in dev_items], idx.cpu().numpy(), ws


@pytest.mark.parametrize("cfg,B", [(2, 1), (2, 2), (5, 1), (5, 2), (2, 4), (5, 8), (6, 1), (6, 2), (6, 8)])
def test_grouped_argmax_workloads(cfg, B):
    """The step's GEMVs and the LM-head argmax in one call (fused into the LM head's launch
    at B <= 2, a separate argmax launch otherwise): logits within the GEMV tolerance, the
    index bit-exact against the oracle's argmax of the GPU's own logits, ws back to zero."""
    gemvs = [synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
             for sp in synth.workload_specs(cfg)]
    am = len(gemvs) - 1
    ys, idx, ws = _grouped_argmax(gemvs, B, am)
    for g, y in zip(gemvs, ys):
        assert np.isfinite(y).all(), g.name
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=f"fused {g.name}")
    assert (idx == oracle.argmax_ref(ys[am])).all(), (idx, oracle.argmax_ref(ys[am]))
    assert (ws.cpu().numpy() == 0).all()


@pytest.mark.parametrize("B", [1, 2, 8])
def test_grouped_argmax_decode_step_stream_contiguous_ranges(B):
    """The 89-GEMV decode-step stream with the LM-head argmax in one call: at B <= 2 about
    38 row groups per wave, so every wave takes one contiguous range of them (the LM head's
    rows go to the first few hundred waves only); at B = 8 the matrix-core launch with the
    argmax keys per workgroup. Every row of every GEMV against the oracle, the index
    bit-exact against the oracle's argmax of the GPU's own logits, ws back to zero."""
    gemvs = synth.make_workload(4, B)
    am = len(gemvs) - 1
    ys, idx, ws = _grouped_argmax(gemvs, B, am)
    for g, y in zip(gemvs, ys):
        assert np.isfinite(y).all(), g.name
        assert_parity(g.fmt, g.w, g.s, g.x, g.M, g.K, B, y, what=f"stream {g.name}")
    assert (idx == oracle.argmax_ref(ys[am])).all(), (idx, oracle.argmax_ref(ys[am]))
    assert (ws.cpu().numpy() == 0).all()


@pytest.mark.parametrize("B", [2, 4, 8])
def test_grouped_argmax_ties_across_workgroups(B):
    """bf16 LM head whose rows give exactly 0 except rows made negative: the maximum 0.0 is
    tied at rows far apart (different waves and workgroups); the lowest index must win,
    with the LM head in the middle of the entry table (batch 2: the register-x launch;
    4 and 8: the matrix-core launch, whose workgroups publish keys and the last one
    finishes the argmax)."""
    M, K = 20000, 2048
    rng = np.random.default_rng(21)
    x = synth.bf16_normal(rng, (B, K), 1.0)
    x[1:] = x[0]
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    w = np.zeros((M, K), np.uint16)
    neg = np.ones(M, bool)
    neg[[5003, 7777, 19999]] = False                      # the zero rows
    # negative rows: w = -0.01 * sign(x), so the dot product is -0.01 * sum|x| < 0
    wrow = synth.round_f32_to_bf16_bits((-0.01 * np.sign(xf[0])).astype(np.float32))
    w[neg] = wrow
    lm = synth.Gemv("lm", synth.BF16, M, K, B, w, None, x, (0, 0, 0))
    other = synth.make_gemv("o", synth.BF16, 2048, 2048, B, 9, 1, "o")
    tail = synth.make_gemv("t", synth.BF16, 100, 1024, B, 9, 2, "qkv")
    ys, idx, ws = _grouped_argmax([other, lm, tail], B, 1)
    y = ys[1]
    assert (y[:, ~neg] == 0).all() and (y[:, neg] < 0).all()
    assert (idx == 5003).all(), idx
    assert (ws.cpu().numpy() == 0).all()


@pytest.mark.parametrize("B", [2, 4, 8])
def test_grouped_argmax_nan_logit_and_workspace_reuse(B):
    """A NaN scale makes that row's logits NaN: the first NaN row wins (NumPy semantics).
    Five calls reuse one workspace, which is zero after each."""
    sp = synth.workload_specs(2)[-1]
    g = synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
    ws = qg.fused_argmax_workspace(B)
    for rows in ([], [30001], [12345, 30001], [0], [31999, 4]):
        s = g.s.copy()
        for r in rows:
            s[r, 7] = 0x7E00                                   # binary16 NaN
        gg = synth.Gemv(g.name, g.fmt, g.M, g.K, B, g.w, s, g.x, g.seeds)
        ys, idx, ws = _grouped_argmax([gg], B, 0, ws)
        want = oracle.argmax_ref(ys[0])
        assert (idx == want).all(), (rows, idx, want)
        if rows:
            assert (idx == min(rows)).all()
        assert (ws.cpu().numpy() == 0).all()


# ------------------------------------------------------------ device quantizer
def gpu_quantize(fmt, w, M, K):
    wb, sb = qg.packed_size(fmt, M, K)
    Wd = dev(np.ascontiguousarray(w))
    C = torch.zeros(wb, dtype=torch.uint8, device=DEV)
    S = torch.zeros(sb // 2, dtype=torch.int16, device=DEV)
    E = torch.zeros(1, dtype=torch.int32, device=DEV)
    print(f"[gpu] qgemv_quantize fmt={qg.FMT_NAMES[fmt]} M={M} K={K}", flush=True)
    qg.quantize(fmt, Wd, M, K, C, S, E)
    torch.cuda.synchronize()
    return C.cpu().numpy(), S.cpu().numpy().view(np.uint16), int(E.cpu().numpy()[0])


def _quant_edge_inputs():
    rng = np.random.default_rng(99)
    w = synth.bf16_normal(rng, (64, 512), 0.02)
    w[0, :128] = 0
    w[1, :32] = synth.round_f32_to_bf16_bits(np.zeros(32, np.float32))
    w[1, 32:64] = 0x8000                                     # all -0.0
    t = np.zeros(32, np.float32); t[3] = -0.5; t[9] = 0.5
    w[2, :32] = synth.round_f32_to_bf16_bits(t)              # |w| tie: the first (negative) wins
    w[2, 32:64] = synth.round_f32_to_bf16_bits(-t)
    w[3, 32:64] = synth.round_f32_to_bf16_bits(np.linspace(-0.3, 0.75, 32).astype(np.float32))
    w[4, :32] = synth.round_f32_to_bf16_bits(np.full(32, 1e-9, np.float32))           # scale rounds to 0
    w[5, :32] = synth.round_f32_to_bf16_bits(np.linspace(-3e-5, 2e-5, 32).astype(np.float32))  # subnormal d
    w[6, :128] = synth.round_f32_to_bf16_bits(np.linspace(-500000, 400000, 128).astype(np.float32))
    w[7, :64] = synth.round_f32_to_bf16_bits(np.arange(64).astype(np.float32) * 0.0625 - 2.0)  # exact halves
    w[8, :128] = synth.round_f32_to_bf16_bits((np.arange(128) - 64).astype(np.float32) * 2.5)  # rint ties
    return w


@pytest.mark.parametrize("fmt", ALL_FMTS[1:], ids=FMT_IDS[1:])
def test_device_quantizer_bit_exact(fmt):
    """qgemv_quantize against the oracle quantizer (and so against qgemv_pack, which the CPU
    tests hold bit-exact to it) on edge groups and on the 2048x2048 workload shape."""
    for w in (_quant_edge_inputs(), synth.bf16_normal(np.random.default_rng(fmt + 1000), (2048, 2048), 0.02)):
        M, K = w.shape
        codes, scales, err = gpu_quantize(fmt, w, M, K)
        o_codes, o_scales = oracle.quantize_from_bf16(fmt, w, M, K)
        assert err == 0
        assert (scales == o_scales.reshape(-1)).all()
        assert (codes == o_codes.reshape(-1).view(np.uint8)).all()


def _random_quant_case(seed):
    """A seeded draw of format, ragged M and K, and bf16 weights whose rows span many
    magnitudes (scales from f16 subnormal to large), with zero groups and repeated
    values (ties in |w|) mixed in."""
    rng = np.random.default_rng(12000 + seed)
    fmt = int(rng.choice(ALL_FMTS[1:]))
    step = synth.K_ALIGN[fmt]
    K = int(step * rng.integers(1, 4096 // step + 1))
    M = int(rng.choice([1, 3, 100, int(rng.integers(1, 3000))]))
    mag = 10.0 ** rng.uniform(-7, 4, size=(M, 1))
    w32 = (rng.standard_normal((M, K)) * mag).astype(np.float32)
    z = rng.random((M, K)) < 0.02
    w32[z] = 0.0
    rep = rng.random((M, K)) < 0.05
    w32[rep] = np.round(w32[rep] * 4) / 4                  # repeated magnitudes within a group
    return fmt, M, K, synth.round_f32_to_bf16_bits(w32)


@pytest.mark.parametrize("seed", range(12))
def test_random_device_quantizer_bit_exact(seed):
    """Seeded random shapes and magnitudes: qgemv_quantize equals the oracle quantizer byte
    for byte (codes and scales)."""
    fmt, M, K, w = _random_quant_case(seed)
    codes, scales, err = gpu_quantize(fmt, w, M, K)
    o_codes, o_scales = oracle.quantize_from_bf16(fmt, w, M, K)
    assert err == 0
    assert (scales == o_scales.reshape(-1)).all()
    assert (codes == o_codes.reshape(-1).view(np.uint8)).all()


def test_device_quantizer_range_errors_flagged():
    w = synth.bf16_normal(np.random.default_rng(5), (4, 128), 0.02)
    _, _, err = gpu_quantize(qg.Q4_0_G32, w, 4, 128)
    assert err == 0
    bad = w.copy(); bad[2, 70] = 0x7F80                          # +inf
    _, _, err = gpu_quantize(qg.Q4_0_G32, bad, 4, 128)
    assert err == qg.ERANGE
    bad = w.copy(); bad[1, 5] = 0x7FC1                           # NaN
    _, _, err = gpu_quantize(qg.INT4_G128, bad, 4, 128)
    assert err == qg.ERANGE
    big = synth.round_f32_to_bf16_bits(np.full((1, 32), 1e7, np.float32))   # scale > 65504
    _, _, err = gpu_quantize(qg.INT8_G32, big, 1, 32)
    assert err == qg.ERANGE


def test_device_quantizer_then_run():
    """Quantize on the device, run the GEMV on those codes: within tolerance of the oracle
    run on the oracle's codes (batch 1 and 8)."""
    rng = np.random.default_rng(17)
    M, K = 1024, 2048
    wbf = synth.bf16_normal(rng, (M, K), 0.02)
    for fmt in ALL_FMTS[1:]:
        codes, scales, err = gpu_quantize(fmt, wbf, M, K)
        assert err == 0
        for B in (1, 8):
            x = synth.bf16_normal(rng, (B, K), 1.0)
            y = gpu_gemv(fmt, codes, scales, x, M, K, B)
            o_codes, o_scales = oracle.quantize_from_bf16(fmt, wbf, M, K)
            assert_parity(fmt, o_codes, o_scales, x, M, K, B, y)


# ------------------------------------------------------------ batch invariance
def gpu_gemv_inv(fmt, Wd, Sd, x, M, K, B):
    Xd = dev(np.ascontiguousarray(x).reshape(B, K))
    Yd = torch.full((B, M), float("nan"), dtype=torch.float32, device=DEV)
    print(f"[gpu] qgemv_run_flags invariant fmt={qg.FMT_NAMES[fmt]} M={M} K={K} B={B}", flush=True)
    qg.run_flags(fmt, Wd, Sd, Xd, Yd, M, K, B, qg.FLAG_BATCH_INVARIANT)
    torch.cuda.synchronize()
    return Yd.cpu().numpy()


# Matrix-core shapes (K a multiple of the format's step) and shapes the
# dot-product kernel takes (short or ragged K), small and large M.
INV_SHAPES = [(2048, 2048), (4100, 1024), (32000, 2048), (65, 384), (1000, 5632), (7, 9216)]


@pytest.mark.parametrize("M,K", INV_SHAPES, ids=[f"{m}x{k}" for m, k in INV_SHAPES])
@pytest.mark.parametrize("fmt", ALL_FMTS, ids=FMT_IDS)
def test_batch_invariant_rows_bitwise_equal(fmt, M, K):
    """With the batch-invariant flag, row b of a batch-B call equals the
    batch-1 call on x[b] bit for bit, for B = 8, 5, 3, 2 (and matches the
    oracle within the usual bound)."""
    if K % synth.K_ALIGN[fmt]:
        K = (K // 128 + 1) * 128
    if 8 * K * 2 + (K if fmt in NIBBLE_FMTS else 0) > 160 * 1024:
        pytest.skip("x of 8 rows does not fit in LDS")
    g = synth.make_gemv("t", fmt, M, K, 8, 13, (3 * M + K) % 983, "gate_up")
    Wd = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
    Sd = dev(g.s.reshape(-1)) if g.s is not None else None
    x = g.x.reshape(8, K)
    singles = np.stack([gpu_gemv_inv(fmt, Wd, Sd, x[b:b + 1], M, K, 1)[0] for b in range(8)])
    assert np.isfinite(singles).all()
    assert_parity(fmt, g.w, g.s, x, M, K, 8, singles, what="singles")
    for B, rows in ((8, range(8)), (5, (7, 0, 3, 6, 1)), (3, (2, 5, 4)), (2, (6, 6))):
        xb = x[list(rows)]
        y = gpu_gemv_inv(fmt, Wd, Sd, xb, M, K, B)
        want = singles[list(rows)]
        assert (y.view(np.uint32) == want.view(np.uint32)).all(), f"B={B} rows={rows}"


def _random_invariant_case(seed):
    """A seeded draw of format, ragged M and K (x of 8 rows within LDS), and the
    batch rows of one batch-B call."""
    rng = np.random.default_rng(11000 + seed)
    fmt = int(rng.choice(ALL_FMTS))
    step = synth.K_ALIGN[fmt]
    K = int(step * rng.integers(1, 6144 // step + 1))
    M = int(rng.choice([1, 5, 64, 333, 2048, int(rng.integers(1, 9000))]))
    B = int(rng.integers(2, 9))
    rows = [int(v) for v in rng.integers(0, 8, size=B)]
    return fmt, M, K, B, rows


@pytest.mark.parametrize("seed", range(16))
def test_random_batch_invariant_call(seed):
    """Seeded random shapes with the batch-invariant flag: each row of a batch-B call
    (rows drawn with repeats) equals the batch-1 call on that row's x bit for bit, and
    every row is within the bound of the oracle."""
    fmt, M, K, B, rows = _random_invariant_case(seed)
    g = synth.make_gemv("t", fmt, M, K, 8, 17, 200 + seed, "gate_up")
    Wd = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
    Sd = dev(g.s.reshape(-1)) if g.s is not None else None
    x = g.x.reshape(8, K)
    singles = {b: gpu_gemv_inv(fmt, Wd, Sd, x[b:b + 1], M, K, 1)[0] for b in set(rows)}
    y = gpu_gemv_inv(fmt, Wd, Sd, x[rows], M, K, B)
    want = np.stack([singles[b] for b in rows])
    assert (y.view(np.uint32) == want.view(np.uint32)).all(), f"seed={seed} B={B} rows={rows}"
    assert_parity(fmt, g.w, g.s, x[rows], M, K, B, y, what="batch call")


def test_batch_invariant_flag_zero_is_run():
    """flags 0 is qgemv_run: same bits."""
    fmt, M, K, B = qg.Q4_0_G32, 2048, 2048, 2
    g = synth.make_gemv("t", fmt, M, K, B, 13, 5, "gate_up")
    y_run = gpu_gemv(fmt, g.w, g.s, g.x, M, K, B)
    Wd = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
    Xd = dev(np.ascontiguousarray(g.x).reshape(B, K))
    Yd = torch.full((B, M), float("nan"), dtype=torch.float32, device=DEV)
    qg.run_flags(fmt, Wd, dev(g.s.reshape(-1)), Xd, Yd, M, K, B, 0)
    torch.cuda.synchronize()
    assert (Yd.cpu().numpy().view(np.uint32) == y_run.view(np.uint32)).all()
