"""Seeded random grouped calls: mixed formats, row lengths (ragged M and K), batch 1..8,
with and without the fused LM-head argmax, every row of each GEMV against the fp64
oracle and the index bit-exact against the oracle's argmax of the GPU's own logits."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bandwidth_bound_quantized_amd as qg  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu

FMTS = [qg.BF16, qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64]
K_STEP = {qg.BF16: 32, qg.INT8_G32: 32, qg.Q4_0_G32: 32, qg.INT4_G128: 128, qg.INT8_ROW: 32, qg.INT4_G64: 64}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 1, 1, 2, 2, 3, 4, 5, 8]))
    n = int(rng.integers(1, 12))
    main = int(rng.choice(FMTS))
    gemvs = []
    for i in range(n):
        fmt = main if rng.random() < 0.7 else int(rng.choice(FMTS))
        step = K_STEP[fmt]
        K = int(step * rng.integers(1, 8192 // step + 1))
        if rng.random() < 0.5:
            K = int(rng.choice([2048, 4096, 5632, 8192])) // step * step
        M = int(rng.choice([1, 7, 63, 65, 1000, 2048, 3001, int(rng.integers(1, 20000))]))
        gemvs.append(synth.make_gemv(f"r{i}", fmt, M, K, B, 6, 900 + seed * 16 + i, "o"))
    return rng, B, gemvs, rng.random() < 0.5, int(rng.integers(0, n))


@pytest.mark.parametrize("seed", range(64))
def test_random_grouped_call(seed):
    rng, B, gemvs, use_am, am = _case(seed)
    items = []
    for g in gemvs:
        W = _dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
        S = _dev(g.s.reshape(-1)) if g.s is not None else None
        X = _dev(np.ascontiguousarray(g.x).reshape(B, g.K))
        Y = torch.full((B, g.M), float("nan"), dtype=torch.float32, device="cuda")
        items.append((g.fmt, W, S, X, Y, g.M, g.K))
    descs = qg.grouped_descs(items)
    shapes = " ".join(f"{qg.FMT_NAMES[g.fmt]}:{g.M}x{g.K}" for g in gemvs)
    print(f"[gpu] seed={seed} B={B} argmax={am if use_am else None} {shapes}", flush=True)
    if use_am:
        ws = qg.fused_argmax_workspace(B)
        idx = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        qg.run_grouped_argmax(descs, B, am, ws, idx)
    else:
        qg.run_grouped(descs, B)
    torch.cuda.synchronize()
    for g, it in zip(gemvs, items):
        y = it[4].cpu().numpy()
        assert np.isfinite(y).all(), g.name
        y_ref, a_ref = oracle.gemv_ref(g.fmt, g.w, g.s, g.x, g.M, g.K)
        rep = oracle.parity_report(y, y_ref, a_ref)
        assert rep["ok"], f"{g.name} {qg.FMT_NAMES[g.fmt]} {g.M}x{g.K} {rep}"
    if use_am:
        ym = items[am][4].cpu().numpy()
        assert (idx.cpu().numpy() == oracle.argmax_ref(ym)).all()
        assert (ws.cpu().numpy() == 0).all()


@pytest.mark.parametrize("B,am", [(1, 3), (1, 66), (2, 3), (4, 3), (8, 66)])
def test_many_entries_grouped_argmax(B, am):
    """70 GEMVs in one call (two launches of the 64-entry table): every workgroup finds its
    entry by the lane-parallel lookup, the argmax entry in the first or the second launch;
    every row of every GEMV and the index against the oracle, and the workspace left zero."""
    rng = np.random.default_rng(4000 + 10 * B + am)
    gemvs = []
    for i in range(70):
        K = 5632 if i % 9 == 4 else 2048
        M = int(rng.choice([64, 100, 257, 1000, 1500, 3001]))
        gemvs.append(synth.make_gemv(f"m{i}", qg.Q4_0_G32, M, K, B, 6, 5000 + 100 * B + i, "o"))
    items = []
    for g in gemvs:
        W = _dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
        S = _dev(g.s.reshape(-1))
        X = _dev(np.ascontiguousarray(g.x).reshape(B, g.K))
        Y = torch.full((B, g.M), float("nan"), dtype=torch.float32, device="cuda")
        items.append((g.fmt, W, S, X, Y, g.M, g.K))
    descs = qg.grouped_descs(items)
    ws = qg.fused_argmax_workspace(B)
    idx = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    print(f"[gpu] many entries B={B} argmax entry {am}", flush=True)
    qg.run_grouped_argmax(descs, B, am, ws, idx)
    torch.cuda.synchronize()
    for g, it in zip(gemvs, items):
        y = it[4].cpu().numpy()
        assert np.isfinite(y).all(), g.name
        y_ref, a_ref = oracle.gemv_ref(g.fmt, g.w, g.s, g.x, g.M, g.K)
        rep = oracle.parity_report(y, y_ref, a_ref)
        assert rep["ok"], f"{g.name} {g.M}x{g.K} {rep}"
    assert (idx.cpu().numpy() == oracle.argmax_ref(items[am][4].cpu().numpy())).all()
    assert bool((ws == 0).all().item())
