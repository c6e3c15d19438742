"""GPU parity of qgemv_run_fused (RMSNorm prologue, residual / SwiGLU
epilogues, fused argmax) against the float64 oracle, through the C ABI.

Shapes reach all three kernels: the register-x kernel (batch <= 2, short
rows), the matrix-core kernel (batch 3..8, K a multiple of its step) and the
LDS dot2 kernel (batch 3..8 with other K, or long rows).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bandwidth_bound_quantized_amd as qg  # noqa: E402
import oracle  # noqa: E402
import oracle.fused as ofused  # noqa: E402
from oracle.gemv import ABS_TOL, REL_TOL  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


class Case:
    """Seeded inputs of one fused GEMV: weights, h (float32 residual stream),
    g (bf16 norm weight), a residual, and a bf16 x for runs without the norm."""

    def __init__(self, fmt, M, K, B, seed):
        self.fmt, self.M, self.K, self.B = fmt, M, K, B
        g = synth.make_gemv("t", fmt, M, K, B, 11, seed % 997, "gate_up")
        self.w, self.s, self.x = g.w, g.s, g.x.reshape(B, K)
        rng = np.random.default_rng(1000 + seed)
        self.h = (rng.standard_normal((B, K)) * 0.8).astype(np.float32)
        self.g = synth.round_f32_to_bf16_bits(rng.uniform(0.5, 1.5, K).astype(np.float32))
        self.res = rng.standard_normal((B, M)).astype(np.float32)
        self.Wd = dev(np.ascontiguousarray(self.w).reshape(-1).view(np.uint8))
        self.Sd = dev(self.s.reshape(-1)) if self.s is not None else None

    def run(self, norm=False, residual=None, swiglu=False, argmax=False, y_init=None):
        B, M, K = self.B, self.M, self.K
        kinds = [k for k, on in (("norm", norm), ("residual", residual is not None),
                                 ("swiglu", swiglu), ("argmax", argmax)) if on]
        print(f"[gpu] qgemv_run_fused fmt={qg.FMT_NAMES[self.fmt]} M={M} K={K} B={B} {'+'.join(kinds)}",
              flush=True)
        kw = {}
        x = None
        if norm:
            kw.update(norm_input=dev(self.h), norm_weight=dev(self.g), eps=EPS)
        else:
            x = dev(self.x)
        y = None
        act = None
        if swiglu:
            act = torch.full((B, M // 2), -1, dtype=torch.int16, device=DEV)
            kw["swiglu_out"] = act
        else:
            y = (torch.full((B, M), float("nan"), dtype=torch.float32, device=DEV) if y_init is None
                 else dev(y_init))
        if residual is not None:
            kw["residual"] = y if residual == "inplace" else dev(self.res)
        idx = ws = None
        if argmax:
            idx = torch.full((B,), -7, dtype=torch.int32, device=DEV)
            ws = qg.fused_argmax_workspace(B)
            kw.update(argmax_idx=idx, argmax_ws=ws)
        qg.run_fused(self.fmt, self.Wd, self.Sd, x, y, M, K, B, **kw)
        torch.cuda.synchronize()
        out = {}
        if y is not None:
            out["y"] = y.cpu().numpy()
        if act is not None:
            out["act"] = act.cpu().numpy().view(np.uint16)
        if idx is not None:
            out["idx"] = idx.cpu().numpy()
            out["ws_zero"] = bool((ws == 0).all().item())
        return out

    def oracle_y(self, norm):
        xb = ofused.rmsnorm_bf16(self.h, self.g, EPS) if norm else self.x
        return oracle.gemv_ref(self.fmt, self.w, self.s, xb, self.M, self.K)


def _parity(y, y_ref, a_ref, what):
    rep = oracle.parity_report(y, y_ref, a_ref)
    assert rep["ok"], f"{what} {rep}"


# (fmt, M, K, B): register-x (B 1, 2), matrix-core (K a multiple of the step,
# B 3..8), LDS dot2 (ragged K at B > 2; long rows at B <= 2)
SHAPES = [
    (qg.Q4_0_G32, 2048, 2048, 1), (qg.Q4_0_G32, 2050, 2048, 2), (qg.Q4_0_G32, 1024, 5632, 1),
    (qg.Q4_0_G32, 2048, 2048, 5), (qg.Q4_0_G32, 1026, 2048 + 32, 3),
    (qg.INT8_G32, 2048, 2048, 1), (qg.INT8_G32, 1536, 8192, 2), (qg.INT8_G32, 2048, 2048, 8),
    (qg.INT8_G32, 1024, 8192, 1),
    (qg.INT4_G128, 2048, 2048, 1), (qg.INT4_G128, 2048, 8192, 4), (qg.INT4_G128, 514, 2048 + 128, 8),
    (qg.BF16, 2048, 2048, 1), (qg.BF16, 1000, 2048, 2), (qg.BF16, 1024, 2048, 3), (qg.BF16, 130, 5664, 6),
    (qg.INT8_ROW, 2048, 2048, 1), (qg.INT8_ROW, 2048, 2048, 8), (qg.INT8_ROW, 512, 2048 + 32, 4),
    (qg.INT4_G64, 2048, 2048, 2), (qg.INT4_G64, 2048, 2048, 5), (qg.INT4_G64, 768, 2048 + 64, 8),
]
IDS = [f"{qg.FMT_NAMES[f]}-{m}x{k}-b{b}" for f, m, k, b in SHAPES]


@pytest.mark.parametrize("fmt,M,K,B", SHAPES, ids=IDS)
def test_fused_norm_residual_swiglu(fmt, M, K, B):
    c = Case(fmt, M, K, B, M + K + B)
    y_ref, a_ref = c.oracle_y(norm=True)
    tol = REL_TOL * a_ref + ABS_TOL

    # RMSNorm prologue, plain store
    y0 = c.run(norm=True)["y"]
    _parity(y0, y_ref, a_ref, "norm")

    # + residual: the same kernel's sums plus one float32 add, bit for bit
    y1 = c.run(norm=True, residual="separate")["y"]
    assert (y1.view(np.uint32) == (c.res + y0).view(np.uint32)).all()
    err = np.abs(y1 - (c.res.astype(np.float64) + y_ref))
    assert (err <= ofused.residual_bound(c.res + y_ref, tol)).all()

    # residual updated in place (residual == y)
    y2 = c.run(norm=True, residual="inplace", y_init=c.res)["y"]
    assert (y2.view(np.uint32) == y1.view(np.uint32)).all()

    # SwiGLU of the paired rows (2i gate, 2i+1 up): y is not written
    act = oracle.bf16_to_f64(c.run(norm=True, swiglu=True)["act"])
    want = ofused.swiglu_ref(y_ref)
    bound = ofused.swiglu_bound(y_ref, tol)
    bad = np.abs(act - want) > bound
    assert not bad.any(), f"swiglu: {bad.sum()} outside the bound, worst {np.max(np.abs(act - want) - bound)}"
    # and against the same kernel's own y: float32 silu and product, one bf16 rounding
    g32, u32 = y0[:, 0::2], y0[:, 1::2]
    mine = (g32 / (np.float32(1) + np.exp(-g32))) * u32
    ulp = np.abs(act - mine.astype(np.float64)) / np.maximum(np.abs(mine.astype(np.float64)), 1e-30)
    assert (ulp <= 2.0 ** -7).all()


@pytest.mark.parametrize("fmt,M,K,B", [(qg.Q4_0_G32, 2048, 2048, 1), (qg.INT8_G32, 2048, 2048, 5),
                                       (qg.BF16, 130, 5664, 6)],
                         ids=["q4-xreg", "int8-mfma", "bf16-lds"])
def test_fused_residual_and_swiglu_without_norm(fmt, M, K, B):
    c = Case(fmt, M, K, B, 7 * M + K)
    y_ref, a_ref = c.oracle_y(norm=False)
    tol = REL_TOL * a_ref + ABS_TOL
    y0 = c.run()["y"]
    _parity(y0, y_ref, a_ref, "plain")
    y1 = c.run(residual="separate")["y"]
    assert (y1.view(np.uint32) == (c.res + y0).view(np.uint32)).all()
    act = oracle.bf16_to_f64(c.run(swiglu=True)["act"])
    assert (np.abs(act - ofused.swiglu_ref(y_ref)) <= ofused.swiglu_bound(y_ref, tol)).all()


@pytest.mark.parametrize("fmt,M,K,B", [(qg.Q4_0_G32, 32000, 2048, 1), (qg.Q4_0_G32, 32000, 2048, 2),
                                       (qg.INT8_G32, 32000, 2048, 8), (qg.BF16, 5000, 2048 + 32, 3)],
                         ids=["q4-b1", "q4-b2", "int8-b8", "bf16-lds-b3"])
def test_fused_lm_head_norm_argmax(fmt, M, K, B):
    """The LM head with its RMSNorm and the argmax of its logits."""
    c = Case(fmt, M, K, B, 3 * M + B)
    for rep in range(2):                          # the workspace is reused
        out = c.run(norm=True, argmax=True)
        assert out["ws_zero"]
        assert (out["idx"] == oracle.argmax_ref(out["y"])).all(), rep
    xb = ofused.rmsnorm_bf16(c.h, c.g, EPS)
    y_ref, a_ref = oracle.gemv_ref(fmt, c.w, c.s, xb, M, K)
    _parity(out["y"], y_ref, a_ref, "lm head")


def test_fused_norm_constant_rows_exact():
    """Constant h rows with eps = 0 normalize to sign(h) * g exactly, so the
    fused result equals a plain run on x = sign(h) * g bit for bit."""
    fmt, M, K, B = qg.Q4_0_G32, 2048, 2048, 2
    c = Case(fmt, M, K, B, 5)
    c.h = np.stack([np.full(K, 0.375, np.float32), np.full(K, -3.0, np.float32)])
    gv = oracle.bf16_to_f64(c.g)
    xb = ofused.f64_to_bf16_bits(np.stack([gv, -gv]))
    kw = dict(norm_input=dev(c.h), norm_weight=dev(c.g), eps=0.0)
    y_n = torch.full((B, M), float("nan"), dtype=torch.float32, device=DEV)
    qg.run_fused(fmt, c.Wd, c.Sd, None, y_n, M, K, B, **kw)
    y_x = torch.full((B, M), float("nan"), dtype=torch.float32, device=DEV)
    qg.run_fused(fmt, c.Wd, c.Sd, dev(xb), y_x, M, K, B)
    torch.cuda.synchronize()
    assert (y_n.cpu().numpy().view(np.uint32) == y_x.cpu().numpy().view(np.uint32)).all()


FUSED_FMTS = [qg.BF16, qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64]
FUSED_K_STEP = {qg.BF16: 32, qg.INT8_G32: 32, qg.Q4_0_G32: 32, qg.INT4_G128: 128, qg.INT8_ROW: 32,
                qg.INT4_G64: 64}


def _random_fused_case(seed):
    """A seeded draw of format, batch, ragged M and K, and the fused operations."""
    rng = np.random.default_rng(7000 + seed)
    fmt = int(rng.choice(FUSED_FMTS))
    B = int(rng.choice([1, 1, 2, 2, 3, 4, 5, 6, 7, 8]))
    step = FUSED_K_STEP[fmt]
    kmax = 8192 if B <= 2 else 4096              # x of the batch staged in LDS where the kernel does
    K = int(step * rng.integers(max(1, 256 // step), kmax // step + 1))
    if rng.random() < 0.4:
        K = int(rng.choice([2048, 4096] + ([5632, 8192] if B <= 2 else []))) // step * step
    epi = str(rng.choice(["plain", "residual", "inplace", "swiglu"]))
    M = int(rng.choice([2, 64, 130, 1000, 2050, 4098, int(rng.integers(1, 6000))]))
    if epi == "swiglu" and M % 2:
        M += 1
    norm = bool(rng.random() < 0.6)
    argmax = epi != "swiglu" and bool(rng.random() < 0.5)
    return fmt, M, K, B, norm, epi, argmax


@pytest.mark.parametrize("seed", range(32))
def test_random_fused_call(seed):
    """Seeded random qgemv_run_fused calls across the three kernels: every row of y
    (or of the SwiGLU activations) against the oracle, the argmax bit-exact on the
    GPU's own logits, and the workspace left zero."""
    fmt, M, K, B, norm, epi, argmax = _random_fused_case(seed)
    c = Case(fmt, M, K, B, 31 * seed + 5)
    y_ref, a_ref = c.oracle_y(norm=norm)
    tol = REL_TOL * a_ref + ABS_TOL
    if epi == "swiglu":
        act = oracle.bf16_to_f64(c.run(norm=norm, swiglu=True)["act"])
        bad = np.abs(act - ofused.swiglu_ref(y_ref)) > ofused.swiglu_bound(y_ref, tol)
        assert not bad.any(), f"swiglu: {int(bad.sum())} outside the bound"
        return
    if epi == "plain":
        out = c.run(norm=norm, argmax=argmax)
        _parity(out["y"], y_ref, a_ref, "plain")
    else:
        out = c.run(norm=norm, argmax=argmax, residual="separate" if epi == "residual" else "inplace",
                    y_init=c.res if epi == "inplace" else None)
        want = c.res.astype(np.float64) + y_ref
        err = np.abs(out["y"] - want)
        assert np.isfinite(out["y"]).all()
        assert (err <= ofused.residual_bound(want, tol)).all(), f"residual: worst {np.max(err)}"
    if argmax:
        assert out["ws_zero"]
        assert (out["idx"] == oracle.argmax_ref(out["y"])).all()
