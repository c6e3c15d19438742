"""A decode step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the TinyLlama decode-step weight stream (89 GEMVs + the LM-head argmax in one
qgemv_run_grouped_argmax call) and the fused layer chain (five dependent
qgemv_run_fused launches), each on two rotation sets with different inputs.

The eager run of the same calls is checked against the float64 oracle (every
row up to 4096 rows, 768 sampled rows of taller outputs - every row of those
shapes is compared in the parity tests); every graph replay must then
reproduce the eager outputs bit for bit (the kernels are deterministic) and
the argmax must equal the oracle's argmax of the replay's own logits. Between
replays the outputs are overwritten with NaN by ordinary eager kernels, so a
replay that skipped a write would show.
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
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def check_rows(M):
    if M <= 4096:
        return None
    rng = np.random.default_rng(M)
    return np.unique(np.concatenate([np.arange(128), np.arange(M - 128, M), rng.choice(M, 512, replace=False)]))


def parity(fmt, w, s, x, M, K, y, what):
    rows = check_rows(M)
    y_ref, a_ref = oracle.gemv_ref(fmt, w, s, x, M, K, rows=rows)
    rep = oracle.parity_report(y if rows is None else y[:, rows], y_ref, a_ref)
    assert rep["ok"], f"{what} {rep}"


def capture(fn):
    """fn(stream) captured into one graph on a side stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn(s)
    torch.cuda.synchronize()
    return g


# ------------------------------------------------- the 89-GEMV decode step
@pytest.mark.parametrize("B", [1, 8])
def test_graph_decode_step_stream_two_sets(B):
    gemvs = synth.make_workload(4, B)
    am = len(gemvs) - 1
    sets = []
    for k in range(2):
        rng = np.random.default_rng(500 + 10 * B + k)
        xs = [synth.bf16_normal(rng, (B, g.K), 1.0) if k else g.x for g in gemvs]
        items = []
        for g, x in zip(gemvs, xs):
            W = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))   # a copy per set
            S = dev(g.s.reshape(-1))
            Y = torch.full((B, g.M), float("nan"), dtype=torch.float32, device=DEV)
            items.append((g.fmt, W, S, dev(x), Y, g.M, g.K))
        ws = qg.fused_argmax_workspace(B)
        idx = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        sets.append((items, qg.grouped_descs(items), ws, idx, xs))

    def step(stream=None):
        for items, descs, ws, idx, _ in sets:
            qg.run_grouped_argmax(descs, B, am, ws, idx, stream=stream)

    def poison():
        for items, _, _, idx, _ in sets:
            for it in items:
                it[4].fill_(float("nan"))
            idx.fill_(-7)

    print(f"[gpu] eager decode step B={B}", flush=True)
    step()
    torch.cuda.synchronize()
    eager = [([it[4].cpu().numpy() for it in items], idx.cpu().numpy()) for items, _, _, idx, _ in sets]
    for (ys, idx), (_, _, ws, _, xs) in zip(eager, sets):
        for g, x, y in zip(gemvs, xs, ys):
            assert np.isfinite(y).all(), g.name
            parity(g.fmt, g.w, g.s, x, g.M, g.K, y, f"eager {g.name}")
        assert (idx == oracle.argmax_ref(ys[am])).all()
        assert bool((ws == 0).all().item())

    graph = capture(step)
    for r in range(REPLAYS):
        poison()
        torch.cuda.synchronize()
        print(f"[gpu] decode step B={B} replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for (ys0, idx0), (items, _, ws, idx, _) in zip(eager, sets):
            for it, y0 in zip(items, ys0):
                assert (it[4].cpu().numpy().view(np.uint32) == y0.view(np.uint32)).all(), r
            got = idx.cpu().numpy()
            assert (got == idx0).all() and (got == oracle.argmax_ref(items[am][4].cpu().numpy())).all(), r
            assert bool((ws == 0).all().item())


# ------------------------------------------------------ the fused chain
class Chain:
    """One TinyLlama-shaped layer and the LM head as five fused launches, every
    intermediate in a buffer of its own so that each op can be checked on the
    GPU's own inputs:
      y_qkv = W_qkv RMSNorm(h0)
      h1    = h0 + W_o x_o
      act   = SwiGLU(W_gate|up RMSNorm(h1))       (gate row 2i, up row 2i+1)
      h2    = h1 + W_down act
      logits = W_lm RMSNorm(h2), idx = argmax(logits)
    """

    def __init__(self, gemvs, B, seed):
        self.gemvs, self.B = gemvs, B
        qkv, o, gu, down, lm = gemvs
        K = qkv.K
        rng = np.random.default_rng(seed)
        self.h0 = rng.standard_normal((B, K)).astype(np.float32)
        self.x_o = synth.bf16_normal(rng, (B, o.K), 1.0)
        self.g = [synth.round_f32_to_bf16_bits(rng.uniform(0.5, 1.5, K).astype(np.float32)) for _ in range(3)]
        self.W = [dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8)) for g in gemvs]
        self.S = [dev(g.s.reshape(-1)) for g in gemvs]
        self.d_h0, self.d_xo = dev(self.h0), dev(self.x_o)
        self.d_g = [dev(x) for x in self.g]
        f32 = dict(dtype=torch.float32, device=DEV)
        self.y_qkv = torch.empty((B, qkv.M), **f32)
        self.h1 = torch.empty((B, o.M), **f32)
        self.act = torch.empty((B, gu.M // 2), dtype=torch.int16, device=DEV)
        self.h2 = torch.empty((B, down.M), **f32)
        self.logits = torch.empty((B, lm.M), **f32)
        self.idx = torch.empty((B,), dtype=torch.int32, device=DEV)
        self.ws = qg.fused_argmax_workspace(B)

    def run(self, stream=None):
        qkv, o, gu, down, lm = self.gemvs
        B = self.B
        qg.run_fused(qkv.fmt, self.W[0], self.S[0], None, self.y_qkv, qkv.M, qkv.K, B,
                     norm_input=self.d_h0, norm_weight=self.d_g[0], eps=EPS, stream=stream)
        qg.run_fused(o.fmt, self.W[1], self.S[1], self.d_xo, self.h1, o.M, o.K, B,
                     residual=self.d_h0, stream=stream)
        qg.run_fused(gu.fmt, self.W[2], self.S[2], None, None, gu.M, gu.K, B,
                     norm_input=self.h1, norm_weight=self.d_g[1], eps=EPS, swiglu_out=self.act, stream=stream)
        qg.run_fused(down.fmt, self.W[3], self.S[3], self.act, self.h2, down.M, down.K, B,
                     residual=self.h1, stream=stream)
        qg.run_fused(lm.fmt, self.W[4], self.S[4], None, self.logits, lm.M, lm.K, B,
                     norm_input=self.h2, norm_weight=self.d_g[2], eps=EPS, argmax_idx=self.idx,
                     argmax_ws=self.ws, stream=stream)

    def outputs(self):
        return {"y_qkv": self.y_qkv.cpu().numpy(), "h1": self.h1.cpu().numpy(),
                "act": self.act.cpu().numpy().view(np.uint16), "h2": self.h2.cpu().numpy(),
                "logits": self.logits.cpu().numpy(), "idx": self.idx.cpu().numpy()}

    def poison(self):
        for t in (self.y_qkv, self.h1, self.h2, self.logits):
            t.fill_(float("nan"))
        self.act.fill_(-1)
        self.idx.fill_(-7)

    def check_against_oracle(self, out):
        qkv, o, gu, down, lm = self.gemvs
        B = self.B
        # qkv on RMSNorm(h0)
        parity(qkv.fmt, qkv.w, qkv.s, ofused.rmsnorm_bf16(self.h0, self.g[0], EPS), qkv.M, qkv.K,
               out["y_qkv"], "qkv+norm")
        # h1 = h0 + W_o x_o (every row: M = 2048)
        y_ref, a_ref = oracle.gemv_ref(o.fmt, o.w, o.s, self.x_o, o.M, o.K)
        want = self.h0.astype(np.float64) + y_ref
        tol = REL_TOL * a_ref + ABS_TOL
        assert (np.abs(out["h1"] - want) <= ofused.residual_bound(want, tol)).all(), "o+residual"
        # act = SwiGLU(W_gu RMSNorm(h1)) on the GPU's own h1
        y_ref, a_ref = oracle.gemv_ref(gu.fmt, gu.w, gu.s, ofused.rmsnorm_bf16(out["h1"], self.g[1], EPS),
                                       gu.M, gu.K)
        act = oracle.bf16_to_f64(out["act"])
        bound = ofused.swiglu_bound(y_ref, REL_TOL * a_ref + ABS_TOL)
        assert (np.abs(act - ofused.swiglu_ref(y_ref)) <= bound).all(), "gate_up+norm+swiglu"
        # h2 = h1 + W_down act, on the GPU's own h1 and act
        y_ref, a_ref = oracle.gemv_ref(down.fmt, down.w, down.s, out["act"], down.M, down.K)
        want = out["h1"].astype(np.float64) + y_ref
        tol = REL_TOL * a_ref + ABS_TOL
        assert (np.abs(out["h2"] - want) <= ofused.residual_bound(want, tol)).all(), "down+residual"
        # logits on RMSNorm of the GPU's own h2; the index bit-exact
        parity(lm.fmt, lm.w, lm.s, ofused.rmsnorm_bf16(out["h2"], self.g[2], EPS), lm.M, lm.K,
               out["logits"], "lm_head+norm")
        assert (out["idx"] == oracle.argmax_ref(out["logits"])).all(), "argmax"
        assert B == out["idx"].size


@pytest.mark.parametrize("B", [1, 8])
def test_graph_fused_chain_two_sets(B):
    gemvs = [synth.make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
             for sp in synth.workload_specs(2)]
    chains = [Chain(gemvs, B, 900 + 10 * B + k) for k in range(2)]
    print(f"[gpu] eager fused chain B={B}", flush=True)
    for c in chains:
        c.run()
    torch.cuda.synchronize()
    eager = [c.outputs() for c in chains]
    for c, out in zip(chains, eager):
        c.check_against_oracle(out)
        assert bool((c.ws == 0).all().item())

    graph = capture(lambda s: [c.run(stream=s) for c in chains])
    for r in range(REPLAYS):
        for c in chains:
            c.poison()
        torch.cuda.synchronize()
        print(f"[gpu] fused chain B={B} replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for c, out0 in zip(chains, eager):
            out = c.outputs()
            for k in ("y_qkv", "h1", "h2", "logits"):
                assert (out[k].view(np.uint32) == out0[k].view(np.uint32)).all(), (r, k)
            assert (out["act"] == out0["act"]).all(), r
            assert (out["idx"] == out0["idx"]).all() and (out["idx"] == oracle.argmax_ref(out["logits"])).all()
            assert bool((c.ws == 0).all().item())


# ------------------------------------------- seeded random captured steps
GRAPH_FMTS = [qg.BF16, qg.INT8_G32, qg.Q4_0_G32, qg.INT4_G128, qg.INT8_ROW, qg.INT4_G64]


def _random_graph_case(seed):
    """A seeded random step: a grouped call (2-8 GEMVs of mixed formats and ragged
    shapes, the fused argmax on one entry) and one decode-attention call."""
    rng = np.random.default_rng(15000 + seed)
    B = int(rng.integers(1, 9))
    gemvs = []
    for i in range(int(rng.integers(2, 9))):
        fmt = int(rng.choice(GRAPH_FMTS))
        step = synth.K_ALIGN[fmt]
        K = int(step * rng.integers(1, 6144 // step + 1))
        M = int(rng.choice([1, 63, 640, 2048, int(rng.integers(1, 9000))]))
        gemvs.append(synth.make_gemv(f"g{i}", fmt, M, K, B, 7, 3000 + 16 * seed + i, "o"))
    am = int(rng.integers(0, len(gemvs)))
    n_kv = int(rng.choice([1, 2, 8]))
    att = (int(rng.integers(1, 9)), n_kv * int(rng.choice([1, 4])), n_kv, int(rng.choice([64, 128])),
           int(rng.choice([33, 512, 2000])))
    return B, gemvs, am, att


@pytest.mark.parametrize("seed", range(8))
def test_graph_random_step(seed):
    """The step eager (against the oracle), then captured in one graph and replayed three
    times with the outputs overwritten in between: every replay reproduces the eager
    outputs bit for bit, the argmax included, and leaves the workspace zero."""
    B, gemvs, am, (Ba, n_q, n_kv, d, T) = _random_graph_case(seed)
    items = []
    for g in gemvs:
        W = dev(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8))
        S = dev(g.s.reshape(-1)) if g.s is not None else None
        Y = torch.full((B, g.M), float("nan"), dtype=torch.float32, device=DEV)
        items.append((g.fmt, W, S, dev(np.ascontiguousarray(g.x).reshape(B, g.K)), Y, g.M, g.K))
    descs = qg.grouped_descs(items)
    ws = qg.fused_argmax_workspace(B)
    idx = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    at = synth.make_attention(Ba, n_q, n_kv, d, T, seed=16000 + seed)
    aq, ak, av, al = dev(at.q), dev(at.k), dev(at.v), dev(at.lens)
    aout = torch.full((Ba, n_q, d), float("nan"), dtype=torch.float32, device=DEV)
    aws = qg.attention_workspace(Ba, n_q, n_kv, d, T)

    def step(stream=None):
        qg.run_grouped_argmax(descs, B, am, ws, idx, stream=stream)
        qg.attention_decode(aq, ak, av, al, aout, Ba, n_q, n_kv, d, T, at.scale, aws, stream=stream)

    def poison():
        for it in items:
            it[4].fill_(float("nan"))
        idx.fill_(-7)
        aout.fill_(float("nan"))

    shapes = " ".join(f"{qg.FMT_NAMES[g.fmt]}:{g.M}x{g.K}" for g in gemvs)
    print(f"[gpu] graph seed={seed} B={B} argmax={am} {shapes} attention B={Ba} {n_q}/{n_kv} d={d} T={T}",
          flush=True)
    step()
    torch.cuda.synchronize()
    ys = [it[4].cpu().numpy() for it in items]
    idx0, a0 = idx.cpu().numpy(), aout.cpu().numpy()
    for g, y in zip(gemvs, ys):
        y_ref, a_ref = oracle.gemv_ref(g.fmt, g.w, g.s, g.x, g.M, g.K)
        rep = oracle.parity_report(y, y_ref, a_ref)
        assert rep["ok"], f"eager {g.name} {rep}"
    assert (idx0 == oracle.argmax_ref(ys[am])).all()
    assert bool((ws == 0).all().item())
    import oracle.attention as oatt
    ref, A = oatt.attention_decode_ref(at.q, at.k, at.v, at.lens, at.scale)
    assert oatt.parity_report(a0, ref, A)["ok"]

    graph = capture(step)
    for r in range(REPLAYS):
        poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for it, y0 in zip(items, ys):
            assert (it[4].cpu().numpy().view(np.uint32) == y0.view(np.uint32)).all(), r
        assert (idx.cpu().numpy() == idx0).all(), r
        assert bool((ws == 0).all().item()), r
        assert (aout.cpu().numpy().view(np.uint32) == a0.view(np.uint32)).all(), r
