"""Bench: fused-dequant decode GEMV throughput on one MI355X (gfx950).

The headline ("step") is the Q4_0-g32 GEMV set at TinyLlama-1.1B decode
shapes (qkv 2560x2048, o 2048x2048, gate_up 11264x2048, down 2048x5632,
lm_head 32000x2048) at batch 1 plus the argmax over the 32000 logits, run as
one qgemv_run_grouped_argmax call. Beside it, the default run measures every
workload the metric names:
  1  bf16 GEMV 2048x2048, batch 1
  2  the headline set at batch 1 (and at batch 8: the matrix-core path)
  3  int8-g32 GEMV set at Llama-3.2-1B shapes, batch 1
  4  the TinyLlama decode-step weight stream (22 layers x 4 GEMVs + LM head
     + argmax) at batch 1, 2, 4, 8
  5  int4-g128 FFN + int8-g32 LM head 128256x2048 + argmax, batch 1 and 8
each GEMV of workloads 1-3 also alone, every figure next to the streaming-read
kernel over the same number of bytes (the size-matched ceiling: what one
launch of that size can reach on this GPU) and the measured peak over 4 GiB.

Inputs are synthetic and seeded (synth), resident in HBM before timing, and
rotated through >= 1 GiB of distinct device copies so that the 256 MB
Infinity Cache cannot serve them. Every figure is timed the same way: a HIP
graph of N calls rotating through the copies is captured once, replayed once
untimed, then replayed in `--trials` trials, each bracketed by events on the
launch stream; a trial's time / N is one sample, and the figure is the
median sample with the 10th and 90th percentiles. The headline's graph holds
exactly --steps steps (after a graph of --warmup steps).

Reported (one JSON line):
  value            algorithmic bytes per step / median time per step (GB/s)
  value_sequential the same GEMVs as a dependent chain: one launch per GEMV,
                   then the argmax launch
  roofline         the dominant kernel (the headline step is one launch)
  configs          per workload: us, GB/s, % of the measured peak, % of the
                   8 TB/s spec, and the size-matched ceiling
  measured_peak    best median rate of the streaming-read kernel over 4 GiB
  cpu_baseline     the fp64 CPU oracle on whole steps, all cores and one thread
  lm_head_alone    a 128256x2048 GEMV (the Llama-3.2-1B LM head shape) alone at
                   batch 1 in bf16, int8-g32 and Q4_0-g32: the per-format
                   fraction of the measured peak at a size one launch can reach
Algorithmic bytes per GEMV = code bytes + scale bytes + x (2*B*K) + y (4*B*M);
a separate argmax = 4*B*V read + 4*B written; a fused argmax = 4*B written.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic.json")
WORKLOAD_KEYS = {1: "bf16_gemv_2048x2048", 2: "q4_0_g32_tinyllama_gemv_set+argmax",
                 3: "int8_g32_llama32_1b_gemv_set", 4: "q4_0_g32_tinyllama_decode_step_89_gemvs+argmax",
                 5: "int4_g128_ffn+int8_g32_lm_head+argmax",
                 6: "q4_0_g32_llama32_1b_layer_gemvs+int8_row_lm_head+argmax"}


def recorded_traffic(kernel_label, workload_name, batch):
    """HBM bytes per launch from the committed counter runs, if they were taken on the
    current GEMV source and this kernel/workload; else None."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    if rec.get("kernel") != kernel_label or rec.get("workload") != workload_name or rec.get("batch") != batch:
        return None
    return int(rec["hbm_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--trials", type=int, default=11, help="timed replays per figure (median, p10, p90)")
    p.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5, 6],
                   help="time only this workload's step (focused run, e.g. under a profiler)")
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peak", action="store_true")
    p.add_argument("--peak-gib", type=float, default=4.0)
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="per CPU leg")
    p.add_argument("--per-kernel", action="store_true", help="focused run: also time every GEMV alone")
    p.add_argument("--no-attention", action="store_true", help="skip the decode-attention measurements")
    p.add_argument("--no-fused-layer", action="store_true", help="skip the fused decode-layer chain")
    p.add_argument("--no-lm-heads", action="store_true", help="skip the 128256x2048 LM heads alone")
    p.add_argument("--pmc-pass", action="store_true",
                   help="only run calibration kernels (a 64 MiB streaming read, a 64 MiB fill) and "
                        "--steps eager steps of --workload, for hardware-counter collection")
    p.add_argument("--size-sweep", action="store_true",
                   help="only time the streaming-read kernel at GEMV-like sizes (size-matched ceilings)")
    return p.parse_args()


def gemv_bytes(qg, fmt, M, K, B):
    w, s = qg.packed_size(fmt, M, K)
    return w + s + 2 * B * K + 4 * B * M


def stats(samples):
    a = np.asarray(samples, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def capture(torch, fn, count):
    """Capture fn(i, stream) for i in range(count) into one graph on a side stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0, s.cuda_stream)          # eager warm call (loads code objects)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(count):
            fn(i, h)
    torch.cuda.synchronize()
    return g


def replay_ms(torch, g):
    """One timed replay of g (events on the stream the graph is launched on)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_calls(torch, fn, count, trials):
    """Median / p10 / p90 over `trials` replays of a graph of `count` calls, in us per call."""
    g = capture(torch, fn, count)
    replay_ms(torch, g)
    samples = [replay_ms(torch, g) * 1e3 / count for _ in range(trials)]
    del g
    return stats(samples)


def rate(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


# ------------------------------------------------------------------ inputs
class Weights:
    """Device copies of a workload's codes and scales, n_sets distinct copies."""

    def __init__(self, torch, gemvs, rotate_bytes):
        self.gemvs = gemvs
        resident = sum(g.w.nbytes + (g.s.nbytes if g.s is not None else 0) for g in gemvs)
        self.resident = resident
        self.n_sets = max(1, math.ceil(rotate_bytes / resident))
        base = []
        for g in gemvs:
            W = torch.from_numpy(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8)).to("cuda")
            S = torch.from_numpy(g.s.reshape(-1).view(np.int16)).to("cuda") if g.s is not None else None
            base.append((W, S))
        self.sets = [base] + [[(W.clone(), None if S is None else S.clone()) for W, S in base]
                              for _ in range(self.n_sets - 1)]
        torch.cuda.synchronize()


class Workload:
    """One workload at one batch: device weights (shared across batches), x, y,
    argmax buffers per rotation set, and the call descriptors."""

    def __init__(self, qg, torch, cfg, B, weights: Weights):
        self.qg, self.torch, self.cfg, self.B = qg, torch, cfg, B
        self.gemvs = weights.gemvs
        self.n_sets = weights.n_sets
        self.has_argmax = synth.WORKLOAD_ARGMAX[cfg]
        self.bytes = [gemv_bytes(qg, g.fmt, g.M, g.K, B) for g in self.gemvs]
        self.argmax_bytes = 4 * B * self.gemvs[-1].M + 4 * B if self.has_argmax else 0
        self.step_bytes = sum(self.bytes) + self.argmax_bytes
        # with the argmax inside the LM head's launch the logits are not read again
        self.fused_bytes = sum(self.bytes) + (4 * B if self.has_argmax else 0)
        self.resident = weights.resident
        dev = "cuda"
        xs = [torch.from_numpy(np.ascontiguousarray(g.x[:B]).view(np.int16)).to(dev) for g in self.gemvs]
        self.sets = []
        for i in range(self.n_sets):
            items = []
            for (W, S), X, g in zip(weights.sets[i], xs, self.gemvs):
                Xi = X if i == 0 else X.clone()
                Y = torch.empty((B, g.M), dtype=torch.float32, device=dev)
                items.append((W, S, Xi, Y))
            ws = qg.fused_argmax_workspace(B) if self.has_argmax else None
            idx = torch.empty(B, dtype=torch.int32, device=dev) if self.has_argmax else None
            self.sets.append((items, ws, idx))
        torch.cuda.synchronize()
        # launch classes of qgemv_run_grouped: one small-batch launch per format,
        # one matrix-core launch per format and K, one launch each for the others
        self.classes = {}
        for j, g in enumerate(self.gemvs):
            cls = qg.grouped_class(g.fmt, g.K, B)
            key = ((g.fmt, "grouped") if cls == qg.GROUP_XREG else
                   (g.fmt, g.K, "mfma") if cls == qg.GROUP_MFMA else ("alone", j))
            self.classes.setdefault(key, []).append(j)
        self.descs = []
        for items, _, _ in self.sets:
            ent = [(g.fmt, W, S, X, Y, g.M, g.K) for (W, S, X, Y), g in zip(items, self.gemvs)]
            self.descs.append(qg.grouped_descs(ent))
        # raw pointers for the launch loop (argument marshalling only)
        self.ptrs = []
        for items, ws, idx in self.sets:
            p = [(W.data_ptr(), None if S is None else S.data_ptr(), X.data_ptr(), Y.data_ptr())
                 for W, S, X, Y in items]
            self.ptrs.append((p, ws.data_ptr() if ws is not None else None,
                              idx.data_ptr() if idx is not None else None))

    def step(self, i, stream_handle):
        """One qgemv_run launch per GEMV (as a chain of dependent GEMVs must run), then
        the argmax launch."""
        qg = self.qg
        p, wsp, ip = self.ptrs[i % self.n_sets]
        for (wp, sp, xp, yp), g in zip(p, self.gemvs):
            qg.run_ptr(g.fmt, wp, sp, xp, yp, g.M, g.K, self.B, stream_handle)
        if self.has_argmax:
            st = qg.lib().qgemv_argmax(p[-1][3], self.gemvs[-1].M, self.B, wsp, ip, stream_handle)
            if st != qg.OK:
                raise qg.QgemvError(st, "qgemv_argmax")

    def step_grouped(self, i, stream_handle):
        """All GEMVs in one qgemv_run_grouped call, then the argmax launch."""
        qg = self.qg
        p, wsp, ip = self.ptrs[i % self.n_sets]
        qg.run_grouped_ptr(self.descs[i % self.n_sets], self.B, stream_handle)
        if self.has_argmax:
            st = qg.lib().qgemv_argmax(p[-1][3], self.gemvs[-1].M, self.B, wsp, ip, stream_handle)
            if st != qg.OK:
                raise qg.QgemvError(st, "qgemv_argmax")

    def step_fused(self, i, stream_handle):
        """The GEMVs and the LM-head argmax in one qgemv_run_grouped_argmax call."""
        p, wsp, ip = self.ptrs[i % self.n_sets]
        self.qg.run_grouped_argmax_ptr(self.descs[i % self.n_sets], self.B, len(self.gemvs) - 1, wsp, ip,
                                       stream_handle)

    def best_step(self):
        """The call a decode step of independent GEMVs uses, and its bytes."""
        if self.has_argmax:
            return self.step_fused, self.fused_bytes
        return self.step_grouped, self.step_bytes

    def launch_one(self, j, i, stream_handle):
        g = self.gemvs[j]
        wp, sp, xp, yp = self.ptrs[i % self.n_sets][0][j]
        self.qg.run_ptr(g.fmt, wp, sp, xp, yp, g.M, g.K, self.B, stream_handle)

    def launch_count(self, k=4, lo=64):
        return max(self.n_sets * k, lo)


class FusedLayer:
    """The decode-layer chain of the TinyLlama set with the fused prologue and
    epilogues ("infer": pipeline figure): qkv = W_qkv RMSNorm(h); h += W_o attn;
    act = SwiGLU(W_gate|up RMSNorm(h)); h += W_down act; logits = W_lm RMSNorm(h)
    and their argmax: five dependent qgemv_run_fused launches. Uses the
    workload's rotation sets (qkv, o, gate_up with gate/up rows paired, down,
    lm_head); h is a float32 residual stream per set, updated in place."""

    def __init__(self, qg, torch, wl):
        assert [g.name for g in wl.gemvs] == ["qkv", "o", "gate_up", "down", "lm_head"]
        self.qg, self.wl, self.B = qg, wl, wl.B
        B, K = wl.B, wl.gemvs[0].K
        rng = np.random.default_rng(77)
        dev = "cuda"
        self.norm_w = [torch.from_numpy(synth.round_f32_to_bf16_bits(
            rng.uniform(0.5, 1.5, K).astype(np.float32)).view(np.int16)).to(dev) for _ in range(3)]
        F = wl.gemvs[2].M // 2
        self.bufs = []
        for items, ws, idx in wl.sets:
            h = torch.from_numpy(rng.standard_normal((B, K)).astype(np.float32)).to(dev)
            act = torch.zeros((B, F), dtype=torch.int16, device=dev)
            self.bufs.append((h, act))
        torch.cuda.synchronize()
        g = wl.gemvs
        w = lambda j: sum(qg.packed_size(g[j].fmt, g[j].M, g[j].K))     # noqa: E731
        self.bytes = (w(0) + 4 * B * K + 2 * K + 4 * B * g[0].M             # qkv: h, g in; y out
                      + w(1) + 2 * B * g[1].K + 8 * B * g[1].M              # o: x in; h read + written
                      + w(2) + 4 * B * K + 2 * K + 2 * B * F                # gate_up: h, g in; act out
                      + w(3) + 2 * B * g[3].K + 8 * B * g[3].M              # down: act in; h read + written
                      + w(4) + 4 * B * K + 2 * K + 4 * B * g[4].M + 4 * B)  # lm_head: h, g in; logits, idx
        self.fusions = []
        for (items, ws, idx), (h, act) in zip(wl.sets, self.bufs):
            f = []
            for kind in range(5):
                fu = qg.Fusion()
                if kind in (0, 2, 4):
                    fu.norm_input = h.data_ptr()
                    fu.norm_weight = self.norm_w[kind // 2].data_ptr()
                    fu.norm_eps = 1e-5
                if kind in (1, 3):
                    fu.residual = h.data_ptr()
                if kind == 2:
                    fu.swiglu_out = act.data_ptr()
                if kind == 4:
                    fu.argmax_idx = idx.data_ptr()
                    fu.argmax_ws = ws.data_ptr()
                f.append(fu)
            self.fusions.append(f)

    NAMES = ["qkv+norm", "o+residual", "gate_up+norm+swiglu", "down+residual", "lm_head+norm+argmax"]

    def op(self, k, i, stream_handle):
        """Launch op k (0..4) of the chain on rotation set i."""
        qg, wl, B = self.qg, self.wl, self.B
        s = i % wl.n_sets
        wp, sp, xp, yp = wl.ptrs[s][0][k]
        h, act = self.bufs[s]
        g = wl.gemvs[k]
        x = {1: xp, 3: act.data_ptr()}.get(k)
        y = {0: yp, 1: h.data_ptr(), 3: h.data_ptr(), 4: yp}.get(k)
        qg.run_fused_ptr(g.fmt, wp, sp, x, y, g.M, g.K, B, self.fusions[s][k], stream_handle)

    def step(self, i, stream_handle):
        for k in range(5):
            self.op(k, i, stream_handle)


# -------------------------------------------------------- streaming reads
class StreamCeiling:
    """The streaming-read kernel over n bytes, rotated through >= rotate_bytes of
    distinct buffers: the size-matched ceiling of a launch that moves n bytes.
    Best median over a small grid x loads-in-flight sweep; one pool, reused."""

    def __init__(self, qg, torch, rotate_bytes, trials):
        self.qg, self.torch, self.trials = qg, torch, trials
        self.rotate_bytes = int(rotate_bytes)
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count
        self.pool = torch.full((self.rotate_bytes // 4 + (1 << 20),), 3, dtype=torch.int32, device="cuda")
        self.sink = torch.zeros(64 * self.cus, dtype=torch.int32, device="cuda")
        self.cache = {}

    def __call__(self, nbytes):
        nbytes = max(4096, int(nbytes) // 4096 * 4096)
        if nbytes in self.cache:
            return self.cache[nbytes]
        qg, torch = self.qg, self.torch
        n = max(2, min(512, self.rotate_bytes // nbytes))
        if n * nbytes > self.pool.numel() * 4:
            n = max(1, self.pool.numel() * 4 // nbytes)
        base = self.pool.data_ptr()
        best = None
        for grid in (2 * self.cus, 4 * self.cus, 8 * self.cus):
            for unroll in (1, 2, 4):
                def fn(i, h, grid=grid, unroll=unroll):
                    st = qg.lib().qgemv_stream_read(base + (i % n) * nbytes, nbytes, self.sink.data_ptr(),
                                                    grid, unroll, h)
                    if st != qg.OK:
                        raise qg.QgemvError(st, "qgemv_stream_read")
                s = time_calls(torch, fn, max(2 * n, 32), self.trials)
                if best is None or s["median"] < best[0]["median"]:
                    best = (s, grid, unroll)
        s, grid, unroll = best
        out = {"us": round(s["median"], 3), "GBps": round(rate(nbytes, s["median"]), 1), "bytes": nbytes,
               "grid": grid, "unroll": unroll}
        self.cache[nbytes] = out
        return out


def measure_peak(qg, torch, gib, trials):
    """Best median streaming-read rate over a gib-GiB buffer, sweeping grid and loads in flight."""
    nbytes = int(gib * (1 << 30)) // 16 * 16
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(64 * cus, dtype=torch.int32, device="cuda")
    best = (0.0, None)
    h = torch.cuda.current_stream().cuda_stream
    for grid_per_cu in (4, 8, 16, 32):
        for unroll in (2, 4, 8, 16):
            grid = grid_per_cu * cus
            qg.stream_read(buf, nbytes, sink, grid=grid, unroll=unroll)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            times = []
            for _ in range(trials):
                e0.record()
                qg.lib().qgemv_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, unroll, h)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = float(np.median(times))
            gbps = nbytes / (ms * 1e-3) / 1e9
            if gbps > best[0]:
                best = (gbps, {"grid": grid, "unroll": unroll, "ms": round(ms, 4),
                               "p10_GBps": round(nbytes / (np.percentile(times, 90) * 1e-3) / 1e9, 1),
                               "p90_GBps": round(nbytes / (np.percentile(times, 10) * 1e-3) / 1e9, 1)})
    del buf
    torch.cuda.empty_cache()
    return best[0], best[1]


def size_sweep(qg, torch, rotate_bytes, trials):
    ceil = StreamCeiling(qg, torch, rotate_bytes, trials)
    for mb in (1, 2, 2.36, 4, 8, 13, 16, 32, 37, 64, 128, 256):
        r = ceil(int(mb * (1 << 20)))
        r["MiB"] = mb
        print(json.dumps(r), flush=True)


def pmc_pass(qg, torch, wl, steps):
    """Kernels of known traffic for scaling the HBM byte counters, then eager steps as
    `value` times them."""
    nbytes = 64 << 20
    buf = torch.full((nbytes // 4,), 7, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    qg.stream_read(buf, nbytes, sink, grid=2048, unroll=1)       # reads exactly 64 MiB
    buf.fill_(3)                                                   # writes exactly 64 MiB
    torch.cuda.synchronize()
    h = torch.cuda.current_stream().cuda_stream
    fn, _ = wl.best_step()
    for i in range(steps):
        fn(i, h)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": True, "calib_bytes": nbytes, "steps": steps,
                      "gemvs": [[g.name, g.M, g.K, b] for g, b in zip(wl.gemvs, wl.bytes)]}), flush=True)


def attention_bench(qg, torch, rotate_bytes, trials):
    """Grouped-query decode attention at Llama-3.2-1B's heads (32 query, 8 key/value,
    head dim 64): the infer page's contexts 512 and 2048 at batch 1, longer contexts,
    and batch 8. Each configuration rotates through >= rotate_bytes of distinct caches;
    bytes per call = the K and V rows read + q + out."""
    n_q, n_kv, d = 32, 8, 64
    out = []
    for B, T in ((1, 512), (1, 2048), (1, 8192), (1, 32768), (8, 2048)):
        per = 2 * B * n_kv * T * d * 2
        n = max(2, math.ceil(rotate_bytes / per))
        at = synth.make_attention(B, n_q, n_kv, d, T, seed=T + B, lens=[T] * B)
        k0 = torch.from_numpy(at.k.view(np.int16)).to("cuda")
        v0 = torch.from_numpy(at.v.view(np.int16)).to("cuda")
        ks = [k0] + [k0.clone() for _ in range(n - 1)]
        vs = [v0] + [v0.clone() for _ in range(n - 1)]
        q = torch.from_numpy(at.q).to("cuda")
        lens = torch.from_numpy(at.lens).to("cuda")
        o = torch.empty((B, n_q, d), dtype=torch.float32, device="cuda")
        ws = qg.attention_workspace(B, n_q, n_kv, d, T)
        torch.cuda.synchronize()

        def fn(i, h):
            st = qg.lib().qgemv_attention_decode(q.data_ptr(), ks[i % n].data_ptr(), vs[i % n].data_ptr(),
                                                 lens.data_ptr(), o.data_ptr(), B, n_q, n_kv, d, T, at.scale,
                                                 ws.data_ptr(), h)
            if st != qg.OK:
                raise qg.QgemvError(st, "qgemv_attention_decode")
        s = time_calls(torch, fn, max(n * 2, 64), trials)
        nbytes = per + 2 * B * n_q * d * 4
        out.append({"batch": B, "ctx": T, "heads": [n_q, n_kv, d], "us": round(s["median"], 3),
                    "p10_us": round(s["p10"], 3), "p90_us": round(s["p90"], 3), "bytes": nbytes,
                    "GBps": round(rate(nbytes, s["median"]), 1)})
        print(f"[bench] attention B={B} ctx={T}: {s['median']:.2f} us, {out[-1]['GBps']} GB/s",
              file=sys.stderr, flush=True)
        del ks, vs
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ CPU baseline
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_leg(gemvs, has_argmax, seconds, threads):
    """The oracle (fp64 dequantize + fp64 GEMV + argmax) on whole steps. threads=None:
    the BLAS/OpenMP pools as the process found them (all the cores it may use)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    def run():
        t0 = time.perf_counter()
        steps = 0
        while True:
            last = None
            for g in gemvs:
                last, _ = oracle.gemv_ref(g.fmt, g.w, g.s, g.x, g.M, g.K)
            if has_argmax:
                oracle.argmax_ref(last.astype(np.float32))
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds or steps >= 50:
                return steps, el
    if threads is None:
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        steps, el = run()
    else:
        with threadpool_limits(threads):
            used = threads
            steps, el = run()
    return steps, el, used


# --------------------------------------------------------------- figures
def figure(nbytes, s, peak, ceil=None):
    us = s["median"]
    gbps = rate(nbytes, us)
    out = {"us": round(us, 3), "p10_us": round(s["p10"], 3), "p90_us": round(s["p90"], 3),
           "bytes": int(nbytes), "GBps": round(gbps, 1), "pct_of_spec_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2)}
    if peak:
        out["pct_of_measured_peak"] = round(100 * gbps / peak, 2)
    if ceil is not None:
        out["stream_ceiling"] = {"us": ceil["us"], "GBps": ceil["GBps"]}
        out["pct_of_size_matched_ceiling"] = round(100 * ceil["us"] / us, 1)
    return out


def workload_figures(qg, torch, cfg, batches, weights, trials, peak, ceil, per_gemv):
    """Every batch of one workload: its decode step as one call (and, at the first
    batch, every GEMV alone when per_gemv)."""
    out = {"workload": WORKLOAD_KEYS[cfg], "gemvs": [[g.name, g.M, g.K] for g in weights.gemvs][:6] +
           ([["...", len(weights.gemvs)]] if len(weights.gemvs) > 6 else []),
           "rotation_sets": weights.n_sets}
    for B in batches:
        wl = Workload(qg, torch, cfg, B, weights)
        fn, nb = wl.best_step()
        s = time_calls(torch, fn, wl.launch_count(2, 32), trials)
        f = figure(nb, s, peak, ceil(nb) if ceil else None)
        f["call"] = "qgemv_run_grouped_argmax" if wl.has_argmax else "qgemv_run_grouped"
        out[f"B{B}"] = f
        print(f"[bench] workload {cfg} B={B}: {f['us']:.2f} us, {f['GBps']} GB/s", file=sys.stderr, flush=True)
        if per_gemv and B == batches[0] and len(wl.gemvs) > 1:
            rows = []
            for j, g in enumerate(wl.gemvs):
                sj = time_calls(torch, lambda i, h, j=j: wl.launch_one(j, i, h), wl.launch_count(4, 64), trials)
                fj = figure(wl.bytes[j], sj, peak, ceil(wl.bytes[j]) if ceil else None)
                fj.update({"name": g.name, "M": g.M, "K": g.K})
                rows.append(fj)
            out[f"B{B}"]["per_gemv"] = rows
        del wl
    torch.cuda.empty_cache()
    return out


def focused(qg, torch, args):
    """--workload N: the step of one workload at one batch (and optionally every GEMV
    alone), for profiler runs."""
    cfg = args.workload
    B = args.batch if args.batch is not None else synth.WORKLOAD_BATCHES[cfg][0]
    weights = Weights(torch, synth.make_workload(cfg, max(B, 1)), args.rotate_gib * (1 << 30))
    wl = Workload(qg, torch, cfg, B, weights)
    if args.pmc_pass:
        pmc_pass(qg, torch, wl, args.steps)
        return
    fn, nb = wl.best_step()
    warm = capture(torch, fn, max(1, args.warmup))
    replay_ms(torch, warm)
    g = capture(torch, fn, args.steps)
    samples = [replay_ms(torch, g) / args.steps for _ in range(args.trials)]
    s = stats(samples)
    out = {"workload": WORKLOAD_KEYS[cfg], "batch": B, "ms_per_step": round(s["median"], 6),
           "p10_ms": round(s["p10"], 6), "p90_ms": round(s["p90"], 6), "bytes_per_step": nb,
           "GBps": round(rate(nb, s["median"] * 1e3), 1)}
    if args.per_kernel:
        out["per_gemv"] = []
        for j, gm in enumerate(wl.gemvs):
            sj = time_calls(torch, lambda i, h, j=j: wl.launch_one(j, i, h), wl.launch_count(4, 64), args.trials)
            out["per_gemv"].append({"name": gm.name, "M": gm.M, "K": gm.K, "us": round(sj["median"], 3),
                                    "GBps": round(rate(wl.bytes[j], sj["median"]), 1)})
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "qgemv runs on one GPU; a step is not sharded across GPUs, "
                          "so --gpus above 1 is not supported",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch
    import bandwidth_bound_quantized_amd as qg

    torch.cuda.set_device(0)
    rotate = args.rotate_gib * (1 << 30)
    if args.size_sweep:
        size_sweep(qg, torch, rotate, args.trials)
        return
    if args.workload is not None:
        focused(qg, torch, args)
        return
    t_start = time.perf_counter()

    peak = None
    if not args.no_peak:
        peak_gbps, peak_cfg = measure_peak(qg, torch, args.peak_gib, max(args.trials, 7))
        peak = {"GBps": round(peak_gbps, 1), "config": peak_cfg, "buffer_GiB": args.peak_gib}
        print(f"[bench] measured streaming-read peak {peak_gbps:.1f} GB/s {peak_cfg}", file=sys.stderr, flush=True)
    pk = peak["GBps"] if peak else None
    ceil = StreamCeiling(qg, torch, rotate, args.trials)

    # ---- the headline: workload 2 at batch 1, graphs of exactly --steps steps
    w2 = Weights(torch, synth.make_workload(2, 8), rotate)
    wl = Workload(qg, torch, 2, 1, w2)
    print(f"[bench] workload 2 B=1: {len(wl.gemvs)} GEMVs, {wl.fused_bytes} B/step, {wl.n_sets} rotation sets",
          file=sys.stderr, flush=True)
    modes = {}
    for mode, fn in (("fused", wl.step_fused), ("grouped", wl.step_grouped), ("sequential", wl.step)):
        warm = capture(torch, fn, max(1, args.warmup))
        replay_ms(torch, warm)
        del warm
        g = capture(torch, fn, args.steps)
        modes[mode] = stats([replay_ms(torch, g) / args.steps for _ in range(args.trials)])
        del g
        nb = wl.fused_bytes if mode == "fused" else wl.step_bytes
        print(f"[bench] {mode}: {modes[mode]['median'] * 1e3:.2f} us/step, "
              f"{rate(nb, modes[mode]['median'] * 1e3):.1f} GB/s", file=sys.stderr, flush=True)
    ms_per_step = modes["fused"]["median"]
    fused_bytes, step_bytes = wl.fused_bytes, wl.step_bytes
    value = rate(fused_bytes, ms_per_step * 1e3)

    # per GEMV alone (the same inputs), and the step's ceiling
    per_gemv = []
    for j, g in enumerate(wl.gemvs):
        sj = time_calls(torch, lambda i, h, j=j: wl.launch_one(j, i, h), wl.launch_count(4, 64), args.trials)
        fj = figure(wl.bytes[j], sj, pk, ceil(wl.bytes[j]))
        fj.update({"name": g.name, "M": g.M, "K": g.K})
        per_gemv.append(fj)

    fused_layer = None
    if not args.no_fused_layer:
        fl = FusedLayer(qg, torch, wl)
        s = time_calls(torch, fl.step, wl.launch_count(2, 32), args.trials)
        fused_layer = {
            "chain": "qkv(RMSNorm) -> o(+=residual) -> gate_up(RMSNorm, SwiGLU of paired rows) -> "
                     "down(+=residual) -> lm_head(RMSNorm, argmax): 5 dependent qgemv_run_fused launches",
            "us_per_step": round(s["median"], 3), "p10_us": round(s["p10"], 3), "p90_us": round(s["p90"], 3),
            "bytes_per_step": fl.bytes, "GBps": round(rate(fl.bytes, s["median"]), 1),
            "plain_sequential_us_per_step": round(modes["sequential"]["median"] * 1e3, 3)}
        print(f"[bench] fused layer chain: {s['median']:.2f} us/step", file=sys.stderr, flush=True)
        del fl
    del wl

    # ---- every workload the metric names
    configs = {}
    w1 = Weights(torch, synth.make_workload(1, 1), rotate)
    configs["1"] = workload_figures(qg, torch, 1, [1], w1, args.trials, pk, ceil, False)
    del w1
    b1 = figure(fused_bytes, {k: v * 1e3 for k, v in modes["fused"].items() if k != "n"}, pk, ceil(fused_bytes))
    b1.update({"call": "qgemv_run_grouped_argmax", "per_gemv": per_gemv})
    configs["2"] = {"workload": WORKLOAD_KEYS[2], "gemvs": [[g.name, g.M, g.K] for g in w2.gemvs],
                    "rotation_sets": w2.n_sets, "B1": b1}
    b8 = workload_figures(qg, torch, 2, [8], w2, args.trials, pk, ceil, False)
    configs["2"]["B8"] = b8["B8"]
    del w2
    torch.cuda.empty_cache()
    w3 = Weights(torch, synth.make_workload(3, 1), rotate)
    configs["3"] = workload_figures(qg, torch, 3, [1], w3, args.trials, pk, ceil, True)
    del w3
    torch.cuda.empty_cache()
    w4 = Weights(torch, synth.make_workload(4, 8), rotate)
    configs["4"] = workload_figures(qg, torch, 4, [1, 2, 4, 8], w4, args.trials, pk, ceil, False)
    del w4
    torch.cuda.empty_cache()
    w5 = Weights(torch, synth.make_workload(5, 8), rotate)
    configs["5"] = workload_figures(qg, torch, 5, [1, 8], w5, args.trials, pk, ceil, False)
    del w5
    torch.cuda.empty_cache()

    # ---- the batch-1 fraction-of-peak targets per format, at a size one launch can reach
    # them: the Llama-3.2-1B LM head shape (128256 x 2048) alone through qgemv_run
    lm_heads = None
    if not args.no_lm_heads:
        lm_heads = {}
        for fmt in (synth.BF16, synth.INT8_G32, synth.Q4_0_G32):
            g = synth.make_gemv("lm_head", fmt, 128256, 2048, 1, 5, 0, "lm_head")
            wh = Weights(torch, [g], rotate)
            wl = Workload(qg, torch, 1, 1, wh)
            s = time_calls(torch, lambda i, h: wl.launch_one(0, i, h), wl.launch_count(4, 32), args.trials)
            f = figure(wl.bytes[0], s, pk, ceil(wl.bytes[0]))
            f.update({"M": g.M, "K": g.K, "call": "qgemv_run", "rotation_sets": wh.n_sets})
            lm_heads[synth.FMT_NAMES[fmt]] = f
            print(f"[bench] {synth.FMT_NAMES[fmt]} 128256x2048 alone: {f['us']:.2f} us, {f['GBps']} GB/s",
                  file=sys.stderr, flush=True)
            del wl, wh, g
            torch.cuda.empty_cache()

    attention = None
    if not args.no_attention:
        attention = attention_bench(qg, torch, rotate, args.trials)

    cpu = None
    if not args.no_cpu_baseline:
        g2 = synth.make_workload(2, 1)
        nbytes = sum(gemv_bytes(qg, g.fmt, g.M, g.K, 1) for g in g2) + 4 * 32000 + 4
        steps_a, el_a, used_a = cpu_leg(g2, True, args.cpu_seconds, None)
        steps_1, el_1, _ = cpu_leg(g2, True, args.cpu_seconds, 1)
        cpu = {"value": round(nbytes * steps_a / el_a / 1e9, 4), "unit": "GB/s", "cores": int(used_a),
               "kind": "oracle",
               "sample": f"{steps_a} whole step(s) of the Q4_0 TinyLlama set at batch 1 (5 GEMVs + argmax), "
                         f"fp64, {el_a:.1f} s, BLAS threads as found ({used_a})",
               "cpu_model": cpu_model(), "cores_available": len(os.sched_getaffinity(0)),
               "one_thread": {"value": round(nbytes * steps_1 / el_1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{steps_1} whole step(s), {el_1:.1f} s"}}
        print(f"[bench] cpu oracle: {cpu['value']} GB/s ({used_a} threads), "
              f"{cpu['one_thread']['value']} GB/s (1 thread)", file=sys.stderr, flush=True)

    traffic = recorded_traffic("qgemv_run_grouped_argmax launch [qkv+o+gate_up+down+lm_head+argmax]",
                               WORKLOAD_KEYS[2], 1)
    dom_us = ms_per_step * 1e3
    out = {
        "metric": "fused-dequant GEMV achieved HBM GB/s and % of peak (bf16/int8/Q4_0, batch 1)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "p10_ms_per_step": round(modes["fused"]["p10"], 6),
        "p90_ms_per_step": round(modes["fused"]["p90"], 6),
        "trials": args.trials,
        "value_sequential": round(rate(step_bytes, modes["sequential"]["median"] * 1e3), 1),
        "ms_per_step_sequential": round(modes["sequential"]["median"], 6),
        "value_grouped_separate_argmax": round(rate(step_bytes, modes["grouped"]["median"] * 1e3), 1),
        "ms_per_step_grouped_separate_argmax": round(modes["grouped"]["median"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0",
        "data": "synthetic (seeded; same shapes and value distributions as the workload)",
        "config": {"workload": WORKLOAD_KEYS[2], "batch": 1,
                   "gemvs": configs["2"]["gemvs"],
                   "bytes_per_step": int(fused_bytes),
                   "execution": "value: the step's independent GEMVs and the LM-head argmax in one "
                                "qgemv_run_grouped_argmax call (one launch; the argmax inside it); "
                                "value_sequential: the dependent-chain figure, one qgemv_run launch per "
                                "GEMV then qgemv_argmax; value_grouped_separate_argmax: qgemv_run_grouped "
                                "+ qgemv_argmax",
                   "timing": f"median (p10, p90) of {args.trials} trials, each one replay of a HIP graph "
                             f"of exactly `steps` steps after a graph of `warmup` steps; events on the "
                             f"launch stream"},
        "pct_of_spec_8TBps": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "gemv_xreg_group_kernel<Q4_0, 1 batch row, argmax> "
                               "(qgemv_run_grouped_argmax: the whole step is this one launch)",
                     "bytes_per_launch": int(fused_bytes), "avg_launch_us": round(dom_us, 3),
                     "timing": "the headline's median step (one launch per step), graph-replayed"},
        "cpu_baseline": cpu,
        "configs": configs,
    }
    if peak is not None:
        out["measured_peak"] = peak
        out["pct_of_measured_peak"] = round(100 * value / peak["GBps"], 2)
        out["roofline"]["pct_of_measured_peak"] = round(100 * value / peak["GBps"], 2)
    out["roofline"]["pct_of_size_matched_ceiling"] = configs["2"]["B1"].get("pct_of_size_matched_ceiling")
    if fused_layer is not None:
        out["fused_layer"] = fused_layer
    if attention is not None:
        out["attention_decode"] = attention
    if lm_heads is not None:
        out["lm_head_alone"] = lm_heads
    out["bench_wall_s"] = round(time.perf_counter() - t_start, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
