"""Bench: fused-dequant decode GEMV throughput on one MI355X (gfx950).

One "step" is one pass of the whole hot path over one batch: every GEMV of
the workload (qgemv_run) and, where the workload ends in an LM head, the
argmax of its logits (qgemv_argmax). The default workload is the Q4_0-g32
GEMV set at TinyLlama-1.1B decode shapes (qkv 2560x2048, o 2048x2048,
gate_up 11264x2048, down 2048x5632, lm_head 32000x2048) at batch 1, plus
the argmax over the 32000 logits.

Inputs are synthetic and seeded (synth), resident in HBM before timing, and
rotated through >= 1 GiB of distinct device copies so that the 256 MB
Infinity Cache cannot serve them. The timed steps are captured once in a
HIP graph (the decode step of the infer page is a CUDA graph too) and
replayed; events on the launch stream bracket exactly --steps steps.

Reported (one JSON line):
  value            algorithmic bytes per step / time per step (GB/s)
  roofline         dominant kernel (largest bytes per launch): its bytes per
                   launch / its average launch duration, against 8 TB/s
  measured_peak    best rate of the streaming-read kernel over 4 GiB
  cpu_baseline     the fp64 CPU oracle on one step, one thread
Algorithmic bytes per GEMV = code bytes + scale bytes + x (2*B*K) + y (4*B*M);
argmax = 4*B*V read + 4*B written.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic.json")


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
    p.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6])
    p.add_argument("--batch", type=int, default=None)
    p.add_argument("--rotate-gib", type=float, default=1.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peak", action="store_true")
    p.add_argument("--peak-gib", type=float, default=4.0)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--per-kernel", action="store_true", help="also time every GEMV of the step alone")
    p.add_argument("--no-attention", action="store_true",
                   help="skip the decode-attention measurements (workload 2)")
    p.add_argument("--no-fused-layer", action="store_true",
                   help="skip the fused decode-layer chain (workload 2)")
    p.add_argument("--pmc-pass", action="store_true",
                   help="only run calibration kernels (a 64 MiB streaming read, a 64 MiB fill) and "
                        "--steps eager steps, for hardware-counter collection")
    p.add_argument("--size-sweep", action="store_true",
                   help="only time the streaming-read kernel at GEMV-like sizes (size-matched ceilings)")
    return p.parse_args()


def gemv_bytes(qg, fmt, M, K, B):
    w, s = qg.packed_size(fmt, M, K)
    return w + s + 2 * B * K + 4 * B * M


class Workload:
    """Device-resident inputs for one workload, replicated n_sets times."""

    def __init__(self, qg, torch, cfg, B, rotate_bytes):
        self.qg, self.torch, self.cfg, self.B = qg, torch, cfg, B
        self.gemvs = synth.make_workload(cfg, B)
        self.has_argmax = synth.WORKLOAD_ARGMAX[cfg]
        self.bytes = [gemv_bytes(qg, g.fmt, g.M, g.K, B) for g in self.gemvs]
        self.argmax_bytes = 4 * B * self.gemvs[-1].M + 4 * B if self.has_argmax else 0
        self.step_bytes = sum(self.bytes) + self.argmax_bytes
        # with the argmax inside the LM head's launch the logits are not read again
        self.fused_bytes = sum(self.bytes) + (4 * B if self.has_argmax else 0)
        resident = sum(g.w.nbytes + (g.s.nbytes if g.s is not None else 0) for g in self.gemvs)
        self.n_sets = max(1, math.ceil(rotate_bytes / resident))
        dev = "cuda"
        self.sets = []
        base = []
        for g in self.gemvs:
            W = torch.from_numpy(np.ascontiguousarray(g.w).reshape(-1).view(np.uint8)).to(dev)
            S = torch.from_numpy(g.s.reshape(-1).view(np.int16)).to(dev) if g.s is not None else None
            X = torch.from_numpy(g.x.view(np.int16)).to(dev)
            base.append((W, S, X))
        for i in range(self.n_sets):
            items = []
            for (W, S, X), g in zip(base, self.gemvs):
                Wi = W if i == 0 else W.clone()
                Si = None if S is None else (S if i == 0 else S.clone())
                Xi = X if i == 0 else X.clone()
                Y = torch.empty((B, g.M), dtype=torch.float32, device=dev)
                items.append((Wi, Si, Xi, Y))
            ws = qg.fused_argmax_workspace(B) if self.has_argmax else None
            idx = torch.empty(B, dtype=torch.int32, device=dev) if self.has_argmax else None
            self.sets.append((items, ws, idx))
        torch.cuda.synchronize()
        # per set: descriptors for one grouped call, and per launch class
        self.classes = {}
        for j, g in enumerate(self.gemvs):
            # qgemv_run_grouped: one small-batch launch per format, one
            # matrix-core launch per format and K, one launch each for the others
            cls = qg.grouped_class(g.fmt, g.K, B)
            key = ((g.fmt, "grouped") if cls == qg.GROUP_XREG else
                   (g.fmt, g.K, "mfma") if cls == qg.GROUP_MFMA else ("alone", j))
            self.classes.setdefault(key, []).append(j)
        self.descs = []
        self.class_descs = []
        for items, _, _ in self.sets:
            ent = [(g.fmt, W, S, X, Y, g.M, g.K) for (W, S, X, Y), g in zip(items, self.gemvs)]
            self.descs.append(qg.grouped_descs(ent))
            self.class_descs.append({k: qg.grouped_descs([ent[j] for j in js])
                                     for k, js in self.classes.items()})
        # raw pointers for the launch loop (argument marshalling only)
        self.ptrs = []
        for items, ws, idx in self.sets:
            p = [(W.data_ptr(), None if S is None else S.data_ptr(), X.data_ptr(), Y.data_ptr())
                 for W, S, X, Y in items]
            self.ptrs.append((p, ws.data_ptr() if ws is not None else None,
                              idx.data_ptr() if idx is not None else None))

    def step(self, i, stream_handle):
        qg = self.qg
        p, wsp, ip = self.ptrs[i % self.n_sets]
        for (wp, sp, xp, yp), g in zip(p, self.gemvs):
            qg.run_ptr(g.fmt, wp, sp, xp, yp, g.M, g.K, self.B, stream_handle)
        if self.has_argmax:
            st = qg.lib().qgemv_argmax(p[-1][3], self.gemvs[-1].M, self.B, wsp, ip, stream_handle)
            if st != qg.OK:
                raise qg.QgemvError(st, "qgemv_argmax")

    def step_grouped(self, i, stream_handle):
        """All GEMVs of the step in one qgemv_run_grouped call, then the argmax."""
        qg = self.qg
        p, wsp, ip = self.ptrs[i % self.n_sets]
        qg.run_grouped_ptr(self.descs[i % self.n_sets], self.B, stream_handle)
        if self.has_argmax:
            st = qg.lib().qgemv_argmax(p[-1][3], self.gemvs[-1].M, self.B, wsp, ip, stream_handle)
            if st != qg.OK:
                raise qg.QgemvError(st, "qgemv_argmax")

    def step_fused(self, i, stream_handle):
        """The step's GEMVs and the LM-head argmax in one qgemv_run_grouped_argmax call
        (the argmax runs inside the LM head's launch where the small-batch kernel takes it)."""
        qg = self.qg
        p, wsp, ip = self.ptrs[i % self.n_sets]
        qg.run_grouped_argmax_ptr(self.descs[i % self.n_sets], self.B, len(self.gemvs) - 1, wsp, ip,
                                  stream_handle)

    def launch_class(self, key, i, stream_handle):
        """One launch class as the step runs it: with the LM-head argmax fused in if the
        class holds the LM head."""
        am = len(self.gemvs) - 1
        descs = self.class_descs[i % self.n_sets][key]
        if self.has_argmax and am in self.classes[key]:
            p, wsp, ip = self.ptrs[i % self.n_sets]
            self.qg.run_grouped_argmax_ptr(descs, self.B, self.classes[key].index(am), wsp, ip,
                                           stream_handle)
        else:
            self.qg.run_grouped_ptr(descs, self.B, stream_handle)

    def class_bytes(self, key):
        return sum(self.bytes[j] for j in self.classes[key])

    def class_label(self, key):
        names = "+".join(self.gemvs[j].name for j in self.classes[key][:6])
        more = f"+{len(self.classes[key]) - 6} more" if len(self.classes[key]) > 6 else ""
        return f"{names}{more}"

    def launch_one(self, j, i, stream_handle):
        g = self.gemvs[j]
        wp, sp, xp, yp = self.ptrs[i % self.n_sets][0][j]
        self.qg.run_ptr(g.fmt, wp, sp, xp, yp, g.M, g.K, self.B, stream_handle)


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


def capture(torch, fn, count):
    """Capture fn(i) for i in range(count) into one graph on a side stream."""
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


def time_graph(torch, g, reps=1):
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_peak(qg, torch, gib):
    """Best streaming-read rate over a gib-GiB buffer, sweeping grid and loads in flight."""
    nbytes = int(gib * (1 << 30)) // 16 * 16
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(64 * cus, dtype=torch.int32, device="cuda")
    best = (0.0, None)
    sweep = []
    for grid_per_cu in (4, 8, 16, 32):
        for unroll in (2, 4, 8, 16):
            grid = grid_per_cu * cus
            h = torch.cuda.current_stream().cuda_stream
            qg.stream_read(buf, nbytes, sink, grid=grid, unroll=unroll)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            times = []
            for _ in range(5):
                e0.record()
                qg.lib().qgemv_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, unroll, h)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = float(np.median(times))
            gbps = nbytes / (ms * 1e-3) / 1e9
            sweep.append({"grid": grid, "unroll": unroll, "GBps": round(gbps, 1)})
            if gbps > best[0]:
                best = (gbps, {"grid": grid, "unroll": unroll, "ms": ms})
    del buf
    torch.cuda.empty_cache()
    return best[0], best[1], sweep


def size_sweep(qg, torch, rotate_bytes):
    """Streaming-read kernel at small sizes, rotated through >= rotate_bytes of distinct
    buffers: the size-matched ceiling a kernel of that many bytes can reach."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for mb in (1, 2, 2.36, 4, 8, 13, 16, 32, 37, 64, 128, 256):
        nbytes = int(mb * (1 << 20)) // 4096 * 4096
        n = max(4, math.ceil(rotate_bytes / nbytes))
        pool = torch.empty(n * nbytes // 4, dtype=torch.int32, device="cuda")
        pool.fill_(3)
        sink = torch.zeros(64 * cus, dtype=torch.int32, device="cuda")
        best = None
        for grid in (cus, 2 * cus, 4 * cus, 8 * cus):
            for unroll in (1, 2, 4):
                base = pool.data_ptr()

                def fn(i, h, grid=grid, unroll=unroll):
                    st = qg.lib().qgemv_stream_read(base + (i % n) * nbytes, nbytes, sink.data_ptr(),
                                                    grid, unroll, h)
                    if st != qg.OK:
                        raise qg.QgemvError(st, "qgemv_stream_read")
                g = capture(torch, fn, n)
                time_graph(torch, g)
                us = time_graph(torch, g, reps=3) * 1e3 / n
                if best is None or us < best[0]:
                    best = (us, grid, unroll)
                del g
        us, grid, unroll = best
        out.append({"MiB": mb, "bytes": nbytes, "us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1),
                    "grid": grid, "unroll": unroll, "rotation": n})
        print(json.dumps(out[-1]), flush=True)
        del pool
        torch.cuda.empty_cache()
    return out


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
    for i in range(steps):
        (wl.step_fused if wl.has_argmax else wl.step_grouped)(i, h)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": True, "calib_bytes": nbytes, "steps": steps,
                      "gemvs": [[g.name, g.M, g.K, b] for g, b in zip(wl.gemvs, wl.bytes)]}), flush=True)


def attention_bench(qg, torch, rotate_bytes):
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
        count = max(n * 2, 64)
        g = capture(torch, fn, count)
        time_graph(torch, g)
        us = time_graph(torch, g, reps=3) * 1e3 / count
        nbytes = per + 2 * B * n_q * d * 4
        out.append({"batch": B, "ctx": T, "heads": [n_q, n_kv, d], "us": round(us, 3), "bytes": nbytes,
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)})
        print(f"[bench] attention B={B} ctx={T}: {us:.2f} us, {out[-1]['GBps']} GB/s", file=sys.stderr, flush=True)
        del g, ks, vs
        torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, seconds):
    """The oracle (fp64 dequantize + fp64 GEMV + argmax) on whole steps, one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        t0 = time.perf_counter()
        steps = 0
        while True:
            last = None
            for g in wl.gemvs:
                last, _ = oracle.gemv_ref(g.fmt, g.w, g.s, g.x, g.M, g.K)
            if wl.has_argmax:
                oracle.argmax_ref(last.astype(np.float32))
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds or steps >= 50:
                break
    return steps, el


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
    if args.size_sweep:
        size_sweep(qg, torch, args.rotate_gib * (1 << 30))
        return
    cfg = args.workload
    B = args.batch if args.batch is not None else synth.WORKLOAD_BATCHES[cfg][0]
    wl = Workload(qg, torch, cfg, B, args.rotate_gib * (1 << 30))
    if args.pmc_pass:
        pmc_pass(qg, torch, wl, args.steps)
        return
    print(f"[bench] workload {cfg} B={B}: {len(wl.gemvs)} GEMVs, {wl.step_bytes} B/step, "
          f"{wl.n_sets} rotation sets", file=sys.stderr, flush=True)

    # ---- timed steps (graph of exactly `steps` steps, rotating through the sets).
    # grouped: the step's GEMVs (independent inputs) in one qgemv_run_grouped call;
    # sequential: one qgemv_run launch per GEMV, as a decode step whose GEMVs
    # depend on each other must run them.
    results = {}
    modes = [("sequential", wl.step), ("grouped", wl.step_grouped)]
    if wl.has_argmax:
        modes.append(("fused", wl.step_fused))
    for mode, fn in modes:
        g_warm = capture(torch, fn, max(1, args.warmup))
        time_graph(torch, g_warm)
        g_steps = capture(torch, fn, args.steps)
        ms = time_graph(torch, g_steps) / args.steps
        results[mode] = ms
        nb = wl.fused_bytes if mode == "fused" else wl.step_bytes
        print(f"[bench] {mode}: {ms * 1e3:.2f} us/step, {nb / (ms * 1e-3) / 1e9:.1f} GB/s",
              file=sys.stderr, flush=True)
        del g_warm, g_steps
    attention = None
    if cfg == 2 and not args.no_attention:
        attention = attention_bench(qg, torch, args.rotate_gib * (1 << 30))
    fused_layer = None
    if cfg == 2 and not args.no_fused_layer:
        fl = FusedLayer(qg, torch, wl)
        g_warm = capture(torch, fl.step, max(1, args.warmup))
        time_graph(torch, g_warm)
        g_steps = capture(torch, fl.step, args.steps)
        ms_fl = time_graph(torch, g_steps) / args.steps
        del g_warm, g_steps
        per_op = []
        if args.per_kernel:
            for k in range(5):
                n = max(wl.n_sets * 4, 64)
                gk = capture(torch, lambda i, h, k=k: fl.op(k, i, h), n)
                time_graph(torch, gk)
                us = time_graph(torch, gk, reps=3) * 1e3 / n
                gp = capture(torch, lambda i, h, k=k: wl.launch_one(k, i, h), n)
                time_graph(torch, gp)
                us_p = time_graph(torch, gp, reps=3) * 1e3 / n
                per_op.append({"op": FusedLayer.NAMES[k], "fused_us": round(us, 3), "plain_gemv_us": round(us_p, 3)})
                del gk, gp
        fused_layer = {
            "chain": "qkv(RMSNorm) -> o(+=residual) -> gate_up(RMSNorm, SwiGLU of paired rows) -> "
                     "down(+=residual) -> lm_head(RMSNorm, argmax): 5 dependent qgemv_run_fused launches",
            "us_per_step": round(ms_fl * 1e3, 3), "bytes_per_step": fl.bytes,
            "GBps": round(fl.bytes / (ms_fl * 1e-3) / 1e9, 1),
            "plain_sequential_us_per_step": round(results["sequential"] * 1e3, 3),
            "plain_sequential_launches": len(wl.gemvs) + 1}
        if per_op:
            fused_layer["per_op"] = per_op
        print(f"[bench] fused layer chain: {ms_fl * 1e3:.2f} us/step, {fused_layer['GBps']} GB/s",
              file=sys.stderr, flush=True)
    ms_per_step = results["fused"] if wl.has_argmax else results["grouped"]
    value = (wl.fused_bytes if wl.has_argmax else wl.step_bytes) / (ms_per_step * 1e-3) / 1e9
    value_seq = wl.step_bytes / (results["sequential"] * 1e-3) / 1e9
    value_grp = wl.step_bytes / (results["grouped"] * 1e-3) / 1e9

    # ---- dominant kernel: the grouped launch with the most bytes, timed alone
    dom_key = max(wl.classes, key=wl.class_bytes)
    n_dom = max(wl.n_sets * 4, 64)
    if dom_key[0] == "alone":
        dom_fn = (lambda i, h, j=dom_key[1]: wl.launch_one(j, i, h))
    else:
        dom_fn = (lambda i, h: wl.launch_class(dom_key, i, h))
    g_dom = capture(torch, dom_fn, n_dom)
    time_graph(torch, g_dom)
    dom_us = time_graph(torch, g_dom, reps=3) * 1e3 / n_dom
    dom_bytes = wl.class_bytes(dom_key)
    dom_gbps = dom_bytes / (dom_us * 1e-6) / 1e9

    per_kernel = []
    if args.per_kernel:
        for j, gm in enumerate(wl.gemvs):
            n = max(wl.n_sets * 4, 64)
            gj = capture(torch, lambda i, h, j=j: wl.launch_one(j, i, h), n)
            time_graph(torch, gj)
            us = time_graph(torch, gj, reps=3) * 1e3 / n
            per_kernel.append({"name": gm.name, "M": gm.M, "K": gm.K, "us": round(us, 3),
                               "GBps": round(wl.bytes[j] / (us * 1e-6) / 1e9, 1)})
            del gj

    peak = None
    if not args.no_peak:
        peak_gbps, peak_cfg, sweep = measure_peak(qg, torch, args.peak_gib)
        peak = {"GBps": round(peak_gbps, 1), "config": peak_cfg, "buffer_GiB": args.peak_gib}
        print(f"[bench] measured streaming-read peak {peak_gbps:.1f} GB/s {peak_cfg}",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        steps, el = cpu_baseline(wl, args.cpu_seconds)
        cpu = {"value": round(wl.step_bytes * steps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{steps} whole step(s) of workload {cfg} (all {len(wl.gemvs)} GEMVs"
                         f"{' + argmax' if wl.has_argmax else ''}), fp64, one thread, {el:.1f} s"}

    names = {1: "bf16_gemv_2048x2048", 2: "q4_0_g32_tinyllama_gemv_set+argmax",
             3: "int8_g32_llama32_1b_gemv_set", 4: "q4_0_g32_tinyllama_decode_step_89_gemvs+argmax",
             5: "int4_g128_ffn+int8_g32_lm_head+argmax",
             6: "q4_0_g32_llama32_1b_layer_gemvs+int8_row_lm_head+argmax"}
    dtypes = {1: "bf16", 2: "q4_0", 3: "int8", 4: "q4_0", 5: "int4/int8", 6: "q4_0/int8"}
    if dom_key[0] == "alone":
        dom_label = f"qgemv_run {wl.gemvs[dom_key[1]].name}"
    elif wl.has_argmax and len(wl.gemvs) - 1 in wl.classes[dom_key]:
        dom_label = f"qgemv_run_grouped_argmax launch [{wl.class_label(dom_key)}+argmax]"
    else:
        dom_label = f"qgemv_run_grouped launch [{wl.class_label(dom_key)}]"
    traffic = recorded_traffic(dom_label, names[cfg], B)
    out = {
        "metric": "fused-dequant GEMV achieved HBM GB/s and % of peak (bf16/int8/Q4_0, batch 1)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "value_sequential": round(value_seq, 1),
        "ms_per_step_sequential": round(results["sequential"], 6),
        "value_grouped_separate_argmax": round(value_grp, 1) if wl.has_argmax else None,
        "ms_per_step_grouped_separate_argmax": round(results["grouped"], 6) if wl.has_argmax else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtypes[cfg],
        "data": "synthetic (seeded; same shapes and value distributions as the workload)",
        "config": {"workload": names[cfg], "batch": B,
                   "gemvs": [[g.name, g.M, g.K] for g in wl.gemvs][:6] + (
                       [["...", len(wl.gemvs)]] if len(wl.gemvs) > 6 else []),
                   "bytes_per_step": wl.fused_bytes if wl.has_argmax else wl.step_bytes,
                   "rotation_sets": wl.n_sets,
                   "rotation_bytes": wl.n_sets * sum(g.w.nbytes + (g.s.nbytes if g.s is not None else 0)
                                                     for g in wl.gemvs),
                   "execution": "value: the step's independent GEMVs (one launch per format) and, "
                                "with an LM head, its argmax in one qgemv_run_grouped_argmax call "
                                "(the argmax inside the LM head's launch at batch <= 2); "
                                "value_grouped_separate_argmax: qgemv_run_grouped + qgemv_argmax; "
                                "value_sequential: one qgemv_run launch per GEMV + qgemv_argmax",
                   "timing": "HIP graph of exactly `steps` steps, events on the launch stream"},
        "pct_of_spec_8TBps": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": dom_label,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3),
                     "launches": n_dom},
        "cpu_baseline": cpu,
    }
    if peak is not None:
        out["measured_peak"] = peak
        out["pct_of_measured_peak"] = round(100 * value / peak["GBps"], 2)
        out["roofline"]["pct_of_measured_peak"] = round(100 * dom_gbps / peak["GBps"], 2)
    if per_kernel:
        out["per_kernel"] = per_kernel
    if fused_layer is not None:
        out["fused_layer"] = fused_layer
    if attention is not None:
        out["attention_decode"] = attention
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
