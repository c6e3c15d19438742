"""Seeded synthetic inputs for the decode-step GEMV workloads.

This module is shared by the tests, the bench and the smoke check. It draws
random bits and lays them out as the raw tensors a decode step reads (bf16
weights, quantized codes, f16 scales, bf16 activations). It holds none of the
GEMV's arithmetic: no dequantization, no dot product, no quantizer.

Value distributions follow the workloads of the pages on bandwidth-bound
decode ("Writing an LLM inference engine from scratch in Rust", the
TinyLlama-1.1B recap and Lesson 1; "infer", the per-kernel tables for the
Llama-3.2-1B shapes, whose numbers were also reproduced on random weights of
the same shapes):

* bf16 weights ~ N(0, 0.02^2), activations ~ N(0, 1): a float32 normal draw
  rounded to bf16 (round to nearest, ties to even).
* 4-bit codes uniform in [0, 15]: every nibble of every packed byte is an
  independent uniform 4-bit draw, so a uniform random byte gives two of them
  regardless of how a format assigns nibbles to elements.
* int8 codes uniform in [-127, 127].
* f16 scales uniform in [lo, hi]: a float64 uniform draw rounded to binary16.

Seeds: ``seed = 1_000_000*cfg + 1_000*layer + 10*proj + tensor`` with
proj in {qkv:0, o:1, gate_up:2, down:3, lm_head:4} and tensor in
{weights:0, scales:1, x:2}; NumPy's PCG64 generator.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

# format ids, mirrored from the C header on purpose: these are names, not math
BF16, INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64 = 0, 1, 2, 3, 4, 5
FMT_NAMES = {BF16: "bf16", INT8_G32: "int8_g32", Q4_0_G32: "q4_0_g32", INT4_G128: "int4_g128",
             INT8_ROW: "int8_row", INT4_G64: "int4_g64"}
FMT_BY_NAME = {v: k for k, v in FMT_NAMES.items()}
# weights per scale (0: one scale per row); K must be a multiple of K_ALIGN
GROUP = {BF16: 1, INT8_G32: 32, Q4_0_G32: 32, INT4_G128: 128, INT8_ROW: 0, INT4_G64: 64}
K_ALIGN = {BF16: 32, INT8_G32: 32, Q4_0_G32: 32, INT4_G128: 128, INT8_ROW: 32, INT4_G64: 64}
ALL_FORMATS = (BF16, INT8_G32, Q4_0_G32, INT4_G128, INT8_ROW, INT4_G64)


def scale_shape(fmt: int, M: int, K: int):
    """Shape of the planar scale array (None for bf16)."""
    if fmt == BF16:
        return None
    return (M,) if GROUP[fmt] == 0 else (M, K // GROUP[fmt])

PROJ = {"qkv": 0, "o": 1, "gate_up": 2, "down": 3, "lm_head": 4}
T_W, T_S, T_X = 0, 1, 2


def seed_for(cfg: int, layer: int, proj: str, tensor: int) -> int:
    return 1_000_000 * cfg + 1_000 * layer + 10 * PROJ[proj] + tensor


def round_f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return round_f32_to_bf16_bits(a)


def f16_uniform(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    a = rng.uniform(lo, hi, size=shape)
    return a.astype(np.float16).view(np.uint16)


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def int8_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


@dataclasses.dataclass
class Gemv:
    """One GEMV's raw inputs in the canonical planar layout.

    w: bf16 -> uint16[M][K]; int8_g32 -> int8[M][K];
       q4_0_g32 -> uint8[M][K/32][16]; int4_g128 -> uint8[M][K/128][64]
    s: uint16 f16 bits [M][K/G] (None for bf16)
    x: uint16 bf16 bits [B][K]
    """
    name: str
    fmt: int
    M: int
    K: int
    B: int
    w: np.ndarray
    s: Optional[np.ndarray]
    x: np.ndarray
    seeds: Tuple[int, int, int]


SCALE_RANGE = {INT8_G32: (1e-4, 4e-4), Q4_0_G32: (0.001, 0.005), INT4_G128: (0.001, 0.005),
               INT8_ROW: (1e-4, 4e-4), INT4_G64: (0.001, 0.005)}


def make_gemv(name: str, fmt: int, M: int, K: int, B: int, cfg: int, layer: int, proj: str,
              w_std: float = 0.02) -> Gemv:
    sw, ss, sx = (seed_for(cfg, layer, proj, t) for t in (T_W, T_S, T_X))
    rw, rs, rx = (np.random.default_rng(s) for s in (sw, ss, sx))
    G = GROUP[fmt]
    if fmt == BF16:
        w = bf16_normal(rw, (M, K), w_std)
        s = None
    elif fmt in (INT8_G32, INT8_ROW):
        w = int8_uniform(rw, (M, K))
        s = f16_uniform(rs, scale_shape(fmt, M, K), *SCALE_RANGE[fmt])
    else:
        w = random_bytes(rw, (M, K // G, G // 2))
        s = f16_uniform(rs, (M, K // G), *SCALE_RANGE[fmt])
    x = bf16_normal(rx, (B, K), 1.0)
    return Gemv(name, fmt, M, K, B, w, s, x, (sw, ss, sx))


# ---------------------------------------------------------------- workloads
TINYLLAMA = [("qkv", 2560, 2048), ("o", 2048, 2048), ("gate_up", 11264, 2048),
             ("down", 2048, 5632)]
TINYLLAMA_HEAD = ("lm_head", 32000, 2048)
LLAMA32_1B = [("qkv", 3072, 2048), ("o", 2048, 2048), ("gate_up", 16384, 2048),
              ("down", 2048, 8192)]


@dataclasses.dataclass
class Spec:
    name: str
    fmt: int
    M: int
    K: int
    cfg: int
    layer: int
    proj: str


def workload_specs(cfg: int) -> List[Spec]:
    """The GEMVs of each decode-step workload, in launch order."""
    if cfg == 1:
        return [Spec("bf16_2048x2048", BF16, 2048, 2048, 1, 0, "o")]
    if cfg == 2:
        return [Spec(p, Q4_0_G32, m, k, 2, 0, p) for p, m, k in TINYLLAMA + [TINYLLAMA_HEAD]]
    if cfg == 3:
        return [Spec(p, INT8_G32, m, k, 3, 0, p) for p, m, k in LLAMA32_1B]
    if cfg == 4:
        out = []
        for layer in range(22):
            out += [Spec(f"L{layer}.{p}", Q4_0_G32, m, k, 4, layer, p) for p, m, k in TINYLLAMA]
        p, m, k = TINYLLAMA_HEAD
        out.append(Spec(p, Q4_0_G32, m, k, 4, 999, p))
        return out
    if cfg == 5:
        return [Spec("gate_up", INT4_G128, 16384, 2048, 5, 0, "gate_up"),
                Spec("down", INT4_G128, 2048, 8192, 5, 0, "down"),
                Spec("lm_head", INT8_G32, 128256, 2048, 5, 0, "lm_head")]
    if cfg == 6:
        return ([Spec(p, Q4_0_G32, m, k, 6, 0, p) for p, m, k in LLAMA32_1B] +
                [Spec("lm_head", INT8_ROW, 128256, 2048, 6, 999, "lm_head")])
    raise ValueError(f"unknown workload {cfg}")


WORKLOAD_NAMES = {
    1: "bf16 GEMV 2048x2048",
    2: "Q4_0-g32 GEMV set, TinyLlama-1.1B decode shapes + argmax",
    3: "int8-g32 GEMV set, Llama-3.2-1B decode shapes",
    4: "Q4_0-g32 TinyLlama-1.1B decode-step weight stream (89 GEMVs) + argmax",
    5: "int4-g128 FFN + int8-g32 LM head (Llama-3.2-1B shapes) + argmax",
    6: "int4-g32 (Q4_0) Llama-3.2-1B layer GEMVs + int8 per-row LM head + argmax",
}
WORKLOAD_BATCHES = {1: [1], 2: [1], 3: [1], 4: [1, 2, 4, 8], 5: [1, 8], 6: [1, 8]}
# workloads whose last GEMV is an LM head followed by argmax over its logits
WORKLOAD_ARGMAX = {1: False, 2: True, 3: False, 4: True, 5: True, 6: True}


def make_workload(cfg: int, B: int) -> List[Gemv]:
    return [make_gemv(sp.name, sp.fmt, sp.M, sp.K, B, sp.cfg, sp.layer, sp.proj)
            for sp in workload_specs(cfg)]


def f32_logits_with_ties(rng: np.random.Generator, B: int, V: int) -> np.ndarray:
    """float32 logits with planted duplicate maxima (argmax tie cases)."""
    a = rng.standard_normal(size=(B, V), dtype=np.float32)
    for b in range(B):
        hi = np.float32(a[b].max() + 1.0)
        pos = np.sort(rng.choice(V, size=min(3, V), replace=False))
        a[b, pos] = hi
    return a


# ------------------------------------------------------- decode attention
@dataclasses.dataclass
class Attention:
    """Inputs of one grouped-query decode-attention call: q float32 [B][n_q][d];
    k, v bf16 bits [B][n_kv][max_ctx][d] (positions past a sequence's length
    hold random values that must not be read); lens int32 [B]."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    lens: np.ndarray
    scale: float


def make_attention(B: int, n_q: int, n_kv: int, d: int, max_ctx: int, seed: int,
                   lens=None) -> Attention:
    """q, k, v ~ N(0, 1) (k, v rounded to bf16); a length mix per sequence:
    uniform in [max_ctx / 4, max_ctx] with the first sequence at max_ctx,
    unless lens is given."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n_q, d), dtype=np.float32)
    k = bf16_normal(rng, (B, n_kv, max_ctx, d), 1.0)
    v = bf16_normal(rng, (B, n_kv, max_ctx, d), 1.0)
    if lens is None:
        lens = rng.integers(max(1, max_ctx // 4), max_ctx + 1, size=B)
        lens[0] = max_ctx
    return Attention(q, k, v, np.asarray(lens, dtype=np.int32), 1.0 / float(np.sqrt(d)))
