"""Shared test helpers: build the hand-built golden cases into raw arrays.

Nothing here computes a GEMV; it only lays out the bytes each case lists.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def load_json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hex16(v):
    return int(v, 16)


def build_case(case):
    """-> (fmt, M, K, w, s, x, y_exact[B][M] as Fractions)."""
    fmt = synth.FMT_BY_NAME[case["fmt"]]
    M, K = case["M"], case["K"]
    G = synth.GROUP[fmt]
    wspec = case["w"]
    if fmt == synth.BF16:
        w = np.zeros((M, K), dtype=np.uint16)
        for r, row in enumerate(wspec["rows_bf16"]):
            w[r, :len(row)] = [_hex16(v) for v in row]
    elif fmt in (synth.INT8_G32, synth.INT8_ROW):
        w = np.zeros((M, K), dtype=np.int8)
        if "fill" in wspec:
            w[:] = wspec["fill"]
        if "alternate" in wspec:
            a, b = wspec["alternate"]
            w[:, 0::2] = a
            w[:, 1::2] = b
        if wspec.get("ramp_minus32"):
            w[:] = (np.arange(K) - 32).astype(np.int8)
        for r, i, v in wspec.get("set", []):
            w[r, i] = v
    else:
        nbytes = K // 2
        w = np.full((M, nbytes), wspec.get("fill", 0), dtype=np.uint8)
        if wspec.get("ramp_0x11"):
            per = G // 2
            j = np.arange(nbytes) % per
            w[:] = (0x11 * j).astype(np.uint8)
        for r, i, v in wspec.get("set", []):
            w[r, i] = v
        w = w.reshape(M, K // G, G // 2)
    s = None
    if case["s"] is not None:
        s = np.array([[_hex16(v) for v in row] for row in case["s"]], dtype=np.uint16)
        if fmt == synth.INT8_ROW:
            s = s.reshape(M)
    xspec = case["x"]
    if "fill_bf16" in xspec:
        x = np.array([[_hex16(xspec["fill_bf16"][0])] * K], dtype=np.uint16)
    elif "block_bf16" in xspec:
        rows = []
        for row in xspec["block_bf16"]:
            per = K // len(row)
            rows.append(np.repeat([_hex16(v) for v in row], per))
        x = np.array(rows, dtype=np.uint16)
    elif "onehot" in xspec:
        x = np.zeros((len(xspec["onehot"]), K), dtype=np.uint16)
        for b, k in enumerate(xspec["onehot"]):
            x[b, k] = 0x3F80
    else:
        x = np.zeros((len(xspec["rows_bf16"]), K), dtype=np.uint16)
        for b, row in enumerate(xspec["rows_bf16"]):
            x[b, :len(row)] = [_hex16(v) for v in row]
    y = [[Fraction(v) for v in row] for row in case["y"]]
    return fmt, M, K, w, s, x, y
