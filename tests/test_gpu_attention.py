"""GPU parity of qgemv_attention_decode (grouped-query decode attention over a
bf16 KV cache) against the float64 oracle, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bandwidth_bound_quantized_amd as qg  # noqa: E402
import oracle.attention as oatt  # noqa: E402
import synth  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def gpu_attention(at, n_q, n_kv, d, max_ctx, ws=None, k=None, v=None):
    B = at.q.shape[0]
    print(f"[gpu] qgemv_attention_decode B={B} n_q={n_q} n_kv={n_kv} d={d} max_ctx={max_ctx} "
          f"lens={list(at.lens)[:4]}", flush=True)
    out = torch.full((B, n_q, d), float("nan"), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = qg.attention_workspace(B, n_q, n_kv, d, max_ctx)
    qg.attention_decode(dev(at.q), dev(at.k if k is None else k), dev(at.v if v is None else v),
                        dev(at.lens), out, B, n_q, n_kv, d, max_ctx, at.scale, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


def check(at, out, what=""):
    ref, A = oatt.attention_decode_ref(at.q, at.k, at.v, at.lens, at.scale)
    rep = oatt.parity_report(out, ref, A)
    assert rep["ok"], f"{what} {rep}"


# (B, n_q, n_kv, head_dim, max_ctx): Llama-3.2-1B (32/8, 64) and TinyLlama
# (32/4, 64) heads at the infer page's contexts, both head sizes and every
# group size, one-split and many-split plans, ragged lengths
SHAPES = [(1, 32, 8, 64, 512), (1, 32, 8, 64, 2048), (4, 32, 8, 64, 2048), (8, 32, 8, 64, 512),
          (1, 32, 4, 64, 2048), (2, 32, 4, 64, 1000), (1, 8, 8, 128, 4096), (3, 16, 8, 128, 777),
          (1, 32, 8, 128, 2048), (2, 64, 8, 128, 1500), (1, 8, 4, 64, 8192), (5, 4, 4, 64, 130),
          # up to 8 splits with more outputs per (sequence, KV head) than merge threads
          (8, 64, 8, 128, 300), (1, 16, 4, 128, 600)]


@pytest.mark.parametrize("B,n_q,n_kv,d,T", SHAPES, ids=[f"b{b}-{q}x{k}-d{d}-ctx{t}" for b, q, k, d, t in SHAPES])
def test_attention_parity(B, n_q, n_kv, d, T):
    at = synth.make_attention(B, n_q, n_kv, d, T, seed=B * 1000 + n_q + T)
    out, ws = gpu_attention(at, n_q, n_kv, d, T)
    check(at, out, f"B={B} {n_q}/{n_kv} d={d} T={T}")
    # the workspace reused as it was left: the same inputs give the same bits
    out2, _ = gpu_attention(at, n_q, n_kv, d, T, ws=ws)
    assert (out.view(np.uint32) == out2.view(np.uint32)).all()


@pytest.mark.parametrize("lens", [[1], [2], [63], [64], [65], [255], [256], [257], [4095], [4096]])
def test_attention_lengths_and_block_edges(lens):
    T = 4096
    at = synth.make_attention(1, 32, 8, 64, T, seed=sum(lens), lens=lens)
    out, _ = gpu_attention(at, 32, 8, 64, T)
    check(at, out, f"len={lens}")


def test_attention_ignores_cache_past_length():
    """NaN in every position past each sequence's length changes nothing."""
    B, n_q, n_kv, d, T = 4, 32, 8, 64, 1024
    at = synth.make_attention(B, n_q, n_kv, d, T, seed=9, lens=[1000, 1, 513, 64])
    out, _ = gpu_attention(at, n_q, n_kv, d, T)
    k, v = at.k.copy(), at.v.copy()
    for b, L in enumerate(at.lens):
        k[b, :, L:] = 0x7FC0
        v[b, :, L:] = 0x7FC0
    out2, _ = gpu_attention(at, n_q, n_kv, d, T, k=k, v=v)
    assert np.isfinite(out2).all()
    assert (out.view(np.uint32) == out2.view(np.uint32)).all()
    check(at, out2)


def test_attention_long_context():
    at = synth.make_attention(1, 32, 8, 64, 32768, seed=5)
    out, _ = gpu_attention(at, 32, 8, 64, 32768)
    check(at, out, "ctx 32768")


def test_attention_peaked_scores():
    """Large scores (one key per head far above the rest): the online softmax's
    rescaling across blocks and splits must keep exp() in range."""
    B, n_q, n_kv, d, T = 2, 32, 8, 64, 4096
    at = synth.make_attention(B, n_q, n_kv, d, T, seed=21, lens=[4096, 3000])
    at.q = (at.q * 8.0).astype(np.float32)          # scores ~ N(0, 64)
    out, _ = gpu_attention(at, n_q, n_kv, d, T)
    assert np.isfinite(out).all()
    check(at, out, "peaked")


def _random_attention_case(seed):
    """A seeded draw of batch, heads (group size 1..8), head size, context and a
    per-sequence length mix (lengths from 1 to the context, block edges included)."""
    rng = np.random.default_rng(9100 + seed)
    B = int(rng.integers(1, 9))
    n_kv = int(rng.choice([1, 2, 4, 8]))
    n_q = n_kv * int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    T = int(rng.choice([1, 63, 64, 65, 300, 1000, 2048, int(rng.integers(1, 6000))]))
    lens = rng.integers(1, T + 1, size=B)
    lens[int(rng.integers(0, B))] = T
    if T > 1 and rng.random() < 0.5:
        lens[int(rng.integers(0, B))] = int(rng.choice([1, min(64, T), T - 1]))
    return B, n_q, n_kv, d, T, [int(v) for v in lens]


@pytest.mark.parametrize("seed", range(24))
def test_random_attention_call(seed):
    """Seeded random shapes and length mixes: every output against the oracle."""
    B, n_q, n_kv, d, T, lens = _random_attention_case(seed)
    at = synth.make_attention(B, n_q, n_kv, d, T, seed=20000 + seed, lens=lens)
    out, _ = gpu_attention(at, n_q, n_kv, d, T)
    check(at, out, f"seed={seed} B={B} {n_q}/{n_kv} d={d} T={T} lens={lens}")
