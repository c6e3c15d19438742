"""qgemv_argmax_noalloc (the argmax with the library's static per-device
workspace) against qgemv_argmax with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller input, then a repeat of the pair
(the static workspace must have been left zero), a one-slice row, and
graph replays of a captured call. Indices must be bit-equal to the other entry
point's and to the oracle's argmax of the same logits."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bandwidth_bound_quantized_amd as qg  # noqa: E402
import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _logits(B, V, seed):
    """Random logits with the row maximum planted twice, in different slices of the
    row (the lower index must win), and a near-maximum elsewhere."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((B, V)).astype(np.float32)
    for b in range(B):
        i, j = sorted(rng.choice(V, 2, replace=False)) if V > 1 else (0, 0)
        a[b, i] = a[b, j] = 9.0
        if V > 2:
            a[b, rng.integers(0, V)] = np.nextafter(np.float32(9.0), np.float32(0))
    return a


def _both(a):
    B, V = a.shape
    L = torch.from_numpy(a).to(DEV)
    idx_na = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    idx_ws = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    ws = qg.argmax_workspace(B)
    print(f"[gpu] qgemv_argmax_noalloc V={V} B={B}", flush=True)
    qg.argmax_noalloc(L, V, B, idx_na)
    qg.argmax(L, V, B, ws, idx_ws)
    torch.cuda.synchronize()
    return idx_na.cpu().numpy(), idx_ws.cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls():
    # 128256 x 8: eight slices per row joined through the static workspace;
    # then 32000 x 3 (smaller): eleven slices per row; then the pair again
    for rep in range(2):
        for B, V, seed in ((8, 128256, 1), (3, 32000, 2)):
            a = _logits(B, V, seed + 10 * rep)
            na, ws = _both(a)
            ref = oracle.argmax_ref(a)
            assert (na == ws).all(), (B, V, na, ws)
            assert (na == ref).all(), (B, V, na, ref)


def test_noalloc_single_slice_and_special_values():
    a = _logits(1, 7, 3)
    na, ws = _both(a)
    assert (na == ws).all() and (na == oracle.argmax_ref(a)).all()
    b = np.full((2, 40000), -np.inf, dtype=np.float32)        # all -inf: index 0
    b[1, 30000] = np.nan                                       # first NaN wins
    b[1, 35000] = np.nan
    na, ws = _both(b)
    assert (na == ws).all() and (na == oracle.argmax_ref(b)).all() and list(na) == [0, 30000]


def test_noalloc_graph_replays():
    B, V = 4, 128256
    L = torch.empty((B, V), dtype=torch.float32, device=DEV)
    idx = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    L.copy_(torch.from_numpy(_logits(B, V, 20)))
    qg.argmax_noalloc(L, V, B, idx)            # eager call first (set-up outside capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        qg.argmax_noalloc(L, V, B, idx, stream=s)
    torch.cuda.synchronize()
    for r in range(4):
        a = _logits(B, V, 30 + r)
        L.copy_(torch.from_numpy(a))
        idx.fill_(-1)
        torch.cuda.synchronize()
        print(f"[gpu] graph replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        assert (got == oracle.argmax_ref(a)).all(), (r, got)
        # eager work between replays, on the same static workspace
        na, ws = _both(_logits(2, 50000, 40 + r))
        assert (na == ws).all()
