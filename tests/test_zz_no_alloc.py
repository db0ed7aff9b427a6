"""qgemm_q4k_noalloc: Q4_K prefill whose K-split partial sums go through the
library's own 32 MiB device array instead of a caller workspace.  Through the
C ABI, two calls in a row (the second smaller, on an array the first left full
of partial sums) must match qgemm_q4k_ws with a fresh NaN-filled workspace bit
for bit, and sampled outputs of each must meet the oracle's prefill bar.
Also: the call captured in a HIP graph and replayed, an unsplit call (no array
used), a call on a second stream, and a call needing more than the array,
refused with QGEMV_E_WORKSPACE.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def q():
    from dequant_gemv_amd import qgemv

    return qgemv


def _inputs(t, m, k, seed):
    w = synth.weights("q4k", m, k, synth.W_SEED + seed)
    xh = np.stack([synth.activations("q4k", k, synth.X_SEED + seed + i) for i in range(t)])
    return w, xh, torch.from_numpy(w).to(DEV), torch.from_numpy(xh.view(np.int16).copy()).to(DEV)


def _nan(t, m):
    return torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)


def _with_workspace(q, w, x, t, m, k):
    n = q.qgemm_workspace_bytes(t, m, k)
    ws = torch.full((max(n, 256) // 4,), float("nan"), dtype=torch.float32, device=DEV) if n else None
    y = _nan(t, m)
    q.qgemm_q4k_ws(w, x, y, t, m, k, ws)
    return y


def _oracle_check(wh, xh, got, t, m, k, seed):
    rng = np.random.default_rng(seed)
    toks = np.unique(np.concatenate([[0, t - 1], rng.integers(0, t, 12)]))
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 40)]))
    yr, ar = oracle.gemm("q4k", wh, xh, t, m, k, tokens=toks, rows=rows)
    g = got.astype(np.float64)[np.ix_(toks, rows)]
    bad = np.argwhere(~(np.abs(g - yr) <= 1e-3 * ar + 1e-5))
    assert bad.size == 0, f"T={t} {m}x{k}: {len(bad)} sampled outputs outside the bar"


def test_noalloc_captured_in_a_graph(q):
    """The graph-capture use: the call recorded in a HIP graph (the first
    no-alloc call of the process when this file runs first in it, so the
    array's address is looked up during the capture), replayed three times
    with eager work between the replays; every replay equals the eager call
    bit for bit."""
    t, m, k = 130, 4096, 4096
    _, _, w, x = _inputs(t, m, k, 920)
    y = _nan(t, m)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        q.qgemm_q4k_noalloc(w, x, y, t, m, k, stream=side)
    outs = []
    for _ in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy().copy())
    ref = _nan(t, m)
    q.qgemm_q4k_noalloc(w, x, ref, t, m, k)
    torch.cuda.synchronize()
    r = ref.cpu().numpy()
    for i, o in enumerate(outs):
        assert np.array_equal(o.view(np.uint32), r.view(np.uint32)), f"replay {i} differs"


# (T, M, K): 32 MiB of partial sums (the whole array), then 24 MiB
CALLS = [(512, 4096, 14336), (130, 4096, 4096)]


def test_noalloc_two_calls_match_workspace_path(q):
    assert q.qgemm_workspace_bytes(*CALLS[0]) == q.NOALLOC_MAX_BYTES
    assert 0 < q.qgemm_workspace_bytes(*CALLS[1]) < q.NOALLOC_MAX_BYTES
    for i, (t, m, k) in enumerate(CALLS):
        print(f"noalloc call {i}: T={t} M={m} K={k}", flush=True)
        wh, xh, w, x = _inputs(t, m, k, 900 + i)
        y = _nan(t, m)
        q.qgemm_q4k_noalloc(w, x, y, t, m, k)
        y_ws = _with_workspace(q, w, x, t, m, k)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), y_ws.cpu().numpy().view(np.uint32)), f"call {i} differs"
        _oracle_check(wh, xh, got, t, m, k, 900 + i)


def test_noalloc_unsplit_and_second_stream(q):
    t, m, k = 7, 5, 512  # one tile, not split: the array is not used
    assert q.qgemm_workspace_bytes(t, m, k) == 0
    _, _, w, x = _inputs(t, m, k, 910)
    y = _nan(t, m)
    q.qgemm_q4k_noalloc(w, x, y, t, m, k)
    ref = _with_workspace(q, w, x, t, m, k)
    t2, m2, k2 = 64, 1000, 2048
    _, _, w2, x2 = _inputs(t2, m2, k2, 911)
    assert q.qgemm_workspace_bytes(t2, m2, k2) > 0
    y2 = _nan(t2, m2)
    torch.cuda.synchronize()  # inputs and y2 are ready before the side stream starts
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        q.qgemm_q4k_noalloc(w2, x2, y2, t2, m2, k2, stream=side)
    side.synchronize()
    ref2 = _with_workspace(q, w2, x2, t2, m2, k2)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    assert np.array_equal(y2.cpu().numpy().view(np.uint32), ref2.cpu().numpy().view(np.uint32))


def test_noalloc_refuses_more_than_the_array(q):
    t, m, k = 4608, 8192, 4096
    assert q.qgemm_workspace_bytes(t, m, k) > q.NOALLOC_MAX_BYTES
    # refused in host code before any launch: the addresses are never used
    w = torch.zeros(256, dtype=torch.uint8, device=DEV)
    a = w.data_ptr()
    assert q.lib().qgemm_q4k_noalloc(a, a + (1 << 40), a + (2 << 40), t, m, k, None) == q.QGEMV_E_WORKSPACE
