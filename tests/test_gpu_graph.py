"""The entry points captured in a HIP graph (the launch pattern the bench
times) and replayed several times, with eager work and synchronisations of
the program between the replays: every replay must give what the eager call
gives (bit for bit where the kernels are deterministic; to the GEMV bar of
the oracle where the prefill's K split adds partial sums with atomics, whose
order varies), and work that clears memory inside a captured sequence (the
prefill's y clear) must clear it again on every replay.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


@pytest.fixture(scope="module")
def q():
    from dequant_gemv_amd import qgemv

    return qgemv


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _capture(fn, stream):
    """Run fn(stream handle) eagerly once, then capture it into a graph."""
    h = stream.cuda_stream
    with torch.cuda.stream(stream):
        fn(h)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn(h)
    torch.cuda.synchronize()
    return g


def _replay(g, stream, disturb):
    """Replay after some eager work of the program (which also overwrites the
    outputs, so a replay that skipped its work would show)."""
    disturb()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt,n,k", [("q4k", 4096, 14336), ("nvfp4", 4096, 14336), ("tq1", 14336, 4096),
                                     ("q4k", 1000, 36864), ("bf16", 700, 4096)])
def test_gemv_graph_replays(q, fmt, n, k):
    # two launches over two weight copies into two outputs, as in the bench
    ws = [_dev(synth.weights(fmt, n, k, synth.W_SEED + 300 + i)) for i in range(2)]
    x = _dev(synth.activations(fmt, k, synth.X_SEED + 300).view(np.int16))
    ys = [torch.full((n,), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    s = torch.cuda.Stream()
    g = _capture(lambda h: [q.GEMV[fmt](ws[i], x, ys[i], n, k, h) for i in range(2)], s)
    want = [y.clone() for y in ys]
    assert not any(torch.isnan(w).any().item() for w in want)
    for r in range(REPLAYS):
        _replay(g, s, lambda: [y.fill_(float(r + 1)) for y in ys])
        for i in range(2):
            assert torch.equal(ys[i].view(torch.int32), want[i].view(torch.int32)), (fmt, r, i)


def test_gemv_ex_in_place_graph_replays_accumulate(q):
    # y (fp16) = v + 0.5 y in place: each replay applies the step once more
    fmt, n, k = "q4k", 2048, 4096
    w = _dev(synth.weights(fmt, n, k, synth.W_SEED + 310))
    x = _dev(synth.activations(fmt, k, synth.X_SEED + 310).view(np.int16))
    y0 = torch.linspace(-1, 1, n, device=DEV).to(torch.float16)
    y = y0.clone()
    s = torch.cuda.Stream()
    g = _capture(lambda h: q.GEMV_EX[fmt](w, x, y, n, k, 1.0, 0.5, y, h), s)
    # the eager reference sequence on a copy, one call per step; _capture made
    # one eager call, so y has had one step
    ref = y0.clone()
    q.GEMV_EX[fmt](w, x, ref, n, k, 1.0, 0.5, ref)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    for r in range(REPLAYS):
        _replay(g, s, lambda: None)
        q.GEMV_EX[fmt](w, x, ref, n, k, 1.0, 0.5, ref)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), r


@pytest.mark.parametrize("fmt,n,k,nrows", [("q4k", 4096, 14336, None), ("tq1", 14336, 4096, None),
                                           ("nvfp4", 4096, 14336, None), ("q4k", 128256, 4096, 512)])
def test_rows_graph_replays(q, fmt, n, k, nrows):
    w = _dev(synth.weights(fmt, n, k, synth.W_SEED + 320))
    rows = None
    if nrows is not None:
        rows = _dev(np.random.default_rng(320).integers(0, n, nrows).astype(np.int32))
    m = n if nrows is None else nrows
    dt = torch.bfloat16 if fmt == "nvfp4" else torch.float16
    out = torch.full((m, k), float("nan"), dtype=dt, device=DEV)
    s = torch.cuda.Stream()
    g = _capture(lambda h: q.GET_ROWS[fmt](w, n, k, rows, m, out, h), s)
    want = out.clone()
    for r in range(REPLAYS):
        _replay(g, s, lambda: out.fill_(float(r)))
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (fmt, r)


@pytest.mark.parametrize("fmt,t,m,k", [
    ("q4k", 5, 300, 2304),         # few tiles: K split, y cleared by a fill kernel, atomics
    ("tq1", 1025, 21888, 2048),    # last round split over K: partial clear, atomics
    ("nvfp4", 512, 14336, 1024),   # no split
])
def test_prefill_graph_replays(q, fmt, t, m, k):
    w = synth.weights(fmt, m, k, synth.W_SEED + 330)
    x = np.stack([synth.activations(fmt, k, synth.X_SEED + 330 + i) for i in range(t)])
    wd, xd = _dev(w), _dev(x.view(np.int16))
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    g = _capture(lambda h: q.GEMM[fmt](wd, xd, y, t, m, k, h), s)
    rng = np.random.default_rng(330)
    toks = np.unique(np.concatenate([[0, t - 1], rng.integers(0, t, 8)]))
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 200)]))
    yr, ar = oracle.gemm(fmt, w, x, t, m, k, tokens=toks, rows=rows)
    for r in range(REPLAYS):
        # non-zero garbage in y first: a replay whose clear did not run would add to it
        _replay(g, s, lambda: y.fill_(1000.0 * (r + 1)))
        got = y.cpu().numpy().astype(np.float64)
        assert not np.isnan(got).any()
        g_ = got[np.ix_(toks, rows)]
        assert np.all(np.abs(g_ - yr) <= 1e-3 * ar + 1e-5), (fmt, t, m, k, r)


@pytest.mark.parametrize("fmt,t,m,k", [
    ("q4k", 130, 4096, 4096),      # every tile split: partials, then the reduction kernel
    ("tq1", 1025, 21888, 2048),    # the last round split
])
def test_prefill_ws_graph_replays(q, fmt, t, m, k):
    # the workspace path in a graph: every replay bit-identical to the eager
    # call, with y and the workspace overwritten between replays
    w = synth.weights(fmt, m, k, synth.W_SEED + 331)
    x = np.stack([synth.activations(fmt, k, synth.X_SEED + 331 + i) for i in range(t)])
    wd, xd = _dev(w), _dev(x.view(np.int16))
    nws = q.qgemm_workspace_bytes(t, m, k)
    assert nws > 0
    ws = torch.empty(nws // 4, dtype=torch.float32, device=DEV)
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    g = _capture(lambda h: q.GEMM_WS[fmt](wd, xd, y, t, m, k, ws, h), s)
    want = y.clone()
    assert not torch.isnan(want).any()
    for r in range(REPLAYS):
        def disturb():
            y.fill_(1000.0 * (r + 1))
            ws.fill_(-7.0)
        _replay(g, s, disturb)
        assert torch.equal(y.view(torch.int32), want.view(torch.int32)), (fmt, r)
