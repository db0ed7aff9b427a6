"""The prefill entry points with a workspace (qgemm_*_ws): the partial sums
of a tile split over K go to the caller's workspace and a second kernel adds
them in a fixed order.  Checked against the fp64 oracle (the same bar as the
other prefill tests), for a result identical bit for bit from call to call
(the second call on a workspace the first left full of partial sums) and
with the atomics path's within the bar.
Shapes: every tile split (few tiles), the split last round of 512-token tiles,
and an unsplit launch that needs no workspace.
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


def _x(fmt, t, k, seed):
    return np.stack([synth.activations(fmt, k, seed + i) for i in range(t)])


def _workspace(q, t, m, k):
    n = q.qgemm_workspace_bytes(t, m, k)
    # NaN-filled: nothing may read it before writing; 256-byte aligned (torch's
    # device allocations are)
    return n, (torch.full((max(n, 256) // 4,), float("nan"), dtype=torch.float32, device=DEV) if n else None)


CASES = [
    # (format, T, M, K, sampled tokens, sampled rows)
    ("q4k", 5, 300, 2304, None, None),        # 3 tiles x 3 splits of 12 steps
    ("q4k", 130, 4096, 4096, 40, 300),        # 32 tiles x 6 splits
    ("nvfp4", 200, 520, 4096, None, None),    # 5 tiles x 6 splits
    ("tq1", 131, 77, 1280, None, None),       # 1 tile x 2 splits (ragged rows and tokens)
    ("q4k", 3, 130, 1 << 20, None, [0, 1, 63, 127, 128, 129]),  # the largest K: 16 splits
    ("q4k", 1025, 21888, 4096, 12, 60),       # 513 tiles of 512 tokens: the last one split 4 ways
]


@pytest.mark.parametrize("fmt,t,m,k,st,sr", CASES)
def test_prefill_ws(q, fmt, t, m, k, st, sr):
    seed = 800 + t + m % 97 + k % 89
    w = torch.from_numpy(synth.weights(fmt, m, k, synth.W_SEED + seed)).to(DEV)
    xh = _x(fmt, t, k, synth.X_SEED + seed)
    x = torch.from_numpy(xh.view(np.int16).copy()).to(DEV)
    nbytes, ws = _workspace(q, t, m, k)
    assert nbytes > 0
    ys = [torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV) for _ in range(2)]
    for y in ys:  # two calls on one workspace
        q.GEMM_WS[fmt](w, x, y, t, m, k, ws)
    y_at = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM[fmt](w, x, y_at, t, m, k)
    torch.cuda.synchronize()
    got = ys[0].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ys[1].cpu().numpy().view(np.uint32)), "second call differs"
    rng = np.random.default_rng(seed)
    toks = np.arange(t) if st is None else np.unique(np.concatenate([[0, t - 1], rng.integers(0, t, st)]))
    rows = (np.arange(m) if sr is None else
            np.unique(np.concatenate([[0, m - 1], np.asarray(sr) if isinstance(sr, list) else rng.integers(0, m, sr)])))
    if t == 1025:  # the split tile: token 1024, rows 21760..
        toks = np.unique(np.concatenate([toks, [1023, 1024]]))
        rows = np.unique(np.concatenate([rows, np.arange(21760, m, 5)]))
    yr, ar = oracle.gemm(fmt, w.cpu().numpy(), xh, t, m, k, tokens=toks, rows=rows)
    bar = 1e-3 * ar + 1e-5
    g = got.astype(np.float64)[np.ix_(toks, rows)]
    bad = np.argwhere(~(np.abs(g - yr) <= bar))
    assert bad.size == 0, (f"{fmt} T={t} {m}x{k}: {len(bad)} outputs off, e.g. token {toks[bad[0][0]]} row "
                           f"{rows[bad[0][1]]}: {g[tuple(bad[0])]} vs {yr[tuple(bad[0])]}")
    ga = y_at.cpu().numpy().astype(np.float64)[np.ix_(toks, rows)]
    assert np.all(np.abs(g - ga) <= 2 * bar)


def test_prefill_ws_unsplit_needs_none(q):
    # enough tiles: nothing split, no workspace, and the result is the plain call's
    fmt, t, m, k = "q4k", 2048, 4096, 512
    assert q.qgemm_workspace_bytes(t, m, k) == 0
    w = torch.from_numpy(synth.weights(fmt, m, k, synth.W_SEED + 5)).to(DEV)
    x = torch.from_numpy(_x(fmt, t, k, synth.X_SEED + 5).view(np.int16).copy()).to(DEV)
    y0 = torch.empty((t, m), dtype=torch.float32, device=DEV)
    y1 = torch.empty((t, m), dtype=torch.float32, device=DEV)
    q.qgemm_q4k_ws(w, x, y0, t, m, k, None)
    q.qgemm_q4k(w, x, y1, t, m, k)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_prefill_ws_too_small_is_refused(q):
    fmt, t, m, k = "q4k", 130, 4096, 4096
    n = q.qgemm_workspace_bytes(t, m, k)
    w = torch.zeros(synth.weight_bytes(fmt, m, k), dtype=torch.uint8, device=DEV)
    x = torch.zeros((t, k), dtype=torch.int16, device=DEV)
    y = torch.zeros((t, m), dtype=torch.float32, device=DEV)
    ws = torch.zeros((n - 256) // 4, dtype=torch.float32, device=DEV)
    with pytest.raises(q.QgemvError) as e:
        q.qgemm_q4k_ws(w, x, y, t, m, k, ws)
    assert e.value.code == -7
