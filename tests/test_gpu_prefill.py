"""Parity of the prefill entry points (many activation rows, matrix cores)
with the fp64 oracle's Y = X . dequant(W)^T.

Bar: |y - y_ref| <= 1e-3 * sum_i |x_i w_i| + 1e-5 per output.  The weights
enter the matrix unit rounded once to the activation type (relative error at
most 2^-11 for fp16, 2^-8 for bf16, the latter only for NVFP4 whose weights
are exact in bf16), which stays inside that bound; accumulation is fp32.
Shapes cover single tokens, ragged token and row tiles (256 or 512 tokens x
128 rows per workgroup), odd and even K step counts, split and unsplit K and
the Llama-8B prefill shapes (sampled outputs there).
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


CASES = [
    # (format, T, M, K, sampled tokens, sampled rows)
    ("q4k", 1, 64, 256, None, None),
    ("q4k", 5, 300, 2304, None, None),
    ("q4k", 128, 128, 512, None, None),
    ("q4k", 200, 520, 4096, None, None),
    ("q4k", 130, 4096, 4096, 40, 300),
    ("q4k", 512, 4096, 14336, 24, 200),
    ("q4k", 512, 14336, 4096, 24, 300),
    ("nvfp4", 1, 64, 64, None, None),
    ("nvfp4", 5, 300, 2112, None, None),
    ("nvfp4", 200, 520, 4096, None, None),
    ("nvfp4", 512, 4096, 14336, 24, 200),
    ("nvfp4", 512, 14336, 4096, 24, 300),
    ("tq1", 1, 64, 256, None, None),
    ("tq1", 5, 300, 2304, None, None),
    ("tq1", 200, 520, 4096, None, None),
    ("tq1", 131, 77, 1280, None, None),
    ("tq1", 512, 4096, 14336, 24, 200),
    ("tq1", 512, 14336, 4096, 24, 300),
    # one past a 256-token tile and a 128-row tile; an odd step count (a zero step at the end)
    ("q4k", 257, 129, 1280, None, None),
    ("nvfp4", 300, 130, 192, None, None),
    ("tq1", 256, 256, 768, None, None),
    # many tiles, no K split
    ("q4k", 2048, 4096, 4096, 24, 200),
    # enough tiles for 512-token tiles: the large prefill shape, and ragged
    # token tiles of that kernel
    ("q4k", 4096, 14336, 4096, 16, 200),
    ("nvfp4", 2049, 16384, 512, 24, 300),
    ("tq1", 1100, 32768, 512, 24, 300),
    # one round of 512-token tiles instead of two of 256 (ragged last tile)
    ("nvfp4", 1000, 14336, 1024, 24, 300),
    ("tq1", 1000, 14336, 768, 24, 300),
    ("q4k", 2560, 4096, 2048, 24, 300),
]


@pytest.mark.parametrize("fmt,t,m,k,st,sr", CASES)
def test_prefill(q, fmt, t, m, k, st, sr):
    seed = 700 + t + m % 97 + k % 89
    w = synth.weights(fmt, m, k, synth.W_SEED + seed)
    x = _x(fmt, t, k, synth.X_SEED + seed)
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM[fmt](torch.from_numpy(w).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV), y, t, m, k)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    toks = np.arange(t) if st is None else np.unique(np.concatenate([[0, t - 1], rng.integers(0, t, st)]))
    rows = np.arange(m) if sr is None else np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, sr)]))
    yr, ar = oracle.gemm(fmt, w, x, t, m, k, tokens=toks, rows=rows)
    g = got[np.ix_(toks, rows)]
    bad = np.argwhere(~(np.abs(g - yr) <= 1e-3 * ar + 1e-5))
    assert bad.size == 0, (f"{fmt} T={t} {m}x{k}: {len(bad)} outputs off, e.g. token {toks[bad[0][0]]} row "
                           f"{rows[bad[0][1]]}: {g[tuple(bad[0])]} vs {yr[tuple(bad[0])]}")


@pytest.mark.parametrize("fmt,t,m,k", [("q4k", 1025, 21888, 4096), ("tq1", 1025, 21888, 2048),
                                       ("nvfp4", 1025, 21888, 2048)])
def test_prefill_tail_round_split(q, fmt, t, m, k):
    # 171 row tiles x 3 token tiles of 512 = 513 tiles: two full rounds on
    # 256 CUs and one tile left, which is split over K (4 parts of 18, 18,
    # 18 and 10 steps for K = 4096, 2 parts of 18 and 14 steps for K = 2048)
    # into token 1024 x rows 21760.. 21887; the other tiles of that token row
    # are stored unsplit over a cleared y
    seed = 900 + k % 89
    w = synth.weights(fmt, m, k, synth.W_SEED + seed)
    x = _x(fmt, t, k, synth.X_SEED + seed)
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM[fmt](torch.from_numpy(w).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV), y, t, m, k)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    toks = np.unique(np.concatenate([[0, 511, 512, 1023, 1024], rng.integers(0, t, 12)]))
    rows = np.unique(np.concatenate([np.arange(21760, m, 3), [0, 127, 21759], rng.integers(0, m, 60)]))
    yr, ar = oracle.gemm(fmt, w, x, t, m, k, tokens=toks, rows=rows)
    g = got[np.ix_(toks, rows)]
    bad = np.argwhere(~(np.abs(g - yr) <= 1e-3 * ar + 1e-5))
    assert bad.size == 0, (f"{fmt} T={t} {m}x{k}: {len(bad)} outputs off, e.g. token {toks[bad[0][0]]} row "
                           f"{rows[bad[0][1]]}: {g[tuple(bad[0])]} vs {yr[tuple(bad[0])]}")
    assert not np.isnan(got).any()


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_prefill_max_k(q, fmt):
    # the largest K the prefill calls accept (2^20): two row tiles, K split
    # 16 ways, 1024 steps per split; sampled rows of both tiles
    t, m, k = 3, 130, 1 << 20
    w = synth.weights(fmt, m, k, synth.W_SEED + 93)
    x = _x(fmt, t, k, synth.X_SEED + 93)
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM[fmt](torch.from_numpy(w).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV), y, t, m, k)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 127, 128, 129])
    yr, ar = oracle.gemm(fmt, w, x, t, m, k, rows=rows)
    got = y.cpu().numpy().astype(np.float64)[:, rows]
    assert np.all(np.abs(got - yr) <= 1e-3 * ar + 1e-5), np.max(np.abs(got - yr) / (1e-3 * ar + 1e-5))


@pytest.mark.parametrize("fmt,k", [("q4k", 256), ("nvfp4", 64), ("tq1", 256)])
def test_prefill_million_rows(q, fmt, k):
    # M = 1,000,003 (7,813 row tiles, the last one ragged) for 3 tokens; the
    # rows repeat a random block of 4099 rows; 2000 sampled rows
    t, m, period = 3, 1_000_003, 4099
    base = synth.weights(fmt, period, k, synth.W_SEED + 97)
    reps = (m + period - 1) // period
    if fmt == "nvfp4":  # nibbles [M][K/2], then scales [M][K/16]
        nib, sc = base[:period * k // 2].reshape(period, k // 2), base[period * k // 2:].reshape(period, k // 16)
        w = np.concatenate([np.tile(nib, (reps, 1))[:m].ravel(), np.tile(sc, (reps, 1))[:m].ravel()])
    else:
        w = np.tile(base.reshape(period, -1), (reps, 1))[:m].ravel()
    x = _x(fmt, t, k, synth.X_SEED + 97)
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM[fmt](torch.from_numpy(w).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV), y, t, m, k)
    torch.cuda.synchronize()
    rng = np.random.default_rng(97)
    rows = np.unique(np.concatenate([[0, 127, 128, m - 3, m - 1], rng.integers(0, m, 2000)]))
    yr, ar = oracle.gemm(fmt, w, x, t, m, k, rows=rows)
    got = y.cpu().numpy().astype(np.float64)[:, rows]
    assert np.all(np.abs(got - yr) <= 1e-3 * ar + 1e-5)


def test_prefill_split_k_unaligned_y(q):
    # few tiles, so K is split and y is cleared first; y starts 4 bytes past
    # a 16-byte boundary and its length is not a multiple of 4 (the clear's
    # loose head and tail floats); the float before y must stay untouched
    fmt, t, m, k = "q4k", 5, 299, 2304
    w = synth.weights(fmt, m, k, synth.W_SEED + 41)
    x = _x(fmt, t, k, synth.X_SEED + 41)
    buf = torch.full((t * m + 8,), 7.0, dtype=torch.float32, device=DEV)
    y = buf[1:1 + t * m].view(t, m)
    q.GEMM[fmt](torch.from_numpy(w).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV), y, t, m, k)
    torch.cuda.synchronize()
    yr, ar = oracle.gemm(fmt, w, x, t, m, k)
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - yr) <= 1e-3 * ar + 1e-5)
    rest = buf.cpu().numpy()
    assert rest[0] == 7.0 and np.all(rest[1 + t * m:] == 7.0)


def test_prefill_empty_is_noop(q):
    w = torch.zeros(144, dtype=torch.uint8, device=DEV)
    y = torch.zeros(1, device=DEV)
    q.qgemm_q4k(w, w, y, 0, 1, 256)
    q.qgemm_q4k(w, w, y, 3, 0, 256)
    torch.cuda.synchronize()
