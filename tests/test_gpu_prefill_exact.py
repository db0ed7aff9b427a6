"""Bit-exact prefill parity: weights whose every dequantised value is exact in
the matrix units' input type and activations -1, 0 or +1, so every product
and partial sum the MFMA tiles form (in any order, with K split or not) is an
integer multiple of the finest product below 2^24 of them, and Y has one
correct fp32 value per output.  The prefill entry points through the C ABI
must return exactly the oracle's value (fp64, converted to fp32 without
rounding) in every checked output: the plain calls (K splits added with
atomics), the workspace calls (K splits added in order by a second kernel)
and, for Q4_K, the allocation-free call.

Weights: Q4_K d = dmin = 1 (every weight s q - m an integer of magnitude
below 2^11, exact in fp16; scales and mins below 16 for long rows); NVFP4
scales 2^-2..2^2 (weights multiples of 2^-3, exact in bf16); TQ1_0 d = +-2^e.
Shapes walk the launch plans: 256-token tiles split over K, several token
and row tiles, 512-token tiles with a K-split last round, the longest rows.
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


# Largest |weight| in units of the format's finest weight step: Q4_K 63 * 15
# (15 * 15 with small scales), NVFP4 6 * 4 in units of 2^-3, TQ1_0 2 in units
# of 2^-2 (d up to 2).
def _max_term(fmt, small):
    return {"q4k": 225 if small else 945, "nvfp4": 192, "tq1": 8}[fmt]


CASES = [
    # (format, T, M, K, sampled tokens, sampled rows)
    ("q4k", 5, 300, 2304, None, None),          # one token tile, K split
    ("q4k", 130, 4096, 4096, 40, 300),          # 32 tiles, K split
    ("q4k", 600, 1000, 4096, None, None),       # 3 x 8 tiles of 256 tokens
    ("q4k", 1100, 2000, 2048, 60, 200),         # 512-token tiles
    ("q4k", 3, 130, 1 << 16, None, None),       # long rows (small scales), 16 splits
    ("q4k", 1025, 21888, 4096, 12, 60),         # 512-token tiles, the last round split over K
    ("nvfp4", 200, 520, 4096, None, None),
    ("nvfp4", 700, 600, 2048, None, None),
    ("tq1", 131, 77, 1280, None, None),
    ("tq1", 600, 1000, 4096, 80, 200),
]


def _random_cases():
    # shapes off the planned grid (fixed seed, so the list is stable)
    rng = np.random.default_rng(777)
    c = []
    for i in range(9):
        fmt = ("q4k", "nvfp4", "tq1")[i % 3]
        kmul = 64 if fmt == "nvfp4" else 256
        t, m = int(rng.integers(1, 1500)), int(rng.integers(1, 6000))
        c.append((fmt, t, m, int(rng.integers(1, 8192 // kmul + 1)) * kmul, 24, 48))
    return c


CASES += _random_cases()


def _sample(t, m, st, sr, seed):
    rng = np.random.default_rng(seed)
    toks = np.arange(t) if st is None else np.unique(np.concatenate([[0, t - 1], rng.integers(0, t, st)]))
    rows = np.arange(m) if sr is None else np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, sr)]))
    if t == 1025:  # the split tile: token 1024, rows 21760..
        toks = np.unique(np.concatenate([toks, [1023, 1024]]))
        rows = np.unique(np.concatenate([rows, np.arange(21760, m, 7)]))
    return toks, rows


@pytest.mark.parametrize("fmt,t,m,k,st,sr", CASES)
def test_prefill_bit_exact(q, fmt, t, m, k, st, sr):
    small = fmt == "q4k" and k > 16384
    assert k * _max_term(fmt, small) < 2 ** 24
    seed = 900 + t + m % 97 + k % 89
    wh = synth.weights_exact(fmt, m, k, seed, small=small)
    xh = np.stack([synth.x_ternary(fmt, k, seed + 1 + i) for i in range(t)])
    w = torch.from_numpy(np.ascontiguousarray(wh)).to(DEV)
    x = torch.from_numpy(xh.view(np.int16).copy()).to(DEV)
    outs = {}
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM[fmt](w, x, y, t, m, k)
    outs["atomics"] = y
    nbytes = q.qgemm_workspace_bytes(t, m, k)
    ws = torch.full((max(nbytes, 256) // 4,), float("nan"), dtype=torch.float32, device=DEV) if nbytes else None
    y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMM_WS[fmt](w, x, y, t, m, k, ws)
    outs["workspace"] = y
    if fmt == "q4k" and nbytes <= q.NOALLOC_MAX_BYTES:
        y = torch.full((t, m), float("nan"), dtype=torch.float32, device=DEV)
        q.qgemm_q4k_noalloc(w, x, y, t, m, k)
        outs["noalloc"] = y
    torch.cuda.synchronize()
    toks, rows = _sample(t, m, st, sr, seed)
    want, _ = oracle.gemm(fmt, wh, xh, t, m, k, tokens=toks, rows=rows)
    assert np.array_equal(want.astype(np.float32).astype(np.float64), want), "inputs not exact"
    for name, yt in outs.items():
        got = yt.cpu().numpy().astype(np.float64)[np.ix_(toks, rows)]
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{fmt} T={t} {m}x{k} {name}: {len(bad)} outputs differ, e.g. token "
                               f"{toks[bad[0][0]]} row {rows[bad[0][1]]}: gpu {got[tuple(bad[0])]!r} "
                               f"oracle {want[tuple(bad[0])]!r}")
