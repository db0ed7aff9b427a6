"""Bit-exact GEMV parity: inputs whose every product and partial sum is exact
in fp32, so the GEMV has one correct fp32 result per row whatever the
summation order, and the HIP path through the C ABI must return exactly the
oracle's value (fp64, converted to fp32 without rounding) in every row.

Weights use unit or power-of-two scale factors (Q4_K d = dmin = 1; NVFP4
scales 2^-2..2^2 with random sign bits; TQ1_0 d = +-2^e; dense integers
-8..8), activations are -1, 0 or +1.  A wrong nibble, digit, scale, group,
block or row then shows up as a non-zero difference in the row it touches,
instead of hiding inside the tolerance that general inputs need.

The shapes walk every dispatch choice of the kernels: each K-chunk count of
the row-streaming kernels with a ragged last chunk, each rows-per-wave and
waves-per-workgroup choice (one wave per SIMD, two, and the many-rows
single-round and multi-round launches), ragged last workgroups, the K-split
kernels for longer rows, and the Llama-8B decode shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# rows that pick each rows-per-wave choice of the row-streaming launch (one
# wave per SIMD, then 1 to 8, 10, 12, 14, 16 rows per wave, then more than
# one round); the larger ones only where the LDS stage allows them
N_ALL = [1000, 1500, 3001, 5001, 7001, 9001, 11001, 13001, 15001, 19001, 23001, 27001, 31001, 40001]
N_SHORT = [1000, 1500, 3001, 5001, 7001, 11001, 13001, 15001, 17001]
N_FEW = [1000, 1500, 3001, 9001]
N_TWO = [1000, 1500, 5001]


def _cases():
    c = []
    # Q4_K: K-chunks of 8 blocks; a ragged last chunk in each
    c += [("q4k", n, 1792) for n in N_ALL]            # 1 chunk (7 blocks)
    c += [("q4k", n, 2816) for n in N_SHORT]          # 2 chunks (11 blocks)
    c += [("q4k", n, k) for k in (5888, 7936) for n in N_FEW]           # 3, 4 chunks
    c += [("q4k", n, k) for k in (9984, 12032, 14080) for n in N_TWO]   # 5, 6, 7 chunks
    c += [("q4k", n, 16128) for n in (1000, 3001)]    # 8 chunks
    c += [("q4k", 4096, 4096), ("q4k", 14336, 4096), ("q4k", 4096, 14336), ("q4k", 6144, 4096),
          ("q4k", 1, 256), ("q4k", 5, 512), ("q4k", 33, 16640), ("q4k", 300, 18432), ("q4k", 65, 36864)]
    # NVFP4: K-chunks of 2048 weights
    c += [("nvfp4", n, 1056) for n in N_ALL]
    c += [("nvfp4", n, 2080) for n in N_SHORT]
    c += [("nvfp4", n, k) for k in (4160, 6240) for n in N_FEW]
    c += [("nvfp4", n, k) for k in (8224, 10272, 12320) for n in N_TWO]
    c += [("nvfp4", n, 14368) for n in (1000, 3001)]
    c += [("nvfp4", 4096, 14336), ("nvfp4", 1, 32), ("nvfp4", 3, 96), ("nvfp4", 33, 16416), ("nvfp4", 65, 36896)]
    # TQ1_0: 16-block segments (K = 2048 is one short segment, 6144 ends in one);
    # K = 4096 over 1024 rows takes the table-driven kernel (every rows-per-wave
    # choice, its ring-buffer stage from 10 rows per wave on)
    c += [("tq1", n, 2048) for n in N_ALL]
    c += [("tq1", n, 4096) for n in N_ALL + [14336, 28672]]
    c += [("tq1", n, k) for k in (6144, 8192) for n in N_SHORT + [19001, 23001]]
    c += [("tq1", 1, 256), ("tq1", 5, 768), ("tq1", 37, 4352), ("tq1", 33, 41216)]
    # dense fp16 / bf16
    c += [(f, n, k) for f in ("f16", "bf16") for n, k in ((37, 1000), (4096, 4096), (2000, 14336), (3, 65536))]
    return c


# Largest |term| of the kernels' intermediate sums per unit activation, in
# units of the finest product: Q4_K d s q and dmin m are summed separately
# (63 * 15 + 63 = 1008, 15 * 15 + 15 = 240 with small scales); NVFP4 e2m1
# times scale in units of 2^-3 (6 * 4 * 8); TQ1_0 d (t - 1) in units of 2^-2
# (2 * 4, and the kernel also sums the activations times d); dense |w| <= 8.
def _max_term(fmt, small):
    return {"q4k": 240 if small else 1008, "nvfp4": 192, "tq1": 16, "f16": 8, "bf16": 8}[fmt]


@pytest.fixture(scope="module")
def q():
    from dequant_gemv_amd import qgemv

    return qgemv


@pytest.mark.parametrize("fmt,n,k", _cases())
def test_gemv_bit_exact(q, fmt, n, k):
    small = fmt == "q4k" and k > 16384
    # every partial sum in any order stays an integer multiple of the finest
    # product below 2^24 of them: exact in fp32
    assert k * _max_term(fmt, small) < 2 ** 24
    seed = 7 * n + k
    w = synth.weights_exact(fmt, n, k, seed, small=small)
    x = synth.x_ternary(fmt, k, seed + 1)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMV[fmt](torch.from_numpy(np.ascontiguousarray(w)).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV),
                y, n, k)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want, _ = oracle.gemv(fmt, w, x, n, k)
    assert np.array_equal(want.astype(np.float32).astype(np.float64), want), "inputs not exact"
    bad = np.flatnonzero(got.astype(np.float64) != want)
    assert bad.size == 0, (f"{fmt} {n}x{k}: {bad.size} rows differ, e.g. row {bad[0]}: gpu {got[bad[0]]!r} "
                           f"oracle {want[bad[0]]!r}")


def _random_cases():
    # shapes off the planned grid: mostly many rows, some a handful; K any
    # multiple of the block up to 16384 (fixed seed, so the list is stable)
    rng = np.random.default_rng(54321)
    c = []
    for fmt, kmul in (("q4k", 256), ("nvfp4", 32), ("tq1", 256)):
        for _ in range(8):
            n = int(rng.integers(1, 40000)) if rng.random() < 0.8 else int(rng.integers(1, 64))
            c.append((fmt, n, int(rng.integers(1, 16384 // kmul + 1)) * kmul))
    return c


@pytest.mark.parametrize("fmt,n,k", _random_cases())
def test_gemv_bit_exact_random_shapes(q, fmt, n, k):
    test_gemv_bit_exact(q, fmt, n, k)


@pytest.mark.parametrize("fmt,n,k", [("q4k", 3001, 2816), ("nvfp4", 1500, 4160), ("tq1", 13001, 2048),
                                     ("q4k", 300, 18432), ("tq1", 37, 4352)])
@pytest.mark.parametrize("y_dtype", ["f32", "f16"])
def test_gemv_ex_bit_exact(q, fmt, n, k, y_dtype):
    # the output stage with alpha = 2, beta = -1 and c = an integer vector:
    # 2 v - c is exact in fp32; for fp16 y, rows whose value fp16 cannot hold
    # exactly get c = 2 v (they then read 0)
    seed = 11 * n + k
    w = synth.weights_exact(fmt, n, k, seed, small=k > 16384)
    x = synth.x_ternary(fmt, k, seed + 1)
    v, _ = oracle.gemv(fmt, w, x, n, k)
    c = np.random.default_rng(seed).integers(-50, 51, size=n).astype(np.float32)
    want = 2.0 * v - c
    if y_dtype == "f16":
        with np.errstate(over="ignore"):
            keep = want.astype(np.float16).astype(np.float64) == want
        want = np.where(keep, want, 0.0)
        c = np.where(keep, c, (2.0 * v).astype(np.float32))
    y = q.gemv_ex(fmt, torch.from_numpy(np.ascontiguousarray(w)).to(DEV), torch.from_numpy(x.view(np.int16).copy()).to(DEV),
                  n, k, alpha=2.0, beta=-1.0, c=torch.from_numpy(c).to(DEV), y_dtype=y_dtype)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{fmt} {n}x{k} {y_dtype}: {bad.size} rows differ, e.g. row {bad[0]}: {got[bad[0]]} vs {want[bad[0]]}"
