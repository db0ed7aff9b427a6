"""Parity of the widened entry points (through the C ABI) with the fp64 oracle:
the dense fp16 / bf16 GEMV, the general output stage y = alpha v + beta c in
fp32 / fp16 / bf16 for every format, and row materialisation (GET_ROWS).

Bars:
- dense GEMV: as for the packed formats, |y - y_ref| <= 1e-3 * sum |x_i w_i| + 1e-5;
- epilogue: |alpha| times that bound, plus 2^-22 (|alpha v| + |beta c|) for the
  fp32 epilogue arithmetic, plus one unit in the last place of the output type
  at the result (its final rounding);
- rows: bit-exact against the oracle's fp16(fp32(w)) / bf16(fp32(w)) / fp32(w),
  NaN matching NaN, and out-of-range indices give exactly the quiet-NaN row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth

pytestmark = pytest.mark.gpu

RTOL = 1e-3
ATOL = 1e-5
DEV = "cuda:0"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def q():
    from dequant_gemv_amd import qgemv

    return qgemv


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _bits_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy()).to(DEV)


def _vec_dev(v, dtype):
    if dtype == "f32":
        return _dev(v.astype(np.float32))
    return _bits_dev(v).view(TORCH[dtype])


def _to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _sample_rows(n, sample, seed):
    if sample is None or sample >= n:
        return None
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, sample)]))


# ---- dense GEMV ----------------------------------------------------------------

DENSE = [
    (1, 8, None), (3, 200, None), (65, 512, None), (300, 4096, None), (2100, 520, None),
    (5000, 1000, 1500), (2049, 4104, 1500), (1100, 14336, 600), (4096, 14336, 1200),
    (14336, 4096, 1500), (70, 65536, None),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("n,k,sample", DENSE)
def test_dense_gemv(q, fmt, n, k, sample):
    seed = 300 + n % 97 + k % 89
    w = synth.weights(fmt, n, k, synth.W_SEED + seed)
    x = synth.activations(fmt, k, synth.X_SEED + seed)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMV[fmt](_dev(w), _bits_dev(x), y, n, k)
    torch.cuda.synchronize()
    got = _to_f64(y)
    rows = _sample_rows(n, sample, seed)
    yr, ar = oracle.gemv(fmt, w, x, n, k, rows=rows)
    if rows is not None:
        got = got[rows]
    bad = np.flatnonzero(~(np.abs(got - yr) <= RTOL * ar + ATOL))
    assert bad.size == 0, f"{fmt} {n}x{k}: {bad.size} rows off, e.g. {bad[0]}: {got[bad[0]]} vs {yr[bad[0]]}"


def test_dense_gemv_empty_is_noop(q):
    w = torch.zeros(16, dtype=torch.uint8, device=DEV)
    y = torch.zeros(1, device=DEV)
    q.qgemv_bf16(w, w, y, 0, 8)
    torch.cuda.synchronize()


# ---- general output stage -----------------------------------------------------

EX_SHAPES = {
    "q4k": [(4096, 14336, 1200), (100, 20480, None)],
    "nvfp4": [(4096, 14336, 1200), (100, 18432, None)],
    "tq1": [(14336, 4096, 1500), (300, 2304, None)],
    "f16": [(1100, 4104, None)],
    "bf16": [(4096, 14336, 1200)],
}
EX_CASES = [(fmt, n, k, s) for fmt, shapes in EX_SHAPES.items() for (n, k, s) in shapes]
COEFS = [(1.0, 0.0), (0.5, 1.0), (-2.0, 0.25)]


def _ulp(v, dtype):
    a = np.abs(v)
    if dtype == "f32":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
        return 2.0 ** (e - 23)
    if dtype == "f16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _check_ex(got, v, bound, alpha, beta, cv, y_dtype, what):
    ref_abs = np.abs(v)
    tol = (abs(alpha) * (RTOL * bound + ATOL)
           + 2.0 ** -22 * (ref_abs + (np.abs(beta * cv) if cv is not None else 0.0))
           + _ulp(np.maximum(ref_abs, np.abs(got)), y_dtype))
    bad = np.flatnonzero(~(np.abs(got - v) <= tol))
    assert bad.size == 0, f"{what}: {bad.size} rows off, e.g. {bad[0]}: {got[bad[0]]!r} vs {v[bad[0]]!r} tol {tol[bad[0]]!r}"


@pytest.mark.parametrize("y_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("fmt,n,k,sample", EX_CASES)
def test_gemv_epilogue(q, fmt, n, k, sample, y_dtype):
    seed = 500 + n % 89 + k % 97
    w = synth.weights(fmt, n, k, synth.W_SEED + seed)
    x = synth.activations(fmt, k, synth.X_SEED + seed)
    wd, xd = _dev(w), _bits_dev(x)
    rows = _sample_rows(n, sample, seed)
    yr, ar = oracle.gemv(fmt, w, x, n, k, rows=rows)
    for ci, c_dtype in enumerate(["f32", "f16", "bf16"]):
        c = synth.vector(n, c_dtype, 900 + seed + ci)
        cd = _vec_dev(c, c_dtype)
        cv_all = oracle.c_values(c, c_dtype)
        cv = cv_all if rows is None else cv_all[rows]
        for alpha, beta in COEFS:
            if beta == 0.0 and ci > 0:
                continue
            y = torch.full((n,), float("nan"), dtype=TORCH[y_dtype], device=DEV)
            q.GEMV_EX[fmt](wd, xd, y, n, k, alpha, beta, cd if beta != 0.0 else None)
            torch.cuda.synchronize()
            got = _to_f64(y)
            if rows is not None:
                got = got[rows]
            v = alpha * yr + (beta * cv if beta != 0.0 else 0.0)
            _check_ex(got, v, ar, alpha, beta, cv if beta != 0.0 else None, y_dtype,
                      f"{fmt} {n}x{k} y {y_dtype} c {c_dtype} alpha {alpha} beta {beta}")


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1", "bf16"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_gemv_epilogue_in_place(q, fmt, dtype):
    # c is y itself: y = alpha v + beta y
    n, k = 2100, 4096
    w = synth.weights(fmt, n, k, 77)
    x = synth.activations(fmt, k, 78)
    c = synth.vector(n, dtype, 79)
    y = _vec_dev(c, dtype).clone()
    alpha, beta = 0.75, -1.5
    q.GEMV_EX[fmt](_dev(w), _bits_dev(x), y, n, k, alpha, beta, y)
    torch.cuda.synchronize()
    v, bound = oracle.gemv_ex(fmt, w, x, n, k, alpha, beta, c, dtype)
    yr, ar = oracle.gemv(fmt, w, x, n, k)
    _check_ex(_to_f64(y), v, ar, alpha, beta, oracle.c_values(c, dtype), dtype, f"{fmt} in place {dtype}")


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1", "f16"])
def test_gemv_epilogue_beta_zero_ignores_c(q, fmt):
    n, k = 700, 2048
    w = synth.weights(fmt, n, k, 81)
    x = synth.activations(fmt, k, 82)
    wd, xd = _dev(w), _bits_dev(x)
    nan_c = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    y = torch.empty(n, dtype=torch.float32, device=DEV)
    q.GEMV_EX[fmt](wd, xd, y, n, k, 1.0, 0.0, nan_c)
    y0 = torch.empty(n, dtype=torch.float32, device=DEV)
    q.GEMV[fmt](wd, xd, y0, n, k)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)  # same kernel arithmetic, c never read


# ---- row materialisation -------------------------------------------------------

NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def _rows_bits(t, dtype):
    a = t.cpu()
    if dtype == "f32":
        return a.view(torch.int32).numpy().view(np.uint32)
    return a.view(torch.int16).numpy().view(np.uint16)


def _check_rows(q, fmt, w, n, k, rows, nrows, dtype):
    out = torch.full((nrows, k), 1.0, dtype=TORCH[dtype], device=DEV)
    rows_d = None if rows is None else _dev(rows.astype(np.int32))
    q.GET_ROWS[fmt](_dev(w), n, k, rows_d, nrows, out)
    torch.cuda.synchronize()
    got = _rows_bits(out, dtype)
    idx = np.arange(nrows) if rows is None else rows.astype(np.int64)
    want = oracle.get_rows(fmt, w, n, k, idx, dtype)
    if dtype == "f32":
        gv, wv = got.view(np.float32), want.view(np.float32)
    else:
        gv = oracle.decode16(dtype, got)
        wv = oracle.decode16(dtype, want)
    same = (got == want) | (np.isnan(gv) & np.isnan(wv))
    invalid = (idx < 0) | (idx >= n)
    if invalid.any():  # the fill is exactly the documented quiet NaN
        assert np.all(got[invalid] == NAN_BITS[dtype])
    if not same.all():
        i = np.argwhere(~same)[0]
        pytest.fail(f"{fmt} rows {dtype} {n}x{k}: {int((~same).sum())} mismatches, first {tuple(i)}: "
                    f"gpu {got[tuple(i)]:#x} oracle {want[tuple(i)]:#x}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("fmt,n,k", [("q4k", 300, 4096), ("q4k", 37, 256), ("nvfp4", 300, 4096),
                                     ("nvfp4", 37, 32), ("tq1", 300, 4096), ("tq1", 37, 256),
                                     ("q4k", 129, 14336), ("nvfp4", 129, 14368)])
def test_get_rows_indexed(q, fmt, n, k, dtype):
    w = synth.weights(fmt, n, k, 600 + n + k)
    rng = np.random.default_rng(n + k)
    rows = np.concatenate([rng.integers(0, n, 40), [0, n - 1, n - 1, -1, n, 2 ** 31 - 1, -(2 ** 31)]])
    _check_rows(q, fmt, w, n, k, rows, rows.size, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_get_rows_all(q, fmt, dtype):
    n, k = (14336, 4096) if fmt == "tq1" else (4096, 14336)
    w = synth.weights(fmt, n, k, 650)
    _check_rows(q, fmt, w, n, k, None, n, dtype)
    _check_rows(q, fmt, w, n, k, None, 1000, dtype)  # a prefix


def test_get_rows_q4k_extreme_bytes(q):
    # random d / dmin bytes: subnormal, negative, Inf and NaN fp16 scales, fp32
    # values beyond fp16's range (they round to Inf) and below its subnormals
    rng = np.random.default_rng(19)
    w = rng.integers(0, 256, (64, 16 * 144), dtype=np.uint8)
    for dtype in ("f16", "bf16"):
        _check_rows(q, "q4k", w, 64, 4096, np.arange(64)[::-1].copy(), 64, dtype)


def test_get_rows_rejects_int64_indices(q):
    w = torch.zeros(144, dtype=torch.uint8, device=DEV)
    out = torch.empty((1, 256), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        q.qget_rows_q4k(w, 1, 256, torch.zeros(1, dtype=torch.int64, device=DEV), 1, out)
