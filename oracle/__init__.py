"""ctypes front end of the fp64 CPU oracle (``oracle.c``).

Test infrastructure only: the test suite, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg are its only users; the HIP library never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT = {"q4k": 0, "nvfp4": 1, "tq1": 2, "f16": 3, "bf16": 4}
# element types of materialised rows, epilogue inputs and outputs
DTYPE = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def build() -> str:
    """Compile oracle.c with gcc: -O2, no fast-math, no FMA contraction, OpenMP."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_f16.restype = ctypes.c_double
    lib.oracle_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16.restype = ctypes.c_double
    lib.oracle_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3.restype = ctypes.c_double
    lib.oracle_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1.restype = ctypes.c_double
    lib.oracle_e2m1.argtypes = [ctypes.c_uint8]
    lib.oracle_round_f16.restype = ctypes.c_uint16
    lib.oracle_round_f16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_get_rows.argtypes = [ctypes.c_int, P, I64, I64, P, I64, ctypes.c_int, P]
    lib.oracle_decode16.argtypes = [ctypes.c_int, P, I64, P]
    lib.oracle_gemm.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, I64, P, I64, P, P]
    lib.oracle_tq1_digit.restype = ctypes.c_int
    lib.oracle_tq1_digit.argtypes = [ctypes.c_uint8, ctypes.c_int]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_dequant.argtypes = [ctypes.c_int, P, I64, I64, P]
    lib.oracle_gemv.argtypes = [ctypes.c_int, P, P, I64, I64, P, I64, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def f16(h: int) -> float:
    return _load().oracle_f16(h)


def bf16(h: int) -> float:
    return _load().oracle_bf16(h)


def e4m3(c: int) -> float:
    return _load().oracle_e4m3(c)


def e2m1(n: int) -> float:
    return _load().oracle_e2m1(n)


def round_f16(v: float) -> int:
    """Bits of the binary16 nearest to ``v`` (ties to even)."""
    return _load().oracle_round_f16(float(v))


def round_bf16(v: float) -> int:
    """Bits of the bfloat16 nearest to ``v`` (ties to even)."""
    return _load().oracle_round_bf16(float(v))


def decode16(dtype: str, h: np.ndarray) -> np.ndarray:
    """fp64 values of 16-bit codes of ``dtype`` ("f16" or "bf16")."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.size, dtype=np.float64)
    if h.size:
        _load().oracle_decode16(DTYPE[dtype], _ptr(h), h.size, _ptr(out))
    return out.reshape(h.shape)


def tq1_digit(b: int, k: int) -> int:
    return _load().oracle_tq1_digit(b, k)


def threads() -> int:
    return _load().oracle_threads()


def set_threads(t: int) -> None:
    _load().oracle_set_threads(t)


def dequant(fmt: str, w: np.ndarray, n: int, k: int) -> np.ndarray:
    """fp64 weights [n, k] of the packed matrix ``w``."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    out = np.empty((n, k), dtype=np.float64)
    _load().oracle_dequant(FMT[fmt], _ptr(w), n, k, _ptr(out))
    return out


def get_rows(fmt: str, w: np.ndarray, n: int, k: int, rows, out_dtype: str) -> np.ndarray:
    """Rows ``rows`` of the weights as [len(rows), k] codes of ``out_dtype``
    (uint32 fp32 bits, or uint16 fp16 / bf16 bits): each weight rounded to
    fp32, then to the output type; an index outside [0, n) gives quiet NaNs."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, k), dtype=np.uint32 if out_dtype == "f32" else np.uint16)
    if rows.size:
        _load().oracle_get_rows(FMT[fmt], _ptr(w), n, k, _ptr(rows), rows.size, DTYPE[out_dtype],
                                _ptr(out))
    return out


def gemv(fmt: str, w: np.ndarray, x: np.ndarray, n: int, k: int, rows=None):
    """(y, a): fp64 y[r] = sum_i x_i w_ri and a[r] = sum_i |x_i w_ri| for the
    listed rows (all rows when ``rows`` is None).  ``x`` holds uint16 bits."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.size == k
    if rows is None:
        cnt = n
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
        cnt = rows.size
        rp = _ptr(rows)
    y = np.empty(cnt, dtype=np.float64)
    a = np.empty(cnt, dtype=np.float64)
    if cnt:
        _load().oracle_gemv(FMT[fmt], _ptr(w), _ptr(x), n, k, rp, cnt, _ptr(y), _ptr(a))
    return y, a


def gemm(fmt: str, w: np.ndarray, x: np.ndarray, t: int, n: int, k: int, tokens=None, rows=None):
    """Prefill form (Y = X . dequant(W)^T for T activation rows): (Y, A) of
    shape [len(tokens), len(rows)] in fp64, A the sum of |x_i w_i| per output.
    ``x`` holds [t][k] 16-bit codes; all tokens / rows when None."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(t, k)
    tokens = np.arange(t) if tokens is None else np.asarray(tokens)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert tokens.size == 0 or (tokens.min() >= 0 and tokens.max() < t)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < n)
    y = np.empty((tokens.size, rows.size), dtype=np.float64)
    a = np.empty_like(y)
    if y.size:
        _load().oracle_gemm(FMT[fmt], _ptr(w), _ptr(x), t, n, k, _ptr(tokens), tokens.size, _ptr(rows),
                            rows.size, _ptr(y), _ptr(a))
    return y, a


def c_values(c: np.ndarray, c_dtype: str) -> np.ndarray:
    """fp64 values of an epilogue input given as fp32 (float32 array) or as
    fp16 / bf16 codes (uint16 array)."""
    if c_dtype == "f32":
        return np.asarray(c, dtype=np.float32).astype(np.float64)
    return decode16(c_dtype, c)


def gemv_ex(fmt: str, w, x, n: int, k: int, alpha: float, beta: float, c=None, c_dtype="f32",
            rows=None):
    """General form of the GEMV ("Writing a high performant GEMV + dequant for
    Metal", section "What is a GEMV"): v = alpha * (x . dequant(w)^T) + beta * c
    in fp64, with c not read when beta == 0.  Returns (v, bound) where bound =
    |alpha| * sum_i |x_i w_ri| + |beta * c_r| scales the tolerance.  ``c`` is
    indexed like the output (rows of ``rows`` when given)."""
    y, a = gemv(fmt, w, x, n, k, rows=rows)
    v = float(alpha) * y
    bound = abs(float(alpha)) * a
    if beta != 0.0:
        cv = c_values(c, c_dtype)
        if rows is not None:
            cv = cv[np.asarray(rows, dtype=np.int64)]
        v = v + float(beta) * cv
        bound = bound + np.abs(float(beta) * cv)
    return v, bound
