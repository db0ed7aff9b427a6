"""Thin ctypes binding of libqgemv (include/qgemv.h).

Same names as the C entry points; the functions only turn torch tensors (or
raw device addresses) into pointers and the current HIP stream, call the
library and raise on a non-zero return code.  Every step of the computation
runs in the library's HIP kernels; there is no fallback path: if the library
is missing this module fails at import.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

QGEMV_OK = 0
QGEMV_E_NULL = -1
QGEMV_E_SHAPE = -2
QGEMV_E_ALIGN = -3
QGEMV_E_HIP = -4
QGEMV_E_ALIAS = -5
QGEMV_E_DTYPE = -6
QGEMV_E_WORKSPACE = -7

# element type codes
QGEMV_F32 = 0
QGEMV_F16 = 1
QGEMV_BF16 = 2
DTYPE_CODE = {"f32": QGEMV_F32, "f16": QGEMV_F16, "bf16": QGEMV_BF16}

# Entry points declared in include/qgemv.h.
GEMV_SYMBOLS = ("qgemv_q4k", "qgemv_nvfp4", "qgemv_tq1", "qgemv_f16", "qgemv_bf16")
GEMV_EX_SYMBOLS = ("qgemv_q4k_ex", "qgemv_nvfp4_ex", "qgemv_tq1_ex", "qgemv_f16_ex", "qgemv_bf16_ex")
DEQUANT_SYMBOLS = ("qdequant_q4k", "qdequant_nvfp4", "qdequant_tq1")
ROWS_SYMBOLS = ("qget_rows_q4k", "qget_rows_nvfp4", "qget_rows_tq1")
GEMM_SYMBOLS = ("qgemm_q4k", "qgemm_nvfp4", "qgemm_tq1")
GEMM_WS_SYMBOLS = ("qgemm_q4k_ws", "qgemm_nvfp4_ws", "qgemm_tq1_ws")
ALL_SYMBOLS = GEMV_SYMBOLS + GEMV_EX_SYMBOLS + DEQUANT_SYMBOLS + ROWS_SYMBOLS + GEMM_SYMBOLS + GEMM_WS_SYMBOLS + (
    "qgemm_q4k_noalloc", "qgemm_workspace_bytes", "qgemv_read_ceiling", "qgemv_read_sink_len", "qgemv_strerror",
    "qgemv_last_hip_error", "qgemv_build_id")


class Epilogue(ctypes.Structure):
    """struct qgemv_epilogue: y = alpha * v + beta * c, stored as y_dtype."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("c", ctypes.c_void_p),
                ("c_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32)]


class QgemvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.qgemv_strerror(code).decode()
        if code == QGEMV_E_HIP:
            msg += f" (hipError {_lib.qgemv_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    for name in GEMV_SYMBOLS:
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, I64, I64, P]
    for name in GEMV_EX_SYMBOLS:
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, I64, I64, ctypes.POINTER(Epilogue), P]
    for name in DEQUANT_SYMBOLS:
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P, P, I64, I64, P]
    for name in ROWS_SYMBOLS:
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P, I64, I64, P, I64, P, ctypes.c_int32, P]
    for name in GEMM_SYMBOLS:
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, I64, I64, I64, P]
    for name in GEMM_WS_SYMBOLS:
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P, P, P, I64, I64, I64, P, I64, P]
    lib.qgemm_q4k_noalloc.restype = ctypes.c_int
    lib.qgemm_q4k_noalloc.argtypes = [P, P, P, I64, I64, I64, P]
    lib.qgemm_workspace_bytes.restype = ctypes.c_int64
    lib.qgemm_workspace_bytes.argtypes = [I64, I64, I64]
    lib.qgemv_read_ceiling.restype = ctypes.c_int
    lib.qgemv_read_ceiling.argtypes = [P, I64, P, P]
    lib.qgemv_read_sink_len.restype = ctypes.c_int64
    lib.qgemv_read_sink_len.argtypes = [I64]
    lib.qgemv_strerror.restype = ctypes.c_char_p
    lib.qgemv_strerror.argtypes = [ctypes.c_int]
    lib.qgemv_last_hip_error.restype = ctypes.c_int
    lib.qgemv_build_id.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _addr(t) -> int:
    """Device address of a torch tensor (must live on the GPU), or an int."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("qgemv takes device memory: move the tensor to the GPU first")
    if not t.is_contiguous():
        raise ValueError("qgemv takes contiguous tensors")
    return t.data_ptr()


# bytes of a packed weight matrix of M rows and K columns, per entry point suffix
def weight_bytes(fmt: str, M: int, K: int) -> int:
    if fmt == "q4k":
        return M * (K // 256) * 144
    if fmt == "nvfp4":
        return M * (K // 2) + M * (K // 16)
    if fmt == "tq1":
        return M * (K // 256) * 54
    return M * K * 2  # f16, bf16


def _need(t, nbytes: int, what: str, where: str, dtype=None) -> None:
    """Raise ValueError if tensor t holds fewer than nbytes bytes (or has the
    wrong element type); raw integer addresses are the caller's to size."""
    if t is None or isinstance(t, int):
        return
    if dtype is not None and t.dtype not in dtype:
        raise ValueError(f"{where}: {what} must be {' or '.join(str(d) for d in dtype)}, not {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{where}: {what} holds {have} bytes, the call needs {nbytes}")


def _f32():
    import torch

    return (torch.float32,)


def _i16():
    import torch

    return (torch.float16, torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream) -> int:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != QGEMV_OK:
        raise QgemvError(rc, where)


def _gemv(name, w, x, y, M, K, stream):
    if M > 0 and K > 0:
        _need(w, weight_bytes(name.split("_")[1], M, K), "w", name)
        _need(x, 2 * K, "x", name, _i16())
        _need(y, 4 * M, "y", name, _f32())
    _check(getattr(_lib, name)(_addr(w), _addr(x), _addr(y), int(M), int(K), _stream(stream)), name)
    return y


def qgemv_q4k(w, x, y, M, K, stream=None):
    """y[M] (fp32) = x[K] (fp16) . dequant_Q4_K(w)^T, enqueued on `stream`."""
    return _gemv("qgemv_q4k", w, x, y, M, K, stream)


def qgemv_nvfp4(w, x, y, M, K, stream=None):
    """y[M] (fp32) = x[K] (bf16) . dequant_NVFP4(w)^T, enqueued on `stream`."""
    return _gemv("qgemv_nvfp4", w, x, y, M, K, stream)


def qgemv_tq1(w, x, y, M, K, stream=None):
    """y[M] (fp32) = x[K] (fp16) . dequant_TQ1_0(w)^T, enqueued on `stream`."""
    return _gemv("qgemv_tq1", w, x, y, M, K, stream)


def qgemv_f16(w, x, y, M, K, stream=None):
    """y[M] (fp32) = x[K] (fp16) . W^T with W [M][K] fp16, enqueued on `stream`."""
    return _gemv("qgemv_f16", w, x, y, M, K, stream)


def qgemv_bf16(w, x, y, M, K, stream=None):
    """y[M] (fp32) = x[K] (bf16) . W^T with W [M][K] bf16, enqueued on `stream`."""
    return _gemv("qgemv_bf16", w, x, y, M, K, stream)


def dtype_code(t) -> int:
    """Element-type code of a torch tensor (fp32 / fp16 / bf16)."""
    import torch

    codes = {torch.float32: QGEMV_F32, torch.float16: QGEMV_F16, torch.bfloat16: QGEMV_BF16}
    if t.dtype not in codes:
        raise ValueError(f"unsupported element type {t.dtype}")
    return codes[t.dtype]


def _gemv_ex(name, w, x, y, M, K, alpha, beta, c, stream):
    if M > 0 and K > 0:
        _need(w, weight_bytes(name.split("_")[1], M, K), "w", name)
        _need(x, 2 * K, "x", name, _i16())
        if y is not None and not isinstance(y, int):
            _need(y, M * y.element_size(), "y", name)
        if beta != 0 and c is not None and not isinstance(c, int):
            _need(c, M * c.element_size(), "c", name)
    ep = Epilogue(float(alpha), float(beta), _addr(c) if c is not None else None,
                  dtype_code(c) if c is not None else QGEMV_F32, dtype_code(y))
    _check(getattr(_lib, name)(_addr(w), _addr(x), _addr(y), int(M), int(K), ctypes.byref(ep),
                               _stream(stream)), name)
    return y


def qgemv_q4k_ex(w, x, y, M, K, alpha=1.0, beta=0.0, c=None, stream=None):
    """y = alpha * (x . dequant_Q4_K(w)^T) + beta * c in y's element type."""
    return _gemv_ex("qgemv_q4k_ex", w, x, y, M, K, alpha, beta, c, stream)


def qgemv_nvfp4_ex(w, x, y, M, K, alpha=1.0, beta=0.0, c=None, stream=None):
    return _gemv_ex("qgemv_nvfp4_ex", w, x, y, M, K, alpha, beta, c, stream)


def qgemv_tq1_ex(w, x, y, M, K, alpha=1.0, beta=0.0, c=None, stream=None):
    return _gemv_ex("qgemv_tq1_ex", w, x, y, M, K, alpha, beta, c, stream)


def qgemv_f16_ex(w, x, y, M, K, alpha=1.0, beta=0.0, c=None, stream=None):
    return _gemv_ex("qgemv_f16_ex", w, x, y, M, K, alpha, beta, c, stream)


def qgemv_bf16_ex(w, x, y, M, K, alpha=1.0, beta=0.0, c=None, stream=None):
    return _gemv_ex("qgemv_bf16_ex", w, x, y, M, K, alpha, beta, c, stream)


def _get_rows(name, w, M, K, rows, nrows, out, stream):
    if rows is not None and not isinstance(rows, int):
        import torch

        if rows.dtype != torch.int32:
            raise ValueError("row indices must be an int32 tensor")
        _need(rows, 4 * nrows, "rows", name)
    if M > 0 and K > 0:
        _need(w, weight_bytes(name.split("_")[2], M, K), "w", name)
    if nrows > 0 and out is not None and not isinstance(out, int):
        _need(out, nrows * K * out.element_size(), "out", name)
    _check(getattr(_lib, name)(_addr(w), int(M), int(K), _addr(rows), int(nrows), _addr(out),
                               dtype_code(out), _stream(stream)), name)
    return out


def qget_rows_q4k(w, M, K, rows, nrows, out, stream=None):
    """out[nrows][K] = rows `rows` (int32 device tensor, or None for 0..nrows-1)
    of dequant_Q4_K(w), in out's element type."""
    return _get_rows("qget_rows_q4k", w, M, K, rows, nrows, out, stream)


def qget_rows_nvfp4(w, M, K, rows, nrows, out, stream=None):
    return _get_rows("qget_rows_nvfp4", w, M, K, rows, nrows, out, stream)


def qget_rows_tq1(w, M, K, rows, nrows, out, stream=None):
    return _get_rows("qget_rows_tq1", w, M, K, rows, nrows, out, stream)


def _gemm_sizes(name, w, x, y, T, M, K):
    if T > 0 and M > 0 and K > 0:
        _need(w, weight_bytes(name.split("_")[1], M, K), "w", name)
        _need(x, 2 * T * K, "x", name, _i16())
        _need(y, 4 * T * M, "y", name, _f32())


def qgemm_q4k(w, x, y, T, M, K, stream=None):
    """Prefill: y[T][M] (fp32) = x[T][K] (fp16) . dequant_Q4_K(w)^T."""
    _gemm_sizes("qgemm_q4k", w, x, y, T, M, K)
    _check(_lib.qgemm_q4k(_addr(w), _addr(x), _addr(y), int(T), int(M), int(K), _stream(stream)), "qgemm_q4k")
    return y


def qgemm_nvfp4(w, x, y, T, M, K, stream=None):
    """Prefill: y[T][M] (fp32) = x[T][K] (bf16) . dequant_NVFP4(w)^T."""
    _gemm_sizes("qgemm_nvfp4", w, x, y, T, M, K)
    _check(_lib.qgemm_nvfp4(_addr(w), _addr(x), _addr(y), int(T), int(M), int(K), _stream(stream)),
           "qgemm_nvfp4")
    return y


def qgemm_tq1(w, x, y, T, M, K, stream=None):
    """Prefill: y[T][M] (fp32) = x[T][K] (fp16) . dequant_TQ1_0(w)^T."""
    _gemm_sizes("qgemm_tq1", w, x, y, T, M, K)
    _check(_lib.qgemm_tq1(_addr(w), _addr(x), _addr(y), int(T), int(M), int(K), _stream(stream)), "qgemm_tq1")
    return y


def qgemm_workspace_bytes(T, M, K) -> int:
    """Bytes of workspace qgemm_*_ws needs for a T x M x K prefill (0: none)."""
    n = _lib.qgemm_workspace_bytes(int(T), int(M), int(K))
    if n < 0:
        raise QgemvError(int(n), "qgemm_workspace_bytes")
    return int(n)


def _gemm_ws(name, w, x, y, T, M, K, ws, stream):
    _gemm_sizes(name, w, x, y, T, M, K)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(getattr(_lib, name)(_addr(w), _addr(x), _addr(y), int(T), int(M), int(K),
                               None if ws is None else _addr(ws), nbytes, _stream(stream)), name)
    return y


def qgemm_q4k_ws(w, x, y, T, M, K, ws, stream=None):
    """Prefill with a run-to-run identical result: K splits go through `ws`
    (a device tensor of at least qgemm_workspace_bytes bytes; None when that
    is 0)."""
    return _gemm_ws("qgemm_q4k_ws", w, x, y, T, M, K, ws, stream)


# Size of the library's own workspace array behind qgemm_q4k_noalloc.
NOALLOC_MAX_BYTES = 32 << 20


def qgemm_q4k_noalloc(w, x, y, T, M, K, stream=None):
    """qgemm_q4k_ws without a caller workspace: the K splits go through a fixed
    32 MiB array per device inside the library, so the call allocates nothing.
    Calls on one device that overlap in time share that array and race."""
    _gemm_sizes("qgemm_q4k_noalloc", w, x, y, T, M, K)
    _check(_lib.qgemm_q4k_noalloc(_addr(w), _addr(x), _addr(y), int(T), int(M), int(K), _stream(stream)),
           "qgemm_q4k_noalloc")
    return y


def qgemm_nvfp4_ws(w, x, y, T, M, K, ws, stream=None):
    """NVFP4 prefill through a workspace (see qgemm_q4k_ws)."""
    return _gemm_ws("qgemm_nvfp4_ws", w, x, y, T, M, K, ws, stream)


def qgemm_tq1_ws(w, x, y, T, M, K, ws, stream=None):
    """TQ1_0 prefill through a workspace (see qgemm_q4k_ws)."""
    return _gemm_ws("qgemm_tq1_ws", w, x, y, T, M, K, ws, stream)


def _dequant(name, w, out, M, K, stream):
    if M > 0 and K > 0:
        _need(w, weight_bytes(name.split("_")[1], M, K), "w", name)
        _need(out, 4 * M * K, "out", name, _f32())
    _check(getattr(_lib, name)(_addr(w), _addr(out), int(M), int(K), _stream(stream)), name)
    return out


def qdequant_q4k(w, out, M, K, stream=None):
    return _dequant("qdequant_q4k", w, out, M, K, stream)


def qdequant_nvfp4(w, out, M, K, stream=None):
    return _dequant("qdequant_nvfp4", w, out, M, K, stream)


def qdequant_tq1(w, out, M, K, stream=None):
    return _dequant("qdequant_tq1", w, out, M, K, stream)


def qgemv_read_sink_len(nbytes: int) -> int:
    return int(_lib.qgemv_read_sink_len(int(nbytes)))


def qgemv_read_ceiling(buf, nbytes, sink, stream=None):
    _check(_lib.qgemv_read_ceiling(_addr(buf), int(nbytes), _addr(sink), _stream(stream)),
           "qgemv_read_ceiling")
    return sink


def qgemv_build_id() -> str:
    return _lib.qgemv_build_id().decode()


def qgemv_strerror(code: int) -> str:
    return _lib.qgemv_strerror(int(code)).decode()


# Convenience: allocate y / out with torch and dispatch by format name.
GEMV = {"q4k": qgemv_q4k, "nvfp4": qgemv_nvfp4, "tq1": qgemv_tq1, "f16": qgemv_f16, "bf16": qgemv_bf16}
GEMV_EX = {"q4k": qgemv_q4k_ex, "nvfp4": qgemv_nvfp4_ex, "tq1": qgemv_tq1_ex, "f16": qgemv_f16_ex,
           "bf16": qgemv_bf16_ex}
DEQUANT = {"q4k": qdequant_q4k, "nvfp4": qdequant_nvfp4, "tq1": qdequant_tq1}
GET_ROWS = {"q4k": qget_rows_q4k, "nvfp4": qget_rows_nvfp4, "tq1": qget_rows_tq1}
GEMM = {"q4k": qgemm_q4k, "nvfp4": qgemm_nvfp4, "tq1": qgemm_tq1}
GEMM_WS = {"q4k": qgemm_q4k_ws, "nvfp4": qgemm_nvfp4_ws, "tq1": qgemm_tq1_ws}


def gemv(fmt: str, w, x, M: int, K: int, y=None, stream=None):
    import torch

    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=w.device)
    return GEMV[fmt](w, x, y, M, K, stream)


def dequant(fmt: str, w, M: int, K: int, out=None, stream=None):
    import torch

    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=w.device)
    return DEQUANT[fmt](w, out, M, K, stream)


def _torch_dtype(name: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def gemv_ex(fmt: str, w, x, M: int, K: int, alpha=1.0, beta=0.0, c=None, y_dtype="f32", y=None,
            stream=None):
    import torch

    if y is None:
        y = torch.empty(M, dtype=_torch_dtype(y_dtype), device=w.device)
    return GEMV_EX[fmt](w, x, y, M, K, alpha, beta, c, stream)


def get_rows(fmt: str, w, M: int, K: int, rows=None, nrows=None, dtype="f16", out=None, stream=None):
    import torch

    if nrows is None:
        nrows = M if rows is None else rows.numel()
    if out is None:
        out = torch.empty((nrows, K), dtype=_torch_dtype(dtype), device=w.device)
    return GET_ROWS[fmt](w, M, K, rows, nrows, out, stream)


def gemm(fmt: str, w, x, T: int, M: int, K: int, y=None, stream=None):
    import torch

    if y is None:
        y = torch.empty((T, M), dtype=torch.float32, device=w.device)
    return GEMM[fmt](w, x, y, T, M, K, stream)
