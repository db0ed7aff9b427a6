"""The C-ABI library without a GPU: it loads, exports every function that
include/qgemv.h declares, carries the build id of its sources, and rejects bad
arguments in host code (these calls return before any HIP call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def q():
    from dequant_gemv_amd import qgemv

    return qgemv


def test_header_symbols_exported(q):
    names = _header_functions()
    assert len(names) == 29, names
    lib = q.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(q.ALL_SYMBOLS) == names


def test_build_id_matches_sources(q):
    from dequant_gemv_amd import build

    assert q.qgemv_build_id() == build.build_id()


def test_strerror(q):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert q.qgemv_strerror(code)
    assert "unknown" in q.qgemv_strerror(42)


A = 0x7F0000000000  # a 16-byte aligned fake device address, never dereferenced


GEMVS = [("qgemv_q4k", 256, 1 << 24), ("qgemv_nvfp4", 32, 1 << 24), ("qgemv_tq1", 256, 1 << 24),
         ("qgemv_f16", 8, 65536), ("qgemv_bf16", 8, 65536)]


@pytest.mark.parametrize("name,kmul,kmax", GEMVS)
def test_gemv_validation(q, name, kmul, kmax):
    f = getattr(q.lib(), name)
    W, X, Y = A, A + (1 << 32), A + (2 << 32)
    assert f(W, X, Y, -1, kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 4, 0, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 4, kmul + kmul // 2, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 4, -kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 4, kmax + kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 1 << 31, kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 0, kmul, None) == q.QGEMV_OK  # empty: no-op, no launch
    assert f(None, X, Y, 4, kmul, None) == q.QGEMV_E_NULL
    assert f(W, None, Y, 4, kmul, None) == q.QGEMV_E_NULL
    assert f(W, X, None, 4, kmul, None) == q.QGEMV_E_NULL
    assert f(W + 8, X, Y, 4, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, X + 2, Y, 4, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, X, Y + 2, 4, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, X, W + 16, 4, kmul, None) == q.QGEMV_E_ALIAS
    assert f(W, X, X, 4, kmul, None) == q.QGEMV_E_ALIAS


GEMMS = [("qgemm_q4k", 256), ("qgemm_nvfp4", 64), ("qgemm_tq1", 256)]


@pytest.mark.parametrize("name,kmul", GEMMS)
def test_gemm_validation(q, name, kmul):
    f = getattr(q.lib(), name)
    W, X, Y = A, A + (1 << 36), A + (2 << 36)
    assert f(W, X, Y, -1, 4, kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 65535 * 128 + 1, 4, kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 3, -1, kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 3, 4, 0, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 3, 4, kmul + kmul // 2, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 3, 4, (1 << 20) + 256, None) == q.QGEMV_E_SHAPE  # K limit of the prefill
    if name == "qgemm_nvfp4":
        assert f(W, X, Y, 3, 4, 96, None) == q.QGEMV_E_SHAPE  # whole 64-weight steps
    assert f(W, X, Y, 0, 4, kmul, None) == q.QGEMV_OK  # empty: no-op, no launch
    assert f(W, X, Y, 3, 0, kmul, None) == q.QGEMV_OK
    assert f(None, X, Y, 3, 4, kmul, None) == q.QGEMV_E_NULL
    assert f(W, None, Y, 3, 4, kmul, None) == q.QGEMV_E_NULL
    assert f(W, X, None, 3, 4, kmul, None) == q.QGEMV_E_NULL
    assert f(W + 8, X, Y, 3, 4, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, X + 2, Y, 3, 4, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, X, Y + 2, 3, 4, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, X, W + 16, 3, 4, kmul, None) == q.QGEMV_E_ALIAS
    assert f(W, X, X + 4, 3, 4, kmul, None) == q.QGEMV_E_ALIAS


def test_gemm_noalloc_validation(q):
    """The argument checks of qgemm_q4k_noalloc all come before it touches its
    device array; a split needing more than the array is refused up front."""
    f = q.lib().qgemm_q4k_noalloc
    W, X, Y = A, A + (1 << 36), A + (2 << 36)
    assert q.qgemm_workspace_bytes(4608, 8192, 4096) > q.NOALLOC_MAX_BYTES
    assert q.qgemm_workspace_bytes(512, 4096, 14336) <= q.NOALLOC_MAX_BYTES
    assert f(W, X, Y, 4608, 8192, 4096, None) == q.QGEMV_E_WORKSPACE
    assert f(W, X, Y, 3, 4, 384, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 65535 * 128 + 1, 4, 256, None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 0, 4, 256, None) == q.QGEMV_OK
    assert f(W, X, Y, 3, 0, 256, None) == q.QGEMV_OK
    assert f(None, X, Y, 130, 4096, 4096, None) == q.QGEMV_E_NULL
    assert f(W, X, Y + 2, 130, 4096, 4096, None) == q.QGEMV_E_ALIGN
    assert f(W, X, X + 4, 130, 4096, 4096, None) == q.QGEMV_E_ALIAS


@pytest.mark.parametrize("name,kmul,kmax", GEMVS)
def test_gemv_ex_validation(q, name, kmul, kmax):
    f = getattr(q.lib(), name + "_ex")
    E = q.Epilogue
    W, X, Y, C = A, A + (1 << 32), A + (2 << 32), A + (3 << 32)
    ok = E(1.0, 0.0, None, q.QGEMV_F32, q.QGEMV_F32)
    assert f(W, X, Y, 4, kmax + kmul, ctypes.byref(ok), None) == q.QGEMV_E_SHAPE
    assert f(W, X, Y, 4, kmul, ctypes.byref(E(1.0, 0.0, None, 0, 3)), None) == q.QGEMV_E_DTYPE
    assert f(W, X, Y, 4, kmul, ctypes.byref(E(1.0, 1.0, C, -1, 0)), None) == q.QGEMV_E_DTYPE
    # c's type is irrelevant (and c not read) when beta == 0
    assert f(W, X, Y, 0, kmul, ctypes.byref(E(1.0, 0.0, None, 7, 0)), None) == q.QGEMV_OK
    assert f(W, X, Y, 0, kmul, None, None) == q.QGEMV_OK  # NULL epilogue = plain
    assert f(W, X, Y, 4, kmul, ctypes.byref(E(1.0, 1.0, None, 0, 0)), None) == q.QGEMV_E_NULL
    assert f(W, X, Y + 2, 4, kmul, ctypes.byref(E(1.0, 0.0, None, 0, q.QGEMV_F32)), None) == q.QGEMV_E_ALIGN
    assert f(W, X, Y + 1, 4, kmul, ctypes.byref(E(1.0, 0.0, None, 0, q.QGEMV_F16)), None) == q.QGEMV_E_ALIGN
    assert f(W, X, Y, 4, kmul, ctypes.byref(E(1.0, 2.0, C + 2, q.QGEMV_F32, 0)), None) == q.QGEMV_E_ALIGN
    assert f(W, X, W + 32, 4, kmul, ctypes.byref(ok), None) == q.QGEMV_E_ALIAS
    # c may be y itself only with the same element type
    assert f(W, X, Y, 4, kmul, ctypes.byref(E(1.0, 1.0, Y + 4, q.QGEMV_F32, q.QGEMV_F32)), None) == q.QGEMV_E_ALIAS
    assert f(W, X, Y, 4, kmul, ctypes.byref(E(1.0, 1.0, Y, q.QGEMV_F16, q.QGEMV_F32)), None) == q.QGEMV_E_ALIAS


@pytest.mark.parametrize("name,kmul", [("qget_rows_q4k", 256), ("qget_rows_nvfp4", 32), ("qget_rows_tq1", 256)])
def test_get_rows_validation(q, name, kmul):
    f = getattr(q.lib(), name)
    W, R, O = A, A + (1 << 32), A + (1 << 36)
    assert f(W, 4, kmul, R, -1, O, 1, None) == q.QGEMV_E_SHAPE
    assert f(W, 4, kmul, None, 5, O, 1, None) == q.QGEMV_E_SHAPE  # rows NULL: nrows <= M
    assert f(W, 4, kmul // 2, R, 2, O, 1, None) == q.QGEMV_E_SHAPE
    assert f(W, 4, kmul, R, 2, O, 3, None) == q.QGEMV_E_DTYPE
    assert f(W, 4, kmul, R, 0, O, 1, None) == q.QGEMV_OK
    assert f(W, 4, kmul, R, 2, None, 1, None) == q.QGEMV_E_NULL
    assert f(None, 4, kmul, R, 2, O, 1, None) == q.QGEMV_E_NULL
    assert f(W, 4, kmul, R, 2, O + 8, 1, None) == q.QGEMV_E_ALIGN
    assert f(W, 4, kmul, R + 2, 2, O, 1, None) == q.QGEMV_E_ALIGN
    assert f(W, 4, kmul, R, 2, W, 0, None) == q.QGEMV_E_ALIAS
    assert f(W, 4, kmul, R, 2, R - 16, 0, None) == q.QGEMV_E_ALIAS


@pytest.mark.parametrize("name,kmul", [("qdequant_q4k", 256), ("qdequant_nvfp4", 32), ("qdequant_tq1", 256)])
def test_dequant_validation(q, name, kmul):
    f = getattr(q.lib(), name)
    W, O = A, A + (1 << 36)
    assert f(W, O, -1, kmul, None) == q.QGEMV_E_SHAPE
    assert f(W, O, 2, kmul // 2, None) == q.QGEMV_E_SHAPE
    assert f(W, O, 0, kmul, None) == q.QGEMV_OK
    assert f(None, O, 2, kmul, None) == q.QGEMV_E_NULL
    assert f(W, None, 2, kmul, None) == q.QGEMV_E_NULL
    assert f(W + 4, O, 2, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, O + 4, 2, kmul, None) == q.QGEMV_E_ALIGN
    assert f(W, W, 2, kmul, None) == q.QGEMV_E_ALIAS


def test_read_ceiling_validation(q):
    f = q.lib().qgemv_read_ceiling
    assert f(A, 15, A + (1 << 32), None) == q.QGEMV_E_SHAPE
    assert f(A, 0, A + (1 << 32), None) == q.QGEMV_OK
    assert f(None, 1024, A + (1 << 32), None) == q.QGEMV_E_NULL
    assert f(A + 4, 1024, A + (1 << 32), None) == q.QGEMV_E_ALIGN
    assert f(A, 1024, A + 512, None) == q.QGEMV_E_ALIAS
    assert q.qgemv_read_sink_len(1) == 1 and q.qgemv_read_sink_len(32768) == 1
    assert q.qgemv_read_sink_len(32769) == 2


def test_binding_rejects_host_tensors(q):
    import torch

    w = torch.zeros(144, dtype=torch.uint8)
    x = torch.zeros(256, dtype=torch.float16)
    y = torch.zeros(1, dtype=torch.float32)
    with pytest.raises(ValueError, match="device memory"):
        q.qgemv_q4k(w, x, y, 1, 256)


def test_binding_checks_tensor_sizes_and_types(q):
    # checked before any address is taken, so host tensors reach these checks
    import torch

    f16, f32, u8 = torch.float16, torch.float32, torch.uint8
    w, x, y = torch.zeros(2 * 144, dtype=u8), torch.zeros(256, dtype=f16), torch.zeros(2, dtype=f32)
    with pytest.raises(ValueError, match="w holds 144 bytes"):
        q.qgemv_q4k(w[:144], x, y, 2, 256)
    with pytest.raises(ValueError, match="x holds"):
        q.qgemv_q4k(w, x[:255], y, 2, 256)
    with pytest.raises(ValueError, match="y holds"):
        q.qgemv_q4k(w, x, y[:1], 2, 256)
    with pytest.raises(ValueError, match="y must be"):
        q.qgemv_q4k(w, x, torch.zeros(2, dtype=f16), 2, 256)
    with pytest.raises(ValueError, match="x must be"):
        q.qgemv_q4k(w, torch.zeros(256, dtype=f32), y, 2, 256)
    with pytest.raises(ValueError, match="w holds"):
        q.qgemv_nvfp4(torch.zeros(2 * 128 + 2 * 16 - 1, dtype=u8), x, y, 2, 256)
    with pytest.raises(ValueError, match="w holds"):
        q.qgemv_bf16(torch.zeros(2 * 256 * 2 - 1, dtype=u8), x, y, 2, 256)
    # output stage: y in its own type, c only when beta != 0
    with pytest.raises(ValueError, match="y holds"):
        q.qgemv_q4k_ex(w, x, torch.zeros(1, dtype=f16), 2, 256)
    with pytest.raises(ValueError, match="c holds"):
        q.qgemv_q4k_ex(w, x, torch.zeros(2, dtype=f16), 2, 256, beta=1.0, c=torch.zeros(1, dtype=f32))
    # prefill, rows, materialisation
    with pytest.raises(ValueError, match="y holds"):
        q.qgemm_q4k(w, torch.zeros(3 * 256, dtype=f16), torch.zeros(5, dtype=f32), 3, 2, 256)
    with pytest.raises(ValueError, match="x holds"):
        q.qgemm_tq1(torch.zeros(2 * 54, dtype=u8), torch.zeros(2 * 256, dtype=f16), torch.zeros(6, dtype=f32),
                    3, 2, 256)
    with pytest.raises(ValueError, match="out holds"):
        q.qget_rows_q4k(w, 2, 256, None, 2, torch.zeros((1, 256), dtype=f16))
    with pytest.raises(ValueError, match="rows holds"):
        q.qget_rows_q4k(w, 2, 256, torch.zeros(1, dtype=torch.int32), 2, torch.zeros((2, 256), dtype=f16))
    with pytest.raises(ValueError, match="out must be"):
        q.qdequant_q4k(w, torch.zeros((2, 256), dtype=f16), 2, 256)
