"""Pins of the oracle's prefill form Y = X . dequant(W)^T (many activation rows;
the Mojo fp4_gemv page's M > 1 matmul path and the TQ1_0 page's prefill).

The dense formats reduce it to a library matrix product of the decoded arrays
(numpy float64 matmul): a transposed operand or a swapped index fails there.
The packed formats must agree, token by token, with the pinned GEMV and with
the pinned dequantisation followed by a library product.
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth


def _x(fmt, t, k, seed):
    return np.stack([synth.activations(fmt, k, seed + i) for i in range(t)])


def _decode(fmt, codes):
    if fmt in ("nvfp4", "bf16"):
        return torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    return codes.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_dense_prefill_is_library_matmul(fmt):
    t, n, k = 7, 11, 72
    w = synth.weights(fmt, n, k, 70)
    x = _x(fmt, t, k, 71)
    y, a = oracle.gemm(fmt, w, x, t, n, k)
    wf = _decode(fmt, w.view(np.uint16).reshape(n, k))
    xf = _decode(fmt, x)
    ref = xf @ wf.T  # [t, n]
    assert y.shape == (t, n)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(xf).max() * np.abs(wf).max() * k)
    assert np.allclose(a, np.abs(xf) @ np.abs(wf).T, rtol=1e-13, atol=0)


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_packed_prefill_matches_dequant_then_matmul(fmt):
    t, n, k = 5, 9, 512
    w = synth.weights(fmt, n, k, 80)
    x = _x(fmt, t, k, 81)
    y, a = oracle.gemm(fmt, w, x, t, n, k)
    ref = _decode(fmt, x) @ oracle.dequant(fmt, w, n, k).T
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * a.max())
    for q in range(t):  # token by token equal to the GEMV
        yq, aq = oracle.gemv(fmt, w, x[q], n, k)
        assert np.array_equal(y[q], yq) and np.array_equal(a[q], aq)


def test_prefill_subsets_and_order():
    fmt, t, n, k = "q4k", 6, 10, 256
    w = synth.weights(fmt, n, k, 90)
    x = _x(fmt, t, k, 91)
    y, a = oracle.gemm(fmt, w, x, t, n, k)
    toks, rows = np.array([5, 0, 3]), np.array([9, 2, 2, 0])
    ys, as_ = oracle.gemm(fmt, w, x, t, n, k, tokens=toks, rows=rows)
    assert np.array_equal(ys, y[np.ix_(toks, rows)]) and np.array_equal(as_, a[np.ix_(toks, rows)])
