"""NVFP4 layout checks and GEMV brute force for all three formats.

NVFP4 (Mojo module "fp4_gemv"): weight = e2m1(nibble) * |e4m3 scale|, one scale
per 16 consecutive weights of a row.  Which nibble of a byte holds the even
element and how the scale bytes are laid out are not on the page: the library
fixes the even element in the low nibble and a plain row-major [N][K/16] scale
array after the [N][K/2] nibble array (parity unpinned for these two
conventions; the one-hot checks below only confirm the oracle follows them).

GEMV ("Writing a high performant GEMV + dequant for Metal", section "What is a
GEMV": y = x W^T with alpha = 1, beta = 0): on tiny shapes the oracle's fp64 y
and |x||w| sum are compared with the exact rational sums.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dequant_gemv_amd import synth


def _nvfp4_buf(n, k, nib, sc):
    return np.concatenate([np.asarray(nib, np.uint8).reshape(-1), np.asarray(sc, np.uint8).reshape(-1)])


def test_nvfp4_one_hot_nibbles_and_scales():
    n, k = 2, 64
    for r in range(n):
        for i in range(k):
            nib = np.zeros((n, k // 2), np.uint8)
            nib[r, i // 2] = 0x2 << (4 * (i % 2))  # e2m1 code 2 = 1.0 in the nibble of element i
            sc = np.full((n, k // 16), 0x38, np.uint8)  # 1.0
            sc[r, i // 16] = 0x40  # 2.0 on the scale block of element i
            w = oracle.dequant("nvfp4", _nvfp4_buf(n, k, nib, sc), n, k)
            want = np.zeros((n, k))
            want[r, i] = 2.0
            assert np.array_equal(w, want), (r, i)


def test_nvfp4_scale_sign_ignored():
    n, k = 1, 32
    rng = np.random.default_rng(3)
    nib = rng.integers(0, 256, (n, k // 2))
    sc = np.array([[0x3A, 0x45]], np.uint8)
    w_pos = oracle.dequant("nvfp4", _nvfp4_buf(n, k, nib, sc), n, k)
    w_neg = oracle.dequant("nvfp4", _nvfp4_buf(n, k, nib, sc | 0x80), n, k)
    assert np.array_equal(w_pos, w_neg)


def test_nvfp4_weights_are_products():
    n, k = 3, 96
    buf = synth.nvfp4_weights(n, k, 31)
    nib = buf[: n * k // 2].reshape(n, k // 2)
    sc = buf[n * k // 2:].reshape(n, k // 16)
    w = oracle.dequant("nvfp4", buf, n, k)
    for r in range(n):
        for i in range(k):
            c = (nib[r, i // 2] >> (4 * (i % 2))) & 15
            assert w[r, i] == oracle.e2m1(int(c)) * abs(oracle.e4m3(int(sc[r, i // 16])))


def _exact(fmt, w, x, n, k):
    wd = oracle.dequant(fmt, w, n, k)
    dec = oracle.bf16 if fmt == "nvfp4" else oracle.f16
    xv = [Fraction(dec(int(v))) for v in x]
    ys, as_ = [], []
    for r in range(n):
        terms = [xv[i] * Fraction(float(wd[r, i])) for i in range(k)]
        ys.append(sum(terms))
        as_.append(sum(abs(t) for t in terms))
    return ys, as_


@pytest.mark.parametrize("fmt,k", [("q4k", 256), ("q4k", 512), ("tq1", 256), ("tq1", 512), ("nvfp4", 32), ("nvfp4", 512)])
@pytest.mark.parametrize("n", [1, 3, 5])
def test_gemv_brute_force(fmt, k, n):
    w = synth.weights(fmt, n, k, 100 + n + k)
    x = synth.activations(fmt, k, 200 + n + k)
    y, a = oracle.gemv(fmt, w, x, n, k)
    ye, ae = _exact(fmt, w, x, n, k)
    for r in range(n):
        # K sequential fp64 additions: error below K * 2^-53 * sum|x w|
        assert abs(Fraction(float(y[r])) - ye[r]) <= Fraction(k, 2 ** 52) * ae[r]
        assert abs(Fraction(float(a[r])) - ae[r]) <= Fraction(k, 2 ** 52) * ae[r]


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_gemv_row_subset_and_sign_symmetry(fmt):
    n, k = 37, 1024
    w = synth.weights(fmt, n, k, 7)
    x = synth.activations(fmt, k, 8)
    y, a = oracle.gemv(fmt, w, x, n, k)
    rows = np.array([36, 0, 17, 17, 5])
    ys, as_ = oracle.gemv(fmt, w, x, n, k, rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(as_, a[rows])
    yn, an = oracle.gemv(fmt, w, x ^ np.uint16(0x8000), n, k)  # x -> -x
    assert np.array_equal(yn, -y) and np.array_equal(an, a)


def test_gemv_matches_dequant_then_matmul():
    # the gemv entry point re-dequantises internally; it must agree with the
    # dequant entry point followed by a library matrix-vector product
    for fmt in ("q4k", "nvfp4", "tq1"):
        n, k = 19, 2048
        w = synth.weights(fmt, n, k, 40)
        x = synth.activations(fmt, k, 41)
        y, a = oracle.gemv(fmt, w, x, n, k)
        wd = oracle.dequant(fmt, w, n, k)
        dec = oracle.bf16 if fmt == "nvfp4" else oracle.f16
        xv = np.array([dec(int(v)) for v in x])
        assert np.allclose(wd @ xv, y, rtol=0, atol=1e-12 * a.max())
        assert np.allclose(np.abs(wd * xv).sum(1), a, rtol=1e-13, atol=0)
