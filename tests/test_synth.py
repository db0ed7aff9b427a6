"""The seeded generators: determinism, shapes and the stated distributions."""
import numpy as np

import oracle
from dequant_gemv_amd import synth


def test_deterministic_and_shaped():
    for fmt in ("q4k", "nvfp4", "tq1"):
        a = synth.weights(fmt, 5, 512, 1)
        b = synth.weights(fmt, 5, 512, 1)
        c = synth.weights(fmt, 5, 512, 2)
        assert np.array_equal(a, b) and not np.array_equal(a, c)
        assert a.dtype == np.uint8 and a.size == synth.weight_bytes(fmt, 5, 512)
        x = synth.activations(fmt, 512, 3)
        assert x.dtype == np.uint16 and x.size == 512


def test_q4k_fields():
    w = synth.q4k_weights(64, 4096, 1000).reshape(64, 16, 144)
    d = w[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    dmin = w[:, :, 2:4].copy().view(np.float16).astype(np.float64)
    assert d.min() >= 0.000999 and d.max() <= 0.01001 and dmin.min() >= 0.000999
    assert 120 < w[:, :, 4:].mean() < 135  # uniform bytes


def test_nvfp4_scales_distribution():
    n, k = 64, 4096
    buf = synth.nvfp4_weights(n, k, 1002)
    sc = buf[n * k // 2:]
    vals = np.array([oracle.e4m3(int(c)) for c in sc])
    assert np.all(vals >= 0) and np.all(np.isfinite(vals))
    assert 0.035 < vals.mean() < 0.045  # E|N(0, 0.05)| = 0.0399
    sub = np.mean((sc & 0x78) == 0)  # exponent field 0: zero or subnormal
    assert 0.2 < sub < 0.3


def test_tq1_trits_uniform():
    n, k = 64, 4096
    w = synth.tq1_weights(n, k, 1003).reshape(n, 16, 54)
    t = np.array([[oracle.tq1_digit(int(b), kk) for kk in range(5)] for b in w[:, :, :48].reshape(-1)])
    frac = np.bincount(t.reshape(-1), minlength=3) / t.size
    assert np.all(np.abs(frac - 1 / 3) < 0.01)
    d = w[:, :, 52:54].copy().view(np.float16).astype(np.float64)
    assert d.min() >= 0.00999 and d.max() <= 0.0501
