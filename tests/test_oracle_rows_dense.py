"""Pins of the oracle's widened paths: correctly rounded fp16 / bf16 encoders,
row materialisation (GET_ROWS), the dense fp16 / bf16 GEMV and the alpha/beta
epilogue.

Sources (page titles): the dense GEMV is the comparison kernel of the Mojo
"fp4_gemv" page; materialising rows is the dequantize template of "metal:
TQ1_0 kernel performance" (section "Prefill") and the fp32 dequant of the Mojo
page; the epilogue is the general form of "Writing a high performant GEMV +
dequant for Metal", section "What is a GEMV".
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth


# ---- encoders ----------------------------------------------------------------


def _f16_bits_numpy(v):
    with np.errstate(over="ignore"):
        return int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])


def test_round_f16_matches_numpy_on_ties_and_neighbours():
    # every binary16 value, the midpoints to its neighbours and points just
    # off those midpoints (numpy converts float64 -> float16 with one rounding)
    codes = np.arange(0, 0x7C00, 7, dtype=np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    nxt = (codes + 1).view(np.float16).astype(np.float64)
    for v, u in zip(vals, nxt):
        mid = (v + u) / 2
        for t in (v, mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid):
            assert oracle.round_f16(t) == _f16_bits_numpy(t), t


def test_round_f16_matches_numpy_random_and_overflow():
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        np.array([65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26]),
    ])
    for t in xs:
        assert oracle.round_f16(t) == _f16_bits_numpy(t), t
        assert oracle.round_f16(-t) == _f16_bits_numpy(-t), t


def test_round_f16_landmarks():
    assert oracle.round_f16(1.0) == 0x3C00
    assert oracle.round_f16(1 + 2.0 ** -11) == 0x3C00      # tie -> even (down)
    assert oracle.round_f16(1 + 3 * 2.0 ** -11) == 0x3C02  # tie -> even (up)
    assert oracle.round_f16(65520.0) == 0x7C00             # halfway past the max: inf
    assert oracle.round_f16(2.0 ** -25) == 0x0000          # tie between 0 and 2^-24
    assert oracle.round_f16(-0.0) == 0x8000
    assert oracle.round_f16(math.inf) == 0x7C00 and oracle.round_f16(-math.inf) == 0xFC00
    assert math.isnan(oracle.f16(oracle.round_f16(math.nan)))


def test_round_bf16_matches_torch_on_float32_values():
    # torch rounds float32 -> bfloat16 to nearest even: compare on float32 bit
    # patterns of every class (random bits, then ties and their neighbours)
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, 20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties, ties + 1, ties - 1])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_round_bf16_landmarks():
    assert oracle.round_bf16(1.0) == 0x3F80
    assert oracle.round_bf16(1 + 2.0 ** -8) == 0x3F80       # tie -> even (down)
    assert oracle.round_bf16(1 + 3 * 2.0 ** -8) == 0x3F82   # tie -> even (up)
    assert oracle.round_bf16(3.3895313892515355e38) == 0x7F7F  # largest finite
    assert oracle.round_bf16(2.0 ** 128) == 0x7F80
    assert oracle.round_bf16(2.0 ** -133) == 0x0001         # smallest subnormal
    assert oracle.round_bf16(2.0 ** -134) == 0x0000         # tie -> even (zero)


# ---- row materialisation ------------------------------------------------------


FMTS = ["q4k", "nvfp4", "tq1", "f16", "bf16"]


def _w(fmt, n, k, seed=11):
    return synth.weights(fmt, n, k, seed)


@pytest.mark.parametrize("fmt", FMTS)
def test_get_rows_f32_is_the_fp32_dequant(fmt):
    n, k = 9, 512
    w = _w(fmt, n, k)
    rows = np.array([3, 0, 8, 3, -1, 9, 5])
    out = oracle.get_rows(fmt, w, n, k, rows, "f32").view(np.float32)
    wd = oracle.dequant(fmt, w, n, k).astype(np.float32)
    for j, r in enumerate(rows):
        if 0 <= r < n:
            assert np.array_equal(out[j], wd[r])
        else:
            assert np.all(out[j].view(np.uint32) == 0x7FC00000)


@pytest.mark.parametrize("fmt", FMTS)
def test_get_rows_16bit_match_library_casts(fmt):
    # fp32 weights cast by numpy (-> fp16) and torch (-> bf16), both round to
    # nearest even
    n, k = 7, 1024
    w = _w(fmt, n, k)
    rows = np.arange(n)[::-1].copy()
    wd = oracle.dequant(fmt, w, n, k).astype(np.float32)[rows]
    h = oracle.get_rows(fmt, w, n, k, rows, "f16")
    assert np.array_equal(h, wd.astype(np.float16).view(np.uint16))
    b = oracle.get_rows(fmt, w, n, k, rows, "bf16")
    ref = torch.from_numpy(wd).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_get_rows_exact_formats():
    # NVFP4 weights (2-bit by 4-bit significands) are exact in fp16 and bf16;
    # TQ1_0 weights are +-d or 0 with d in fp16, exact in fp16; dense weights
    # come back bit for bit in their own type.
    n, k = 5, 2048
    w = _w("nvfp4", n, k)
    wd = oracle.dequant("nvfp4", w, n, k)
    rows = np.arange(n)
    assert np.array_equal(oracle.decode16("f16", oracle.get_rows("nvfp4", w, n, k, rows, "f16")), wd)
    assert np.array_equal(oracle.decode16("bf16", oracle.get_rows("nvfp4", w, n, k, rows, "bf16")), wd)
    w = _w("tq1", n, k)
    assert np.array_equal(oracle.decode16("f16", oracle.get_rows("tq1", w, n, k, rows, "f16")),
                          oracle.dequant("tq1", w, n, k))
    for fmt in ("f16", "bf16"):
        w = _w(fmt, n, k)
        assert np.array_equal(oracle.get_rows(fmt, w, n, k, rows, fmt), w.view(np.uint16).reshape(n, k))


def test_get_rows_q4k_rounds_the_fp32_weight():
    # The 16-bit materialisation rounds the fp32 weight.  A Q4_K weight needs
    # more than 24 significant bits when d*s*q and dmin*m are far apart in
    # magnitude: with d = 1 and dmin = 2^-14 * (1 + 2^-10) every weight with
    # s*q and m both non-zero is inexact in fp32.  The oracle must round those
    # twice (fp32, then fp16), as numpy's two casts do.
    n, k = 4, 1024
    w = _w("q4k", n, k, 21).reshape(n, k // 256, 144).copy()
    w[:, :, 0:2] = np.array([0x3C00], np.uint16).view(np.uint8)  # d = 1.0
    w[:, :, 2:4] = np.array([0x0401], np.uint16).view(np.uint8)  # dmin = 2^-14 (1 + 2^-10)
    w = w.reshape(n, -1)
    wd = oracle.dequant("q4k", w, n, k)
    assert (wd != wd.astype(np.float32).astype(np.float64)).mean() > 0.5
    h = oracle.get_rows("q4k", w, n, k, np.arange(n), "f16")
    assert np.array_equal(h, wd.astype(np.float32).astype(np.float16).view(np.uint16))
    b = oracle.get_rows("q4k", w, n, k, np.arange(n), "bf16")
    ref = torch.from_numpy(wd.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


# ---- dense GEMV -------------------------------------------------------------


@pytest.mark.parametrize("fmt,k", [("f16", 8), ("f16", 200), ("bf16", 64), ("bf16", 136)])
@pytest.mark.parametrize("n", [1, 4])
def test_dense_gemv_brute_force(fmt, k, n):
    w = synth.weights(fmt, n, k, 300 + n + k)
    x = synth.activations(fmt, k, 400 + n + k)
    y, a = oracle.gemv(fmt, w, x, n, k)
    wv = w.view(np.uint16).reshape(n, k)
    if fmt == "f16":
        wf = wv.view(np.float16).astype(np.float64)
        xf = x.view(np.float16).astype(np.float64)
    else:
        wf = torch.from_numpy(wv.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
        xf = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for r in range(n):
        terms = [Fraction(float(xf[i])) * Fraction(float(wf[r, i])) for i in range(k)]
        ye = sum(terms)
        ae = sum(abs(t) for t in terms)
        assert abs(Fraction(float(y[r])) - ye) <= Fraction(k, 2 ** 52) * ae
        assert abs(Fraction(float(a[r])) - ae) <= Fraction(k, 2 ** 52) * ae


def test_dense_activation_type_follows_format():
    # x of a dense fp16 GEMV is read as fp16, of a bf16 GEMV as bf16: one-hot
    # weights pick out x_i decoded in that type
    k = 32
    x = np.full(k, 0x4000, np.uint16)  # fp16 2.0; bf16 2.0 is 0x4000 as well
    x[5] = 0x3E00                      # fp16 1.5, bf16 0.125
    for fmt, want in (("f16", 1.5), ("bf16", 0.125)):
        w = np.zeros((1, k), np.uint16)
        w[0, 5] = 0x3C00 if fmt == "f16" else 0x3F80  # 1.0
        y, _ = oracle.gemv(fmt, w.view(np.uint8), x, 1, k)
        assert y[0] == want


# ---- epilogue -----------------------------------------------------------------


@pytest.mark.parametrize("c_dtype", ["f32", "f16", "bf16"])
def test_gemv_ex_exact(c_dtype):
    n, k = 3, 256
    w = synth.weights("q4k", n, k, 501)
    x = synth.activations("q4k", k, 502)
    c = synth.vector(n, c_dtype, 503)
    alpha, beta = -0.75, 1.5
    v, bound = oracle.gemv_ex("q4k", w, x, n, k, alpha, beta, c, c_dtype)
    wd = oracle.dequant("q4k", w, n, k)
    xv = [Fraction(oracle.f16(int(t))) for t in x]
    if c_dtype == "f32":
        cv = [Fraction(float(t)) for t in c]
    else:
        dec = oracle.f16 if c_dtype == "f16" else oracle.bf16
        cv = [Fraction(dec(int(t))) for t in c]
    for r in range(n):
        terms = [xv[i] * Fraction(float(wd[r, i])) for i in range(k)]
        exact = Fraction(alpha) * sum(terms) + Fraction(beta) * cv[r]
        b = abs(Fraction(alpha)) * sum(abs(t) for t in terms) + abs(Fraction(beta) * cv[r])
        assert abs(Fraction(float(v[r])) - exact) <= Fraction(k + 2, 2 ** 52) * b
        assert abs(Fraction(float(bound[r])) - b) <= Fraction(k + 2, 2 ** 52) * b


def test_gemv_ex_beta_zero_does_not_read_c():
    n, k = 4, 256
    w = synth.weights("tq1", n, k, 7)
    x = synth.activations("tq1", k, 8)
    y, a = oracle.gemv("tq1", w, x, n, k)
    c = np.full(n, np.nan, np.float32)
    v, bound = oracle.gemv_ex("tq1", w, x, n, k, 2.0, 0.0, c)
    assert np.array_equal(v, 2.0 * y) and np.array_equal(bound, 2.0 * a)
    v1, _ = oracle.gemv_ex("tq1", w, x, n, k, 1.0, 0.0, None)
    assert np.array_equal(v1, y)
