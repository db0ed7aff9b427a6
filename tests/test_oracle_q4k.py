"""Pins of the Q4_K oracle against "Writing a high performant GEMV + dequant for
Metal".

The oracle indexes bytes and nibbles directly.  The checks here read the same
144-byte block the way the page's kernel addresses it instead, through 16-bit
little-endian words and masks:

* section "Kernel code": the first half-word of the block is d, the second dmin
  (d multiplies the scale terms, dmin the min terms); the 12 scale bytes start
  at byte 4 and the 128 nibble bytes at byte 16;
* the scale words are masked with 0x3f3f, 0x0f0f and 0xc0c0, the top two bits
  of the first eight bytes becoming bits 4-5 of the scales and mins of groups
  4..7;
* the nibble word at byte 16 + 2u holds, in bits 0-3 / 8-11 / 4-7 / 12-15, the
  quants of elements e, e+1, e+32, e+33 with e = 64 (u div 16) + 2 (u mod 16),
  which is where that kernel fetches the matching activations from;
* section "Compute": the block dot product factors as
  d * sum_g s_g Q_g - dmin * sum_g m_g X_g.
"""
from fractions import Fraction

import numpy as np

import oracle
from dequant_gemv_amd import synth


def _words(b, lo, n):
    """n little-endian 16-bit words starting at byte offset lo of each block."""
    return b[..., lo:lo + 2 * n].astype(np.uint32).reshape(b.shape[:-1] + (n, 2)) @ np.array([1, 256], np.uint32)


def word_decode(blocks):
    """(d, dmin, s[8], m[8], q[256]) of Q4_K blocks, read through 16-bit words."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    hw = _words(blocks, 0, 2).astype(np.uint16)
    d = hw[..., 0].view(np.float16).astype(np.float64)
    dmin = hw[..., 1].view(np.float16).astype(np.float64)
    sw = _words(blocks, 4, 6)  # six scale words
    s = np.zeros(blocks.shape[:-1] + (8,), np.int64)
    m = np.zeros_like(s)
    for iq in range(2):  # each word pair covers two consecutive groups
        lo_s = sw[..., iq] & 0x3F3F
        lo_m = sw[..., iq + 2] & 0x3F3F
        hi_s = (sw[..., iq + 4] & 0x0F0F) | ((sw[..., iq] & 0xC0C0) >> 2)
        hi_m = ((sw[..., iq + 4] >> 4) & 0x0F0F) | ((sw[..., iq + 2] & 0xC0C0) >> 2)
        for half in range(2):
            g = 2 * iq + half
            s[..., g] = (lo_s >> (8 * half)) & 0xFF
            m[..., g] = (lo_m >> (8 * half)) & 0xFF
            s[..., 4 + g] = (hi_s >> (8 * half)) & 0xFF
            m[..., 4 + g] = (hi_m >> (8 * half)) & 0xFF
    qw = _words(blocks, 16, 64)
    q = np.zeros(blocks.shape[:-1] + (256,), np.int64)
    u = np.arange(64)
    e = 64 * (u // 16) + 2 * (u % 16)
    q[..., e] = qw & 0x000F
    q[..., e + 1] = (qw & 0x0F00) >> 8
    q[..., e + 32] = (qw & 0x00F0) >> 4
    q[..., e + 33] = (qw & 0xF000) >> 12
    return d, dmin, s, m, q


def _blocks(nblk, seed):
    return synth.q4k_weights(1, 256 * nblk, seed).reshape(nblk, 144)


def test_dequant_equals_word_reading():
    # w_i = d s_g q_i - dmin m_g (section "Compute") with every field read the
    # kernel's way; both sides are exact in fp64.
    blk = _blocks(64, 11)
    d, dmin, s, m, q = word_decode(blk)
    g = np.arange(256) // 32
    ref = d[:, None] * s[:, g] * q - dmin[:, None] * m[:, g]
    got = oracle.dequant("q4k", blk.reshape(1, -1), 1, 256 * 64).reshape(64, 256)
    assert np.array_equal(got, ref)


def test_gemv_equals_factored_form_exactly():
    # Section "Compute": y_block = d sum_g s_g Q_g - dmin sum_g m_g X_g with
    # Q_g = sum x_i q_i and X_g = sum x_i over group g.  Compared exactly in
    # rationals against the oracle's plain sum of x_i * w_i.
    nblk = 6
    blk = _blocks(nblk, 12)
    x = synth.x_f16(256 * nblk, 13)
    xv = [Fraction(float(v)) for v in x.view(np.float16).astype(np.float64)]
    d, dmin, s, m, q = word_decode(blk)
    fact = Fraction(0)
    for b in range(nblk):
        sq = Fraction(0)
        mx = Fraction(0)
        for gi in range(8):
            Q = sum(xv[256 * b + i] * int(q[b, i]) for i in range(32 * gi, 32 * gi + 32))
            X = sum(xv[256 * b + i] for i in range(32 * gi, 32 * gi + 32))
            sq += int(s[b, gi]) * Q
            mx += int(m[b, gi]) * X
        fact += Fraction(float(d[b])) * sq - Fraction(float(dmin[b])) * mx
    w = oracle.dequant("q4k", blk.reshape(1, -1), 1, 256 * nblk)[0]
    plain = sum(xv[i] * Fraction(float(w[i])) for i in range(256 * nblk))
    assert plain == fact
    y, a = oracle.gemv("q4k", blk.reshape(1, -1), x, 1, 256 * nblk)
    assert abs(Fraction(float(y[0])) - fact) <= Fraction(2.0 ** -50) * Fraction(float(a[0]))


def _block(d=0x3C00, dmin=0x3C00, scales=None, qs=None):
    b = np.zeros(144, np.uint8)
    b[0:2] = [d & 0xFF, d >> 8]
    b[2:4] = [dmin & 0xFF, dmin >> 8]
    if scales is not None:
        b[4:16] = scales
    if qs is not None:
        b[16:] = qs
    return b


def test_zero_scales_give_zero_weights():
    rng = np.random.default_rng(5)
    b = _block(qs=rng.integers(0, 256, 128))
    assert np.all(oracle.dequant("q4k", b[None], 1, 256) == 0.0)


def test_d_zero_leaves_minus_dmin_m():
    rng = np.random.default_rng(6)
    b = _block(d=0x0000, dmin=0x3C00, scales=rng.integers(0, 256, 12), qs=rng.integers(0, 256, 128))
    w = oracle.dequant("q4k", b[None], 1, 256)[0]
    _, _, _, m, _ = word_decode(b[None])
    assert np.array_equal(w, -np.repeat(m[0], 32).astype(np.float64))


def test_scale_min_bits_form_a_bijection():
    # The 12 scale bytes hold 16 six-bit values (8 scales, 8 mins): every one of
    # the 96 bits lands in exactly one bit of one value.  Read the values back
    # from the oracle with d = 1, dmin = 0, all quants 1 (w = s_g) and with
    # d = 0, dmin = -1 (w = m_g).
    seen = set()
    for byte in range(12):
        for bit in range(8):
            sc = np.zeros(12, np.uint8)
            sc[byte] = 1 << bit
            ws = oracle.dequant("q4k", _block(0x3C00, 0x0000, sc, np.full(128, 0x11))[None], 1, 256)[0]
            wm = oracle.dequant("q4k", _block(0x0000, 0xBC00, sc, np.zeros(128))[None], 1, 256)[0]
            vals = [("s", g, int(ws[32 * g])) for g in range(8)] + [("m", g, int(wm[32 * g])) for g in range(8)]
            hit = [(k, g, v) for k, g, v in vals if v != 0]
            assert len(hit) == 1, (byte, bit, hit)
            k, g, v = hit[0]
            assert v & (v - 1) == 0 and v < 64
            seen.add((k, g, v.bit_length() - 1))
    assert len(seen) == 96


def test_single_nibble_lands_on_the_word_reading_element():
    # One non-zero quant at a time: the weight appears at exactly the element
    # the word-level addressing assigns it.
    sc = np.full(12, 0x01, np.uint8)  # s_g = m_g = 1 for g < 4, s = m = 17 for g >= 4
    for byte in range(128):
        for shift in (0, 4):
            qs = np.zeros(128, np.uint8)
            qs[byte] = 1 << shift
            b = _block(0x3C00, 0x0000, sc, qs)
            w = oracle.dequant("q4k", b[None], 1, 256)[0]
            nz = np.flatnonzero(w)
            _, _, _, _, q = word_decode(b[None])
            assert list(nz) == list(np.flatnonzero(q[0])), (byte, shift)
            assert len(nz) == 1


def test_power_of_two_scaling_of_d_and_dmin():
    # Doubling d and dmin (fp16 exponent + 1) doubles every weight and y exactly.
    w = synth.q4k_weights(3, 512, 21)
    x = synth.x_f16(512, 22)
    w2 = w.copy().reshape(3, 2, 144)
    for lo in (0, 2):
        h = w2[:, :, lo].astype(np.uint16) | (w2[:, :, lo + 1].astype(np.uint16) << 8)
        h = h + (1 << 10)  # values are normal fp16 well below the top binade
        w2[:, :, lo] = h & 0xFF
        w2[:, :, lo + 1] = h >> 8
    y1, _ = oracle.gemv("q4k", w, x, 3, 512)
    y2, _ = oracle.gemv("q4k", w2.reshape(3, -1), x, 3, 512)
    assert np.array_equal(2 * y1, y2)
