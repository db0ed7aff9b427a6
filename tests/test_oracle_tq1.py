"""Pins of the TQ1_0 oracle against "metal: TQ1_0 kernel performance".

* The oracle's digit is floor(3 ((3^k b) mod 256) / 256).  The page states the
  digit through the floor pair floor(3^(k+1) b / 256) - 3 floor(3^k b / 256)
  (sections 1, 2 and "Not applicable"); both must agree on all 256 bytes.
* Section 1's zero-padded collapse: sum_k y_k t_k = sum_{k=1..5} g_k f_k with
  g_k = y_{k-1} - 3 y_k, y_5 = 0, f_k = floor(3^k b / 256); padding the fifth
  activation with zero gives the four-digit form (g_5 = 0, g_4 = y_3).
* Section "Not applicable": doing the floor pair in fp16 is wrong for 17 of the
  1280 digits, byte 79 digit 3 among them (tests/golden).
* Section 2's element order, restated as an index map: element 32 k + j is
  digit k of qs[j] (j < 32), element 160 + 16 k + i is digit k of qs[32 + i]
  (i < 16), and the last 16 elements come from the qh tail.  The order inside
  that tail is not on the page: elements 240 + 4k + m take digit k of qh[m]
  (parity unpinned for that order, a convention).
"""
import os
from fractions import Fraction

import numpy as np

import oracle
from dequant_gemv_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def floor_pair(b, k):
    return (3 ** (k + 1) * b) // 256 - 3 * ((3 ** k * b) // 256)


def test_digit_equals_floor_pair_all_bytes():
    for b in range(256):
        for k in range(5):
            assert oracle.tq1_digit(b, k) == floor_pair(b, k), (b, k)


def test_digits_are_base3_of_scaled_byte():
    # floor(3^k b/256) = floor(floor(243 b/256) / 3^(5-k)), so the five digits
    # are the base-3 digits (most significant first) of v = floor(243 b / 256).
    for b in range(256):
        v = (243 * b) // 256
        want = [(v // 3 ** (4 - k)) % 3 for k in range(5)]
        assert [oracle.tq1_digit(b, k) for k in range(5)] == want


def test_packed_digit_recurrence_all_byte_pairs():
    # The GEMV's digit arithmetic: both bytes of a pair in one 32-bit word,
    # L_0 = b, t = 3 L_k, digit_k << 8 = t & 0xFF00 per 16-bit half, L_{k+1} =
    # t & 0xFF; checked against the oracle's digit for every byte pair (no
    # carry may cross between the halves).
    b0 = np.repeat(np.arange(256, dtype=np.uint64), 256)
    b1 = np.tile(np.arange(256, dtype=np.uint64), 256)
    L = b0 | (b1 << np.uint64(16))
    want = np.array([[oracle.tq1_digit(b, k) for k in range(5)] for b in range(256)], dtype=np.uint64)
    for k in range(5):
        t = (L * np.uint64(3)) & np.uint64(0xFFFFFFFF)
        d = t & np.uint64(0xFF00FF00)
        assert np.array_equal(d & np.uint64(0xFFFF), want[b0.astype(np.int64), k] << np.uint64(8)), k
        assert np.array_equal(d >> np.uint64(16), want[b1.astype(np.int64), k] << np.uint64(8)), k
        L = t & np.uint64(0x00FF00FF)


def test_collapse_identity_all_bytes_exact():
    rng = np.random.default_rng(7)
    for b in range(256):
        y = [Fraction(int(v), 97) for v in rng.integers(-500, 500, 5)]
        t = [oracle.tq1_digit(b, k) for k in range(5)]
        f = [(3 ** k * b) // 256 for k in range(6)]  # f_0 .. f_5
        yy = y + [Fraction(0)]
        g = [None] + [yy[k - 1] - 3 * yy[k] for k in range(1, 6)]
        assert sum(y[k] * t[k] for k in range(5)) == sum(g[k] * f[k] for k in range(1, 6))
        # zero-padded fifth activation: the four-digit form
        y4 = y[:4] + [Fraction(0), Fraction(0)]
        g4 = [None] + [y4[k - 1] - 3 * y4[k] for k in range(1, 6)]
        assert g4[5] == 0 and g4[4] == y4[3]
        assert sum(y4[k] * t[k] for k in range(4)) == sum(g4[k] * f[k] for k in range(1, 6))


def _golden(name):
    out = {}
    with open(os.path.join(HERE, "golden", name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = int(v)
    return out


def test_fp16_floor_pair_negative_control():
    g = _golden("tq1_fp16_digit_errors.txt")

    def f16_floor(j, b):
        return np.floor(np.float16(np.float16(3 ** j) * np.float16(b)) / np.float16(256))

    wrong = []
    for b in range(256):
        for k in range(5):
            d16 = int(f16_floor(k + 1, b) - 3 * f16_floor(k, b))
            if d16 != oracle.tq1_digit(b, k):
                wrong.append((b, k, d16))
    assert 256 * 5 == g["total_pairs"]
    assert len(wrong) == g["wrong_pairs"]
    b, k = g["example_byte"], g["example_digit"]
    assert (b, k, g["example_fp16"]) in wrong
    assert oracle.tq1_digit(b, k) == g["example_exact"]


def test_generator_codes_round_trip():
    c5 = synth.tq1_codes(5)
    tuples = {tuple(oracle.tq1_digit(int(c), k) for k in range(5)) for c in c5}
    assert len(c5) == 243 and len(tuples) == 243
    c4 = synth.tq1_codes(4)
    assert len(c4) == 81
    for c in c4:
        assert oracle.tq1_digit(int(c), 4) == 0
    assert len({tuple(oracle.tq1_digit(int(c), k) for k in range(4)) for c in c4}) == 81
    non_codes = sorted(set(range(256)) - set(int(c) for c in c5))
    assert non_codes == [1, 20, 40, 60, 79, 99, 119, 138, 158, 178, 197, 217, 237]


def element_of(pos, k):
    """Element fed by digit k of payload byte pos, from section 2's il rule."""
    for il in range(15):
        for e in range(16):
            if il < 10:
                byte, dig = 16 * (il % 2) + e, il // 2
            else:
                byte, dig = 32 + e, il - 10
            if (byte, dig) == (pos, k):
                return 16 * il + e
    assert 48 <= pos < 52
    return None if k == 4 else 240 + 4 * k + (pos - 48)  # qh tail: a convention


def _one_hot_block(pos, k):
    # every trit 1 (weight 0) except digit k of byte pos, which is 2 (weight +d)
    blk = np.full(54, 0, np.uint8)
    ones5 = int(synth.tq1_codes(5)[121])  # digits 1,1,1,1,1
    ones4 = int(synth.tq1_codes(4)[40])  # digits 1,1,1,1,(0)
    blk[:48] = ones5
    blk[48:52] = ones4
    digits = [1, 1, 1, 1, 1 if pos < 48 else 0]
    digits[k] = 2
    v = sum(t * 3 ** (4 - j) for j, t in enumerate(digits))
    blk[pos] = (256 * v + 242) // 243
    blk[52:54] = [0x00, 0x3C]  # d = 1.0
    return blk


def test_element_map_one_hot():
    for pos in range(52):
        for k in range(5 if pos < 48 else 4):
            w = oracle.dequant("tq1", _one_hot_block(pos, k)[None], 1, 256)[0]
            assert list(np.flatnonzero(w)) == [element_of(pos, k)], (pos, k)
            assert w[element_of(pos, k)] == 1.0


def test_dequant_coverage_77824_elements():
    # 304 blocks; every byte value (codes and the 13 non-codes, 0 and 255
    # included) appears at every payload position; compared with the section-2
    # element rule and the floor-pair digits, elementwise and exactly.
    nblk = 304
    rng = np.random.default_rng(8)
    blk = np.empty((nblk, 54), np.uint8)
    for pos in range(52):
        blk[:, pos] = np.concatenate([np.arange(256), rng.integers(0, 256, nblk - 256)])[rng.permutation(nblk)]
    d = rng.uniform(-5e-2, 5e-2, nblk).astype(np.float16)
    blk[:, 52:54] = d.view(np.uint8).reshape(nblk, 2)
    got = oracle.dequant("tq1", blk.reshape(1, -1), 1, 256 * nblk).reshape(nblk, 256)
    want = np.zeros((nblk, 256))
    for pos in range(52):
        for k in range(5 if pos < 48 else 4):
            e = element_of(pos, k)
            t = np.array([floor_pair(int(b), k) for b in blk[:, pos]])
            want[:, e] = d.astype(np.float64) * (t - 1)
    assert got.size == 77824
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
