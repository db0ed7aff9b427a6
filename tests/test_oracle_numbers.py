"""Pins of the oracle's scalar decoders against library routines and closed forms."""
import math

import numpy as np
import pytest
import torch

import oracle


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


def test_f16_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    for c in range(0, 65536, 1):
        assert _same(oracle.f16(c), float(ref[c])), hex(c)


def test_bf16_all_codes_match_torch():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    ref = codes.to(torch.float64).numpy()
    for c in range(65536):
        assert _same(oracle.bf16(c), float(ref[c])), hex(c)


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    # The OCP E4M3 "fn" flavour: bias 7, subnormals, NaN only at S.1111.111.
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e4m3(c), float(ref[c])), hex(c)


def test_e4m3_closed_form_landmarks():
    assert oracle.e4m3(0x38) == 1.0            # exponent field 7 = bias
    assert oracle.e4m3(0x7E) == 448.0          # largest finite
    assert oracle.e4m3(0x01) == 2.0 ** -9      # smallest subnormal
    assert oracle.e4m3(0x08) == 2.0 ** -6      # smallest normal
    nans = [c for c in range(256) if math.isnan(oracle.e4m3(c))]
    assert nans == [0x7F, 0xFF]
    assert all(math.isfinite(oracle.e4m3(c)) for c in range(256) if c not in nans)


# E2M1 element values of the OCP Microscaling (MX) formats specification:
# magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, sign in bit 3.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    vals = [oracle.e2m1(n) for n in range(16)]
    assert vals[:8] == E2M1_MAGNITUDES
    for n in range(8):
        assert vals[8 + n] == -vals[n]
    assert math.copysign(1.0, vals[8]) == -1.0  # code 8 is -0
    # Mojo fp4_gemv page: every E2M1 value is exact in fp16, +-0.5 included.
    for v in vals:
        assert float(np.float16(v)) == v
    assert 0.5 in vals and -0.5 in vals


def test_e2m1_times_e4m3_exact_in_fp32():
    # Basis of the bit-exact dequantisation claim (Mojo fp4_gemv page): every
    # e2m1 * |e4m3| product is representable in fp32.
    for n in range(16):
        for c in range(256):
            s = oracle.e4m3(c)
            if math.isnan(s):
                continue
            p = oracle.e2m1(n) * abs(s)
            assert float(np.float32(p)) == p
