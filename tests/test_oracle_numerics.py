"""Pins of the 16-bit decoders: all 65 536 patterns against the format definitions."""

import math

import numpy as np
import pytest

from oracle.numerics import bf16_bits_to_f64, e8m0_bits_to_f64, f16_bits_to_f64, fp8_bits_to_f64
from tests import pins


def ieee_value(bits, exp_bits, man_bits):
    """Value of an IEEE-style binary pattern from sign, biased exponent and fraction."""
    sign = -1.0 if (bits >> (exp_bits + man_bits)) & 1 else 1.0
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    m = bits & ((1 << man_bits) - 1)
    bias = (1 << (exp_bits - 1)) - 1
    if e == (1 << exp_bits) - 1:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, 1 - bias - man_bits)
    return sign * math.ldexp((1 << man_bits) + m, e - bias - man_bits)


@pytest.mark.parametrize("fmt,fn,exp_bits,man_bits", [
    ("binary16", f16_bits_to_f64, 5, 10),
    ("bfloat16", bf16_bits_to_f64, 8, 7),
])
def test_decode_exhaustive(fmt, fn, exp_bits, man_bits):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = fn(bits)
    for p in range(1 << 16):
        want = ieee_value(p, exp_bits, man_bits)
        g = float(got[p])
        if math.isnan(want):
            assert math.isnan(g), (fmt, hex(p))
        else:
            assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), (fmt, hex(p), g, want)


def test_decode_spot_values():
    assert f16_bits_to_f64(np.array([0x3C00], np.uint16))[0] == 1.0
    assert f16_bits_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -24
    assert f16_bits_to_f64(np.array([0x7BFF], np.uint16))[0] == 65504.0
    assert bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert bf16_bits_to_f64(np.array([0xC040], np.uint16))[0] == -3.0
    assert bf16_bits_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -133


def test_fp8_decode_against_torch_and_extremes():
    pins.pin_fp8_decode(fp8_bits_to_f64)


def test_e8m0_decode_against_torch():
    import torch
    bits = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(bits).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = e8m0_bits_to_f64(bits)
    assert np.array_equal(got[:255], want[:255]) and np.isnan(got[255]) and np.isnan(want[255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_synth_fp8_encoder_round_trips_and_rounds_to_nearest_even():
    import synth
    for fmt in ("e4m3", "e5m2"):
        bits = np.arange(256, dtype=np.uint8)
        vals = fp8_bits_to_f64(bits, fmt)
        finite = np.isfinite(vals)
        enc = synth.fp8_bits(vals[finite].astype(np.float32), fmt)
        # every finite value encodes to its own pattern (-0 included)
        assert np.array_equal(enc, bits[finite])
        # midpoints of adjacent positive values round to the one with an even fraction
        pos = np.sort(np.unique(vals[finite & (vals >= 0)]))
        mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
        exact_mid = mid.astype(np.float64) == (pos[:-1] + pos[1:]) / 2
        got = fp8_bits_to_f64(synth.fp8_bits(mid[exact_mid], fmt), fmt)
        lo, hi = pos[:-1][exact_mid], pos[1:][exact_mid]
        lo_bits = synth.fp8_bits(lo.astype(np.float32), fmt)
        want = np.where(lo_bits % 2 == 0, lo, hi)
        assert np.array_equal(got, want), fmt
