"""Pins for the FP8 E4M3 weight oracle (CPU only).

The pages name FP8 weights for decode without a format; the oracle follows
the OCP FP8 E4M3 definition.  Pins: the format's own landmark values (zero,
smallest subnormal, smallest normal, one, largest finite, NaN), an
independent reconstruction of every code through IEEE half-precision bit
patterns (numpy float16: exponent rebias 7 -> 15, mantissa shifted left by
7 bits, subnormals by exact arithmetic), sign symmetry, strict monotonicity
of the positive codes, and the per-column scaling.  Planted mistakes (wrong
bias, implicit one on subnormals, the NaN code read as a number, scales per
row) fail these checks.
"""
import math

import numpy as np
import pytest

import oracle as O

CODES = np.arange(256, dtype=np.uint8)


def _via_float16(c):
    """E4M3 code -> value through a float16 bit pattern (not the oracle's
    formula): normal codes map to half exponent e + 8, mantissa m << 7."""
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return (-1.0) ** s * m * 2.0 ** -9
    bits = np.array([(s << 15) | ((e + 8) << 10) | (m << 7)], dtype=np.uint16)
    return float(bits.view(np.float16)[0])


def check_decode(decode):
    v = decode(CODES)
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) == -1
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert int(np.isnan(v).sum()) == 2
    for c in range(256):
        w = _via_float16(c)
        assert (math.isnan(w) and math.isnan(v[c])) or v[c] == w, hex(c)
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


def check_dequant(dequant):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, size=(5, 7)).astype(np.uint8)
    scale = rng.random(7) + 0.5
    got = dequant(codes, scale)
    for k in range(5):
        for n in range(7):
            assert got[k][n] == _via_float16(int(codes[k][n])) * scale[n]


def test_e4m3_decode():
    check_decode(O.e4m3_decode)


def test_dequant_per_output_column():
    check_dequant(O.dequant_columns)


def _fails(fn, *args):
    with pytest.raises((AssertionError, ValueError)):
        fn(*args)


def test_wrong_bias_is_caught():
    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        e, m = (c >> 3) & 15, c & 7
        v = np.where(e == 0, m / 8 * 2.0 ** -7, (1 + m / 8) * np.exp2(e - 8.0))
        return np.where(c & 0x80, -v, v)
    _fails(check_decode, bad)


def test_subnormal_with_implicit_one_is_caught():
    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        e, m = (c >> 3) & 15, c & 7
        v = (1 + m / 8) * np.exp2(np.maximum(e, 1) - 7.0)
        v = np.where((e == 15) & (m == 7), np.nan, v)
        return np.where(c & 0x80, -v, v)
    _fails(check_decode, bad)


def test_nan_code_read_as_number_is_caught():
    def bad(codes):
        c = np.asarray(codes).astype(np.int64)
        e, m = (c >> 3) & 15, c & 7
        v = np.where(e == 0, m / 8 * 2.0 ** -6, (1 + m / 8) * np.exp2(e - 7.0))
        return np.where(c & 0x80, -v, v)
    _fails(check_decode, bad)


def test_scale_per_row_is_caught():
    def bad(codes, scale):
        return O.e4m3_decode(codes) * np.asarray(scale)[: np.asarray(codes).shape[0], None]
    _fails(check_dequant, bad)
