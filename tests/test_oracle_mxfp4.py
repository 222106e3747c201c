"""Pins of the oracle's MXFP4 encoding.

The e2m1 values come from the bit layout (sign, 2-bit exponent with bias 1,
1-bit mantissa, exponent 0 subnormal: OCP MX v1.0, section 5.3); ties and
saturation are checked against a brute-force nearest search written here;
dequantization against ldexp over every scale byte and code.
"""

import math

import numpy as np
import pytest

from oracle import mxfp4

# Tie and saturation cases worked by hand from the OCP MX v1.0 conversion rule
# (round to nearest, ties to the even mantissa, saturate at the largest normal;
# the sign is kept, so small negatives give -0): (value, expected code).
TIES = [
    (0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6),
    (5.0, 0x6), (7.0, 0x7), (1e30, 0x7), (0.0, 0x0), (-0.0, 0x8), (-0.25, 0x8),
    (-0.75, 0xA), (-5.0, 0xE), (-6.5, 0xF), (0.2499, 0x0), (0.2501, 0x1),
    (5.0001, 0x7), (4.9999, 0x6),
]


def bit_formula(code):
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * 0.5 * m
    return s * 2.0 ** (e - 1) * (1 + 0.5 * m)


def test_e2m1_table_from_bits():
    for code in range(16):
        assert mxfp4.e2m1_value(code) == bit_formula(code)


def brute_round(v):
    """Nearest e2m1 magnitude; ties to even code; above 6 -> 6."""
    m = abs(v)
    best, bestd = None, None
    for code in range(8):
        d = abs(m - bit_formula(code))
        if best is None or d < bestd or (d == bestd and code % 2 == 0):
            best, bestd = code, d
    sign = 8 if math.copysign(1.0, v) < 0 else 0
    return sign | best


def test_ties_fixture():
    for value, code in TIES:
        assert int(mxfp4.round_e2m1(np.array([value]))[0]) == code, (value, code)


def test_rounding_brute_force():
    g = np.random.default_rng(1)
    v = np.concatenate([g.uniform(-8, 8, 4000),
                        np.arange(-32, 33) * 0.25,        # every quarter: all ties
                        [0.0, -0.0, 1e-300, -1e-300, 6.0, -6.0, 7.999, -100.0]])
    got = mxfp4.round_e2m1(v)
    for x, q in zip(v, got):
        assert int(q) == brute_round(float(x)), x


def test_shared_exponent():
    assert mxfp4.shared_exponent(0.0) == 0
    for j in range(-120, 120, 7):
        for m in (1.0, 1.5, 1.999):
            amax = np.float32(m * 2.0 ** j)
            assert mxfp4.shared_exponent(amax) == j - 2 + 127
    assert mxfp4.shared_exponent(np.float32(2.0 ** -126)) == 0       # -128 + 127 clamps at 0
    assert mxfp4.shared_exponent(np.float32(1e-45)) == 0
    assert mxfp4.shared_exponent(np.finfo(np.float32).max) == 127 + 125


def test_dequant_every_scale_and_code():
    codes = np.arange(16, dtype=np.uint8)
    byte_row = mxfp4.pack(np.tile(codes, 2))                 # 32 codes -> 16 bytes
    packed = np.tile(byte_row, (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    got = mxfp4.dequantize(packed, scales, 32)
    for s in range(256):
        for c in range(16):
            x = got[s, c]
            if s == 255:
                assert np.isnan(x)
                continue
            with np.errstate(over="ignore"):
                ref = np.float32(math.ldexp(bit_formula(c), s - 127)) if not (
                    abs(bit_formula(c)) * 2.0 ** (s - 127) > np.finfo(np.float32).max) else np.float32(
                    math.copysign(math.inf, bit_formula(c)))
            assert x.view(np.uint32) == ref.view(np.uint32) or (x == ref), (s, c, x, ref)
    # s = 0 scales to the float32 subnormal 2^-128 for code 1 (0.5)
    assert got[0, 1] == np.float32(2.0 ** -128)
    # negative zero is kept
    assert math.copysign(1.0, float(got[127, 8])) == -1.0


def test_nibble_order():
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, 0] = 6.0            # amax 6: e = 2 - 2 = 0, s = 127, code 7
    blk[0, 1] = -1.0           # code 0xA
    packed, s = mxfp4.quantize(blk)
    assert s[0, 0] == 127
    assert packed[0, 0] == 0xA7   # element 0 in the LOW nibble


def test_round_trip():
    g = np.random.default_rng(2)
    w = (g.standard_normal((8, 256)) * 0.02).astype(np.float32)
    p, s = mxfp4.quantize(w)
    w2 = mxfp4.dequantize(p, s, 256)
    p2, s2 = mxfp4.quantize(w2)
    assert np.array_equal(p, p2) and np.array_equal(s, s2)


def test_saturation_fraction():
    # values scaled into (6, 8) saturate; a small share of N(0, s) values do
    g = np.random.default_rng(4)
    w = (g.standard_normal((256, 1024)) * 0.02).astype(np.float32)
    p, s = mxfp4.quantize(w)
    blocks = w.reshape(-1, 32).astype(np.float64)
    scaled = np.abs(blocks) / np.ldexp(1.0, s.reshape(-1).astype(np.int64) - 127)[:, None]
    frac = float(np.mean(scaled > 6.0))
    assert 0.005 < frac < 0.04
    q = mxfp4.unpack(p).reshape(-1, 32)
    assert np.all((q[scaled > 6.0] & 7) == 7)


@pytest.mark.parametrize("bad", [np.inf, np.nan])
def test_rejects_non_finite(bad):
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 3] = bad
    with pytest.raises(ValueError):
        mxfp4.quantize(w)
