"""Pins of the oracle quantizer: exact-code vectors, closed forms, special cases and the
dequantization bound (|x - x_hat| <= scale/2 up to float32 rounding of the sub/mul)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant

BITS = [8, 4, 2]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("e", [0, 3, 7, 10])
def test_exact_code_vectors(bits, e):
    # x_i = c_i * 2^-e with min code 0 and max code Lq: the scale is exactly 2^-e and the
    # codes come back unchanged (all arithmetic exact)
    lq = 2 ** bits - 1
    rng = np.random.default_rng(bits * 100 + e)
    c = rng.integers(0, lq + 1, size=(6, 128))
    c[:, 0] = 0
    c[:, 1] = lq
    x = (c * 2.0 ** -e).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), c * 2.0 ** -e)      # exact in fp16
    codes, s, z = quant.quantize_rows(x, bits)
    assert np.all(s == np.float16(2.0 ** -e))
    assert np.all(z == 0)
    assert np.array_equal(codes, c)
    # an offset row: zero becomes the minimum, codes unchanged
    x2 = (c * 2.0 ** -e - 3.0).astype(np.float16)
    if np.array_equal(x2.astype(np.float64), c * 2.0 ** -e - 3.0):
        codes2, s2, z2 = quant.quantize_rows(x2, bits)
        assert np.all(z2 == np.float16(-3.0))
        assert np.array_equal(codes2, c)


def test_constant_row():
    x = np.full((3, 128), np.float16(0.7))
    for bits in BITS:
        codes, s, z = quant.quantize_rows(x, bits)
        assert np.all(codes == 0) and np.all(s == 0) and np.all(z == np.float16(0.7))
        xh = quant.dequantize_rows(codes, s, z)
        assert np.all(xh == np.float32(np.float16(0.7)))


def test_non_representable_scale_hand_worked():
    # row = {-1, +1, 0...}, 8 bits: s32 = fl32(2/255); fp16(2/255) = 2056 * 2^-18 = 257/32768
    # (2/255 * 2^18 = 2056.03 -> 2056); inv = fl32(32768/257) = 127.50194..; code(0) =
    # rint(127.50194) = 128; code(1) = rint(fl32(2*inv)) = 255; code(-1) = 0
    x = np.zeros((1, 128), np.float16)
    x[0, 0], x[0, 1] = -1, 1
    codes, s, z = quant.quantize_rows(x, 8)
    assert Fraction(float(s[0])) == Fraction(257, 32768)
    assert float(z[0]) == -1.0
    assert codes[0, 0] == 0 and codes[0, 1] == 255 and np.all(codes[0, 2:] == 128)


def test_subnormal_scale_floor():
    # range 2^-24 at 8 bits: s32 = 2^-24/255 rounds to fp16 zero, so the scale is set to
    # the smallest subnormal 2^-24; inv = 2^24; the top element gets code 1
    x = np.zeros((1, 128), np.float16)
    x[0, 5] = np.float16(2.0 ** -24)
    codes, s, z = quant.quantize_rows(x, 8)
    assert float(s[0]) == 2.0 ** -24 and float(z[0]) == 0.0
    assert codes[0, 5] == 1 and codes[0].sum() == 1


@pytest.mark.parametrize("bits", BITS)
def test_extremes_and_bound_random(bits):
    lq = 2 ** bits - 1
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((2000, 128)).astype(np.float16)
    x[:500] *= np.float16(8)
    codes, s, z = quant.quantize_rows(x, bits)
    assert codes.max() <= lq
    xf = x.astype(np.float32)
    amin, amax = xf.argmin(1), xf.argmax(1)
    r = np.arange(len(x))
    assert np.all(codes[r, amin] == 0)
    assert np.all(codes[r, amax] == lq)     # normal-range scales: fp16 rounding excess < 0.5
    xh = quant.dequantize_rows(codes, s, z)
    sf = s.astype(np.float64)[:, None]
    ulp = np.spacing(np.abs(xf)).astype(np.float64)
    err = np.abs(xf.astype(np.float64) - xh.astype(np.float64))
    assert np.all(err <= sf * (0.5 + 2.0 ** -12) + ulp)


def test_dequantize_is_a_single_rounding():
    # fl32(c*s + z) computed from exact rationals
    rng = np.random.default_rng(1)
    c = rng.integers(0, 256, size=(4, 128))
    s = rng.standard_normal(4).astype(np.float16) ** 2
    z = rng.standard_normal(4).astype(np.float16)
    got = quant.dequantize_rows(c.astype(np.uint8), s, z)
    for i in range(4):
        for j in range(0, 128, 17):
            exact = Fraction(int(c[i, j])) * Fraction(float(s[i])) + Fraction(float(z[i]))
            assert Fraction(float(got[i, j])) == Fraction(float(np.float32(float(exact))))


def test_requantize_demotion_is_quantize_of_fp16_reconstruction():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 128)).astype(np.float16)
    c8, s8, z8 = quant.quantize_rows(x, 8)
    c4, s4, z4 = quant.requantize_from(c8, s8, z8, 4)
    xh = quant.dequantize_rows(c8, s8, z8).astype(np.float16)
    e4 = quant.quantize_rows(xh, 4)
    assert np.array_equal(c4, e4[0]) and np.array_equal(s4, e4[1]) and np.array_equal(z4, e4[2])
    # the reconstruction keeps min and max exactly (codes 0 and 255 map back to z, z+255s)
    assert np.all(z4 == z8)


def test_demotion_hand_worked_vector():
    # keys on a grid of 1/16 with a zero point of -3: x_i = -3 + c_i / 16, c_i in 0..255 with
    # both ends present.  At 8 bits the range is 255/16, the scale exactly 1/16 and the codes
    # the c_i themselves, so the reconstruction is x itself.  Demoted to 4 bits: range
    # 15.9375, scale 15.9375 / 15 = 1.0625 (exact in fp16), zero -3, and code_i =
    # rint((c_i / 16) / 1.0625) = rint(c_i / 17), never a tie (c_i / 17 is at least 1/34 from
    # a half-integer)
    c = np.array(list(range(0, 256, 2)), np.int64)
    c[-1] = 255
    x = (np.float64(-3.0) + c / 16.0).astype(np.float16)[None]
    c8, s8, z8 = quant.quantize_rows(x, 8)
    assert float(s8[0]) == 1.0 / 16 and float(z8[0]) == -3.0
    assert np.array_equal(c8[0], c)
    c4, s4, z4 = quant.requantize_from(c8, s8, z8, 4)
    assert float(s4[0]) == 1.0625 and float(z4[0]) == -3.0
    # a few by hand: 8/17 = 0.47 -> 0, 10/17 = 0.59 -> 1, 24/17 = 1.41 -> 1, 26/17 = 1.53 -> 2,
    # 252/17 = 14.82 -> 15, 255/17 = 15 -> 15
    hand = {0: 0, 8: 0, 10: 1, 24: 1, 26: 2, 128: 8, 252: 15, 255: 15}
    for ci, want in hand.items():
        assert c4[0, list(c).index(ci)] == want, ci
    assert np.array_equal(c4[0], np.floor(c / 17.0 + 0.5).astype(np.int64))
    # values on a grid of 1/4, codes 0..15 (V4), demoted to 2 bits: range 3.75, scale 1.25
    # (exact), code = rint(c / 5): 0..2 -> 0, 3..7 -> 1, 8..12 -> 2, 13..15 -> 3
    cv = np.tile(np.arange(16), 8)
    xv = (cv / 4.0).astype(np.float16)[None]
    v4, sv4, zv4 = quant.quantize_rows(xv, 4)
    assert float(sv4[0]) == 0.25 and np.array_equal(v4[0], cv)
    v2, sv2, zv2 = quant.requantize_from(v4, sv4, zv4, 2)
    assert float(sv2[0]) == 1.25 and float(zv2[0]) == 0.0
    want = np.array([0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 2, 2, 2, 3, 3, 3])
    assert np.array_equal(v2[0], np.tile(want, 8))


def test_fp16_rounding_is_nearest_even():
    # numpy's float32 -> float16 conversion (used for scales) agrees with torch's on ties
    import torch
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # ties: exact midpoints between adjacent fp16 values
    h = rng.integers(0, 0x7BFF, size=5000).astype(np.uint16).view(np.float16)
    mids = ((h.astype(np.float64) + np.nextafter(h, np.float16(np.inf)).astype(np.float64)) / 2).astype(np.float32)
    allf = np.concatenate([f, mids])
    a = allf.astype(np.float16).view(np.uint16)
    b = torch.from_numpy(allf).to(torch.float16).numpy().view(np.uint16)
    assert np.array_equal(a, b)
    # a tie rounds to the even neighbour
    one = np.float32(1.0) + np.float32(2.0 ** -11)      # halfway between 1 and 1+2^-10
    assert np.float16(one) == np.float16(1.0)


def test_scale_on_an_fp16_tie_rounds_to_even():
    # row min -1.7587890625, max 34.4375 at 4 bits: the range 36.1962890625 is exact in float32
    # and range / 15 = 2.4130859375 exactly, the midpoint of the fp16 neighbours 2.412109375
    # (mantissa 211) and 2.4140625 (mantissa 212): the float32 quotient is the tie itself and
    # the fp16 rounding takes the even mantissa
    x = np.zeros((1, 128), np.float16)
    x[0, 0], x[0, 1] = -1.7587890625, 34.4375
    assert Fraction(float(x[0, 1])) - Fraction(float(x[0, 0])) == Fraction(36.1962890625)
    assert Fraction(36.1962890625) / 15 == (Fraction(2.412109375) + Fraction(2.4140625)) / 2
    codes, s, z = quant.quantize_rows(x, 4)
    assert float(s[0]) == 2.4140625 and float(z[0]) == -1.7587890625
    assert codes[0, 0] == 0 and codes[0, 1] == 15
