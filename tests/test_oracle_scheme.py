"""Pins of the precision-scheme oracle: hand-derived packed bytes, round trips, exact bit
coverage of a page's code region, the capacity rule, the quantizer at 1 and 2 bits, and the
K8V4-K4V2 scheme's reconstructions equal to the ones of the default layout's oracle."""
import numpy as np
import pytest

from oracle import place, quant, scheme as osch


def test_hand_packed_bytes():
    c = np.zeros(128, np.uint8)
    c[:4] = [1, 2, 3, 0]
    # 2 bits: byte 0 = 1 | 2 << 2 | 3 << 4 | 0 << 6
    assert osch.pack_codes(c, 2)[0] == 0b00111001
    # 4 bits: low nibble first
    assert osch.pack_codes(c, 4)[0] == 0x21 and osch.pack_codes(c, 4)[1] == 0x03
    # 1 bit: code i at bit i
    b = np.zeros(128, np.uint8)
    b[[0, 3, 8, 127]] = 1
    p = osch.pack_codes(b, 1)
    assert p[0] == 0b1001 and p[1] == 1 and p[15] == 0x80 and p.sum() == 0b1001 + 1 + 0x80
    # 8 bits: bytes as they are
    e = np.arange(128, dtype=np.uint8)
    assert np.array_equal(osch.pack_codes(e, 8), e)


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_round_trip(b):
    rng = np.random.default_rng(b)
    c = rng.integers(0, 2 ** b, size=(5, 128)).astype(np.uint8)
    assert np.array_equal(osch.unpack_codes(osch.pack_codes(c, b), b), c)


@pytest.mark.parametrize("high,low", [("K8V4", "K4V2"), ("K4V8", "K2V4"), ("K8V2", "K4V1"),
                                      ("K4V2", "K4V2"), ("K2V4", "K4V1")])
def test_page_bit_coverage(high, low):
    # all-ones codes light exactly slots * 16 (kb + vb) bytes; nothing else in the code region
    sc = osch.Scheme.named(high, low)
    for tier in (osch.HIGH, osch.LOW):
        kb, vb = sc.bits[tier]
        S = osch.SLOTS[tier]
        ones_k = np.full((S, 128), 2 ** kb - 1, np.uint8)
        ones_v = np.full((S, 128), 2 ** vb - 1, np.uint8)
        z = np.zeros(S, np.float16)
        page = osch.build_page(sc, tier, ones_k, ones_v, z, z, z, z, np.arange(S))
        n = S * 16 * (kb + vb)
        assert np.all(page[:n] == 0xFF) and np.all(page[n:osch.CODE_BYTES] == 0)
        k, v, *_, pos = osch.read_page(page, sc, tier, S)
        assert np.array_equal(k, ones_k) and np.array_equal(v, ones_v)
        assert np.array_equal(pos, np.arange(S))


def test_hand_placed_fields():
    # K4V2 in a LOW page (32 slots): slot 1's key code 3 sits at byte 64 (16 * 4 * 1), low
    # nibble.  Its value code for channel 5 (block 0, g = 0, r = 1, n = 0, c = 5: lane 5's
    # 8 bytes from 2048 + 40, bit 16 (r odd) + 0) is at byte 2048 + 42, bits 0..1
    sc = osch.Scheme.named("K8V4", "K4V2")
    k = np.zeros((2, 128), np.uint8)
    v = np.zeros((2, 128), np.uint8)
    k[1, 0] = 3
    v[1, 5] = 2
    z = np.zeros(2, np.float16)
    page = osch.build_page(sc, osch.LOW, k, v, z, z, z, z, [7, 9])
    assert page[64] == 3 and page[2048 + 42] == 2
    assert np.count_nonzero(page[:osch.CODE_BYTES]) == 2
    # K8V4 in a HIGH page: slot 15 = g 3, r 3; channel 0 = n 0, c 0: lane 48's 16 bytes from
    # 2048 + 768; r = 3 puts the code at bit 16 + 4 = 20: byte 770, high nibble
    k2 = np.zeros((16, 128), np.uint8)
    v2 = np.zeros((16, 128), np.uint8)
    v2[15, 0] = 0xF
    z2 = np.zeros(16, np.float16)
    page = osch.build_page(sc, osch.HIGH, k2, v2, z2, z2, z2, z2, np.arange(16))
    assert page[2048 + 770] == 0xF0 and np.count_nonzero(page[:osch.CODE_BYTES]) == 1
    # K4V8 in a HIGH page: an 8-bit code sits in one byte; slot 6 = g 1, r 2 of channel 37
    # (n 2, c 5): lane 21's 32 bytes from 16 * 4 * 16 + 32 * 21 = 1696, word 2, bit 8: byte 1705
    sc8 = osch.Scheme.named("K4V8", "K2V4")
    v3 = np.zeros((16, 128), np.uint8)
    v3[6, 37] = 0xA5
    page = osch.build_page(sc8, osch.HIGH, k2, v3, z2, z2, z2, z2, np.arange(16))
    assert page[1705] == 0xA5 and np.count_nonzero(page[:osch.CODE_BYTES]) == 1


def test_value_bits_are_a_bijection():
    # every (slot, channel) code of every width lands on its own vb bits inside the region
    for vb in (1, 2, 4, 8):
        for S in (16, 32):
            if 16 * vb * S > osch.CODE_BYTES:
                continue
            starts = sorted(osch.value_bit(vb, s, d) for s in range(S) for d in range(128))
            assert starts == list(range(0, 16 * vb * S * 8, vb))


def test_capacity_rule():
    assert osch.fits(osch.HIGH, 8, 4) and osch.fits(osch.HIGH, 4, 8)
    assert not osch.fits(osch.HIGH, 8, 8)          # 16 * 16 * 16 = 4096 > 3072
    assert osch.fits(osch.LOW, 4, 2) and osch.fits(osch.LOW, 2, 4) and osch.fits(osch.LOW, 4, 1)
    assert not osch.fits(osch.LOW, 4, 4) and not osch.fits(osch.LOW, 8, 2)
    assert not osch.fits(osch.HIGH, 3, 4)
    with pytest.raises(ValueError):
        osch.Scheme(8, 8, 4, 2)


@pytest.mark.parametrize("b", [1, 2])
def test_low_bit_quantizer(b):
    # codes stay in 0 .. 2^b - 1, the row's min and max map to 0 and 2^b - 1, and the
    # reconstruction is within half a step (plus rounding) of the input
    rng = np.random.default_rng(10 + b)
    x = rng.standard_normal((6, 128)).astype(np.float16)
    c, s, z = quant.quantize_rows(x, b)
    assert c.max() <= 2 ** b - 1
    for r in range(6):
        assert c[r, np.argmin(x[r])] == 0 and c[r, np.argmax(x[r])] == 2 ** b - 1
    xh = quant.dequantize_rows(c, s, z)
    step = s.astype(np.float64)[:, None]
    xf = x.astype(np.float32)
    ulp = np.spacing(np.abs(xf)).astype(np.float64)     # the float32 rounding of c*s + z
    err = np.abs(xh.astype(np.float64) - xf.astype(np.float64))
    assert np.all(err <= step * (0.5 + 2 ** -12) + ulp)


def test_default_scheme_matches_default_layout_reconstruction():
    # under K8V4-K4V2 the reconstructions are the default path's (only the byte layout differs)
    rng = np.random.default_rng(7)
    k = rng.standard_normal((90, 128)).astype(np.float16)
    v = rng.standard_normal((90, 128)).astype(np.float16)
    tier = rng.choice([0, 1, 2], size=90).astype(np.uint8)
    sc = osch.Scheme.named("K8V4", "K4V2")
    a = osch.head_dequantized(k, v, tier, sc)
    b = place.head_dequantized(k, v, tier)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
