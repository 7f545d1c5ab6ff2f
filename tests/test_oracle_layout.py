"""Pins of the unified page format: hand-derived bytes, bit coverage and round trips."""
import numpy as np
import pytest

from oracle import layout


def test_field_coverage_is_exact():
    # every code bit of the 3072-byte code area is used by exactly one (slot, channel)
    for tier, kb, vb in ((2, 8, 4), (1, 4, 2)):
        used = np.zeros(3072 * 8, np.int64)
        (kbyte, kshift), (vbyte, vshift) = layout._MAPS[tier]
        for byte, shift, nb in ((kbyte, kshift, kb), (vbyte, vshift, vb)):
            for bit in range(nb):
                np.add.at(used, (byte * 8 + shift + bit).ravel(), 1)
        assert np.all(used == 1)


def test_k4_word_hand_derived():
    # channels 0..7 with codes 0..7: channel e sits in nibble (e&1) + 2(e>>2) + 4((e>>1)&1),
    # so nibbles 0..7 hold codes 0,1,4,5,2,3,6,7 -> word 0x76325410 -> bytes 10 54 32 76
    k = np.zeros((1, 128), np.uint8)
    k[0, :8] = np.arange(8)
    page = layout.build_page(1, k, np.zeros((1, 128), np.uint8), [0], [0], [0], [0], [9])
    assert page[:4].tolist() == [0x10, 0x54, 0x32, 0x76]
    assert np.all(page[4:64] == 0)


def test_k8_rows_hand_derived():
    k = np.arange(2 * 128).reshape(2, 128).astype(np.uint8)
    page = layout.build_page(2, k, np.zeros((2, 128), np.uint8), [0, 0], [0, 0], [0, 0], [0, 0], [0, 1])
    assert np.array_equal(page[:128], k[0]) and np.array_equal(page[128:256], k[1])


def test_v4_unit_hand_derived():
    # HIGH value unit (j=0, l=0) holds slots 0..3 of channels 0,16,...,112.  Give slot r of
    # channel 16n the code (n + 4r) % 16 ... only for n in {0,1}: word 0 nibbles are
    # (n=0,r=0)->0, (0,1)->4, (0,2)->1, (0,3)->5, (1,0)->2, (1,1)->6, (1,2)->3, (1,3)->7
    v = np.zeros((4, 128), np.uint8)
    vals = {(0, 0): 1, (0, 1): 2, (0, 2): 3, (0, 3): 4, (1, 0): 5, (1, 1): 6, (1, 2): 7, (1, 3): 8}
    for (n, r), c in vals.items():
        v[r, 16 * n] = c
    page = layout.build_page(2, np.zeros((4, 128), np.uint8), v, [0] * 4, [0] * 4, [0] * 4, [0] * 4, range(4))
    # nibble index -> code: 0:1, 1:3, 2:5, 3:7, 4:2, 5:4, 6:6, 7:8 -> word 0x86427531
    word = int.from_bytes(bytes(page[2048:2052]), "little")
    assert word == 0x86427531
    assert np.all(page[2052:3072] == 0)


def test_v2_unit_hand_derived():
    # LOW value unit (j=0, l=0), word 0 = half f=0, channels n=0..3: field 2n + (r>>1) + 8(r&1)
    v = np.zeros((32, 128), np.uint8)
    v[0, 0] = 1      # n=0 r=0 -> field 0
    v[1, 0] = 2      # n=0 r=1 -> field 8
    v[2, 16] = 3     # n=1 r=2 -> field 3
    v[16, 32] = 1    # half 1, n=2, r=0 -> word 2, field 4
    page = layout.build_page(1, np.zeros((32, 128), np.uint8), v, [0] * 32, [0] * 32, [0] * 32,
                             [0] * 32, range(32))
    w0 = int.from_bytes(bytes(page[2048:2052]), "little")
    w2 = int.from_bytes(bytes(page[2056:2060]), "little")
    assert w0 == (1 << 0) | (2 << 16) | (3 << 6)
    assert w2 == (1 << 8)


@pytest.mark.parametrize("tier", [1, 2])
@pytest.mark.parametrize("m", [1, 7, 16, 32])
def test_round_trip_and_dead_slots(tier, m):
    per = layout.SLOTS[tier]
    if m > per:
        pytest.skip("more tokens than slots")
    rng = np.random.default_rng(tier * 100 + m)
    kb, vb = (8, 4) if tier == 2 else (4, 2)
    k = rng.integers(0, 2 ** kb, size=(m, 128)).astype(np.uint8)
    v = rng.integers(0, 2 ** vb, size=(m, 128)).astype(np.uint8)
    ks, kz, vs, vz = (rng.standard_normal(m).astype(np.float16) for _ in range(4))
    pos = rng.integers(0, 10 ** 6, size=m)
    page = layout.build_page(tier, k, v, ks, kz, vs, vz, pos)
    k2, v2, ks2, kz2, vs2, vz2, pos2 = layout.read_page(page, tier, m)
    assert np.array_equal(k, k2) and np.array_equal(v, v2)
    for a, b in ((ks, ks2), (kz, kz2), (vs, vs2), (vz, vz2)):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(pos, pos2)
    # dead slots: zero codes and parameters, position -1
    kd, vd, *prm, posd = layout.read_page(page, tier, per)
    assert np.all(kd[m:] == 0) and np.all(vd[m:] == 0)
    for p in prm:
        assert np.all(p[m:] == 0)
    assert np.all(posd[m:] == -1)
    assert np.all(page[3072 + 8 * per:3328] == 0)


def test_bytes_per_token_and_memory_fraction():
    # Referee report, 'Significance': with K8V4/K4V2 a 27.4% memory fraction means about
    # 46% high-precision and 54% low-precision tokens.  Code bytes per token: HIGH
    # 128 + 64 = 192, LOW 64 + 32 = 96 of fp16's 512 -> 0.375 h + 0.1875 (1 - h) = 0.274
    hi = (layout.K_ROW[2] + 64) / 512
    lo = (layout.K_ROW[1] + 32) / 512
    assert hi == 0.375 and lo == 0.1875
    h = (0.274 - lo) / (hi - lo)
    assert abs(h - 0.461) < 1e-3
    # a page holds 3072 code bytes for 16 HIGH or 32 LOW tokens: LOW costs half a HIGH
    assert layout.SLOTS[2] * (layout.K_ROW[2] + 64) == 3072
    assert layout.SLOTS[1] * (layout.K_ROW[1] + 32) == 3072
