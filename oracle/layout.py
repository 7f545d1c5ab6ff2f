"""Oracle: the unified page format, bit by bit (test infrastructure only).

Source: DiffKV review page, "Core claim" -- one GPU-resident manager with *unified* pages
shared by both precision tiers.  The page prints no byte layout; this module is the
layout this project defines, written out independently of the
GPU code so that page images can be compared byte for byte.

One page is 3456 bytes and holds either 16 HIGH (K8V4) tokens or 32 LOW (K4V2) tokens:

  [   0, 2048)  key codes, one row per slot
                  HIGH: slot s at 128*s, byte i = 8-bit code of channel i
                  LOW : slot s at  64*s, 16 little-endian 32-bit words; word w holds
                        channels 8w..8w+7, channel 8w+e in nibble
                        (e & 1) + 2*(e >> 2) + 4*((e >> 1) & 1)
  [2048, 3072)  value codes, 64 units of 16 bytes; unit u = 16*j + l (j in 0..3, l in 0..15)
                at 2048 + 16*u, four little-endian 32-bit words q = 0..3
                  HIGH (4-bit): slot s = 4*j + r, channel c = 16*n + l,
                        word q = n >> 1, nibble 2*(n & 1) + (r >> 1) + 4*(r & 1)
                  LOW  (2-bit): slot s = 16*f + 4*j + r (f = 0,1), channel c = 16*n + l,
                        word q = 2*f + (n >> 2), 2-bit field 2*(n & 3) + (r >> 1) + 8*(r & 1)
  [3072, 3328)  per-slot parameters, 8 bytes per slot: key scale, key zero, value scale,
                value zero (fp16, little-endian)
  [3328, 3456)  per-slot token position (int32, little-endian)

Slots a page does not hold live tokens in are all-zero codes and parameters, position -1.
"""
import numpy as np

D = 128
PAGE_BYTES = 3456
K_OFF, V_OFF, PARAM_OFF, POS_OFF = 0, 2048, 3072, 3328
SLOTS = {2: 16, 1: 32}          # tier -> slots per page (HIGH 16, LOW 32)
K_ROW = {2: 128, 1: 64}         # tier -> key bytes per slot


def _k_map(tier):
    """(byte, shift) of the key code of (slot, channel), arrays [slots][128]."""
    n = SLOTS[tier]
    byte = np.zeros((n, D), np.int64)
    shift = np.zeros((n, D), np.int64)
    for s in range(n):
        for c in range(D):
            if tier == 2:
                byte[s, c] = K_OFF + 128 * s + c
                shift[s, c] = 0
            else:
                w, e = c // 8, c % 8
                nib = (e & 1) + 2 * (e >> 2) + 4 * ((e >> 1) & 1)
                byte[s, c] = K_OFF + 64 * s + 4 * w + nib // 2
                shift[s, c] = 4 * (nib % 2)
    return byte, shift


def _v_map(tier):
    """(byte, shift) of the value code of (slot, channel), arrays [slots][128]."""
    n = SLOTS[tier]
    byte = np.zeros((n, D), np.int64)
    shift = np.zeros((n, D), np.int64)
    for s in range(n):
        for c in range(D):
            nn, l = c // 16, c % 16
            if tier == 2:
                j, r = s // 4, s % 4
                q = nn >> 1
                field = 2 * (nn & 1) + (r >> 1) + 4 * (r & 1)   # 4-bit field index in word
                bit = 4 * field
            else:
                f, j, r = s // 16, (s % 16) // 4, s % 4
                q = 2 * f + (nn >> 2)
                field = 2 * (nn & 3) + (r >> 1) + 8 * (r & 1)   # 2-bit field index in word
                bit = 2 * field
            u = 16 * j + l
            byte[s, c] = V_OFF + 16 * u + 4 * q + bit // 8
            shift[s, c] = bit % 8
    return byte, shift


_MAPS = {t: (_k_map(t), _v_map(t)) for t in (1, 2)}
_KBITS = {2: 8, 1: 4}
_VBITS = {2: 4, 1: 2}


def build_page(tier, k_codes, v_codes, k_scale, k_zero, v_scale, v_zero, pos):
    """Page image (uint8 [3456]) of `m` live tokens placed in slots 0..m-1.

    k_codes/v_codes uint8 [m][128]; scales/zeros fp16 [m]; pos int [m]; m <= slots(tier).
    """
    m = len(pos)
    assert m <= SLOTS[tier]
    page = np.zeros(PAGE_BYTES, np.uint8)
    (kb, ks), (vb, vs) = _MAPS[tier]
    acc = np.zeros(PAGE_BYTES, np.int64)
    # the fields of different (slot, channel) pairs never overlap, so adding is OR-ing
    np.add.at(acc, kb[:m].ravel(), (np.asarray(k_codes, np.int64)[:m] << ks[:m]).ravel())
    np.add.at(acc, vb[:m].ravel(), (np.asarray(v_codes, np.int64)[:m] << vs[:m]).ravel())
    page[:PARAM_OFF] = acc[:PARAM_OFF].astype(np.uint8)
    params = np.zeros((32, 4), np.float16)
    params[:m, 0] = k_scale
    params[:m, 1] = k_zero
    params[:m, 2] = v_scale
    params[:m, 3] = v_zero
    page[PARAM_OFF:POS_OFF] = params.view(np.uint8).ravel()   # little-endian host
    posv = np.full(32, -1, np.int32)
    posv[:m] = pos
    page[POS_OFF:PAGE_BYTES] = posv.view(np.uint8)
    return page


def read_page(page, tier, m):
    """Inverse of build_page for the first m slots: codes, parameters and positions."""
    page = np.asarray(page, np.uint8)
    (kb, ks), (vb, vs) = _MAPS[tier]
    kmask = (1 << _KBITS[tier]) - 1
    vmask = (1 << _VBITS[tier]) - 1
    k = ((page[kb[:m]].astype(np.int64) >> ks[:m]) & kmask).astype(np.uint8)
    v = ((page[vb[:m]].astype(np.int64) >> vs[:m]) & vmask).astype(np.uint8)
    params = page[PARAM_OFF:POS_OFF].copy().view(np.float16).reshape(32, 4)[:m]
    pos = page[POS_OFF:PAGE_BYTES].copy().view(np.int32)[:m]
    return k, v, params[:, 0], params[:, 1], params[:, 2], params[:, 3], pos
