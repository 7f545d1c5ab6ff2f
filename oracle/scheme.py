"""Oracle: precision-scheme variants of the two tiers and their page images (test
infrastructure only; nothing in the library imports it).

Source: DiffKV review page.  The free-parameter ledger says the K8V4-K4V2 scheme was chosen by
comparing K8V4, K4V8, K8V2, K4V2, K2V4 and K4V1; the reading notes report that mirror
configurations giving values more bits than keys collapse in accuracy; the referee report
(minor comment 5) lists the configurations K8V4-K4V2, K8V4-K4V2-Pr and K8V4-Prune.

Readings taken: a scheme gives each tier its own key and value bit widths (1, 2, 4 or 8),
quantized with the same per-token min/max quantizer as K8V4/K4V2 (``quant.py``) at 2^b - 1
levels.  Pages keep their geometry (3456 bytes; 16 HIGH or 32 LOW slots, so allocation is
unchanged); a tier's format must fit its slots into the first 3072 bytes:
slots * 16 * (kb + vb) <= 3072.  The page layout of these variants (this project's own, with
bits counted little-endian from a field's first byte):
* keys slot-major: slot s's 128 codes at bytes [16 kb s, 16 kb (s + 1)), code i at bits
  [i kb, (i + 1) kb);
* values from byte 16 kb S (S = 16 or 32 slots) in blocks of 16 slots (a HIGH page has one,
  a LOW page two), 256 vb bytes each, in the decode's operand order: block f's bytes
  [4 vb L, 4 vb (L + 1)) (L = 16 g + c, g < 4, c < 16) hold the codes of channels 16 n + c
  (n < 8) for slots 16 f + 4 g + r (r < 4); with p = 8 / vb channels-groups per 32-bit word,
  code (n, r) sits at bit 32 (n // p) + 16 (r % 2) + vb (2 (n % p) + r // 2) of that range
  (each pair of codes that the decode converts together lies 16 bits apart in one word);
* the bytes after the values up to 3072 are zero; parameters (k scale, k zero, v scale,
  v zero as fp16) at 3072 + 8 s and positions (int32, -1 when empty) at 3328 + 4 s for all 32
  slot indices, as in the K8V4/K4V2 layout.
"""
import numpy as np

from . import quant

D = 128
PAGE_BYTES = 3456
CODE_BYTES = 3072
PARAM_OFF, POS_OFF = 3072, 3328
HIGH, LOW = 2, 1
SLOTS = {HIGH: 16, LOW: 32}
BITS = (1, 2, 4, 8)

# the single-tier formats the pages compare, as (key bits, value bits)
FORMATS = {"K8V4": (8, 4), "K4V8": (4, 8), "K8V2": (8, 2), "K4V2": (4, 2), "K2V4": (2, 4),
           "K4V1": (4, 1)}


def fits(tier, kb, vb):
    """Whether a (key bits, value bits) format fits a tier's slots in one page."""
    return kb in BITS and vb in BITS and SLOTS[tier] * 16 * (kb + vb) <= CODE_BYTES


class Scheme:
    """Bit widths of the two tiers: HIGH (kh, vh), LOW (kl, vl)."""

    def __init__(self, kh, vh, kl, vl):
        if not (fits(HIGH, kh, vh) and fits(LOW, kl, vl)):
            raise ValueError("format does not fit the tier's page")
        self.bits = {HIGH: (kh, vh), LOW: (kl, vl)}

    @classmethod
    def named(cls, high, low):
        return cls(*FORMATS[high], *FORMATS[low])

    def slot_bytes(self, tier):
        kb, vb = self.bits[tier]
        return 16 * (kb + vb)


def pack_codes(codes, b):
    """codes uint8 [..., 128] of b bits -> bytes [..., 16 b], code i at bits i b .. i b + b - 1."""
    codes = np.asarray(codes, np.int64)
    n = codes.shape[-1]
    bits = ((codes[..., :, None] >> np.arange(b)) & 1).reshape(codes.shape[:-1] + (n * b,))
    weights = 1 << np.arange(8)
    return (bits.reshape(codes.shape[:-1] + (n * b // 8, 8)) * weights).sum(-1).astype(np.uint8)


def unpack_codes(data, b, n=D):
    """Inverse of pack_codes."""
    data = np.asarray(data, np.int64)
    bits = ((data[..., :, None] >> np.arange(8)) & 1).reshape(data.shape[:-1] + (data.shape[-1] * 8,))
    bits = bits[..., :n * b].reshape(data.shape[:-1] + (n, b))
    return (bits * (1 << np.arange(b))).sum(-1).astype(np.uint8)


def value_bit(vb, s, d):
    """Bit index, from the start of the value region, of slot s's code for channel d."""
    f, g, r = s // 16, (s % 16) // 4, s % 4
    n, c = d // 16, d % 16
    p = 8 // vb
    lane = 16 * g + c
    return 8 * (256 * vb * f + 4 * vb * lane) + 32 * (n // p) + 16 * (r % 2) + vb * (2 * (n % p) + r // 2)


def pack_values(v_codes, vb):
    """v_codes uint8 [S][128] (S = 16 or 32) -> the value region's bytes [16 vb S]."""
    S = v_codes.shape[0]
    bits = np.zeros(16 * vb * S * 8, np.uint8)
    for s in range(S):
        for d in range(D):
            b0 = value_bit(vb, s, d)
            code = int(v_codes[s, d])
            for k in range(vb):
                bits[b0 + k] = (code >> k) & 1
    return (bits.reshape(-1, 8).astype(np.int64) << np.arange(8)).sum(1).astype(np.uint8)


def unpack_values(data, vb, S):
    """Inverse of pack_values: bytes [16 vb S] -> uint8 [S][128]."""
    bits = ((np.asarray(data, np.int64)[:, None] >> np.arange(8)) & 1).reshape(-1)
    out = np.zeros((S, D), np.uint8)
    for s in range(S):
        for d in range(D):
            b0 = value_bit(vb, s, d)
            out[s, d] = int((bits[b0:b0 + vb] << np.arange(vb)).sum())
    return out


def build_page(scheme, tier, k_codes, v_codes, k_scale, k_zero, v_scale, v_zero, pos):
    """Page image (uint8 [3456]) of m live tokens in slots 0..m-1 of a scheme's tier."""
    kb, vb = scheme.bits[tier]
    m = len(pos)
    S = SLOTS[tier]
    assert m <= S
    page = np.zeros(PAGE_BYTES, np.uint8)
    for s in range(m):
        page[16 * kb * s:16 * kb * (s + 1)] = pack_codes(k_codes[s], kb)
    vs_all = np.zeros((S, D), np.uint8)
    vs_all[:m] = np.asarray(v_codes, np.uint8)[:m]
    v0 = 16 * kb * S
    page[v0:v0 + 16 * vb * S] = pack_values(vs_all, vb)
    params = np.zeros((32, 4), np.float16)
    params[:m, 0] = k_scale
    params[:m, 1] = k_zero
    params[:m, 2] = v_scale
    params[:m, 3] = v_zero
    page[PARAM_OFF:POS_OFF] = params.view(np.uint8).ravel()
    posv = np.full(32, -1, np.int32)
    posv[:m] = pos
    page[POS_OFF:PAGE_BYTES] = posv.view(np.uint8)
    return page


def read_page(page, scheme, tier, m):
    """Codes, parameters and positions of the first m slots of a page image."""
    kb, vb = scheme.bits[tier]
    S = SLOTS[tier]
    page = np.asarray(page, np.uint8)
    k = np.stack([unpack_codes(page[16 * kb * s:16 * kb * (s + 1)], kb) for s in range(m)]) \
        if m else np.zeros((0, D), np.uint8)
    v0 = 16 * kb * S
    v = unpack_values(page[v0:v0 + 16 * vb * S], vb, S)[:m]
    params = page[PARAM_OFF:POS_OFF].copy().view(np.float16).reshape(32, 4)[:m]
    pos = page[POS_OFF:PAGE_BYTES].copy().view(np.int32)[:m]
    return k, v, params[:, 0], params[:, 1], params[:, 2], params[:, 3], pos


def head_pages(k_rows, v_rows, tier_col, scheme):
    """Prompt placement of one head under a scheme: {HIGH: [images], LOW: [images]}, tokens in
    ascending position order within each tier (as for K8V4/K4V2)."""
    out = {}
    for tier in (HIGH, LOW):
        kb, vb = scheme.bits[tier]
        pos = np.nonzero(np.asarray(tier_col) == tier)[0]
        kc, ks, kz = quant.quantize_rows(k_rows[pos], kb)
        vc, vs, vz = quant.quantize_rows(v_rows[pos], vb)
        per = SLOTS[tier]
        out[tier] = [build_page(scheme, tier, kc[p0:p0 + per], vc[p0:p0 + per], ks[p0:p0 + per],
                                kz[p0:p0 + per], vs[p0:p0 + per], vz[p0:p0 + per],
                                pos[p0:p0 + per]) for p0 in range(0, len(pos), per)]
    return out


def head_dequantized(k_rows, v_rows, tier_col, scheme):
    """float32 keys and values of one head's live tokens under a scheme, HIGH tokens first then
    LOW tokens, each in ascending position order."""
    ks, vs = [], []
    for tier in (HIGH, LOW):
        kb, vb = scheme.bits[tier]
        pos = np.nonzero(np.asarray(tier_col) == tier)[0]
        kc, s, z = quant.quantize_rows(k_rows[pos], kb)
        ks.append(quant.dequantize_rows(kc, s, z))
        vc, s, z = quant.quantize_rows(v_rows[pos], vb)
        vs.append(quant.dequantize_rows(vc, s, z))
    return np.concatenate(ks), np.concatenate(vs)
