"""Oracle: the page images one head must hold after quantize_and_place.

Test infrastructure only.

Source: DiffKV review page, "Core claim" (K8V4 for important tokens, K4V2 for moderately
important ones, unified pages) and "What carries the argument" (each head owns its own
high- and low-precision pages).  Reading taken: within one head and one tier,
tokens take slots in ascending position order, so HIGH token number s (counting from 0 in
position order) sits in slot s % 16 of the head's HIGH page s // 16 (row position s // 16),
and LOW token number s in slot s % 32 of LOW page s // 32 (row position C-1 - s // 32).
"""
import numpy as np

from . import layout, quant

HIGH, LOW = 2, 1


def head_tokens(tier_col, want):
    """Positions (ascending) of the tokens of one head whose tier is `want`."""
    return np.nonzero(np.asarray(tier_col) == want)[0]


def head_pages(k_rows, v_rows, tier_col):
    """Prompt placement of one head.

    k_rows, v_rows fp16 [N][128] (positions 0..N-1 of one request, one KV head);
    tier_col uint8 [N].  Returns {HIGH: [page images], LOW: [page images]} where list
    index = page number within the tier (row position p for HIGH, C-1-p for LOW).
    """
    out = {}
    for tier in (HIGH, LOW):
        pos = head_tokens(tier_col, tier)
        kc, ks, kz = quant.quantize_rows(k_rows[pos], quant.K_BITS[tier])
        vc, vs, vz = quant.quantize_rows(v_rows[pos], quant.V_BITS[tier])
        per = layout.SLOTS[tier]
        pages = []
        for p0 in range(0, len(pos), per):
            sl = slice(p0, min(p0 + per, len(pos)))
            pages.append(layout.build_page(tier, kc[sl], vc[sl], ks[sl], kz[sl], vs[sl],
                                           vz[sl], pos[sl]))
        out[tier] = pages
    return out


def head_dequantized(k_rows, v_rows, tier_col):
    """float32 dequantized keys and values of one head's live tokens, HIGH tokens first
    (ascending position) then LOW tokens (ascending position)."""
    ks, vs = [], []
    for tier in (HIGH, LOW):
        pos = head_tokens(tier_col, tier)
        kc, s, z = quant.quantize_rows(k_rows[pos], quant.K_BITS[tier])
        ks.append(quant.dequantize_rows(kc, s, z))
        vc, s, z = quant.quantize_rows(v_rows[pos], quant.V_BITS[tier])
        vs.append(quant.dequantize_rows(vc, s, z))
    return np.concatenate(ks), np.concatenate(vs)


def dequantize_pages(images, tier, n):
    """float32 keys and values of the first n tokens stored in a tier's page images."""
    per = layout.SLOTS[tier]
    ks, vs = [], []
    for p, img in enumerate(images):
        m = min(per, n - p * per)
        if m <= 0:
            break
        kc, vc, ksc, kz, vsc, vz, _ = layout.read_page(img, tier, m)
        ks.append(quant.dequantize_rows(kc, ksc, kz))
        vs.append(quant.dequantize_rows(vc, vsc, vz))
    if not ks:
        return np.zeros((0, layout.D), np.float32), np.zeros((0, layout.D), np.float32)
    return np.concatenate(ks), np.concatenate(vs)
