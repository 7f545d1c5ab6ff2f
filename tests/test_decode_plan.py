"""The decode's split plan, restated from its documented rule and checked on the CPU: the
number of workgroup slots per head agrees with the size of the library's decode workspace, and
the geometries of the GPU edge tests really reach the paths they are meant to reach (a wave
slice longer than the 64 page ids a wave preloads).

Rule (the decode kernel's header and the workspace layout): s0 = clamp(ceil(2048 / heads), 16,
64); wt = clamp(ceil(Wmax / s0), 128, 256) work units per workgroup, Wmax = 3 (C + 1) the units
of the largest head the row capacity allows; splits = min(s0, ceil(Wmax / wt),
floor(8192 / heads)), at least 1.  A head of nh HIGH and nl LOW tokens weighs 3 units per HIGH
tile (16 tokens, one page) and 2 per LOW tile (16 tokens, half a page), uses
SH = clamp(ceil(W / wt), 1, splits) workgroups of 4 waves, and wave c of the SH * 4 takes the
tiles between unit boundaries W c / (4 SH) and W (c + 1) / (4 SH), rounded up to a tile and,
in the LOW tier, to an even LOW tile.
"""
import math

from mixed_precision_paged_score_amd import kvc

UH, UL, WAVES, PART_STRIDE = 3, 2, 4, 132


def plan(heads, C):
    s0 = min(max(-(-2048 // heads), 16), 64)
    wmax = UH * (C + 1)
    wt = min(max(-(-wmax // s0), 128), 256)
    splits = min(s0, -(-wmax // wt), 8192 // heads)
    return max(splits, 1), wt


def wave_slices(nh, nl, splits, wt):
    qH, tL = -(-nh // 16), -(-nl // 16)
    WH = UH * qH
    W = WH + UL * tL
    SH = min(max(-(-W // wt), 1), splits)
    NC = SH * WAVES

    def tile_of(x):
        t = -(-x // UH) if x <= WH else qH + -(-(x - WH) // UL)
        if t > qH:
            t = qH + ((t - qH + 1) & ~1)
        return min(t, qH + tL)
    out = []
    for c in range(NC):
        u0, u1 = tile_of(W * c // NC), tile_of(W * (c + 1) // NC)
        out.append(((u0, min(u1, qH)), (max(u0, qH) - qH, u1 - qH)))
    return SH, out


def splits_from_workspace(B, Hq, Hkv, C):
    g = kvc.make_geom(1, B, Hq, Hkv, C, 1 << 16)
    part = kvc.workspace_bytes(g, kvc.OP_DECODE)
    per_split = 4 * PART_STRIDE * B * Hq
    return part // per_split


def test_plan_matches_library_workspace():
    for B, Hq, Hkv, C in [(16, 64, 8, 2049), (64, 64, 8, 2049), (256, 64, 8, 2049),
                          (1, 32, 8, 33), (16, 64, 8, 257), (3, 16, 4, 40), (512, 8, 8, 20)]:
        s, _ = plan(B * Hkv, C)
        assert splits_from_workspace(B, Hq, Hkv, C) == s, (B, Hq, Hkv, C)


def test_slices_tile_every_head_exactly_once():
    for nh, nl in [(0, 0), (1, 0), (0, 1), (16384, 16384), (100, 3000), (5000, 7)]:
        for heads, C in [(128, 2049), (2048, 2049), (4, 129)]:
            s, wt = plan(heads, C)
            SH, sl = wave_slices(nh, nl, s, wt)
            qH, tL = -(-nh // 16), -(-nl // 16)
            hs = sorted(a for a, _ in sl if a[0] < a[1])
            ls = sorted(b for _, b in sl if b[0] < b[1])
            assert sum(b - a for a, b in hs) == qH and sum(b - a for a, b in ls) == tL
            for (a, b), (c, d) in zip(hs, hs[1:]):
                assert b <= c
            for (a, b), (c, d) in zip(ls, ls[1:]):
                assert b <= c
            for a, _ in ls:
                assert a % 2 == 0          # LOW pairs stay within a page


def test_2048_head_edge_case_spans_more_than_one_page_chunk():
    # the geometry of the GPU test: 256 requests x 8 KV heads, C for 32,768 tokens, one head
    # with 16,384 HIGH and 16,384 LOW tokens
    C = -(-32768 // 16) + 1
    s, wt = plan(2048, C)
    assert s == 4 and wt == 256
    SH, sl = wave_slices(16384, 16384, s, wt)
    assert SH == 4
    high_tiles = max(b - a for (a, b), _ in sl)
    low_pages = max(math.ceil(d / 2) - c // 2 for _, (c, d) in sl if d > c)
    # a wave preloads the ids of 64 pages: 64 HIGH tiles or 128 LOW tiles
    assert high_tiles > 64, high_tiles
    assert low_pages > 64, low_pages


def test_small_edge_case_has_several_pairs_per_wave():
    # the large-value test: each wave must see several pairs so the lazy running max lags
    C = -(-2048 // 16) + 1
    s, wt = plan(4, C)
    SH, sl = wave_slices(1024 + 32, 992, s, wt)
    assert all((b - a) >= 4 or (d - c) >= 4 for (a, b), (c, d) in sl)


def _lazy_max_peak_pv(lens, Hkv, G, W, v_amp, bits_v):
    """Replays the decode's running-max rule on the large-value test's inputs: per wave slice
    the pairs of tiles in order, a rescale of every column when some column's pair max passes
    its running max by more than 8 (log2); returns the largest p * scale_v a token reaches (the
    value the decode would round to fp16 without its overflow guard)."""
    import numpy as np
    from oracle import quant
    from test_gpu_decode_edges import block_tiers, ramp_inputs, HIGH, LOW
    tiers = np.concatenate([block_tiers(n, Hkv, 32, W) for n in lens])
    k, v, q = ramp_inputs(lens, Hkv, G, tiers, 7.5 / 32, v_amp, seed=72)
    k, v, q = k.numpy(), v.numpy(), q.numpy()
    C = -(-max(lens) // 16) + 1
    s, wt = plan(len(lens) * Hkv, C)
    scale_log2 = np.log2(np.e) / np.sqrt(128)
    peak = 0.0
    o = 0
    for b, n in enumerate(lens):
        for h in range(Hkv):
            tiles = {}
            for x in (HIGH, LOW):
                idx = np.nonzero(tiers[o:o + n, h] == x)[0]
                kc, ks, kz = quant.quantize_rows(k[o + idx, h], quant.K_BITS[x])
                kd = quant.dequantize_rows(kc, ks, kz).astype(np.float64)
                _, vs, _ = quant.quantize_rows(v[o + idx, h], bits_v[x])
                L = (q[b, h * G:(h + 1) * G].astype(np.float64) @ kd.T) * scale_log2  # [G][n]
                tiles[x] = [(L[:, i:i + 16], vs[i:i + 16].astype(np.float64))
                            for i in range(0, len(idx), 16)]
            nh = int((tiers[o:o + n, h] == HIGH).sum())
            nl = int((tiers[o:o + n, h] == LOW).sum())
            _, slices = wave_slices(nh, nl, s, wt)
            for (a0, a1), (l0, l1) in slices:
                m = np.full(G, -1e30)
                for x, (t0, t1) in ((HIGH, (a0, a1)), (LOW, (l0, l1))):
                    for t in range(t0, t1, 2):
                        pair = tiles[x][t:min(t + 2, t1)]
                        Lp = np.concatenate([p[0] for p in pair], axis=1)
                        vsp = np.concatenate([p[1] for p in pair])
                        cmax = Lp.max(axis=1)
                        if np.any(cmax > m + 8.0):
                            m = np.maximum(m, cmax)
                        peak = max(peak, float((np.exp2(Lp - m[:, None]) * vsp[None]).max()))
        o += n
    return peak


def test_large_value_test_inputs_would_overflow_fp16_without_the_guard():
    # the default decode's tiers: K8V4 HIGH, K4V2 LOW
    from test_gpu_decode_edges import HIGH, LOW
    peak = _lazy_max_peak_pv([2048, 1500], 2, 8, 64, {HIGH: 3500.0, LOW: 700.0},
                             {HIGH: 4, LOW: 2})
    assert peak > 65504.0, peak
