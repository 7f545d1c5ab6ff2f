"""Pins of the oracle's generation phase: appends, monotone re-tier rounds, survivors keep
their codes, demotions re-quantize from the K8V4 reconstruction, and with nothing ever
demoted the pages equal a prompt placement of the whole sequence."""
import numpy as np

from oracle import generation as ogen, place, quant, score as osc


def _data(rng, B, H, n):
    k = rng.standard_normal((n, H, 128)).astype(np.float16)
    v = rng.standard_normal((n, H, 128)).astype(np.float16)
    return k, v


def test_all_high_generation_equals_prompt_of_the_whole_sequence():
    rng = np.random.default_rng(0)
    B, H, n0, steps = 2, 2, 40, 30
    ks, vs = zip(*[_data(rng, 1, H, n0 + steps) for _ in range(B)])
    g = ogen.Generation(B, H, 16, 400)
    cu = np.array([0, n0, 2 * n0])
    k0 = np.concatenate([k[:n0] for k in ks])
    v0 = np.concatenate([v[:n0] for v in vs])
    tier0 = np.full((2 * n0, H), ogen.HIGH, np.uint8)
    g.prompt(k0, v0, tier0, cu)
    for s in range(steps):
        g.append(np.stack([k[n0 + s] for k in ks]), np.stack([v[n0 + s] for v in vs]))
        if s % 10 == 9:
            n = n0 + s + 1
            acc = np.ones((B * n, 2 * H), np.float32)        # alpha_h = 0: everything HIGH
            g.retier(acc, 0.0, 0.0, 4)
    g.pool.check_invariants()
    for b in range(B):
        for h in range(H):
            want = place.head_pages(ks[b][:, h], vs[b][:, h], np.full(n0 + steps, ogen.HIGH))
            got = g.head_pages(b, h)
            assert len(got[ogen.HIGH]) == len(want[ogen.HIGH])
            for a, e in zip(got[ogen.HIGH], want[ogen.HIGH]):
                assert np.array_equal(a, e)


def test_rounds_are_monotone_survivors_keep_codes_demotions_requantize():
    rng = np.random.default_rng(1)
    B, H, G, n0 = 2, 2, 2, 60
    k0, v0 = _data(rng, B, H, B * n0)
    acc0 = (rng.random((B * n0, H * G)) * np.arange(B * n0)[::-1, None] * 0.05).astype(np.float32)
    cu = np.array([0, n0, 2 * n0])
    tier0, _, _ = osc.score_tokens(acc0, cu, H, 1.0, 0.2, 8)
    g = ogen.Generation(B, H, 16, 800)
    g.prompt(k0, v0, tier0, cu)
    first = {(b, h): dict(g.rec[b][h]) for b in range(B) for h in range(H)}
    prev_tiers = [t.copy() for t in g.tiers]
    for rnd in range(3):
        for s in range(16):
            kn, vn = _data(rng, B, H, B)
            g.append(kn, vn)
            for b in range(B):
                for h in range(H):
                    pos = len(g.tiers[b]) - 1
                    first[(b, h)][pos] = g.rec[b][h][pos]
        n = len(g.tiers[0])
        acc = (rng.random((B * n, H * G)) * np.arange(n)[::-1][None].repeat(B, 0).reshape(-1, 1)
               * 0.08).astype(np.float32)
        g.retier(acc, 1.0, 0.2, 8)
        g.pool.check_invariants()
        for b in range(B):
            old = prev_tiers[b]
            new = g.tiers[b][:len(old)]
            assert np.all(new <= old)          # never promoted
            prev_tiers[b] = g.tiers[b].copy()
            for h in range(H):
                for pos, r in g.rec[b][h].items():
                    orig = first[(b, h)][pos]
                    if r[0] == orig[0]:
                        assert all(np.array_equal(x, y) for x, y in zip(r[1:], orig[1:]))
                    else:                       # demoted HIGH -> LOW: re-quantized once
                        assert orig[0] == ogen.HIGH and r[0] == ogen.LOW
                        kc, kscale, kz = quant.requantize_from(orig[1][None], np.array([orig[2]]),
                                                               np.array([orig[3]]), 4)
                        assert np.array_equal(r[1], kc[0]) and r[2] == kscale[0]
                for pos in range(len(g.tiers[b])):
                    kept = int(g.tiers[b][pos, h]) in (ogen.HIGH, ogen.LOW)
                    assert kept == (pos in g.rec[b][h])
