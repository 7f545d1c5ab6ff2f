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


# ---- the per-step policy ---------------------------------------------------------------

def _prompted(rng, B, H, G, n0, W, alpha=(1.0, 0.2)):
    k0, v0 = _data(rng, B, H, B * n0)
    acc0 = (rng.random((B * n0, H * G)) * np.arange(B * n0)[::-1, None] * 0.05).astype(np.float32)
    cu = np.array([n0 * b for b in range(B + 1)])
    tier0, _, _ = osc.score_tokens(acc0, cu, H, alpha[0], alpha[1], W)
    g = ogen.Generation(B, H, 64, 4000)
    g.prompt(k0, v0, tier0, cu)
    return g, tier0


def _acc_rows(rng, g, G):
    n = sum(g.lens) + g.B                                  # rows after the new tokens
    return (rng.random((n, g.H * G)) * 2.0).astype(np.float32)


def test_step_with_zero_thresholds_is_an_append():
    # every leaving token scores >= 0 = alpha/N: it stays HIGH and the step is an append
    rng = np.random.default_rng(7)
    B, H, G, n0, W = 2, 2, 2, 50, 8
    a, _ = _prompted(rng, B, H, G, n0, W)
    b_, _ = _prompted(np.random.default_rng(7), B, H, G, n0, W)
    for s in range(40):
        kn, vn = _data(rng, B, H, B)
        dec = a.step(kn, vn, _acc_rows(rng, a, G), 0.0, 0.0, W)
        b_.append(kn, vn)
        assert np.all(dec == ogen.HIGH)
    for b in range(B):
        assert np.array_equal(a.tiers[b], b_.tiers[b])
        for h in range(H):
            pa, pb = a.head_pages(b, h), b_.head_pages(b, h)
            for t in (ogen.HIGH, ogen.LOW):
                assert len(pa[t]) == len(pb[t])
                for x, y in zip(pa[t], pb[t]):
                    assert np.array_equal(x, y)
    assert a.pool.head == b_.pool.head and a.pool.tail == b_.pool.tail


def test_step_with_infinite_thresholds_keeps_only_old_tiers_and_the_window():
    # nothing reaches alpha/N = inf: every token leaving the window is pruned; the head keeps
    # its prompt tokens that were outside the prompt's window and the last W tokens
    rng = np.random.default_rng(8)
    B, H, G, n0, W, steps = 2, 3, 2, 40, 6, 25
    g, tier0 = _prompted(rng, B, H, G, n0, W)
    for s in range(steps):
        kn, vn = _data(rng, B, H, B)
        dec = g.step(kn, vn, _acc_rows(rng, g, G), np.inf, np.inf, W)
        assert np.all(dec == ogen.PRUNE)
    N = n0 + steps
    for b in range(B):
        for h in range(H):
            live = sorted(g.rec[b][h])
            old = [t for t in range(n0 - W) if tier0[b * n0 + t, h] != ogen.PRUNE]
            assert live == old + list(range(N - W, N))
            assert g.count[b, h, 0] == sum(tier0[b * n0 + t, h] == ogen.HIGH
                                           for t in range(n0 - W)) + W
    g.pool.check_invariants()


def test_step_demotion_requantizes_the_k8v4_codes():
    # alpha_h = inf, alpha_l = 0: every leaving token goes LOW, with the codes a demotion of
    # its stored K8V4 codes gives
    rng = np.random.default_rng(9)
    B, H, G, n0, W = 1, 2, 2, 30, 5
    g, _ = _prompted(rng, B, H, G, n0, W)
    before = {h: dict(g.rec[0][h]) for h in range(H)}
    for s in range(12):
        kn, vn = _data(rng, B, H, B)
        dec = g.step(kn, vn, _acc_rows(rng, g, G), np.inf, 0.0, W)
        assert np.all(dec == ogen.LOW)
        for h in range(H):
            before[h][n0 + s] = g.rec[0][h][n0 + s]
    for h in range(H):
        for t in range(n0 - W, n0 - W + 12):
            r0, r1 = before[h][t], g.rec[0][h][t]
            assert r0[0] == ogen.HIGH and r1[0] == ogen.LOW
            k2 = quant.requantize_from(r0[1][None], np.array([r0[2]]), np.array([r0[3]]), 4)
            v2 = quant.requantize_from(r0[4][None], np.array([r0[5]]), np.array([r0[6]]), 2)
            assert np.array_equal(r1[1], k2[0][0]) and r1[2] == k2[1][0] and r1[3] == k2[2][0]
            assert np.array_equal(r1[4], v2[0][0]) and r1[5] == v2[1][0] and r1[6] == v2[2][0]


def test_step_decisions_follow_the_prompt_scoring_rule():
    # the tier given to t_c is the one score_tokens gives that token for the same
    # accumulators (t_c is just outside the window there)
    rng = np.random.default_rng(10)
    B, H, G, n0, W = 2, 2, 4, 64, 8
    g, _ = _prompted(rng, B, H, G, n0, W)
    seen = set()
    for s in range(30):
        kn, vn = _data(rng, B, H, B)
        acc = _acc_rows(rng, g, G) * np.float32(0.06)
        cu = np.concatenate([[0], np.cumsum([n + 1 for n in g.lens])])
        want, _, _ = osc.score_tokens(acc, cu, H, 1.0, 0.5, W)
        dec = g.step(kn, vn, acc, 1.0, 0.5, W)
        for b in range(B):
            t_c = g.lens[b] - 1 - W
            assert np.array_equal(dec[b], want[cu[b] + t_c])
        seen |= set(dec.ravel().tolist())
    assert seen == {ogen.PRUNE, ogen.LOW, ogen.HIGH}
    g.pool.check_invariants()


# ---- precision schemes in the generation phase ---------------------------------------------

def test_scheme_all_high_generation_equals_scheme_prompt_of_the_whole_sequence():
    # with nothing demoted or pruned, appends and rounds under a scheme leave exactly the
    # pages a scheme prompt placement of the whole sequence writes (oracle/scheme.head_pages,
    # pinned by hand-packed bytes in test_oracle_scheme)
    from oracle import scheme as osch
    rng = np.random.default_rng(20)
    B, H, n0, steps = 2, 2, 21, 40
    sc = osch.Scheme.named("K4V8", "K2V4")
    ks, vs = zip(*[_data(rng, 1, H, n0 + steps) for _ in range(B)])
    g = ogen.Generation(B, H, 16, 400, scheme=sc)
    cu = np.array([0, n0, 2 * n0])
    g.prompt(np.concatenate([k[:n0] for k in ks]), np.concatenate([v[:n0] for v in vs]),
             np.full((2 * n0, H), ogen.HIGH, np.uint8), cu)
    for s in range(steps):
        g.append(np.stack([k[n0 + s] for k in ks]), np.stack([v[n0 + s] for v in vs]))
        if s % 16 == 15:
            n = n0 + s + 1
            g.retier(np.ones((B * n, 2 * H), np.float32), 0.0, 0.0, 4)
    for b in range(B):
        for h in range(H):
            want = osch.head_pages(ks[b][:, h], vs[b][:, h], np.full(n0 + steps, ogen.HIGH), sc)
            got = g.head_pages(b, h)
            assert len(got[ogen.HIGH]) == len(want[ogen.HIGH]) and not got[ogen.LOW]
            for a, e in zip(got[ogen.HIGH], want[ogen.HIGH]):
                assert np.array_equal(a, e)


def test_scheme_demotion_requantizes_the_high_reconstruction_read_from_the_page():
    # under K8V2-K4V1 a token demoted by a round carries, in its LOW page, the codes of its
    # HIGH page's reconstruction (read back from the page bytes before the round) rounded to
    # fp16 and quantized at 4 / 1 bits; survivors keep their page bytes' codes
    from oracle import scheme as osch
    rng = np.random.default_rng(21)
    B, H, G, n0 = 1, 2, 2, 64
    sc = osch.Scheme.named("K8V2", "K4V1")
    k0, v0 = _data(rng, B, H, n0)
    cu = np.array([0, n0])
    g = ogen.Generation(B, H, 16, 400, scheme=sc)
    g.prompt(k0, v0, np.full((n0, H), ogen.HIGH, np.uint8), cu)

    def read_all(h):
        out = {}
        pages = g.head_pages(0, h)
        for t in (ogen.HIGH, ogen.LOW):
            for img in pages[t]:
                pos = img[osch.POS_OFF:].copy().view(np.int32)
                m = int((pos >= 0).sum())
                kc, vc, ks_, kz, vs_, vz, ps = osch.read_page(img, sc, t, m)
                for n in range(m):
                    out[int(ps[n])] = (t, kc[n], ks_[n], kz[n], vc[n], vs_[n], vz[n])
        return out
    before = {h: read_all(h) for h in range(H)}
    acc = np.full((n0, H * G), 1e-6, np.float32)
    acc[::3] = 10.0                    # every third token keeps HIGH, the rest fall to LOW
    tier, _, _ = g.retier(acc, 1.0, 1e-30, 4)
    n_dem = 0
    for h in range(H):
        after = read_all(h)
        for pos, r in after.items():
            old = before[h][pos]
            if r[0] == old[0]:
                assert all(np.array_equal(x, y) for x, y in zip(r[1:], old[1:]))
                continue
            assert old[0] == ogen.HIGH and r[0] == ogen.LOW
            n_dem += 1
            xk = (old[1].astype(np.float64) * np.float64(old[2]) + np.float64(old[3]))
            xv = (old[4].astype(np.float64) * np.float64(old[5]) + np.float64(old[6]))
            kc, kscale, kzero = quant.quantize_rows(xk.astype(np.float32).astype(np.float16)[None], 4)
            vc, vscale, vzero = quant.quantize_rows(xv.astype(np.float32).astype(np.float16)[None], 1)
            assert np.array_equal(r[1], kc[0]) and r[2] == kscale[0] and r[3] == kzero[0]
            assert np.array_equal(r[4], vc[0]) and r[5] == vscale[0] and r[6] == vzero[0]
            assert set(np.unique(r[4])) <= {0, 1} and r[1].max() <= 15
    assert n_dem > 20


def test_default_scheme_generation_dequantizes_as_the_default_layout():
    # the K8V4-K4V2 scheme stores the same codes as the default layout in another byte order:
    # the same steps give the same live tokens, codes and dequantized rows
    from oracle import scheme as osch
    rng = np.random.default_rng(22)
    B, H, G, n0, W = 2, 2, 2, 50, 6
    k0, v0 = _data(rng, B, H, B * n0)
    acc0 = (rng.random((B * n0, H * G)) * np.arange(B * n0)[::-1, None] * 0.05).astype(np.float32)
    cu = np.array([0, n0, 2 * n0])
    tier0, _, _ = osc.score_tokens(acc0, cu, H, 1.0, 0.2, W)
    a = ogen.Generation(B, H, 16, 800)
    b_ = ogen.Generation(B, H, 16, 800, scheme=osch.Scheme.named("K8V4", "K4V2"))
    a.prompt(k0, v0, tier0, cu)
    b_.prompt(k0, v0, tier0, cu)
    for s in range(20):
        kn, vn = _data(rng, B, H, B)
        acc = (rng.random((sum(a.lens) + B, H * G)) * 2.0).astype(np.float32)
        da = a.step(kn, vn, acc, 1.0, 0.2, W)
        db = b_.step(kn, vn, acc, 1.0, 0.2, W)
        assert np.array_equal(da, db)
    for b in range(B):
        for h in range(H):
            ka, va = a.head_dequantized(b, h)
            kb, vb = b_.head_dequantized(b, h)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
            pa, pb = a.head_pages(b, h), b_.head_pages(b, h)
            for t in (ogen.HIGH, ogen.LOW):
                assert len(pa[t]) == len(pb[t])
