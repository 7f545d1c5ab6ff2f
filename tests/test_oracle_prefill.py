"""Pins of the prefill oracle (causal attention + strictly-later column sums) against facts
fixed by the mathematics: explicit loops on tiny inputs, closed forms for identical keys,
row-stochastic masses, a scipy softmax recomputation and the sampled helpers."""
import math

import numpy as np
import scipy.special

from oracle import prefill as op


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float16)


def test_brute_force_loops_tiny():
    # every weight written out with scalar exp and sums, no numpy softmax
    rng = np.random.default_rng(0)
    cu = [0, 5, 9]
    q, k, v = _rand(rng, (9, 4, 8)), _rand(rng, (9, 2, 8)), _rand(rng, (9, 2, 8))
    scale = 0.3
    out, acc = op.prefill(q, k, v, cu, 2, scale)
    want_out = np.zeros_like(out)
    want_acc = np.zeros_like(acc)
    for b in range(2):
        lo, hi = cu[b], cu[b + 1]
        for hq in range(4):
            h = hq // 2
            for i in range(hi - lo):
                logits = [sum(float(q[lo + i, hq, e]) * float(k[lo + j, h, e]) for e in range(8))
                          * scale for j in range(i + 1)]
                mx = max(logits)
                ws = [math.exp(x - mx) for x in logits]
                tot = sum(ws)
                for j in range(i + 1):
                    p = ws[j] / tot
                    for e in range(8):
                        want_out[lo + i, hq, e] += p * float(v[lo + j, h, e])
                    if j < i:
                        want_acc[lo + j, hq] += p
    assert np.allclose(out, want_out, rtol=1e-12, atol=1e-12)
    assert np.allclose(acc, want_acc, rtol=1e-12, atol=1e-12)


def test_identical_keys_give_harmonic_tails():
    # all keys equal: row i is uniform over i+1 keys, so acc[t] = sum_{i=t+1}^{n-1} 1/(i+1)
    # = H_n - H_{t+1}, and the output is the running mean of v
    rng = np.random.default_rng(1)
    n = 40
    q = _rand(rng, (n, 2, 16))
    k = np.tile(_rand(rng, (1, 1, 16)), (n, 1, 1))
    v = _rand(rng, (n, 1, 16))
    out, acc = op.prefill(q, k, v, [0, n], 1, 0.125)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    for t in range(n):
        assert abs(acc[t, 0] - (H[n] - H[t + 1])) < 1e-12
        assert abs(acc[t, 1] - (H[n] - H[t + 1])) < 1e-12
    running = np.cumsum(v[:, 0].astype(np.float64), axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(out[:, 0], running, atol=1e-12)


def test_mass_and_edges():
    # each row sums to one, so the column sums total n - sum of the diagonal; the first query
    # puts all of its mass on itself, the last token receives nothing, an empty request is empty
    rng = np.random.default_rng(2)
    cu = [0, 0, 33, 34]
    q, k, v = _rand(rng, (34, 3, 32)), _rand(rng, (34, 1, 32)), _rand(rng, (34, 1, 32))
    out, acc = op.prefill(q, k, v, cu, 1, 1 / math.sqrt(32))
    for hq in range(3):
        p = op.causal_rows(q[0:33, hq], k[0:33, 0], 1 / math.sqrt(32))
        assert np.allclose(p.sum(axis=1), 1.0)
        assert abs(acc[0:33, hq].sum() - (33 - np.trace(p))) < 1e-9
        assert acc[32, hq] == 0.0
        assert acc[33, hq] == 0.0                   # single-token request
        assert np.allclose(out[33, hq], v[33, 0].astype(np.float64))
        assert np.allclose(out[0, hq], v[0, 0].astype(np.float64))


def test_rows_against_scipy_softmax():
    rng = np.random.default_rng(3)
    n = 50
    q, k, v = _rand(rng, (n, 4, 64)), _rand(rng, (n, 2, 64)), _rand(rng, (n, 2, 64))
    scale = 1 / 8
    out, _ = op.prefill(q, k, v, [0, n], 2, scale)
    for hq in (0, 3):
        h = hq // 2
        for i in (0, 7, n - 1):
            s = q[i, hq].astype(np.float64) @ k[:i + 1, h].astype(np.float64).T * scale
            w = scipy.special.softmax(s)
            assert np.allclose(out[i, hq], w @ v[:i + 1, h].astype(np.float64), atol=1e-12)


def test_sampled_helpers_match_full():
    rng = np.random.default_rng(4)
    cu = [0, 70, 131]
    q, k, v = _rand(rng, (131, 4, 32)), _rand(rng, (131, 2, 32)), _rand(rng, (131, 2, 32))
    out, acc = op.prefill(q, k, v, cu, 2, 0.2)
    rows = [0, 5, 60]
    assert np.allclose(op.prefill_rows(q, k, v, cu, 2, 0.2, 1, 3, rows), out[70 + np.array(rows), 3],
                       atol=1e-12)
    cols = [0, 1, 30, 60]
    assert np.allclose(op.prefill_colsums(q, k, cu, 2, 0.2, 1, 2, cols), acc[70 + np.array(cols), 2],
                       atol=1e-12)


def test_blocked_head_matches_full_and_closed_form():
    # the row-blocked form (for 32K-token checks) against the unblocked definition on a ragged
    # size that leaves a partial last block, and against the harmonic closed form
    rng = np.random.default_rng(5)
    n = 300
    q, k, v = _rand(rng, (n, 1, 32)), _rand(rng, (n, 1, 32)), _rand(rng, (n, 1, 32))
    out, acc = op.prefill(q, k, v, [0, n], 1, 0.17)
    for block in (1, 64, 77, 1024):
        bo, ba = op.prefill_head(q[:, 0], k[:, 0], v[:, 0], 0.17, block=block)
        assert np.allclose(bo, out[:, 0], atol=1e-12)
        assert np.allclose(ba, acc[:, 0], atol=1e-12)
    kk = np.tile(_rand(rng, (1, 32)), (n, 1))
    _, ba = op.prefill_head(q[:, 0], kk, v[:, 0], 0.17, block=64)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    assert np.allclose(ba, H[n] - H[1:], atol=1e-12)


def test_planted_mistake_is_caught():
    # counting the diagonal (a token's own query) breaks the harmonic closed form
    n = 6
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    p = np.tril(np.ones((n, n))) / np.arange(1, n + 1)[:, None]
    wrong = p.sum(axis=0)
    assert not np.allclose(wrong, H[n] - H[1:])
    assert np.allclose(p.sum(axis=0) - np.diagonal(p), H[n] - H[1:])
