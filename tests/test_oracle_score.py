"""Pins of the oracle's score/tier step against the page's definitions, special cases and
hand-worked values (DiffKV review page: 'What carries the argument', free-parameter
ledger, referee major comments 2-3)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import score as osc
from mixed_precision_paged_score_amd import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "score_tiny.json")) as f:
        return json.load(f)


def test_hand_worked_example():
    g = _gold()
    acc = np.array(g["acc_sum"], np.float32)
    tier, count, changed = osc.score_tokens(acc, g["cu_seqlens"], g["num_kv_heads"],
                                            g["alpha_h"], g["alpha_l"], g["window"])
    assert tier.tolist() == g["tier"]
    assert count.tolist() == g["count"]
    assert changed.tolist() == [[0, 0]]


def test_hand_worked_example_monotone_retier():
    g = _gold()
    acc = np.array(g["acc_sum"], np.float32)
    prev = np.array(g["prev_tier"], np.uint8)
    tier, count, changed = osc.score_tokens(acc, g["cu_seqlens"], g["num_kv_heads"],
                                            g["alpha_h"], g["alpha_l"], g["window"], prev)
    assert tier.tolist() == g["tier_with_prev"]
    assert count.tolist() == g["count_with_prev"]
    assert changed.tolist() == g["changed_with_prev"]


def _random_case(seed, n=37, hq=8, hkv=2):
    rng = np.random.default_rng(seed)
    acc = (rng.random((n, hq)) * 0.2 * np.arange(n - 1, -1, -1)[:, None]).astype(np.float32)
    return acc, [0, n], hkv


def test_alpha_l_zero_never_prunes():
    # free-parameter ledger: alpha_l = 0 for most models -> nothing below the low threshold
    for seed in range(5):
        acc, cu, hkv = _random_case(seed)
        tier, _, _ = osc.score_tokens(acc, cu, hkv, 1.0, 0.0, 4)
        assert not np.any(tier == osc.PRUNE)


def test_alpha_l_equal_alpha_h_has_no_low_tier():
    # the "K8V4-Prune" configuration named in referee minor comment 5
    for seed in range(5):
        acc, cu, hkv = _random_case(seed)
        tier, count, _ = osc.score_tokens(acc, cu, hkv, 1.0, 1.0, 4)
        assert not np.any(tier == osc.LOW)
        assert np.all(count[..., 1] == 0)


def test_infinite_thresholds_keep_only_window_and_last():
    acc, cu, hkv = _random_case(3)
    n = cu[1]
    tier, _, _ = osc.score_tokens(acc, cu, hkv, np.inf, np.inf, 5)
    assert np.all(tier[n - 5:] == osc.HIGH)
    assert np.all(tier[:n - 5] == osc.PRUNE)


def test_window_covering_everything_is_all_high():
    acc, cu, hkv = _random_case(4)
    tier, count, _ = osc.score_tokens(acc, cu, hkv, 1e9, 1e9, 10 ** 6)
    assert np.all(tier == osc.HIGH)
    assert np.all(count[..., 0] == cu[1])


def test_zero_window_last_token_still_high():
    # the last token has no later query: score +inf, HIGH even without a window
    acc, cu, hkv = _random_case(5)
    tier, _, _ = osc.score_tokens(acc, cu, hkv, 1e9, 0.0, 0)
    assert np.all(tier[-1] == osc.HIGH)
    assert np.all(tier[:-1] == osc.LOW)


@pytest.mark.parametrize("k", [3, 6, 9])
def test_exact_tie_at_one_over_n_goes_high(k):
    # N = 2^k and acc = cnt * 2^-k exactly: every mean equals 1/N = alpha_h/N
    n = 2 ** k
    cnt = np.arange(n - 1, -1, -1, dtype=np.float64)
    acc = np.repeat((cnt * 2.0 ** -k)[:, None], 4, axis=1).astype(np.float32)
    tier, _, _ = osc.score_tokens(acc, [0, n], 2, 1.0, 0.0, 0)
    assert np.all(tier == osc.HIGH)
    # one ulp below the tie drops to LOW
    below = np.nextafter(acc, np.float32(0), dtype=np.float32)
    below[-1] = 0
    tier, _, _ = osc.score_tokens(below, [0, n], 2, 1.0, 0.0, 0)
    assert np.all(tier[:-1] == osc.LOW)


def test_group_max_is_max_over_query_heads():
    # G = 1 is the identity; with G > 1 one hot query head lifts the whole group
    n, hkv, G = 16, 2, 4
    acc = np.zeros((n, hkv * G), np.float32)
    acc[3, 1 * G + 2] = 100.0     # KV head 1, query head 2 of its group
    tier, _, _ = osc.score_tokens(acc, [0, n], hkv, 1.0, 0.5, 0)
    assert tier[3, 1] == osc.HIGH and tier[3, 0] == osc.PRUNE
    # permuting query heads inside a group does not change tiers
    rng = np.random.default_rng(0)
    acc2 = (rng.random((n, hkv * G)) * 2).astype(np.float32)
    perm = np.concatenate([h * G + rng.permutation(G) for h in range(hkv)])
    t1, _, _ = osc.score_tokens(acc2, [0, n], hkv, 1.0, 0.5, 2)
    t2, _, _ = osc.score_tokens(acc2[:, perm], [0, n], hkv, 1.0, 0.5, 2)
    assert np.array_equal(t1, t2)


def test_power_of_two_scale_invariance():
    # scaling accumulators and both alphas by 2 is exact in float32: same tiers
    acc, cu, hkv = _random_case(7)
    t1, _, _ = osc.score_tokens(acc, cu, hkv, 1.0, 0.25, 3)
    t2, _, _ = osc.score_tokens(acc * np.float32(2), cu, hkv, 2.0, 0.5, 3)
    assert np.array_equal(t1, t2)


def test_ragged_batch_is_per_request():
    # each request is tiered with its own N; concatenation changes nothing
    rng = np.random.default_rng(11)
    lens = [5, 0, 12, 1, 30]
    accs = [(rng.random((n, 4)) * 3).astype(np.float32) for n in lens]
    cu = np.concatenate([[0], np.cumsum(lens)])
    tier, count, _ = osc.score_tokens(np.concatenate(accs), cu, 2, 1.0, 0.3, 2)
    for b, n in enumerate(lens):
        tb, cb, _ = osc.score_tokens(accs[b], [0, n], 2, 1.0, 0.3, 2)
        assert np.array_equal(tier[cu[b]:cu[b + 1]], tb)
        assert np.array_equal(count[b], cb[0])


def test_causal_accumulator_brute_force():
    # the accumulator recipe: for every token, the sum over strictly later query positions
    # of its softmax weight, recomputed with explicit loops in float64
    w = workloads.Workload("tiny", 1, 1, 4, 2, [9], 1.0, 0.2, 2, 64, "causal", seed=5)
    k, _ = workloads.make_kv(w)
    acc = workloads.make_acc(w, k).numpy()
    # regenerate the same queries the recipe drew
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed * 1000 + 300)
    qp = torch.randn((9, 4, 128), generator=g, dtype=torch.float32).to(torch.float16)
    qp = qp.double().numpy()
    kk = k.double().numpy()
    for hq in range(4):
        h = hq // 2
        for t in range(9):
            total = 0.0
            for i in range(t + 1, 9):
                logits = [float(np.dot(qp[i, hq], kk[j, h])) / math.sqrt(128) for j in range(i + 1)]
                mx = max(logits)
                den = sum(math.exp(x - mx) for x in logits)
                total += math.exp(logits[t] - mx) / den
            assert abs(acc[t, hq] - total) <= 1e-6 * max(1.0, total)
    # the mean is at most 1 and the last token receives nothing
    assert np.all(acc[-1] == 0)
