"""Pins of the oracle decode attention: special cases with closed forms and a library
softmax (scipy) recomputation."""
import numpy as np
from scipy.special import softmax

from oracle import attention as oatt


def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 128)).astype(np.float32)
    k = rng.standard_normal((1, 128)).astype(np.float32)
    q = rng.standard_normal(128).astype(np.float16)
    assert np.array_equal(oatt.decode_one(q, k, v, 0.3), v[0].astype(np.float64))


def test_identical_keys_give_mean_value():
    rng = np.random.default_rng(1)
    k = np.repeat(rng.standard_normal((1, 128)).astype(np.float32), 50, axis=0)
    v = rng.standard_normal((50, 128)).astype(np.float32)
    q = rng.standard_normal(128).astype(np.float16)
    out = oatt.decode_one(q, k, v, 128 ** -0.5)
    assert np.allclose(out, v.astype(np.float64).mean(0), rtol=0, atol=1e-12)


def test_zero_scale_gives_mean_value_and_empty_gives_zero():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((9, 128)).astype(np.float32)
    v = rng.standard_normal((9, 128)).astype(np.float32)
    q = rng.standard_normal(128).astype(np.float16)
    assert np.allclose(oatt.decode_one(q, k, v, 0.0), v.astype(np.float64).mean(0), atol=1e-12)
    assert np.all(oatt.decode_one(q, k[:0], v[:0], 1.0) == 0)


def test_matches_library_softmax():
    rng = np.random.default_rng(3)
    for n in (2, 17, 300):
        k = (rng.standard_normal((n, 128)) * 2).astype(np.float32)
        v = rng.standard_normal((n, 128)).astype(np.float32)
        q = rng.standard_normal((4, 128)).astype(np.float16)
        out = oatt.decode_group(q, k, v, 128 ** -0.5)
        for g in range(4):
            p = softmax(k.astype(np.float64) @ q[g].astype(np.float64) / np.sqrt(128))
            assert np.allclose(out[g], p @ v.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_weights_match_library_softmax_and_output():
    # the accumulated weights are the softmax the output uses: p @ v reproduces decode_group
    rng = np.random.default_rng(4)
    k = (rng.standard_normal((33, 128)) * 3).astype(np.float32)
    v = rng.standard_normal((33, 128)).astype(np.float32)
    q = rng.standard_normal((8, 128)).astype(np.float16)
    w = oatt.attention_weights(q, k, 128 ** -0.5)
    assert w.shape == (8, 33)
    for g in range(8):
        p = softmax(k.astype(np.float64) @ q[g].astype(np.float64) / np.sqrt(128))
        assert np.allclose(w[g], p, rtol=1e-12, atol=1e-15)
    assert np.allclose(w @ v.astype(np.float64), oatt.decode_group(q, k, v, 128 ** -0.5),
                       rtol=1e-12, atol=1e-12)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    assert oatt.attention_weights(q, k[:0], 1.0).shape == (8, 0)


def test_accumulate_adds_one_unit_per_query_head_at_the_right_positions():
    # two requests, two KV heads, G = 2; identical keys share the weight equally
    rng = np.random.default_rng(5)
    cu = np.array([0, 5, 9])
    q = rng.standard_normal((2, 4, 128)).astype(np.float16)
    key = rng.standard_normal(128).astype(np.float32)
    pos = {(0, 0): [0, 3], (0, 1): [1, 2, 4], (1, 0): [], (1, 1): [0, 1, 2, 3]}
    k_of = lambda b, h: np.repeat(key[None], len(pos[(b, h)]), axis=0)  # noqa: E731
    acc = np.zeros((9, 4))
    oatt.accumulate(acc, q, k_of, lambda b, h: pos[(b, h)], cu, 2, 128 ** -0.5)
    want = np.zeros((9, 4))
    for (b, h), ps in pos.items():
        for p in ps:
            want[cu[b] + p, 2 * h:2 * h + 2] = 1.0 / len(ps)
    assert np.allclose(acc, want, rtol=0, atol=1e-15)
