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
