"""Oracle: decode attention over one head's dequantized live tokens (test infra only).

Source: DiffKV review page -- the abstract's memory manager serves attention over the
compressed, paged KV cache, and "Assumptions" lists standard causal multi-head attention
(the page's Eq. 1).  Reading taken: one new query per request attends to every
live cached token of its KV head (all of them precede it, so there is no mask), with
softmax scale 1/sqrt(128); query head hq reads KV head hq // G.  Keys and values are the
float32 reconstructions code*scale + zero.  Accumulation is float64; a head with no live
token yields a zero vector.
"""
import numpy as np


def decode_one(q, k_hat, v_hat, scale):
    """q fp16/float [d]; k_hat, v_hat float32 [n][d] -> float64 [d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v_hat, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[-1], np.float64)
    s = (k @ q) * float(scale)
    m = s.max()
    p = np.exp(s - m)
    return (p @ v) / p.sum()


def decode_group(q_group, k_hat, v_hat, scale):
    """All G query heads of one KV head: q_group [G][d] -> float64 [G][d]."""
    return np.stack([decode_one(qg, k_hat, v_hat, scale) for qg in q_group])
