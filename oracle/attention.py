"""Oracle: decode attention over one head's dequantized live tokens (test infra only).

Source: DiffKV review page -- the abstract's memory manager serves attention over the
compressed, paged KV cache, and "Assumptions" lists standard causal multi-head attention
(the page's Eq. 1).  Reading taken: one new query per request attends to every
live cached token of its KV head (all of them precede it, so there is no mask), with
softmax scale 1/sqrt(128); query head hq reads KV head hq // G.  Keys and values are the
float32 reconstructions code*scale + zero.  Accumulation is float64; a head with no live
token yields a zero vector.

Score accumulation (the same page, "What carries the argument": a token's significance is the
mean of the attention it receives from subsequent tokens): a decode query is a later token for
every cached token, so each of its softmax weights is added to that token's accumulator.
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


def attention_weights(q_group, k_hat, scale):
    """Softmax weights of one decode query per query head over a head's live tokens:
    q_group [G][d], k_hat float32 [n][d] -> float64 [G][n] (rows in k_hat's order)."""
    q = np.asarray(q_group, dtype=np.float64)
    k = np.asarray(k_hat, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], 0), np.float64)
    s = (q @ k.T) * float(scale)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def accumulate(acc, q, k_hat_of, positions_of, cu, num_kv_heads, scale):
    """acc float64 [T][Hq] += every live token's weight from the request's decode query.
    k_hat_of(b, h) -> float32 [n][d] and positions_of(b, h) -> int [n] give one head's live
    tokens in the same order; q [B][Hq][d]."""
    Hq = q.shape[1]
    G = Hq // num_kv_heads
    for b in range(q.shape[0]):
        for h in range(num_kv_heads):
            pos = np.asarray(positions_of(b, h), np.int64)
            w = attention_weights(q[b, h * G:(h + 1) * G], k_hat_of(b, h), scale)
            for g in range(G):
                acc[int(cu[b]) + pos, h * G + g] += w[g]
    return acc
