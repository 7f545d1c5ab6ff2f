"""Oracle: causal prefill attention and the prompt's significance accumulators (test
infrastructure only; nothing in the library imports it).

Source: DiffKV review page.  "Assumptions" lists standard causal multi-head attention (the
page's Eq. 1); "What carries the argument" defines a token's significance as the mean of the
attention it receives from subsequent tokens, and the referee report (major comment 2) counts
those as the N - i later queries.  The accumulators the scoring step reads are the sums of
those weights, so the step before the path is the prompt's own causal attention, which also
emits, for every key token, the sum of its softmax weights over strictly later queries.

Readings taken: per request and query head hq (KV head hq // G), row i of the softmax runs
over keys j <= i of the same request with logits q_i . k_j * scale; the output row is
sum_j p_ij v_j; acc[t][hq] = sum over i > t of p_it (the token's own query is not a later
one).  Everything in float64 from the fp16 inputs.
"""
import numpy as np


def causal_rows(q, k, scale):
    """Softmax rows of one request and query head: q, k [n][d] -> float64 [n][n], row i over
    columns 0..i (zeros above the diagonal)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    s = (q @ k.T) * float(scale)
    s[np.triu_indices(n, 1)] = -np.inf
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def prefill(q, k, v, cu, num_kv_heads, scale):
    """q fp16 [T][Hq][d], k and v fp16 [T][Hkv][d], cu [B+1] -> (out float64 [T][Hq][d],
    acc float64 [T][Hq])."""
    T, Hq, d = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((T, Hq, d), np.float64)
    acc = np.zeros((T, Hq), np.float64)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        for hq in range(Hq):
            h = hq // G
            p = causal_rows(q[lo:hi, hq], k[lo:hi, h], scale)
            out[lo:hi, hq] = p @ np.asarray(v[lo:hi, h], dtype=np.float64)
            acc[lo:hi, hq] = p.sum(axis=0) - np.diagonal(p)
    return out, acc


def prefill_rows(q, k, v, cu, num_kv_heads, scale, b, hq, rows):
    """Output rows `rows` (positions within request b) of query head hq, float64 [len][d]:
    for sampled checks at sizes where the full prefill is too slow."""
    lo = int(cu[b])
    G = q.shape[1] // num_kv_heads
    h = hq // G
    res = []
    for i in rows:
        qi = np.asarray(q[lo + i, hq], dtype=np.float64)
        kk = np.asarray(k[lo:lo + i + 1, h], dtype=np.float64)
        s = (kk @ qi) * float(scale)
        p = np.exp(s - s.max())
        res.append((p @ np.asarray(v[lo:lo + i + 1, h], dtype=np.float64)) / p.sum())
    return np.stack(res)


def prefill_colsums(q, k, cu, num_kv_heads, scale, b, hq, cols):
    """acc of positions `cols` of request b, query head hq (float64 [len]): each later query's
    softmax row is computed on its own, for sampled checks."""
    lo, hi = int(cu[b]), int(cu[b + 1])
    n = hi - lo
    G = q.shape[1] // num_kv_heads
    h = hq // G
    kk = np.asarray(k[lo:hi, h], dtype=np.float64)
    qq = np.asarray(q[lo:hi, hq], dtype=np.float64)
    cols = np.asarray(cols, np.int64)
    res = np.zeros(len(cols), np.float64)
    first = int(cols.min()) + 1 if len(cols) else n
    for i in range(first, n):
        s = (kk[:i + 1] @ qq[i]) * float(scale)
        p = np.exp(s - s.max())
        p /= p.sum()
        sel = cols < i
        res[sel] += p[cols[sel]]
    return res


def prefill_head(q, k, v, scale, block=1024):
    """One request and query head, the same definition as prefill() taken a block of query rows
    at a time so that no n x n matrix is held: q, k, v [n][d] -> (out float64 [n][d],
    acc float64 [n]).  Row i's softmax runs over keys 0..i; acc[t] sums p_it over rows i > t."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    out = np.zeros((n, q.shape[1]), np.float64)
    acc = np.zeros(n, np.float64)
    for i0 in range(0, n, block):
        i1 = min(n, i0 + block)
        s = (q[i0:i1] @ k[:i1].T) * float(scale)              # rows i0..i1-1, keys 0..i1-1
        rows = np.arange(i0, i1)[:, None]
        s[np.arange(i1)[None, :] > rows] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[i0:i1] = p @ v[:i1]
        p[np.arange(i1 - i0), np.arange(i0, i1)] = 0.0         # a token's own query
        acc[:i1] += p.sum(axis=0)
    return out, acc
