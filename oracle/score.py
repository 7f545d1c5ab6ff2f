"""Oracle: significance score and three-tier decision (test infrastructure only).

Source: DiffKV review page, "What carries the argument" -- a token's significance is the
average attention score it receives from subsequent tokens, max-aggregated across the GQA
heads that share its KV head, compared with the theoretical average 1/N: at or above
alpha_h/N it is kept at high precision (K8V4), between alpha_l/N and alpha_h/N at low
precision (K4V2), below alpha_l/N it is pruned.  "Core claim": thresholds adjust with
sequence length.  Free-parameter ledger: the most recent W = 64 tokens are always kept at
high precision.  Referee major comment 3: a token leaving the window is irreversibly
demoted or pruned, so a re-tier never promotes.

Readings taken where the page is silent:
  * "subsequent tokens" = strictly later query positions, so token t of a length-N request
    is averaged over cnt = N-1-t queries; the caller supplies the sum (acc_sum), the
    division happens here.
  * the last token (cnt = 0) has score +inf.
  * the threshold base N is the request's current length; a tie goes to the higher tier.
  * arithmetic is float32 with round-to-nearest-even: mean = acc / cnt and th = alpha / N
    are each one correctly rounded float32 division.
"""
import numpy as np

PRUNE, LOW, HIGH, FRESH = 0, 1, 2, 3


def score_tokens(acc_sum, cu_seqlens, num_kv_heads, alpha_h, alpha_l, window,
                 prev_tier=None):
    """Tier every (token, KV head).

    acc_sum    float32 [T][Hq]  -- sum of the softmax weight token t received from strictly
                                   later queries of each query head
    cu_seqlens int      [B+1]   -- request b owns rows cu[b] .. cu[b+1]-1 (positions 0..N-1)
    prev_tier  uint8 [T][Hkv] or None; FRESH (3) marks a token that has no tier yet

    Returns (tier uint8 [T][Hkv], count int32 [B][Hkv][2] = (#HIGH, #LOW),
             changed uint8 [B][Hkv] = 1 where some already-tiered token dropped a tier or a
             fresh token was kept, i.e. where the head's pages are rebuilt).
    """
    acc_sum = np.asarray(acc_sum, dtype=np.float32)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, Hq = acc_sum.shape
    Hkv = int(num_kv_heads)
    assert Hq % Hkv == 0
    G = Hq // Hkv
    B = len(cu) - 1
    tier = np.zeros((T, Hkv), np.uint8)
    count = np.zeros((B, Hkv, 2), np.int32)
    changed = np.zeros((B, Hkv), np.uint8)
    a_h = np.float32(alpha_h)
    a_l = np.float32(alpha_l)
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        N = hi - lo
        if N == 0:
            continue
        th = a_h / np.float32(N)          # one float32 division each
        tl = a_l / np.float32(N)
        t = np.arange(N)
        cnt = (N - 1 - t).astype(np.float32)   # number of strictly later queries
        last = cnt == 0
        safe_cnt = np.where(last, np.float32(1), cnt)
        for h in range(Hkv):
            # mean attention received from each query head of the group (float32 division) ...
            means = acc_sum[lo:hi, h * G:(h + 1) * G] / safe_cnt[:, None]
            # ... max-aggregated over the GQA group; the last token has no later query
            score = np.where(last, np.float32(np.inf), means.max(axis=1))
            x = np.where(score >= th, HIGH, np.where(score >= tl, LOW, PRUNE)).astype(np.uint8)
            x[t >= N - int(window)] = HIGH       # recent window: always high precision
            if prev_tier is not None:
                p = np.asarray(prev_tier[lo:hi, h], dtype=np.uint8)
                tiered = p != FRESH
                # the head must be rebuilt if a tiered token drops or a fresh one is kept
                if np.any(tiered & (x < p)) or np.any(~tiered & (x != PRUNE)):
                    changed[b, h] = 1
                x = np.where(tiered, np.minimum(x, p), x).astype(np.uint8)   # never promote
            tier[lo:hi, h] = x
            count[b, h, 0] = int(np.sum(x == HIGH))
            count[b, h, 1] = int(np.sum(x == LOW))
    return tier, count, changed
