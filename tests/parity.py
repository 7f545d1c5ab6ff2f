"""Parity helpers: run the oracle on the same seeded inputs the HIP path received and compare
element by element (shared by the GPU tests, smoke() and nothing else)."""
import numpy as np
import torch

from oracle import attention as oatt, place, pool as opool, score as osc

ATOL, RTOL_L2 = 2e-3, 1e-3


def np_(t):
    return t.detach().cpu().numpy()


def oracle_score(w, acc, prev_tier=None):
    return osc.score_tokens(np_(acc) if torch.is_tensor(acc) else acc, w.cu_seqlens(),
                            w.num_kv_heads, w.alpha_h, w.alpha_l, w.window, prev_tier)


def compare_pool(gpu_pool, opl, layer=None):
    """Bit-exact comparison of page table, counts, reverse map, ring and counters."""
    rows = np_(gpu_pool.page_table)
    cnt = np_(gpu_pool.count)
    if layer is None:
        assert np.array_equal(rows, opl.rows), "page table differs"
        assert np.array_equal(cnt, opl.count), "counts differ"
    else:
        assert np.array_equal(rows[layer], opl.rows[layer]), "page table differs"
        assert np.array_equal(cnt[layer], opl.count[layer]), "counts differ"
    assert np.array_equal(np_(gpu_pool.owner), opl.owner), "owner map differs"
    ctr = np_(gpu_pool.ring_ctr)
    assert int(ctr[0]) == opl.head and int(ctr[1]) == opl.tail, "ring counters differ"
    P = opl.P
    n = opl.tail - opl.head
    ring = np_(gpu_pool.free_ring)
    idx = (opl.head + np.arange(n)) % P
    assert np.array_equal(ring[idx], opl.ring[idx]), "free ring differs"
    assert gpu_pool.status() == opl.status, f"status {gpu_pool.status()} vs {opl.status}"


def compare_head_pages(w, gpu_pool, layer, b, h, k, v, tier):
    """Every byte of every page of head (b, h) against the oracle's page images."""
    cu = w.cu_seqlens()
    lo, hi = int(cu[b]), int(cu[b + 1])
    imgs = place.head_pages(k[lo:hi, h], v[lo:hi, h], tier[lo:hi, h])
    row = np_(gpu_pool.page_table[layer, b, h])
    C = w.row_capacity
    ids = [int(row[p]) for p in range(len(imgs[place.HIGH]))] + \
          [int(row[C - 1 - p]) for p in range(len(imgs[place.LOW]))]
    want = imgs[place.HIGH] + imgs[place.LOW]
    if not ids:
        return 0
    got = np_(gpu_pool.pages[torch.tensor(ids, device=gpu_pool.pages.device)])
    for n, (g, e) in enumerate(zip(got, want)):
        if not np.array_equal(g, e):
            bad = np.nonzero(g != e)[0]
            raise AssertionError(f"head ({b},{h}) page #{n} (id {ids[n]}): {len(bad)} bytes "
                                 f"differ, first at {bad[:8].tolist()}: got {g[bad[:8]].tolist()} "
                                 f"want {e[bad[:8]].tolist()}")
    return len(ids)


def oracle_attention(w, b, h, k, v, tier, q, scale):
    cu = w.cu_seqlens()
    lo, hi = int(cu[b]), int(cu[b + 1])
    kd, vd = place.head_dequantized(k[lo:hi, h], v[lo:hi, h], tier[lo:hi, h])
    G = w.group
    return oatt.decode_group(q[b, h * G:(h + 1) * G], kd, vd, scale)


def assert_close_attention(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    assert err.max() <= ATOL, f"max abs error {err.max():.3e}"
    den = np.linalg.norm(want)
    if den > 0:
        rel = np.linalg.norm(got - want) / den
        assert rel <= RTOL_L2, f"relative L2 error {rel:.3e}"
    return float(err.max())
