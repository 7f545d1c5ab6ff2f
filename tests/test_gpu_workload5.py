"""Full-model shape on one GPU (MI355X only): 64 layers x 64 requests (lengths log-uniform in
[1K, 32K]) x 64 query / 8 KV heads, compacted layer by layer into one global pool.

* With the literal 2^20-page pool the demand outgrows the pool after a few layers: the
  compaction of that layer must set POOL_EXHAUSTED at the same layer as the oracle and leave
  the pool unchanged (all or nothing), and later calls must be no-ops.
* With 2^24 pages (58 GB) all 64 layers fit: tiers, counts, page table, reverse map and free
  ring are compared with the oracle for every head of every layer; page bytes and decode
  attention on a seeded sample of (layer, request) pairs.
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import pool as opool  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _layer_inputs(w, layer):
    k, v = workloads.make_kv(w, DEV, layer)
    acc = workloads.make_acc(w, None, DEV, layer)
    return k, v, acc


def test_workload5_literal_pool_exhausts_all_or_nothing():
    from mixed_precision_paged_score_amd import kvc, pipeline
    w = workloads.workload(5)
    path = pipeline.PromptPath(w, DEV)           # P = 2^20
    opl = opool.Pool(w.num_layers, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    failed_at = None
    for layer in range(w.num_layers):
        print(f"[w5/2^20] layer {layer}", flush=True)
        k, v, acc = _layer_inputs(w, layer)
        tier, count, _ = parity.oracle_score(w, acc)
        names = ("page_table", "free_ring", "owner", "ring_ctr", "count")
        before = {n: getattr(path.pool, n).clone() for n in names}
        path.prompt(layer, acc, k, v)
        opl.compact(layer, count)
        torch.cuda.synchronize()
        assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
        if opl.status:
            failed_at = layer
            assert path.pool.status() == opl.status == kvc.DEV_POOL_EXHAUSTED
            for n in names:
                assert torch.equal(getattr(path.pool, n), before[n]), n
            # sticky: the next layer is a no-op too
            path.prompt(layer + 1, acc, k, v) if layer + 1 < w.num_layers else None
            torch.cuda.synchronize()
            assert torch.equal(path.pool.ring_ctr, before["ring_ctr"])
            break
        parity.compare_pool(path.pool, opl)
        del k, v, acc
    assert failed_at is not None and 1 <= failed_at < w.num_layers
    print(f"[w5/2^20] exhausted at layer {failed_at} (free pages left "
          f"{opl.tail - opl.head})", flush=True)


def test_workload5_big_pool_all_layers():
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.workload(5, num_pages=1 << 24)
    path = pipeline.PromptPath(w, DEV)
    opl = opool.Pool(w.num_layers, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    rng = np.random.default_rng(w.seed)
    sample_layers = sorted(rng.choice(w.num_layers, 4, replace=False).tolist())
    sample = {l: sorted(rng.choice(w.batch, 8, replace=False).tolist()) for l in sample_layers}
    kept = {}
    for layer in range(w.num_layers):
        print(f"[w5/2^24] layer {layer}", flush=True)
        k, v, acc = _layer_inputs(w, layer)
        tier, count, _ = parity.oracle_score(w, acc)
        path.prompt(layer, acc, k, v)
        opl.compact(layer, count)
        torch.cuda.synchronize()
        assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
        assert path.pool.status() == 0
        if layer in sample:
            cu = w.cu_seqlens()
            for b in sample[layer]:
                lo, hi = int(cu[b]), int(cu[b + 1])
                kept[(layer, b)] = (parity.np_(k[lo:hi]), parity.np_(v[lo:hi]), tier[lo:hi])
        del k, v, acc
    parity.compare_pool(path.pool, opl)
    # page bytes and decode attention of the sampled (layer, request) pairs
    ws = dict(w.__dict__)
    for layer in sample_layers:
        q = workloads.make_queries(w, DEV, 0, layer)
        out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
        path.decode(layer, q, out)
        torch.cuda.synchronize()
        qc = parity.np_(q)
        for b in sample[layer]:
            kb, vb, tb = kept[(layer, b)]
            wb = workloads.Workload("one", 1, 1, w.num_q_heads, w.num_kv_heads, [len(tb)],
                                    w.alpha_h, w.alpha_l, w.window, w.num_pages, "zipf")
            for h in range(w.num_kv_heads):
                _compare_request_head(path, layer, b, h, kb, vb, tb, w.row_capacity)
                want = parity.oracle_attention(wb, 0, h, kb, vb, tb, qc[b:b + 1], path.scale)
                G = w.group
                parity.assert_close_attention(parity.np_(out[b, h * G:(h + 1) * G]), want)
    print(f"[w5/2^24] ok: ring head {opl.head}, sampled layers {sample_layers}", flush=True)
    del ws


def _compare_request_head(path, layer, b, h, k, v, tier, C):
    from oracle import place
    imgs = place.head_pages(k[:, h], v[:, h], tier[:, h])
    row = parity.np_(path.pool.page_table[layer, b, h])
    ids = [int(row[p]) for p in range(len(imgs[place.HIGH]))] + \
          [int(row[C - 1 - p]) for p in range(len(imgs[place.LOW]))]
    want = imgs[place.HIGH] + imgs[place.LOW]
    got = parity.np_(path.pool.pages[torch.tensor(ids, device=DEV)])
    for n, (g, e) in enumerate(zip(got, want)):
        assert np.array_equal(g, e), f"layer {layer} head ({b},{h}) page #{n} differs"
