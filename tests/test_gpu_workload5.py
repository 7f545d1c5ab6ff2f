"""Full-model shape on one GPU (MI355X only): 64 layers x 64 requests (lengths log-uniform in
[1K, 32K]) x 64 query / 8 KV heads, compacted layer by layer into one global pool.

* With the literal 2^20-page pool the demand outgrows the pool after a few layers: the
  compaction of that layer must set POOL_EXHAUSTED at the same layer as the oracle and leave
  the pool unchanged (all or nothing), and later calls must be no-ops.
* With 2^24 pages (58 GB) all 64 layers fit: tiers, counts, page table, reverse map and free
  ring are compared with the oracle for every head of every layer; after the whole model's
  compaction one decode step runs on every layer, and page bytes and attention are compared on
  two seeded requests of every layer.
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
    """All 64 layers compacted into one 2^24-page pool, then one decode step of every layer.
    Tiers and allocator state of every head of every layer bit-exact; for two seeded requests
    of every layer (all 8 KV heads) every page byte right after the layer's round, the same
    pages again (by digest) once all layers are placed, and the attention of all their query
    heads in the decode that follows the whole compaction."""
    import hashlib
    from oracle import attention as oatt, place
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.workload(5, num_pages=1 << 24)
    path = pipeline.PromptPath(w, DEV)
    opl = opool.Pool(w.num_layers, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    rng = np.random.default_rng(w.seed)
    sample = {l: sorted(rng.choice(w.batch, 2, replace=False).tolist())
              for l in range(w.num_layers)}
    C, G = w.row_capacity, w.group
    cu = w.cu_seqlens()
    expect = {}             # (layer, b, h) -> (page ids, digest of the oracle's page images)
    expect_o = {}           # (layer, b) -> oracle attention [Hq][128]
    for layer in range(w.num_layers):
        k, v, acc = _layer_inputs(w, layer)
        tier, count, _ = parity.oracle_score(w, acc)
        path.prompt(layer, acc, k, v)
        opl.compact(layer, count)
        torch.cuda.synchronize()
        assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
        assert path.pool.status() == 0
        q = parity.np_(workloads.make_queries(w, DEV, 0, layer))
        for b in sample[layer]:
            lo, hi = int(cu[b]), int(cu[b + 1])
            kb, vb, tb = parity.np_(k[lo:hi]), parity.np_(v[lo:hi]), tier[lo:hi]
            want_o = np.zeros((w.num_q_heads, 128))
            for h in range(w.num_kv_heads):
                imgs = place.head_pages(kb[:, h], vb[:, h], tb[:, h])
                row = parity.np_(path.pool.page_table[layer, b, h])
                ids = [int(row[p]) for p in range(len(imgs[place.HIGH]))] + \
                      [int(row[C - 1 - p]) for p in range(len(imgs[place.LOW]))]
                want = imgs[place.HIGH] + imgs[place.LOW]
                if ids:
                    got = parity.np_(path.pool.pages[torch.tensor(ids, device=DEV)])
                    for n, (gp, e) in enumerate(zip(got, want)):
                        assert np.array_equal(gp, e), \
                            f"layer {layer} head ({b},{h}) page #{n} differs"
                    expect[(layer, b, h)] = (ids, hashlib.sha256(np.stack(want).tobytes()).digest())
                kd, vd = place.head_dequantized(kb[:, h], vb[:, h], tb[:, h])
                want_o[h * G:(h + 1) * G] = oatt.decode_group(q[b, h * G:(h + 1) * G], kd, vd,
                                                              path.scale)
            expect_o[(layer, b)] = want_o
        print(f"[w5/2^24] layer {layer}: round ok, requests {sample[layer]} "
              f"(lengths {[w.seqlens[b] for b in sample[layer]]}) pages ok", flush=True)
        del k, v, acc
    parity.compare_pool(path.pool, opl)
    for (layer, b, h), (ids, dig) in expect.items():
        got = parity.np_(path.pool.pages[torch.tensor(ids, device=DEV)])
        assert hashlib.sha256(got.tobytes()).digest() == dig, f"layer {layer} head ({b},{h})"
    # the decode step of every layer, after the whole model's compaction
    out = torch.empty((w.num_layers, w.batch, w.num_q_heads, 128), dtype=torch.float32,
                      device=DEV)
    for layer in range(w.num_layers):
        path.decode(layer, workloads.make_queries(w, DEV, 0, layer), out[layer])
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    got = parity.np_(out)
    assert np.all(np.isfinite(got))
    worst = 0.0
    for (layer, b), want_o in expect_o.items():
        worst = max(worst, parity.assert_close_attention(got[layer, b], want_o))
    print(f"[w5/2^24] ok: ring head {opl.head}, decode of all {w.num_layers} layers, "
          f"{len(expect_o)} (layer, request) pairs within tolerance (max err {worst:.2e})",
          flush=True)
