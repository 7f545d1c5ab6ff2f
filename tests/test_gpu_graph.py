"""Captured HIP graphs of the hot path (MI355X only): a prompt round (score, compact in prompt
mode, which returns the layer's previous pages to the ring, quantize/place) and a run of decode
steps are captured once and replayed several times, with
eager work and synchronizations between the replays.  Every replay must leave exactly the
state an eager run with the same history leaves: pool arrays, page bytes and decode outputs
bit for bit (the kernels are deterministic), and the first replay is also checked against the
oracle."""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import pool as opool  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
POOL_ARRAYS = ("pages", "page_table", "count", "owner", "free_ring", "ring_ctr", "dev_status")


def _same_pool(a, b):
    for n in POOL_ARRAYS:
        assert torch.equal(getattr(a.pool, n), getattr(b.pool, n)), n


@pytest.mark.parametrize("wid", [1, 2])
def test_graph_replays_match_eager(wid):
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.workload(wid)
    print(f"[graph] {w.name} B={w.batch} P={w.num_pages}", flush=True)
    k, v = workloads.make_kv(w, DEV)
    acc = workloads.make_acc(w, k, DEV)
    qs = [workloads.make_queries(w, DEV, s) for s in range(3)]
    shape = (w.batch, w.num_q_heads, 128)
    ga, gb = pipeline.PromptPath(w, DEV), pipeline.PromptPath(w, DEV)
    out_a = torch.empty(shape, dtype=torch.float32, device=DEV)
    out_b = torch.empty(shape, dtype=torch.float32, device=DEV)
    # page bytes of never-allocated pages are whatever the allocator left there: clear them
    # so that whole pools compare; then one eager round on both so that the replayed rounds
    # have pages to return
    for p in (ga, gb):
        p.pool.pages.zero_()
        p.prompt(0, acc, k, v)
    torch.cuda.synchronize()
    g_prompt = ga.capture_prompt(0, acc, k, v)
    g_dec = ga.capture_decode(0, qs, out_a)
    torch.cuda.synchronize()
    _same_pool(ga, gb)                     # capturing ran nothing
    for r in range(3):
        g_prompt.replay()
        gb.prompt(0, acc, k, v)
        torch.cuda.synchronize()
        _same_pool(ga, gb)
        g_dec.replay()
        for q in qs:
            gb.decode(0, q, out_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"replay {r}: decode output differs"
        # eager work between replays on the graph's own path: a decode with another query
        ga.decode(0, qs[0], out_b)
        gb.decode(0, qs[0], out_b)
        torch.cuda.synchronize()
        if r == 0:
            tier, count, _ = parity.oracle_score(w, acc)
            opl = opool.Pool(w.num_layers, w.batch, w.num_kv_heads, w.row_capacity,
                             w.num_pages)
            opl.compact(0, count)      # first eager round
            opl.compact(0, count)      # the replayed round
            parity.compare_pool(ga.pool, opl)
    assert ga.pool.status() == 0
    print(f"[graph] ok: 3 replays match eager", flush=True)
