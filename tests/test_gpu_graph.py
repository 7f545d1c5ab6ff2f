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


def test_generation_loop_graph_replays_match_eager():
    # the generation loop of one layer (decode with score accumulation into a padded buffer,
    # then the per-step policy, positions advancing on the device) captured once and replayed
    # from restored state three times: pools, accumulators, outputs and decisions bit for bit
    # equal to an eager run of the same steps
    from mixed_precision_paged_score_amd import kvc, pipeline
    w = workloads.Workload("graph-gen", 1, 3, 16, 4, [300, 70, 517], 1.0, 0.2, 16, 2048, "zipf",
                           seed=71)
    steps = 12
    k, v = workloads.make_kv(w, DEV)
    acc = workloads.make_acc(w, k, DEV)
    paths = []
    for _ in range(2):
        p = pipeline.GenerationPath(w, max(w.seqlens) + steps, DEV)
        p.pool.pages.zero_()
        p.prompt(0, acc, k, v)
        paths.append(p)
    ga, gb = paths
    cap = ga.seqlen_cap
    cu_pad = ga.padded_cu()
    cu = w.cu_seqlens()
    accs = []
    for _ in range(2):
        a = torch.zeros((w.batch * cap, w.num_q_heads), dtype=torch.float32, device=DEV)
        for b, n in enumerate(w.seqlens):
            a[b * cap:b * cap + n] = acc[int(cu[b]):int(cu[b + 1])]
        accs.append(a)
    qs = [workloads.make_queries(w, DEV, 40 + s) for s in range(steps)]
    g = torch.Generator(device=DEV).manual_seed(72)
    kn = [torch.randn((w.batch, w.num_kv_heads, 128), generator=g, device=DEV).to(torch.float16)
          for _ in range(steps)]
    vn = [torch.randn((w.batch, w.num_kv_heads, 128), generator=g, device=DEV).to(torch.float16)
          for _ in range(steps)]
    outs = [torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
            for _ in range(2)]
    decs = [torch.empty((steps, w.batch, w.num_kv_heads), dtype=torch.uint8, device=DEV)
            for _ in range(2)]
    poss = [torch.tensor(w.seqlens, dtype=torch.int32, device=DEV) for _ in range(2)]
    wss = [(kvc.workspace(p.geom, kvc.OP_DECODE_ACC, cap, device=DEV),
            kvc.workspace(p.geom, kvc.OP_GENERATE, device=DEV)) for p in paths]

    def run(j):
        p, a, out, dec, pos, (wsa, wsg) = paths[j], accs[j], outs[j], decs[j], poss[j], wss[j]
        for s in range(steps):
            kvc.paged_decode_attention_acc(p.geom, 0, p.pool, qs[s], p.scale, out, a, cu_pad, cap,
                                           wsa)
            kvc.generation_step(p.geom, 0, p.pool, kn[s], vn[s], pos, a, cu_pad, w.alpha_h,
                                w.alpha_l, w.window, dec[s], wsg)
            pos.add_(1)

    state = [getattr(ga.pool, n) for n in POOL_ARRAYS] + [accs[0], poss[0]]
    snap = [t.clone() for t in state]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(0)
    torch.cuda.synchronize()
    for r in range(3):
        for t, s0 in zip(state, snap):
            t.copy_(s0)
        graph.replay()
        torch.cuda.synchronize()
        if r == 0:
            run(1)                         # the eager reference, once
            torch.cuda.synchronize()
        _same_pool(ga, gb)
        assert torch.equal(accs[0], accs[1]), f"replay {r}: accumulators differ"
        assert torch.equal(outs[0], outs[1]), f"replay {r}: output differs"
        assert torch.equal(decs[0], decs[1]), f"replay {r}: decisions differ"
        assert torch.equal(poss[0], poss[1])
    assert ga.pool.status() == 0
    d = decs[0].cpu()
    print(f"[graph] generation loop ok: {int((d == 1).sum())} demoted, {int((d == 0).sum())} "
          f"pruned over {steps} steps", flush=True)
