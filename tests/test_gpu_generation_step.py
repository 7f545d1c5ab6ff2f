"""Per-step generation policy on the GPU (kvc_generation_step) vs the oracle's Generation.step
(MI355X only): every step appends one token per (request, KV head) and gives the token that
leaves the recent window its tier from that step's accumulators.  The decisions are compared
every step; the allocator state and the page images of the tracked heads bit-exactly every
`check_every` steps and at the end; decode attention over the final state within the
attention tolerance (2e-3 max-abs, 1e-3 relative L2)."""
import dataclasses
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import attention as oatt, generation as ogen  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402
from test_gpu_generation import _compare_heads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_steps(w, steps, sample_heads=None, check_every=1, acc_device="cpu", scheme=None):
    """scheme: (HIGH format, LOW format) names, or None for the default layout."""
    from mixed_precision_paged_score_amd import pipeline, kvc
    from oracle import scheme as osch
    print(f"[step] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"prompt={w.seqlens[:6]} W={w.window} alpha=({w.alpha_h},{w.alpha_l}) steps={steps} "
          f"P={w.num_pages} scheme={scheme}", flush=True)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    path = pipeline.GenerationPath(w, max(w.seqlens) + steps, DEV,
                                   scheme=kvc.make_scheme(*scheme) if scheme else None)
    path.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    tier0, _, _ = parity.oracle_score(w, acc)
    if isinstance(sample_heads, int):
        rng = np.random.default_rng(w.seed)
        allh = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
        sample_heads = [allh[i] for i in rng.choice(len(allh), sample_heads, replace=False)]
    gen = ogen.Generation(w.batch, w.num_kv_heads, path.geom.row_capacity, path.geom.num_pages,
                          track=sample_heads,
                          scheme=osch.Scheme.named(*scheme) if scheme else None)
    gen.prompt(k.numpy(), v.numpy(), tier0, w.cu_seqlens())
    g = torch.Generator().manual_seed(w.seed + 77)
    seen = np.zeros(256, np.int64)
    for s in range(steps):
        kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
        vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
        ws = dataclasses.replace(w, seqlens=[n + 1 for n in path.lens],
                                 seed=w.seed + 1000 * (s + 1))
        acc_s = workloads.make_acc_zipf(ws, acc_device)
        path.step(0, kn.to(DEV), vn.to(DEV), acc_s.to(DEV))
        dec_o = gen.step(kn.numpy(), vn.numpy(), acc_s.cpu().numpy(), w.alpha_h, w.alpha_l,
                         w.window)
        dec_g = parity.np_(path.decided)
        if not np.array_equal(dec_g, dec_o):
            bad = np.argwhere(dec_g != dec_o)
            raise AssertionError(f"step {s}: {len(bad)} decisions differ, first {bad[:4].tolist()}")
        seen += np.bincount(dec_o.ravel(), minlength=256)
        if (s + 1) % check_every == 0:
            assert path.pool.status() == 0, f"step {s}: status {path.pool.status()}"
            parity.compare_pool(path.pool, gen.pool)
            _compare_heads(w, path, gen, sample_heads)
            assert np.array_equal(parity.np_(path.packed_state()),
                                  np.concatenate(gen.tiers)), f"step {s}: tier state"
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    parity.compare_pool(path.pool, gen.pool)
    _compare_heads(w, path, gen, sample_heads)
    q = workloads.make_queries(w, "cpu", 5)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    path.decode(0, q.to(DEV), out)
    torch.cuda.synchronize()
    G = w.group
    heads = sample_heads or [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    for (b, h) in heads:
        kd, vd = gen.head_dequantized(b, h)
        want = oatt.decode_group(q.numpy()[b, h * G:(h + 1) * G], kd, vd, path.scale)
        parity.assert_close_attention(parity.np_(out[b, h * G:(h + 1) * G]), want)
    counts = {name: int(seen[t]) for name, t in
              (("high", kvc.HIGH), ("low", kvc.LOW), ("pruned", kvc.PRUNE),
               ("none", kvc.NO_TOKEN))}
    print(f"[step] ok: {counts}, ring head {gen.pool.head}", flush=True)
    return counts


def test_ragged_short_and_empty_prompts():
    # a request with no prompt and one shorter than the window: no token leaves the window
    # for their first steps; HIGH pages fill and LOW pages open during the run
    w = workloads.Workload("step-ragged", 1, 4, 16, 4, [300, 0, 9, 517], 1.0, 0.2, 16, 2048,
                           "zipf", seed=51)
    c = run_steps(w, steps=80)
    assert min(c["high"], c["low"], c["pruned"], c["none"]) > 0, c


@pytest.mark.parametrize("window,hq,hkv,alpha_l", [(1, 8, 8, 0.5), (64, 16, 2, 0.5),
                                                   (112, 32, 4, 0.3)])
def test_windows_and_group_sizes(window, hq, hkv, alpha_l):
    # window 1 (the previous token is scored), the 64-token window, the largest window (the
    # rewritten HIGH tail spans 8 pages); group sizes 1, 8 and 8
    w = workloads.Workload(f"step-w{window}", 1, 3, hq, hkv, [200, 129, 64], 1.0, alpha_l,
                           window, 4096, "zipf", seed=52 + window)
    c = run_steps(w, steps=70, check_every=7)
    assert c["low"] > 0 and c["pruned"] > 0, c


def test_exhausted_pool_changes_nothing():
    # a pool with no free page: the first step that needs one sets KVC_DEV_POOL_EXHAUSTED and
    # leaves pages, table, counts and ring as they were.  Zero thresholds keep every token
    # HIGH, so request 0's 64 tokens fill four HIGH pages per head and its new token needs a
    # fifth.
    from mixed_precision_paged_score_amd import pipeline, kvc
    w = workloads.Workload("step-full", 1, 2, 16, 4, [64, 47], 0.0, 0.0, 16, 4096, "zipf",
                           seed=53)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    tier0, count0, _ = parity.oracle_score(w, acc)
    need = int(sum(-(-int(c[0]) // 16) + -(-int(c[1]) // 32) for c in count0.reshape(-1, 2)))
    wf = dataclasses.replace(w, num_pages=need)
    path = pipeline.GenerationPath(wf, max(w.seqlens) + 4, DEV, num_pages=need)
    path.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    before = [parity.np_(t).copy() for t in (path.pool.pages, path.pool.page_table,
                                             path.pool.count, path.pool.free_ring,
                                             path.pool.ring_ctr)]
    g = torch.Generator().manual_seed(5)
    kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
    ws = dataclasses.replace(w, seqlens=[n + 1 for n in w.seqlens], seed=w.seed + 1)
    path.step(0, kn.to(DEV), kn.to(DEV), workloads.make_acc_zipf(ws).to(DEV))
    torch.cuda.synchronize()
    assert path.pool.status() & kvc.DEV_POOL_EXHAUSTED
    after = [parity.np_(t) for t in (path.pool.pages, path.pool.page_table, path.pool.count,
                                     path.pool.free_ring, path.pool.ring_ctr)]
    for x, y in zip(before, after):
        assert np.array_equal(x, y)


def test_more_heads_than_one_scan_tile():
    # 40 requests x 8 KV heads = 320 heads: more than one workgroup's worth, so the step takes
    # the general path (separate decision launch and the three allocation launches) rather
    # than the fused one used up to 256 heads
    rng = np.random.default_rng(58)
    lens = [int(x) for x in rng.integers(20, 160, 40)]
    w = workloads.Workload("step-wide", 1, 40, 16, 8, lens, 1.0, 0.3, 16, 8192, "zipf", seed=58)
    c = run_steps(w, steps=40, sample_heads=8, check_every=10)
    assert c["low"] > 0 and c["pruned"] > 0, c


def test_workload4_shape_sampled():
    # 16 requests x 4096-token prompts, 64 query / 8 KV heads, the 64-token window: 512 steps
    # of the per-step policy; decisions of all 128 heads every step, allocator state every 64
    # steps, codes and attention on 6 sampled heads
    w = workloads.workload(4)
    run_steps(w, steps=512, sample_heads=6, check_every=64, acc_device=DEV)


def test_decode_acc_padded_layout_matches_packed():
    # the accumulating decode over a padded [B][cap][Hq] buffer (cu = b * cap) adds the same
    # values, bit for bit, as over the packed [T][Hq] layout, and leaves the padding rows as
    # they were
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.Workload("acc-pad", 1, 3, 16, 4, [300, 1, 517], 1.0, 0.2, 16, 2048, "zipf",
                           seed=54)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    path = pipeline.GenerationPath(w, max(w.seqlens) + 40, DEV)
    path.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    cap = path.seqlen_cap
    packed = torch.zeros((path.T, w.num_q_heads), dtype=torch.float32, device=DEV)
    padded = torch.zeros((w.batch * cap, w.num_q_heads), dtype=torch.float32, device=DEV)
    for b, n in enumerate(w.seqlens):
        padded[b * cap + n:(b + 1) * cap] = 0.25         # padding rows: must stay as they are
    out_a = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    out_b = torch.empty_like(out_a)
    for s in range(2):
        q = workloads.make_queries(w, DEV, s)
        path.decode_acc(0, q, out_a, packed)
        path.decode_acc(0, q, out_b, padded, cu=path.padded_cu())
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    assert torch.equal(out_a, out_b)
    cu = w.cu_seqlens()
    for b, n in enumerate(w.seqlens):
        assert torch.equal(padded[b * cap:b * cap + n], packed[int(cu[b]):int(cu[b + 1])]), b
        assert torch.all(padded[b * cap + n:(b + 1) * cap] == 0.25)


def test_full_loop_on_padded_accumulators():
    # the per-step loop of one layer as a caller runs it: decode attention with score
    # accumulation into one padded buffer, then the policy step reading the same buffer.  The
    # oracle's step gets the same accumulator values (read back), so decisions, allocator state
    # and pages must agree bit for bit; the decode output agrees with the oracle's attention
    # over its state before each step.
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.Workload("loop-pad", 1, 3, 16, 4, [300, 5, 200], 1.0, 0.2, 16, 2048, "zipf",
                           seed=55)
    steps = 60
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    path = pipeline.GenerationPath(w, max(w.seqlens) + steps, DEV)
    path.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    cap = path.seqlen_cap
    cu_pad = path.padded_cu()
    acc_pad = torch.zeros((w.batch * cap, w.num_q_heads), dtype=torch.float32, device=DEV)
    cu = w.cu_seqlens()
    for b, n in enumerate(w.seqlens):
        acc_pad[b * cap:b * cap + n] = acc[int(cu[b]):int(cu[b + 1])].to(DEV)
    tier0, _, _ = parity.oracle_score(w, acc)
    gen = ogen.Generation(w.batch, w.num_kv_heads, path.geom.row_capacity, path.geom.num_pages)
    gen.prompt(k.numpy(), v.numpy(), tier0, cu)
    g = torch.Generator().manual_seed(56)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    G = w.group
    seen = np.zeros(256, np.int64)
    for s in range(steps):
        q = workloads.make_queries(w, "cpu", 100 + s)
        kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
        vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
        path.decode_acc(0, q.to(DEV), out, acc_pad, cu=cu_pad)
        if s % 10 == 0:
            torch.cuda.synchronize()
            for b in range(w.batch):
                for h in range(w.num_kv_heads):
                    kd, vd = gen.head_dequantized(b, h)
                    want = oatt.decode_group(q.numpy()[b, h * G:(h + 1) * G], kd, vd, path.scale)
                    parity.assert_close_attention(parity.np_(out[b, h * G:(h + 1) * G]), want)
        lens = list(path.lens)
        path.step(0, kn.to(DEV), vn.to(DEV), acc_pad, cu=cu_pad)
        a_np = parity.np_(acc_pad)
        packed = np.concatenate([a_np[b * cap:b * cap + n + 1] for b, n in enumerate(lens)])
        dec_o = gen.step(kn.numpy(), vn.numpy(), packed, w.alpha_h, w.alpha_l, w.window)
        assert np.array_equal(parity.np_(path.decided), dec_o), f"step {s}"
        seen += np.bincount(dec_o.ravel(), minlength=256)
        if (s + 1) % 10 == 0:
            assert path.pool.status() == 0
            parity.compare_pool(path.pool, gen.pool)
            _compare_heads(w, path, gen)
    assert path.pool.status() == 0
    print(f"[loop] decisions high {seen[2]} low {seen[1]} pruned {seen[0]} none {seen[255]}",
          flush=True)
    assert seen[2] > 0 and seen[1] > 0


# ---- precision schemes --------------------------------------------------------------------

@pytest.mark.parametrize("scheme", [("K4V8", "K2V4"), ("K8V2", "K4V1"), ("K2V4", "K4V2")])
def test_scheme_steps_ragged(scheme):
    # the per-step policy on scheme pages: the HIGH tail rewritten in the scheme's layout, the
    # demoted token set into its LOW slot at the LOW widths
    w = workloads.Workload("step-ragged-sch", 1, 4, 16, 4, [300, 0, 9, 517], 1.0, 0.2, 16, 2048,
                           "zipf", seed=61)
    c = run_steps(w, steps=80, check_every=4, scheme=scheme)
    assert min(c["high"], c["low"], c["pruned"]) > 0, c


def test_scheme_steps_largest_window():
    w = workloads.Workload("step-w112-sch", 1, 3, 32, 4, [200, 129, 64], 1.0, 0.3, 112, 4096,
                           "zipf", seed=62)
    c = run_steps(w, steps=70, check_every=7, scheme=("K4V2", "K4V1"))
    assert c["low"] > 0 and c["pruned"] > 0, c
