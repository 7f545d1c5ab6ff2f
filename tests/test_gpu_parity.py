"""HIP path vs oracle, element by element, on seeded inputs (MI355X only)."""
import math
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


def _log(msg):
    print(msg, flush=True)


def _inputs(w, gen_device, layer=0):
    k, v = workloads.make_kv(w, gen_device, layer)
    acc = workloads.make_acc(w, k, gen_device, layer)
    q = workloads.make_queries(w, gen_device, 0, layer)
    return k.to(DEV), v.to(DEV), acc.to(DEV), q.to(DEV)


def run_prompt_and_check(w, gen_device="cpu", sample_heads=None, decode=True):
    from mixed_precision_paged_score_amd import pipeline
    _log(f"[parity] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
         f"lens={w.seqlens[:6]}{'...' if len(w.seqlens) > 6 else ''} W={w.window} "
         f"alpha=({w.alpha_h},{w.alpha_l}) P={w.num_pages}")
    k, v, acc, q = _inputs(w, gen_device)
    path = pipeline.PromptPath(w, DEV)
    path.prompt(0, acc, k, v)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    if decode:
        path.decode(0, q, out)
    torch.cuda.synchronize()
    # tiers and counts
    tier, count, _ = parity.oracle_score(w, acc)
    g_tier = parity.np_(path.tier[:w.total_tokens])
    assert np.array_equal(g_tier, tier), f"tiers differ at {np.argwhere(g_tier != tier)[:5]}"
    assert np.array_equal(parity.np_(path.new_count), count)
    # allocator state
    opl = opool.Pool(w.num_layers, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    opl.compact(0, count)
    parity.compare_pool(path.pool, opl)
    # page bytes and attention
    kc, vc, qc = parity.np_(k), parity.np_(v), parity.np_(q)
    heads = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    if sample_heads is not None and sample_heads < len(heads):
        rng = np.random.default_rng(w.seed)
        heads = [heads[i] for i in rng.choice(len(heads), sample_heads, replace=False)]
    npages = 0
    worst = 0.0
    for (b, h) in heads:
        npages += parity.compare_head_pages(w, path.pool, 0, b, h, kc, vc, tier)
        if decode:
            want = parity.oracle_attention(w, b, h, kc, vc, tier, qc, path.scale)
            G = w.group
            worst = max(worst, parity.assert_close_attention(
                parity.np_(out[b, h * G:(h + 1) * G]), want))
    _log(f"[parity] ok: {len(heads)} heads, {npages} pages bit-exact, attention max err {worst:.2e}")
    return path


def test_workload1_full():
    run_prompt_and_check(workloads.workload(1))


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (16, 2), (32, 2)])
def test_ragged_batch_group_sizes(hq, hkv):
    w = workloads.Workload(f"ragged-{hq}-{hkv}", 1, 5, hq, hkv, [1, 0, 37, 300, 777], 1.0, 0.3,
                           64, 2048, "zipf", seed=hq * 10 + hkv)
    run_prompt_and_check(w)


@pytest.mark.parametrize("ah,al,win", [(1.0, 0.0, 64), (1.0, 1.0, 64), (math.inf, 0.2, 0),
                                       (1.0, 0.2, 0), (1.0, 0.2, 100000), (3.0, 0.04, 16)])
def test_threshold_and_window_edges(ah, al, win):
    w = workloads.Workload("edges", 1, 3, 16, 4, [600, 129, 1000], ah, al, win, 4096, "zipf",
                           seed=7)
    run_prompt_and_check(w)


def test_single_token_and_empty_requests():
    w = workloads.Workload("tiny", 1, 6, 8, 2, [1, 1, 0, 2, 1, 0], 1.0, 0.2, 0, 64, "zipf", seed=3)
    run_prompt_and_check(w)


def test_causal_accumulators_outliers():
    w = workloads.Workload("causal-outliers", 1, 2, 16, 4, [700, 1100], 1.0, 0.25, 64, 4096,
                           "causal", k_outlier_channels=4, k_outlier_factor=8.0, seed=11)
    run_prompt_and_check(w)


def test_fp16_output_matches_fp32_rounded():
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.workload(1)
    k, v, acc, q = _inputs(w, "cpu")
    path = pipeline.PromptPath(w, DEV)
    path.prompt(0, acc, k, v)
    o32 = torch.empty((1, 32, 128), dtype=torch.float32, device=DEV)
    o16 = torch.empty((1, 32, 128), dtype=torch.float16, device=DEV)
    path.decode(0, q, o32)
    path.decode(0, q, o16)
    assert torch.equal(o32.to(torch.float16), o16)


def test_score_prev_tier_monotone():
    from mixed_precision_paged_score_amd import kvc, pipeline
    w = workloads.Workload("retier", 1, 3, 16, 4, [300, 1, 517], 1.0, 0.2, 8, 1024, "zipf", seed=5)
    _, _, acc, _ = _inputs(w, "cpu")
    rng = np.random.default_rng(0)
    prev = rng.integers(0, 4, size=(w.total_tokens, w.num_kv_heads)).astype(np.uint8)
    path = pipeline.PromptPath(w, DEV)
    changed = torch.empty((w.batch, w.num_kv_heads), dtype=torch.uint8, device=DEV)
    prev_d = torch.from_numpy(prev).to(DEV)
    kvc.score_tokens(path.geom, acc, path.cu, path.T, path.max_seqlen, w.alpha_h, w.alpha_l,
                     w.window, path.tier, path.new_count, prev_tier=prev_d, changed=changed)
    tier, count, ch = parity.oracle_score(w, acc, prev)
    assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
    assert np.array_equal(parity.np_(path.new_count), count)
    assert np.array_equal(parity.np_(changed), ch)


def test_pool_exhaustion_is_all_or_nothing():
    from mixed_precision_paged_score_amd import kvc, pipeline
    w = workloads.Workload("exhaust", 1, 4, 16, 4, [800, 900, 1000, 1100], 1.0, 0.2, 64, 300,
                           "zipf", seed=9)
    k, v, acc, q = _inputs(w, "cpu")
    path = pipeline.PromptPath(w, DEV)
    names = ("page_table", "free_ring", "owner", "ring_ctr", "count", "pages")
    before = {n: getattr(path.pool, n).clone() for n in names}
    path.prompt(0, acc, k, v)
    torch.cuda.synchronize()
    assert path.pool.status() & kvc.DEV_POOL_EXHAUSTED
    for n in names:
        assert torch.equal(getattr(path.pool, n), before[n]), f"{n} changed on a failed compaction"
    # sticky: a call that would fit is a no-op until the status is cleared
    path.release(0)
    torch.cuda.synchronize()
    assert torch.equal(path.pool.ring_ctr, before["ring_ctr"])
    tier, count, _ = parity.oracle_score(w, acc)
    opl = opool.Pool(1, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    opl.compact(0, count)
    assert opl.status & opool.ST_POOL_EXHAUSTED
    path.pool.clear_status()


def test_repeated_rounds_recycle_pages_through_the_ring():
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.Workload("recycle", 1, 3, 16, 4, [900, 400, 1500], 1.0, 0.2, 64, 700, "zipf",
                           seed=21)
    k, v, acc, q = _inputs(w, "cpu")
    tier, count, _ = parity.oracle_score(w, acc)
    path = pipeline.PromptPath(w, DEV)
    opl = opool.Pool(1, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    for it in range(4):
        path.release(0)
        opl.compact(0, np.zeros((w.batch, w.num_kv_heads, 2)))
        path.prompt(0, acc, k, v)
        opl.compact(0, count)
        torch.cuda.synchronize()
        parity.compare_pool(path.pool, opl)
        opl.check_invariants()
    assert opl.head > w.num_pages      # the ring wrapped around
    kc, vc = parity.np_(k), parity.np_(v)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            parity.compare_head_pages(w, path.pool, 0, b, h, kc, vc, tier)


def test_row_overflow_sets_status():
    from mixed_precision_paged_score_amd import kvc, pipeline
    w = workloads.Workload("overflow", 1, 1, 4, 4, [200], 1.0, 0.2, 200, 1024, "zipf", seed=1)
    k, v, acc, q = _inputs(w, "cpu")
    path = pipeline.PromptPath(w, DEV)
    path.geom.row_capacity = 5           # 200 HIGH tokens need 13 pages
    path.pool = kvc.Pool(path.geom, DEV)
    path.pool.init()
    path.score(acc)
    path.compact(0)
    torch.cuda.synchronize()
    assert path.pool.status() == kvc.DEV_ROW_OVERFLOW
    assert int(path.pool.ring_ctr[0].item()) == 0


# 16 requests x 8 KV heads give the decode 16 workgroup slots per head.  With every token
# HIGH (alpha_h = 0) the heads of the two 16K-token requests fill all 16 slots and keep their
# slot order, while the heads of the short and empty requests use one or two slots and turn
# their splits by head index; with (1.0, 0.2) the long heads use fewer than 16.  Every head's
# attention must still be the oracle's.
SPLIT_LENS = [16384, 0, 1, 37, 300, 777, 2048, 16384, 5000, 100, 64, 65, 3000, 15, 900, 4000]


@pytest.mark.parametrize("ah,al", [(0.0, 0.0), (1.0, 0.2)])
def test_decode_split_plan_long_and_short_heads(ah, al):
    w = workloads.Workload(f"split-plan-{ah}-{al}", 1, 16, 64, 8, SPLIT_LENS, ah, al, 64,
                           1 << 16, "zipf", seed=29)
    run_prompt_and_check(w, gen_device=DEV)


def test_decode_split_plan_many_heads():
    """2,048 KV heads (256 requests x 8): the decode grid is capped at 4 slots per head, fewer
    than the 8 XCDs; short heads turn their splits by head index and the longest ones fill
    all 4 slots."""
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 160, size=256)]
    lens[3], lens[100], lens[200] = 3000, 2500, 0
    w = workloads.Workload("split-plan-2048-heads", 1, 256, 16, 8, lens, 1.0, 0.2, 16, 1 << 16,
                           "zipf", seed=43)
    run_prompt_and_check(w, gen_device=DEV, sample_heads=96)


def test_workload2_full():
    run_prompt_and_check(workloads.workload(2), gen_device=DEV)


def test_workload3_full():
    """16 requests x 32,768 tokens, 64 query / 8 KV heads, Zipf(1.1) accumulators: tiers,
    counts and allocator state of every head, every byte of every page of all 128 heads, and
    attention of every query head on 4 of the workload's 64 decode steps (first, last and two
    between), each with its own fresh queries."""
    from mixed_precision_paged_score_amd import pipeline
    from oracle import attention as oatt, place
    w = workloads.workload(3)
    _log(f"[parity] {w.name} full: all heads' pages, attention on 4 decode steps")
    k, v, acc, _ = _inputs(w, DEV)
    path = pipeline.PromptPath(w, DEV)
    path.prompt(0, acc, k, v)
    steps = [0, 21, 42, 63]
    outs = []
    for s in steps:
        q = workloads.make_queries(w, DEV, s)
        out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
        path.decode(0, q, out)
        outs.append((parity.np_(q), out))
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    tier, count, _ = parity.oracle_score(w, acc)
    assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
    assert np.array_equal(parity.np_(path.new_count), count)
    opl = opool.Pool(1, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    opl.compact(0, count)
    parity.compare_pool(path.pool, opl)
    kc, vc = parity.np_(k), parity.np_(v)
    del k, v, acc
    got = [parity.np_(o) for _, o in outs]
    cu = w.cu_seqlens()
    G = w.group
    npages, worst = 0, 0.0
    for b in range(w.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in range(w.num_kv_heads):
            npages += parity.compare_head_pages(w, path.pool, 0, b, h, kc, vc, tier)
            kd, vd = place.head_dequantized(kc[lo:hi, h], vc[lo:hi, h], tier[lo:hi, h])
            # the 4 steps' query groups in one call: rows are (step, query head)
            qg = np.concatenate([qn[b, h * G:(h + 1) * G] for qn, _ in outs])
            want = oatt.decode_group(qg, kd, vd, path.scale).reshape(len(steps), G, 128)
            for n in range(len(steps)):
                worst = max(worst, parity.assert_close_attention(
                    got[n][b, h * G:(h + 1) * G], want[n]))
        _log(f"[parity] w3 request {b}: pages and attention ok")
    _log(f"[parity] w3 full ok: {npages} pages bit-exact, attention on steps {steps} "
         f"max err {worst:.2e}")
