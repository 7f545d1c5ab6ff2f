"""The fused compaction round (kvc_compaction_round) against the three calls it replaces
(kvc_score_tokens -> kvc_compact_pages -> kvc_quantize_and_place) on the GPU (MI355X only):
tiers, counts, changed flags, page table, counts, reverse map, free ring, counters, status
and the bytes of every live page identical, in prompt mode and in re-tier mode; one case per
mode also against the oracle.  Up to 1024 KV heads (the planning workgroup's limit)."""
import dataclasses
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


def _live_pages(pool):
    rows = pool.page_table.reshape(-1)
    ids = torch.unique(rows[rows >= 0])
    return ids, pool.pages[ids.long()]


def assert_same_state(a, b, tier_rows):
    """Two paths' outputs and pool states bit for bit."""
    assert torch.equal(a.tier[:tier_rows], b.tier[:tier_rows]), "tiers differ"
    assert torch.equal(a.new_count, b.new_count), "new counts differ"
    for name in ("page_table", "count", "owner", "free_ring", "ring_ctr", "dev_status"):
        assert torch.equal(getattr(a.pool, name), getattr(b.pool, name)), f"{name} differs"
    ia, pa = _live_pages(a.pool)
    ib, pb = _live_pages(b.pool)
    assert torch.equal(ia, ib) and torch.equal(pa, pb), "live page bytes differ"


def _inputs(w, layer=0):
    gen = "cpu" if w.total_tokens * w.num_q_heads < (1 << 22) else DEV
    k, v = workloads.make_kv(w, gen, layer)
    acc = workloads.make_acc(w, k, gen, layer)
    return k.to(DEV), v.to(DEV), acc.to(DEV)


def run_prompt_pair(w, rounds=1, check_oracle=False):
    from mixed_precision_paged_score_amd import pipeline
    print(f"[round] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"lens={w.seqlens[:6]} L={w.num_layers} rounds={rounds}", flush=True)
    a = pipeline.PromptPath(w, DEV)
    b = pipeline.PromptPath(w, DEV)
    opl = opool.Pool(w.num_layers, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages) \
        if check_oracle else None
    for r in range(rounds):
        layer = r % w.num_layers
        wr = dataclasses.replace(w, seed=w.seed + 31 * r)
        k, v, acc = _inputs(wr, layer)
        a.prompt(layer, acc, k, v)
        b.prompt_fused(layer, acc, k, v)
        torch.cuda.synchronize()
        assert_same_state(a, b, w.total_tokens)
        if opl is not None:
            tier, count, _ = parity.oracle_score(wr, acc.cpu())
            assert np.array_equal(parity.np_(b.tier[:w.total_tokens]), tier)
            opl.compact(layer, count)
            parity.compare_pool(b.pool, opl)
    return a, b


def test_workload1_against_three_calls_and_oracle():
    run_prompt_pair(workloads.workload(1), rounds=3, check_oracle=True)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4), (32, 4), (64, 4)])
def test_ragged_batches_repeated_rounds(hq, hkv):
    # empty and single-token requests, group sizes 1, 4, 8, 16; rounds wrap the ring
    w = workloads.Workload(f"round-{hq}-{hkv}", 2, 5, hq, hkv, [1, 0, 37, 300, 777], 1.0, 0.2,
                           16, 1024, "causal", seed=81)
    run_prompt_pair(w, rounds=6)


@pytest.mark.parametrize("ah,al,win", [(0.0, 0.0, 0), (1.0, 1.0, 3), (np.inf, np.inf, 64)])
def test_threshold_and_window_edges(ah, al, win):
    w = workloads.Workload("round-edges", 1, 4, 16, 4, [64, 65, 129, 500], ah, al, win, 4096,
                           "causal", seed=82)
    run_prompt_pair(w, rounds=2)


def test_workload3_full():
    run_prompt_pair(workloads.workload(3), rounds=2)


def test_workload5_shape_512_heads():
    # 64 requests x 8 KV heads: the planning workgroup takes two heads per thread; three layers
    # into a pool that holds them
    w = dataclasses.replace(workloads.workload(5), num_layers=3, num_pages=1 << 20)
    run_prompt_pair(w, rounds=3)


def test_1024_heads():
    # 128 requests x 8 KV heads of 20..400 tokens: four heads per planning thread
    rng = np.random.default_rng(83)
    lens = [int(x) for x in rng.integers(20, 401, size=128)]
    w = workloads.Workload("round-1024", 1, 128, 64, 8, lens, 1.0, 0.2, 64, 1 << 16, "zipf",
                           seed=83)
    run_prompt_pair(w, rounds=2)


def test_pool_exhaustion_changes_nothing():
    # a pool too small for both layers: the round that does not fit sets the same status bit
    # on both paths and leaves the pool as it was
    w = workloads.Workload("round-full", 2, 4, 16, 4, [300, 200, 500, 400], 1.0, 0.2, 16, 300,
                           "causal", seed=84)
    from mixed_precision_paged_score_amd import pipeline
    a = pipeline.PromptPath(w, DEV)
    b = pipeline.PromptPath(w, DEV)
    for layer in range(2):
        k, v, acc = _inputs(w, layer)
        a.prompt(layer, acc, k, v)
        b.prompt_fused(layer, acc, k, v)
        torch.cuda.synchronize()
        assert_same_state(a, b, w.total_tokens)
    assert b.pool.status() != 0


def test_request_longer_than_max_seqlen_sets_status():
    from mixed_precision_paged_score_amd import kvc, pipeline
    w = workloads.Workload("round-seqlen", 1, 3, 16, 4, [100, 300, 50], 1.0, 0.2, 16, 1024,
                           "causal", seed=85)
    k, v, acc = _inputs(w)
    a = pipeline.PromptPath(w, DEV)
    b = pipeline.PromptPath(w, DEV)
    for p in (a, b):
        p.max_seqlen = 200            # shorter than request 1
        p.tier.fill_(7)               # request 1's tier rows are not written
    # the fused round reports the score's status bit in the pool's status, so the round does
    # not commit: the three calls do the same when the score reports there too
    a.score_status = a.pool.dev_status
    a.prompt(0, acc, k, v)
    b.prompt_fused(0, acc, k, v)
    torch.cuda.synchronize()
    assert b.pool.status() & kvc.DEV_SEQLEN
    assert_same_state(a, b, w.total_tokens)
    assert int((b.pool.page_table >= 0).sum()) == 0          # nothing committed


def run_retier_pair(w, steps, round_every, repeat=False):
    """Two generation runs in lockstep: appends on both, rounds through the three calls on one
    and the fused round on the other; everything compared after every round.  With repeat,
    every round is run a second time on the same accumulators, where no head changes."""
    from mixed_precision_paged_score_amd import pipeline
    print(f"[round] re-tier {w.name} B={w.batch} steps={steps} round={round_every}", flush=True)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    max_len = max(w.seqlens) + steps
    a = pipeline.GenerationPath(w, max_len, DEV)
    b = pipeline.GenerationPath(w, max_len, DEV)
    for p in (a, b):
        p.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert_same_state(a, b, a.T)
    g = torch.Generator().manual_seed(w.seed + 99)
    acc_cur, lens_prev, rounds = acc, list(w.seqlens), 0
    for s in range(steps):
        kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16).to(DEV)
        vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16).to(DEV)
        a.append(0, kn, vn)
        b.append(0, kn, vn)
        if (s + 1) % round_every == 0:
            rounds += 1
            wr = dataclasses.replace(w, seqlens=list(a.lens), seed=w.seed + 1000 * (s + 1))
            acc_cur = workloads.make_acc_zipf_round(wr, acc_cur, lens_prev, "cpu", rounds)
            lens_prev = list(a.lens)
            acc_r = acc_cur.to(DEV)
            a.retier(0, acc_r)
            b.retier_fused(0, acc_r)
            torch.cuda.synchronize()
            assert torch.equal(a.changed, b.changed), f"round {rounds}: changed flags differ"
            assert_same_state(a, b, a.T)
            assert b.pool.status() == 0
            if repeat:
                a.retier(0, acc_r)
                b.retier_fused(0, acc_r)
                torch.cuda.synchronize()
                assert int(b.changed.sum()) == 0, f"round {rounds} repeated: a head changed"
                assert torch.equal(a.changed, b.changed)
                assert_same_state(a, b, a.T)
                assert b.pool.status() == 0
    print(f"[round] re-tier ok: {rounds} rounds", flush=True)


def test_retier_ragged():
    w = workloads.Workload("round-gen", 1, 3, 16, 4, [300, 160, 500], 1.0, 0.2, 16, 2048, "zipf",
                           seed=86)
    run_retier_pair(w, steps=96, round_every=32)


def test_retier_repeated_round_changes_nothing():
    w = workloads.Workload("round-gen-rep", 1, 2, 16, 4, [200, 420], 1.0, 0.2, 16, 2048, "zipf",
                           seed=87)
    run_retier_pair(w, steps=64, round_every=32, repeat=True)


def test_retier_workload4_shape():
    run_retier_pair(workloads.workload(4), steps=512, round_every=128)
