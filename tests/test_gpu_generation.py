"""Generation phase on the GPU vs the oracle's record simulation (MI355X only): per-step
appends (kvc_append_tokens) and re-tier rounds (score with previous tiers, compact with the
rebuilt heads, quantize/place in re-tier mode), compared bit-exactly after every round; the
chain-of-thought workload runs its full 16,384 generated tokens (128 rounds).  The same runs
under precision schemes (kvc_append_tokens_scheme, kvc_quantize_and_place_scheme in re-tier
mode, the scheme decode) against the oracle's scheme generation."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import attention as oatt, generation as ogen  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _compare_heads(w, path, gen, heads=None):
    C = path.geom.row_capacity
    heads = heads if heads is not None else [(b, h) for b in range(w.batch)
                                             for h in range(w.num_kv_heads)]
    for (b, h) in heads:
        want = gen.head_pages(b, h)
        row = parity.np_(path.pool.page_table[0, b, h])
        ids = [int(row[p]) for p in range(len(want[ogen.HIGH]))] + \
              [int(row[C - 1 - p]) for p in range(len(want[ogen.LOW]))]
        imgs = want[ogen.HIGH] + want[ogen.LOW]
        if not ids:
            continue
        got = parity.np_(path.pool.pages[torch.tensor(ids, device=DEV)])
        for n, (gp, e) in enumerate(zip(got, imgs)):
            if not np.array_equal(gp, e):
                bad = np.nonzero(gp != e)[0]
                raise AssertionError(f"head ({b},{h}) page #{n}: {len(bad)} bytes differ, "
                                     f"first {bad[:6].tolist()}")


def _check_attention(w, path, gen, sample_heads, seed):
    """Decode attention of the current state (fresh queries) on the tracked heads."""
    q = workloads.make_queries(w, "cpu", seed)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    path.decode(0, q.to(DEV), out)
    torch.cuda.synchronize()
    G = w.group
    heads = sample_heads or [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    worst = 0.0
    for (b, h) in heads:
        kd, vd = gen.head_dequantized(b, h)
        want = oatt.decode_group(q.numpy()[b, h * G:(h + 1) * G], kd, vd, path.scale)
        worst = max(worst, parity.assert_close_attention(parity.np_(out[b, h * G:(h + 1) * G]),
                                                         want))
    print(f"[generation] attention ok at lengths {path.lens[:3]}...: {len(heads)} heads, "
          f"max err {worst:.2e}", flush=True)


def run_generation(w, steps, round_every, sample_heads=None, check_every_round=True,
                   attn_every=None, acc_device="cpu", scheme=None):
    """scheme: (HIGH format, LOW format) names, e.g. ("K4V8", "K2V4"), or None (K8V4-K4V2 in
    the default layout)."""
    from mixed_precision_paged_score_amd import kvc, pipeline
    from oracle import scheme as osch
    print(f"[generation] B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"prompt={w.seqlens} steps={steps} round={round_every} P={w.num_pages} "
          f"scheme={scheme}", flush=True)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    max_len = max(w.seqlens) + steps
    path = pipeline.GenerationPath(w, max_len, DEV,
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
    g = torch.Generator().manual_seed(w.seed + 99)
    rounds = 0
    acc_cur, lens_prev = acc.to(acc_device), list(w.seqlens)
    for s in range(steps):
        kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
        vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g).to(torch.float16)
        path.append(0, kn.to(DEV), vn.to(DEV))
        gen.append(kn.numpy(), vn.numpy())
        if (s + 1) % round_every == 0:
            import dataclasses
            wr = dataclasses.replace(w, seqlens=list(path.lens), seed=w.seed + 1000 * (s + 1))
            # the round's weights added to the sums (drawn where it is cheapest; both sides
            # receive the same float32 values)
            acc_cur = workloads.make_acc_zipf_round(wr, acc_cur, lens_prev, acc_device,
                                                    rounds + 1)
            lens_prev = list(path.lens)
            acc_r = acc_cur.to(DEV)
            path.retier(0, acc_r)
            tier_o, _, changed_o = gen.retier(parity.np_(acc_r), w.alpha_h, w.alpha_l, w.window)
            rounds += 1
            if check_every_round:
                torch.cuda.synchronize()
                assert np.array_equal(parity.np_(path.changed), changed_o)
                assert np.array_equal(parity.np_(path.tier[:path.T]), tier_o)
                parity.compare_pool(path.pool, gen.pool)
                _compare_heads(w, path, gen, sample_heads)
                print(f"[generation] step {s + 1}: round {rounds} ok, "
                      f"{int(changed_o.sum())} heads rebuilt, ring head {gen.pool.head}",
                      flush=True)
        if attn_every and (s + 1) % attn_every == 0:
            _check_attention(w, path, gen, sample_heads, seed=s + 1)
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    parity.compare_pool(path.pool, gen.pool)
    _compare_heads(w, path, gen, sample_heads)
    # decode attention over the final state
    _check_attention(w, path, gen, sample_heads, seed=7)
    n_demoted = sum(int((t == ogen.LOW).sum()) for t in gen.tiers)
    print(f"[generation] ok: {rounds} rounds, {n_demoted} LOW tokens, ring head {gen.pool.head}",
          flush=True)
    return path, gen


def test_generation_small_ragged():
    w = workloads.Workload("gen-small", 1, 3, 16, 4, [300, 160, 500], 1.0, 0.2, 16, 2048, "zipf",
                           seed=31)
    run_generation(w, steps=96, round_every=32)


def test_generation_group8_with_pruning_and_page_boundaries():
    # appends cross HIGH page boundaries (16 slots) many times; alpha_l prunes
    w = workloads.Workload("gen-g8", 1, 2, 16, 2, [129, 77], 1.0, 0.5, 8, 1024, "zipf", seed=32)
    run_generation(w, steps=70, round_every=20)


def test_workload4_full_length():
    # 16 requests x (4096-token prompt + 16,384 generated tokens), 64 query / 8 KV heads, a
    # re-tier round every 128 steps (128 rounds), 2^18 pages, in lockstep with the oracle:
    # after every round the rebuilt-head flags, the tiers of every position and the allocator
    # state of all 128 heads bit-exact, and every page byte of 6 sampled heads; decode
    # attention of those heads every 1,024 steps
    w = workloads.workload(4)
    run_generation(w, steps=16384, round_every=128, sample_heads=6, attn_every=1024,
                   acc_device=DEV)


# ---- precision schemes --------------------------------------------------------------------

@pytest.mark.parametrize("scheme", [("K4V8", "K2V4"), ("K8V2", "K4V1"), ("K4V2", "K4V1"),
                                    ("K2V4", "K4V2")])
def test_scheme_generation_small_ragged(scheme):
    # every bit width in both tiers: appends set single slots of the value blocks, rounds copy
    # survivors, re-quantize demotions at the LOW widths and return the old pages
    w = workloads.Workload("gen-small-sch", 1, 3, 16, 4, [300, 160, 500], 1.0, 0.2, 16, 2048,
                           "zipf", seed=51)
    run_generation(w, steps=96, round_every=32, scheme=scheme, attn_every=48)


def test_scheme_generation_group8_with_pruning_and_page_boundaries():
    w = workloads.Workload("gen-g8-sch", 1, 2, 16, 2, [129, 77], 1.0, 0.5, 8, 1024, "zipf",
                           seed=52)
    run_generation(w, steps=70, round_every=20, scheme=("K8V2", "K4V1"))


def test_scheme_generation_workload4_shape():
    # workload 4's shape (16 x 4,096-token prompts, 64 query / 8 KV heads) for 512 steps and
    # 4 rounds in the K4V8-K2V4 scheme: allocator state of all heads after every round, page
    # bytes and attention of 6 sampled heads
    w = workloads.workload(4)
    run_generation(w, steps=512, round_every=128, sample_heads=6, attn_every=256,
                   acc_device=DEV, scheme=("K4V8", "K2V4"))
