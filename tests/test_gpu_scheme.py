"""Precision-scheme variants on the GPU (MI355X only): prompt placement with
kvc_quantize_and_place_scheme and decode with kvc_paged_decode_attention_scheme against the
oracle's scheme pages (every byte of every page of every head) and its float64 attention over
the scheme's reconstructions (2e-3 max-abs, 1e-3 relative L2).  Tiers and the allocator are the
default path's (the schemes keep the page geometry)."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import attention as oatt, pool as opool, scheme as osch  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SCHEMES = [("K8V4", "K4V2"), ("K4V8", "K2V4"), ("K8V2", "K4V1"), ("K4V2", "K4V2"),
           ("K2V4", "K4V1"), ("K4V1", "K2V4")]


def run_scheme(w, high, low, heads=None):
    from mixed_precision_paged_score_amd import kvc, pipeline
    print(f"[scheme] {high}-{low} {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"lens={w.seqlens[:6]}", flush=True)
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    q = workloads.make_queries(w)
    sc = kvc.make_scheme(high, low)
    path = pipeline.PromptPath(w, DEV)
    path.prompt_scheme(0, acc.to(DEV), k.to(DEV), v.to(DEV), sc)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    path.decode_scheme(0, q.to(DEV), out, sc)
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    tier, count, _ = parity.oracle_score(w, acc)
    assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
    opl = opool.Pool(1, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    opl.compact(0, count)
    parity.compare_pool(path.pool, opl)
    osc = osch.Scheme.named(high, low)
    cu = w.cu_seqlens()
    C = path.geom.row_capacity
    kn, vn, qn = k.numpy(), v.numpy(), q.numpy()
    G = w.group
    heads = heads or [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    for (b, h) in heads:
        lo, hi = int(cu[b]), int(cu[b + 1])
        want = osch.head_pages(kn[lo:hi, h], vn[lo:hi, h], tier[lo:hi, h], osc)
        row = parity.np_(path.pool.page_table[0, b, h])
        ids = [int(row[p]) for p in range(len(want[osch.HIGH]))] + \
              [int(row[C - 1 - p]) for p in range(len(want[osch.LOW]))]
        if ids:
            got = parity.np_(path.pool.pages[torch.tensor(ids, device=DEV)])
            for n, (gp, e) in enumerate(zip(got, want[osch.HIGH] + want[osch.LOW])):
                bad = np.nonzero(gp != e)[0]
                assert bad.size == 0, f"({b},{h}) page #{n}: {bad.size} bytes differ, first {bad[:6]}"
        kd, vd = osch.head_dequantized(kn[lo:hi, h], vn[lo:hi, h], tier[lo:hi, h], osc)
        want_o = oatt.decode_group(qn[b, h * G:(h + 1) * G], kd, vd, path.scale)
        parity.assert_close_attention(parity.np_(out[b, h * G:(h + 1) * G]), want_o)
    return path, out


@pytest.mark.parametrize("high,low", SCHEMES)
def test_ragged_all_heads(high, low):
    w = workloads.Workload("scheme-ragged", 1, 4, 16, 4, [1, 0, 300, 517], 1.0, 0.2, 16, 2048,
                           "zipf", seed=61)
    run_scheme(w, high, low)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 2)])
def test_group_sizes(hq, hkv):
    # G = 1 and G = 16 (the widest group one workgroup handles)
    w = workloads.Workload(f"scheme-g{hq // hkv}", 1, 2, hq, hkv, [129, 64], 1.0, 0.2, 16, 2048,
                           "zipf", seed=62)
    run_scheme(w, "K8V2", "K4V1")


def test_default_scheme_decode_matches_default_path():
    # K8V4-K4V2 in the slot-major layout gives the default layout's attention (the same
    # reconstructions; only summation order differs)
    from mixed_precision_paged_score_amd import pipeline
    w = workloads.Workload("scheme-same", 1, 3, 32, 8, [70, 300, 129], 1.0, 0.2, 64, 2048,
                           "causal", seed=63)
    path, out_s = run_scheme(w, "K8V4", "K4V2")
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    p2 = pipeline.PromptPath(w, DEV)
    p2.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    out_d = torch.empty_like(out_s)
    p2.decode(0, workloads.make_queries(w).to(DEV), out_d)
    torch.cuda.synchronize()
    assert torch.allclose(out_s, out_d, rtol=0, atol=1e-4)


def test_prune_and_no_prune_configurations():
    # K8V4-Prune: alpha_l = alpha_h leaves no LOW token; no-prune: alpha_l = 0 leaves no PRUNE
    w1 = workloads.Workload("k8v4-prune", 1, 2, 16, 4, [300, 517], 1.0, 1.0, 16, 2048, "zipf",
                            seed=64)
    path, _ = run_scheme(w1, "K8V4", "K4V2")
    t = parity.np_(path.tier[:w1.total_tokens])
    assert not np.any(t == 1) and np.any(t == 0)
    w2 = workloads.Workload("no-prune", 1, 2, 16, 4, [300, 517], 1.0, 0.0, 16, 2048, "zipf",
                            seed=65)
    path, _ = run_scheme(w2, "K8V2", "K4V1")
    t = parity.np_(path.tier[:w2.total_tokens])
    assert not np.any(t == 0) and np.any(t == 1)


@pytest.mark.parametrize("hq", [64, 128])
def test_split_plan_long_and_short_heads(hq):
    """16 requests x 8 KV heads, every token HIGH: the two 8K-token requests' heads fill all
    16 workgroup slots of the decode, the short and empty ones use one or two (8 and 16
    query heads per KV head: both decode kernels)."""
    lens = [8192, 0, 1, 37, 300, 777, 2048, 8192, 5000, 100, 64, 65, 3000, 15, 900, 4000]
    w = workloads.Workload(f"scheme-split-plan-{hq}", 1, 16, hq, 8, lens, 0.0, 0.0, 64, 1 << 16,
                           "zipf", seed=31)
    heads = [(0, h) for h in range(8)] + [(b, (3 * b) % 8) for b in range(1, 16)]
    run_scheme(w, "K8V4", "K4V2", heads=heads)


def test_workload2_sampled():
    w = workloads.workload(2)
    rng = np.random.default_rng(5)
    heads = [(int(b), int(h)) for b, h in zip(rng.integers(0, 8, 6), rng.integers(0, 8, 6))]
    run_scheme(w, "K4V8", "K4V1", heads=heads)
