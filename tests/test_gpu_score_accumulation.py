"""Score accumulation inside decode attention (MI355X only): kvc_paged_decode_attention_acc
adds every cached token's softmax weight from the decode query into acc_sum[cu[b] + pos][hq]
and returns the same attention output as kvc_paged_decode_attention.  Compared with the
oracle's float64 weights over the same dequantized keys (relative 1e-4 per weight; the
weights are recomputed from identical codes, only rounding order differs), and at full size
with the invariant that each query head's weights over its request sum to one."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import attention as oatt, place  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL_W, ATOL_W = 1e-4, 1e-7


def _oracle_delta(w, k, v, tier, q, scale, heads=None, scheme=None):
    """scheme: an oracle.scheme.Scheme whose widths the keys were stored at (None: K8V4/K4V2)"""
    from oracle import scheme as osch
    cu = w.cu_seqlens()
    delta = np.zeros((w.total_tokens, w.num_q_heads))

    def rows(b, h):
        lo, hi = int(cu[b]), int(cu[b + 1])
        return lo, hi

    def k_of(b, h):
        lo, hi = rows(b, h)
        if scheme is not None:
            return osch.head_dequantized(k[lo:hi, h], v[lo:hi, h], tier[lo:hi, h], scheme)[0]
        return place.head_dequantized(k[lo:hi, h], v[lo:hi, h], tier[lo:hi, h])[0]

    def pos_of(b, h):
        lo, hi = rows(b, h)
        return np.concatenate([place.head_tokens(tier[lo:hi, h], place.HIGH),
                               place.head_tokens(tier[lo:hi, h], place.LOW)])
    if heads is None:
        return oatt.accumulate(delta, q, k_of, pos_of, cu, w.num_kv_heads, scale)
    G = w.group
    for (b, h) in heads:
        wts = oatt.attention_weights(q[b, h * G:(h + 1) * G], k_of(b, h), scale)
        for g in range(G):
            delta[int(cu[b]) + pos_of(b, h), h * G + g] += wts[g]
    return delta


def _check(got, want, mask=None):
    err = np.abs(got - want)
    bound = RTOL_W * np.abs(want) + ATOL_W
    if mask is not None:
        err, bound = err[mask], bound[mask]
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{len(bad)} weights off, worst {err.max():.3e}"


def run_case(w, steps=1, sample_heads=None, scheme=None):
    """scheme: (HIGH format, LOW format) names: the prompt placed in that scheme's layout,
    the accumulating scheme decode against the plain scheme decode and the oracle's weights
    over the scheme's dequantized keys."""
    from mixed_precision_paged_score_amd import kvc, pipeline
    from oracle import scheme as osch
    print(f"[acc] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"lens={w.seqlens[:6]} steps={steps} scheme={scheme}", flush=True)
    gen = "cpu" if w.total_tokens * w.num_q_heads < (1 << 22) else DEV
    k, v = workloads.make_kv(w, gen)
    acc = workloads.make_acc(w, k, gen)
    k, v, acc = k.to(DEV), v.to(DEV), acc.to(DEV)
    path = pipeline.PromptPath(w, DEV)
    if scheme is None:
        path.prompt(0, acc, k, v)
    else:
        path.scheme = kvc.make_scheme(*scheme)      # decode_acc then takes the scheme decode
        path.prompt_scheme(0, acc, k, v, path.scheme)
    tier = parity.np_(path.tier[:w.total_tokens])
    acc_gpu = torch.zeros_like(acc)     # accumulators start at zero: the sums stay exact
    out_a = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    out_p = torch.empty_like(out_a)
    qs = [workloads.make_queries(w, DEV, s) for s in range(steps)]
    for q in qs:
        path.decode_acc(0, q, out_a, acc_gpu)
        if scheme is None:
            path.decode(0, q, out_p)
        else:
            path.decode_scheme(0, q, out_p, path.scheme)
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    # the output is the plain decode's
    assert torch.allclose(out_a, out_p, rtol=0, atol=1e-6)
    delta = parity.np_(acc_gpu).astype(np.float64)
    kc, vc = parity.np_(k), parity.np_(v)
    heads = None
    if sample_heads is not None:
        rng = np.random.default_rng(w.seed)
        allh = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
        heads = [allh[i] for i in rng.choice(len(allh), sample_heads, replace=False)]
    want = np.zeros_like(delta)
    osc_ = osch.Scheme.named(*scheme) if scheme else None
    for q in qs:
        want += _oracle_delta(w, kc, vc, tier, parity.np_(q), path.scale, heads, osc_)
    if heads is None:
        _check(delta, want)
    else:
        cu = w.cu_seqlens()
        G = w.group
        mask = np.zeros(delta.shape, bool)
        for (b, h) in heads:
            mask[int(cu[b]):int(cu[b + 1]), h * G:(h + 1) * G] = True
        _check(delta, want, mask)
    # every query head's weights over its request's live tokens sum to one per step
    cu = w.cu_seqlens()
    counts = parity.np_(path.new_count)
    for b in range(w.batch):
        s = delta[int(cu[b]):int(cu[b + 1])].sum(0)
        live = (counts[b].sum(1) > 0).repeat(w.group)
        assert np.allclose(s[live], steps, rtol=0, atol=1e-4 * steps), (b, s[live][:4])
        assert np.all(s[~live] == 0)
    print(f"[acc] ok: max weight {want.max():.3e}", flush=True)


def test_workload1_full():
    run_case(workloads.workload(1))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (6, 2), (16, 4), (32, 4), (32, 2)])
def test_ragged_group_sizes_and_two_steps(hq, hkv):
    w = workloads.Workload(f"acc-{hq}-{hkv}", 1, 5, hq, hkv, [1, 0, 37, 300, 777], 1.0, 0.2,
                           16, 4096, "causal", seed=41)
    run_case(w, steps=2)


def test_workload2_full():
    run_case(workloads.workload(2))


def test_workload3_sampled():
    run_case(workloads.workload(3), sample_heads=6)


@pytest.mark.parametrize("scheme", [("K4V8", "K2V4"), ("K8V2", "K4V1"), ("K2V4", "K4V2")])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 4), (32, 4)])
def test_scheme_pages_ragged(scheme, hq, hkv):
    # the accumulating decode over precision-scheme pages (groups of 1, 4 and 8 query heads)
    w = workloads.Workload(f"acc-sch-{hq}-{hkv}", 1, 5, hq, hkv, [1, 0, 37, 300, 777], 1.0, 0.2,
                           16, 4096, "causal", seed=43)
    run_case(w, steps=2, scheme=scheme)


def test_scheme_pages_workload2_full():
    run_case(workloads.workload(2), scheme=("K4V8", "K2V4"))
