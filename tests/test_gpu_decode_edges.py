"""Decode attention edge paths on the GPU (MI355X only), against the oracle.

* Large value ranges with rising logits.  The decode keeps a lazy running max (moved only when
  a pair of tiles exceeds it by more than 8 in log2 units), so a token's weight p can reach
  2^8 before the rescale, and P' = p * scale_v enters the value product in fp16.  Value rows
  spanning ~1,400 (LOW, 2-bit codes) and ~7,000 (HIGH, 4-bit codes) have scales near 470, so
  p * scale_v would pass fp16's 65,504 without the kernel's overflow guard.  Keys are a ramp
  along a fixed sign pattern that the queries follow, so each tier's logits rise by ~7.5
  (log2) per pair of tiles and p comes close to 2^7.5 on every other pair of a wave.
* A wave slice longer than one 64-page chunk.  With more than 512 KV heads the plan gives each
  head at most 8,192 / heads workgroups (4 at 2,048 heads) while the work per workgroup stays
  sized for 16, so a 32,768-token head is cut into 16 wave slices of ~320 work units: about
  107 HIGH tiles or 160 LOW tiles each, past the 64 pages whose ids a wave preloads.  The
  kernel then reloads the page ids for every further chunk of its slice.
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import attention as oatt, place, pool as opool, scheme as osch  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HIGH, LOW, PRUNE = 2, 1, 0


def acc_for_tiers(tiers, seqlens, G, alpha_h, alpha_l):
    """Accumulators that make kvc_score_tokens give `tiers` ([T][Hkv], outside the window):
    the sum over later queries is cnt * score with score 4 alpha_h / N (HIGH), the midpoint of
    alpha_l / N and alpha_h / N (LOW) or 0 (PRUNE), the same for every query head of a group."""
    T, H = tiers.shape
    acc = np.zeros((T, H * G), np.float64)
    o = 0
    for n in seqlens:
        cnt = (n - 1 - np.arange(n, dtype=np.float64))[:, None]
        t = tiers[o:o + n]
        sc = np.where(t == HIGH, 4.0 * alpha_h / n,
                      np.where(t == LOW, 0.5 * (alpha_h + alpha_l) / n, 0.0))
        acc[o:o + n] = np.repeat(cnt * sc, G, axis=1)
        o += n
    return torch.from_numpy(acc.astype(np.float32))


def run_prompt_and_decode(w, k, v, acc, q, check_heads, scheme=None):
    """Prompt round and one decode through the C ABI; tiers and allocator state of every head
    bit-exact; page bytes (default layout) and attention of `check_heads` against the oracle.
    Returns the largest absolute error and the largest |v_hat| seen."""
    from mixed_precision_paged_score_amd import kvc, pipeline
    path = pipeline.PromptPath(w, DEV)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=DEV)
    if scheme is None:
        path.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
        path.decode(0, q.to(DEV), out)
    else:
        sc = kvc.make_scheme(*scheme)
        path.prompt_scheme(0, acc.to(DEV), k.to(DEV), v.to(DEV), sc)
        path.decode_scheme(0, q.to(DEV), out, sc)
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    tier, count, _ = parity.oracle_score(w, acc)
    assert np.array_equal(parity.np_(path.tier[:w.total_tokens]), tier)
    opl = opool.Pool(1, w.batch, w.num_kv_heads, w.row_capacity, w.num_pages)
    opl.compact(0, count)
    parity.compare_pool(path.pool, opl)
    kn, vn, qn = k.numpy(), v.numpy(), q.numpy()
    cu = w.cu_seqlens()
    G = w.group
    got_all = parity.np_(out)
    worst, vmax = 0.0, 0.0
    for (b, h) in check_heads:
        lo, hi = int(cu[b]), int(cu[b + 1])
        if scheme is None:
            parity.compare_head_pages(w, path.pool, 0, b, h, kn, vn, tier)
            kd, vd = place.head_dequantized(kn[lo:hi, h], vn[lo:hi, h], tier[lo:hi, h])
        else:
            osc = osch.Scheme.named(*scheme)
            kd, vd = osch.head_dequantized(kn[lo:hi, h], vn[lo:hi, h], tier[lo:hi, h], osc)
        want = oatt.decode_group(qn[b, h * G:(h + 1) * G], kd, vd, path.scale)
        got = got_all[b, h * G:(h + 1) * G]
        assert np.all(np.isfinite(got)), f"head ({b},{h}): non-finite output"
        vm = float(np.abs(vd).max()) if len(vd) else 0.0
        vmax = max(vmax, vm)
        # the absolute bound is the one stated for unit-scale data; with values of magnitude
        # up to vm the float32 sums' rounding grows in proportion, so it scales with vm here
        err = np.abs(got.astype(np.float64) - want)
        assert err.max() <= 2e-3 * max(1.0, vm), (b, h, float(err.max()), vm)
        den = np.linalg.norm(want)
        if den > 0:
            assert np.linalg.norm(got - want) / den <= 1e-3, (b, h)
        worst = max(worst, float(err.max()))
    return worst, vmax


def ramp_inputs(seqlens, Hkv, G, tiers, step_log2, v_amp, seed):
    """Keys k_t = r_t * s_h (s_h a fixed +-1 pattern per KV head) with r_t rising by
    `step_log2` (in log2 units of q.k / sqrt(128) for q = s_h) per token of the same tier, in
    position order; values uniform in [-A, A] with A = v_amp[tier]; queries s_h plus N(0, 0.05)
    per query head, so every head of a group sees the ramp."""
    rng = np.random.default_rng(seed)
    T = sum(seqlens)
    s = rng.choice([-1.0, 1.0], size=(Hkv, 128))
    k = np.zeros((T, Hkv, 128))
    v = np.zeros((T, Hkv, 128))
    per_unit = 128 / np.sqrt(128) * np.log2(np.e)   # log2 logit per unit of r
    o = 0
    for n in seqlens:
        for h in range(Hkv):
            t = tiers[o:o + n, h]
            for x in (HIGH, LOW):
                idx = np.nonzero(t == x)[0]
                r = np.arange(len(idx)) * step_log2 / per_unit
                k[o + idx, h] = r[:, None] * s[h][None, :]
                v[o + idx, h] = rng.uniform(-v_amp[x], v_amp[x], size=(len(idx), 128))
        o += n
    q = s[None, :, None, :] + rng.normal(0, 0.05, size=(len(seqlens), Hkv, G, 128))
    q = q.reshape(len(seqlens), Hkv * G, 128)
    return (torch.from_numpy(k).to(torch.float16), torch.from_numpy(v).to(torch.float16),
            torch.from_numpy(q).to(torch.float16))


def block_tiers(n, H, block, window):
    """HIGH / LOW in alternating position blocks, the last `window` positions HIGH."""
    t = np.where((np.arange(n) // block) % 2 == 0, HIGH, LOW).astype(np.uint8)
    t[max(0, n - window):] = HIGH
    return np.repeat(t[:, None], H, axis=1)


@pytest.mark.parametrize("G", [8, 4])
def test_large_value_ranges_no_fp16_overflow(G):
    lens, Hkv, W = [2048, 1500], 2, 64
    w = workloads.Workload(f"edge-bigv-g{G}", 1, len(lens), Hkv * G, Hkv, lens, 1.0, 0.2, W,
                           4096, "zipf", seed=71)
    print(f"[edge] large value ranges, G={G}, lens={lens}", flush=True)
    tiers = np.concatenate([block_tiers(n, Hkv, 32, W) for n in lens])
    k, v, q = ramp_inputs(lens, Hkv, G, tiers, 7.5 / 32, {HIGH: 3500.0, LOW: 700.0}, seed=72)
    acc = acc_for_tiers(tiers, lens, G, w.alpha_h, w.alpha_l)
    heads = [(b, h) for b in range(w.batch) for h in range(Hkv)]
    worst, vmax = run_prompt_and_decode(w, k, v, acc, q, heads)
    assert vmax > 3000.0     # the value rows do reach the overflowing scales
    print(f"[edge] large values ok: max abs err {worst:.3e}, max |v_hat| {vmax:.0f}", flush=True)


def test_large_8bit_value_ranges_scheme_decode():
    # K4V8 HIGH pages hold 8-bit values, which the scheme decode multiplies by p unscaled:
    # rows spanning ~131,000 give scales near 514
    lens, Hkv, G, W = [1024, 777], 2, 8, 64
    w = workloads.Workload("edge-bigv8", 1, len(lens), Hkv * G, Hkv, lens, 1.0, 0.2, W, 4096,
                           "zipf", seed=73)
    print(f"[edge] scheme K4V8-K2V4 large 8-bit values, lens={lens}", flush=True)
    tiers = np.concatenate([block_tiers(n, Hkv, 32, W) for n in lens])
    k, v, q = ramp_inputs(lens, Hkv, G, tiers, 7.5 / 32, {HIGH: 65000.0, LOW: 700.0}, seed=74)
    acc = acc_for_tiers(tiers, lens, G, w.alpha_h, w.alpha_l)
    heads = [(b, h) for b in range(w.batch) for h in range(Hkv)]
    worst, vmax = run_prompt_and_decode(w, k, v, acc, q, heads, scheme=("K4V8", "K2V4"))
    assert vmax > 60000.0
    print(f"[edge] scheme large values ok: max abs err {worst:.3e}", flush=True)


def _many_heads_workload(seed):
    """256 requests x 8 KV heads (2,048 heads, G = 8): 255 of 50..300 tokens and one of
    32,768 tokens whose tiers alternate HIGH / LOW in 16-position blocks (16,384 + 16,384
    tokens: 1,024 HIGH pages and 512 LOW pages)."""
    rng = np.random.default_rng(seed)
    B, Hkv, G, W = 256, 8, 8, 64
    long_b = 77
    lens = [int(x) for x in rng.integers(50, 301, size=B)]
    lens[long_b] = 32768
    w = workloads.Workload("edge-2048heads", 1, B, Hkv * G, Hkv, lens, 1.0, 0.2, W, 1 << 16,
                           "zipf", seed=seed)
    parts = []
    for b, n in enumerate(lens):
        if b == long_b:
            parts.append(block_tiers(n, Hkv, 16, W))
        else:
            t = rng.choice([HIGH, LOW, PRUNE], size=(n, Hkv), p=[0.5, 0.4, 0.1]).astype(np.uint8)
            t[max(0, n - W):] = HIGH
            parts.append(t)
    tiers = np.concatenate(parts)
    acc = acc_for_tiers(tiers, lens, G, w.alpha_h, w.alpha_l)
    k, v = workloads.make_kv(w)
    q = workloads.make_queries(w)
    heads = [(long_b, h) for h in range(Hkv)]
    heads += [(int(b), int(h)) for b, h in zip(rng.choice([x for x in range(B) if x != long_b],
                                                          16, replace=False),
                                               rng.integers(0, Hkv, 16))]
    return w, k, v, acc, q, heads


def test_long_head_among_2048_heads_spans_page_chunks():
    w, k, v, acc, q, heads = _many_heads_workload(75)
    print(f"[edge] 2,048 heads with one 32,768-token head (default decode)", flush=True)
    worst, _ = run_prompt_and_decode(w, k, v, acc, q, heads)
    print(f"[edge] chunked slices ok: max abs err {worst:.3e}", flush=True)


def test_long_head_among_2048_heads_scheme_decode():
    w, k, v, acc, q, heads = _many_heads_workload(75)
    print(f"[edge] 2,048 heads with one 32,768-token head (scheme decode K8V4-K4V2)", flush=True)
    worst, _ = run_prompt_and_decode(w, k, v, acc, q, heads, scheme=("K8V4", "K4V2"))
    print(f"[edge] scheme chunked slices ok: max abs err {worst:.3e}", flush=True)
