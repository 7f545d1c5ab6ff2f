"""Benchmark of the DiffKV-style compaction + mixed-precision paged decode hot path on one
MI355X.

A step is one pass of the whole path over one batch of synthetic input resident in HBM:
score_tokens -> compact_pages (prompt mode: the layer's previous pages go back to the ring,
new ones are assigned) -> quantize_and_place for the full prompt, then the workload's decode
steps of paged_decode_attention (fresh queries).  Default workload: one layer, 16 requests x
32,768 tokens, 64 query / 8 KV heads, Zipf(1.1) accumulators, 64 decode steps; the pool has
room for two layouts of the layer (2 x 2^18 pages).  The step's library calls are captured
into two HIP graphs (prompt round, decode steps) and replayed; --eager launches them from
Python instead.  Each step starts with a ~200 us GPU spin outside the timed region, so that
the host has queued the step before the GPU reaches it.

Prints one JSON line.  `value` = KV token-heads compacted per second over the compaction
part of the step; `decode_GBps` = algorithmic bytes of paged decode attention per second;
`roofline` is for the dominant work, the decode-attention call (main + combine kernel),
timed with HIP events around the replayed decode steps on the stream they run on, divided
by the number of calls; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.  Beside the step: `decode_with_score_accumulation` (the same decode calls adding
every cached token's weight into the accumulators) and `generation_loop` (64 generation steps
of the layer after the prompt: decode with score accumulation into one padded accumulator
buffer, then kvc_generation_step, captured as one graph) and `prefill` (the causal prefill
attention of the workload's prompts with the accumulators, kvc_prefill_attention, against the
fp16 matrix-core peak) and `precision_schemes` (decode over pages placed in other precision
schemes, kvc_quantize_and_place_scheme + kvc_paged_decode_attention_scheme) and, for a
workload with re-tier rounds, `retier_round` (one round after `round_every` appended tokens:
re-score with the previous tiers as ceiling, compact the changed heads, rebuild their pages).
"""
import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0      # dense fp16 matrix-core peak of MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-acc", action="store_true",
                    help="skip the extra timing of decode attention with score accumulation")
    ap.add_argument("--cpu-sample-requests", type=int, default=16)
    ap.add_argument("--gen-steps", type=int, default=64,
                    help="steps of the generation loop (decode with score accumulation, then "
                         "the per-step policy) timed after the main steps (0: skip)")
    ap.add_argument("--no-retier", action="store_true",
                    help="skip the timing of a re-tier round (workloads with one)")
    ap.add_argument("--no-schemes", action="store_true",
                    help="skip the precision-scheme decode timings")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the causal prefill (prompt accumulator producer) timing")
    ap.add_argument("--eager", action="store_true",
                    help="launch every library call from Python instead of replaying HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch, 4 launches.
    Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its per-dispatch counters give the factor
    that turns those counters into bytes."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    evs = []
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    print(json.dumps({"copy_calibration_bytes_per_launch": {"read": n, "write": n},
                      "launches": 4, "median_ms": ms[len(ms) // 2],
                      "copy_GBps_read_plus_write": 2 * n / (ms[len(ms) // 2] / 1e3) / 1e9}),
          flush=True)


def measure_ceilings():
    """Streaming rates of plain device kernels on the same GPU, for context beside the path's
    GB/s: a 1 GiB device copy (read + write), an elementwise add over 1 GiB of fp16 (read +
    write) and a 1 GiB fill (write); the median of 10 launches each, outside the timed steps."""
    n = 1 << 30
    a = torch.ones(n // 2, dtype=torch.float16, device="cuda:0")
    b = torch.empty_like(a)

    def rate(fn, nbytes):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = sorted(x.elapsed_time(y) for x, y in evs)[5]
        return nbytes / (ms / 1e3) / 1e9

    res = {"copy_GBps": rate(lambda: b.copy_(a), 2 * n),
           "stream_add_GBps": rate(lambda: torch.add(a, 1.0, out=b), 2 * n),
           "fill_GBps": rate(lambda: b.fill_(2.0), n)}
    del a, b
    torch.cuda.empty_cache()
    return res


def spin_cycles(stream, target_us=200.0):
    """Argument of torch.cuda._sleep that keeps the GPU busy for about target_us: queued
    before a timed region, it lets the host submit the region's whole graph first, so that the
    events time the GPU's work and not the host's submission of each node (which shows when a
    long graph before has left the GPU idle)."""
    probe = 1 << 20
    torch.cuda._sleep(probe)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(probe)
    e1.record(stream)
    torch.cuda.synchronize()
    us = max(e0.elapsed_time(e1) * 1e3, 1.0)
    return int(probe * target_us / us)


def time_retier_round(w, k, v, acc, ev, stream, spin, reps=3):
    """A re-tier round of a generation run (the chain-of-thought growth workload has one every
    128 decode steps).  Setup,
    outside the timed region and redone for every round timed: the prompt, then `round_every`
    appended tokens per (request, KV head) and that round's Zipf accumulators over the live
    positions.  Timed with HIP events on the stream: score_tokens with the previous tiers as
    ceiling, compact_pages with the changed heads, quantize_and_place in re-tier mode (pages of
    changed heads rebuilt from their old pages).  Returns (us per round, token-heads re-scored,
    heads rebuilt)."""
    from mixed_precision_paged_score_amd import kvc, pipeline, workloads
    R = int(w.extra["round_every"])
    times, heads = [], 0
    for rep in range(reps + 1):                      # the first round is a warm-up
        g = torch.Generator(device="cuda").manual_seed(w.seed + 99)
        path = pipeline.GenerationPath(w, max(w.seqlens) + R, "cuda:0")
        path.prompt(0, acc, k, v)
        for _ in range(R):
            kn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g, device="cuda")
            vn = torch.randn((w.batch, w.num_kv_heads, 128), generator=g, device="cuda")
            path.append(0, kn.half(), vn.half())
        wr = dataclasses.replace(w, seqlens=list(path.lens), seed=w.seed + 1000 * R)
        acc_r = workloads.make_acc_zipf(wr, "cuda:0")
        prev = path.packed_state()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        torch.cuda._sleep(spin)
        e0.record(stream)
        kvc.score_tokens(path.geom, acc_r, path.cu, path.T, path.max_seqlen, w.alpha_h,
                         w.alpha_l, w.window, path.tier, path.new_count, prev_tier=prev,
                         changed=path.changed, dev_status=path.score_status)
        kvc.compact_pages(path.geom, 0, path.pool, path.new_count, path.ws_compact,
                          changed=path.changed, old_rows=path.old_rows, old_count=path.old_count)
        kvc.quantize_and_place(path.geom, 0, path.pool, None, None, path.cu, path.T,
                               path.max_seqlen, path.tier, path.ws_quant, prev_tier=prev,
                               changed=path.changed, old_rows=path.old_rows,
                               old_count=path.old_count)
        e1.record(stream)
        torch.cuda.synchronize()
        assert path.pool.status() == 0, f"re-tier round status {path.pool.status()}"
        if rep > 0:
            times.append(e0.elapsed_time(e1) * 1e3)
        heads = int(path.changed.sum().item())
        token_heads = path.T * w.num_kv_heads
        # algorithmic bytes: the accumulators, previous and new tiers, and for every rebuilt
        # head its old pages read and its new pages written whole
        chg = path.changed.cpu().numpy().astype(bool)
        old_c = path.old_count.cpu().numpy()[chg]
        new_c = path.new_count.cpu().numpy()[chg]

        def pages(cnt):
            return int((-(-cnt[:, 0] // 16)).sum() + (-(-cnt[:, 1] // 32)).sum())
        nbytes = (path.T * w.num_q_heads * 4 + 2 * token_heads
                  + (pages(old_c) + pages(new_c)) * kvc.PAGE_BYTES)
        del path, acc_r, prev
    return float(np.median(times)), token_heads, heads, nbytes


def time_decode_acc(a, path, qs, out, nsteps_dec, ev, stream):
    """Decode attention with score accumulation (every cached token's weight added into fp32
    accumulators), the same decode steps, replayed as one graph outside the timed steps;
    returns microseconds per call."""
    acc = torch.zeros((path.T, path.w.num_q_heads), dtype=torch.float32, device=out.device)
    if a.eager:
        def run():
            for q in qs:
                path.decode_acc(0, q, out, acc)
    else:
        path.decode_acc(0, qs[0], out, acc)          # workspace made before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for q in qs:
                path.decode_acc(0, q, out, acc)
        run = g.replay
    for _ in range(max(a.warmup, 1)):
        run()
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(a.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (a.steps * nsteps_dec)


def time_generation_loop(a, w, k, v, acc, ev, stream, nsteps):
    """The generation phase of one layer, `nsteps` steps after the workload's prompt, as a
    caller runs it: each step is a decode with score accumulation (a fresh query per request
    and query head) into one padded accumulator buffer [B][N + nsteps][Hq], then
    kvc_generation_step on the same buffer (append the new tokens, score the token leaving
    the window).  The steps are captured into one graph (positions advance on the device);
    before each replay the pool, the accumulators and the positions are restored from a
    snapshot taken after the prompt (outside the timed region).  Returns microseconds per step,
    the policy step alone per step, and the decisions of the last replay."""
    from mixed_precision_paged_score_amd import kvc, pipeline, workloads
    B, Hkv, Hq, W = w.batch, w.num_kv_heads, w.num_q_heads, w.window
    N = max(w.seqlens)
    dev = k.device
    gp = pipeline.GenerationPath(w, N + nsteps, dev)
    gp.prompt(0, acc, k, v)
    cap = gp.seqlen_cap
    cu_pad = gp.padded_cu()
    acc_pad = torch.zeros((B * cap, Hq), dtype=torch.float32, device=dev)
    cu = w.cu_seqlens()
    for b, n in enumerate(w.seqlens):
        acc_pad[b * cap:b * cap + n] = acc[int(cu[b]):int(cu[b + 1])]
    pos = torch.tensor(w.seqlens, dtype=torch.int32, device=dev)
    qs = [workloads.make_queries(w, dev, 1000 + s) for s in range(nsteps)]
    gen = torch.Generator(device=dev).manual_seed(w.seed + 4243)
    kn = [torch.randn((B, Hkv, 128), generator=gen, device=dev).to(torch.float16)
          for _ in range(nsteps)]
    vn = [torch.randn((B, Hkv, 128), generator=gen, device=dev).to(torch.float16)
          for _ in range(nsteps)]
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    ws_acc = kvc.workspace(gp.geom, kvc.OP_DECODE_ACC, cap, device=dev)
    ws_gen = kvc.workspace(gp.geom, kvc.OP_GENERATE, device=dev)
    decided = torch.empty((nsteps, B, Hkv), dtype=torch.uint8, device=dev)
    pool = gp.pool
    state = [pool.pages, pool.page_table, pool.count, pool.owner, pool.free_ring,
             pool.ring_ctr, pool.dev_status, acc_pad, pos]
    snap = [t.clone() for t in state]

    def restore():
        for t, s0 in zip(state, snap):
            t.copy_(s0)

    def run_steps(with_decode=True):
        for s in range(nsteps):
            if with_decode:
                kvc.paged_decode_attention_acc(gp.geom, 0, pool, qs[s], gp.scale, out, acc_pad,
                                               cu_pad, cap, ws_acc)
            kvc.generation_step(gp.geom, 0, pool, kn[s], vn[s], pos, acc_pad, cu_pad,
                                w.alpha_h, w.alpha_l, W, decided[s], ws_gen)
            pos.add_(1)

    def timed(with_decode):
        restore()
        run_steps(with_decode)             # eager once: checks the sequence before capture
        torch.cuda.synchronize()
        status = pool.status()
        restore()
        if a.eager:
            run = lambda: run_steps(with_decode)  # noqa: E731
        else:
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_steps(with_decode)
            run = g.replay
        times = []
        for _ in range(max(a.steps, 1)):
            restore()
            e0, e1 = ev(), ev()
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / nsteps)
        return float(np.mean(times)), status | pool.status()

    policy_us, st0 = timed(False)      # the policy step alone (prompt accumulators only)
    step_us, st1 = timed(True)
    d = decided.cpu().numpy()
    counts = {"kept_high": int((d == kvc.HIGH).sum()), "demoted_low": int((d == kvc.LOW).sum()),
              "pruned": int((d == kvc.PRUNE).sum())}
    del gp, snap, acc_pad
    return step_us, policy_us, counts, st0 | st1


def prefill_flops(seqlens, Hq):
    """Matrix flops of the causal prefill with column sums: the forward pass multiplies
    q.k and p.v over the N(N+1)/2 causal pairs (4 d flops per pair); the column-sum pass
    recomputes q.k over the N(N-1)/2 strictly-later pairs (2 d flops each)."""
    fwd = sum(n * (n + 1) / 2 for n in seqlens) * Hq * 4 * 128
    cs = sum(n * (n - 1) / 2 for n in seqlens) * Hq * 2 * 128
    return fwd, cs


def time_prefill(a, w, k, v, ev, stream):
    """kvc_prefill_attention on the workload's prompts (fresh fp16 queries, fp16 output, the
    accumulators): milliseconds per call over a few calls after one warmup."""
    from mixed_precision_paged_score_amd import kvc
    dev = k.device
    T, Hq = w.total_tokens, w.num_q_heads
    g = torch.Generator(device=dev).manual_seed(w.seed + 5151)
    q = torch.randn((T, Hq, 128), generator=g, device=dev).to(torch.float16)
    out = torch.empty((T, Hq, 128), dtype=torch.float16, device=dev)
    acc = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    cu = torch.tensor(w.cu_seqlens(), device=dev)
    ms = max(w.seqlens)
    geom = kvc.make_geom(1, w.batch, Hq, w.num_kv_heads, 1, 1)
    ws = kvc.workspace(geom, kvc.OP_PREFILL, ms, device=dev)
    scale = 1.0 / math.sqrt(128)
    kvc.prefill_attention(geom, q, k, v, cu, ms, scale, out, acc, ws)
    torch.cuda.synchronize()
    reps = max(1, min(a.steps, 3))
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(reps):
        kvc.prefill_attention(geom, q, k, v, cu, ms, scale, out, acc, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps
    del q, out, acc, ws
    torch.cuda.empty_cache()
    return t


SCHEME_PAIRS = [("K8V4", "K4V2"), ("K4V8", "K2V4"), ("K8V2", "K4V1"), ("K4V2", "K4V1")]


def time_schemes(a, w, k, v, acc, qs, ev, stream):
    """Decode attention over pages in each precision scheme's slot-major layout (the prompt
    placed with kvc_quantize_and_place_scheme, then the workload's decode steps with
    kvc_paged_decode_attention_scheme): microseconds per call and algorithmic bytes, a live
    token costing 16 (k + v) code bytes, 8 parameter bytes and 4 position bytes."""
    from mixed_precision_paged_score_amd import kvc, pipeline
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=k.device)
    res = {}
    path = pipeline.PromptPath(w, k.device)
    for high, low in SCHEME_PAIRS:
        sc = kvc.make_scheme(high, low)
        path.prompt_scheme(0, acc, k, v, sc)
        for q in qs[:2]:
            path.decode_scheme(0, q, out, sc)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for q in qs:
            path.decode_scheme(0, q, out, sc)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / len(qs)
        count = path.new_count.cpu().numpy()
        nh, nl = int(count[..., 0].sum()), int(count[..., 1].sum())
        pages = int(np.ceil(count[..., 0] / 16).sum() + np.ceil(count[..., 1] / 32).sum())
        kh, vh = kvc.FORMATS[high]
        kl, vl = kvc.FORMATS[low]
        byts = (nh * (16 * (kh + vh) + 12) + nl * (16 * (kl + vl) + 12) + 4 * pages +
                w.batch * w.num_q_heads * 128 * 6)
        res[f"{high}-{low}"] = {"us_per_call": us, "algorithmic_bytes": byts,
                                "GBps": byts / (us * 1e-6) / 1e9,
                                "frac_hbm": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                "status": path.pool.status()}
    del path
    torch.cuda.empty_cache()
    return res


def traffic_record(workload):
    """HBM bytes per decode call and per compaction round from the committed rocprofv3
    counter summary (profiles/traffic_<workload>.md), each kept only while the kernel sources
    it was measured on are unchanged."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    none = {"decode": None, "compaction": None, "decode_acc": None}
    if not os.path.exists(path):
        return none
    text = open(path).read()
    try:
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return none
    csrc = os.path.join(ROOT, "mixed_precision_paged_score_amd", "csrc")

    def same(names):
        for n in names:
            f = os.path.join(csrc, n)
            if not os.path.exists(f) or n not in rec["kernel_sources_sha256"]:
                return False
            if hashlib.sha256(open(f, "rb").read()).hexdigest() != rec["kernel_sources_sha256"][n]:
                return False
        return True
    dec_src = same(["attention.hip", "page_load.h", "workspace.h", "kvc_internal.h"])
    out = dict(none)
    if dec_src:
        out["decode"] = rec["decode_call_bytes"]["total"]
        out["decode_acc"] = rec.get("decode_acc_call_bytes", {}).get("total")
    if same(["score.hip", "compact.hip", "compact_dev.h", "quantize.hip", "quant_row.h",
             "page_io.h", "workspace.h", "kvc_internal.h"]):
        out["compaction"] = rec["compaction_round_bytes"]["total"]
    return out


def decode_algorithmic_bytes(count, B, Hq):
    """Bytes the decode must move per call, per live token-head 204 (HIGH: 128 + 64 code bytes,
    8 bytes of scale/zero, 4 of position) or 108 (LOW: 64 + 32 + 8 + 4), 4 per page id, the
    fp16 query and the fp32 output."""
    nh = count[..., 0].astype(np.int64)
    nl = count[..., 1].astype(np.int64)
    pages = -(-nh // 16) + -(-nl // 32)
    return int((nh * 204 + nl * 108 + pages * 4).sum() + B * Hq * 128 * (2 + 4))


def compaction_algorithmic_bytes(count, T, Hkv, Hq):
    """Per token-head: read K+V fp16 (512 B) and the accumulators (4 B per query head); write
    204 B per HIGH and 108 B per LOW token-head (codes, scale/zero, position); 4 B per page of
    page-table, ring and reverse-map traffic."""
    nh = count[..., 0].astype(np.int64)
    nl = count[..., 1].astype(np.int64)
    pages = int((-(-nh // 16) + -(-nl // 32)).sum())
    return int(T * Hkv * 512 + T * Hq * 4 + nh.sum() * 204 + nl.sum() * 108 + pages * 4)


def cpu_baseline(w, k, v, acc, qs, nreq):
    """Oracle (as it is) on the first `nreq` requests: score, allocation, page images and one
    decode step; returns (token-heads per second, seconds, description)."""
    from oracle import attention as oatt, place, pool as opool, score as osc
    import dataclasses
    ws = dataclasses.replace(w, batch=nreq, seqlens=w.seqlens[:nreq])
    T = ws.total_tokens
    kc = k[:T].cpu().numpy()
    vc = v[:T].cpu().numpy()
    ac = acc[:T].cpu().numpy()
    qc = qs[0][:nreq].cpu().numpy()
    t0 = time.perf_counter()
    tier, count, _ = osc.score_tokens(ac, ws.cu_seqlens(), ws.num_kv_heads, ws.alpha_h,
                                      ws.alpha_l, ws.window)
    pl = opool.Pool(1, nreq, ws.num_kv_heads, ws.row_capacity, ws.num_pages)
    pl.compact(0, count)
    cu = ws.cu_seqlens()
    G = ws.group
    for b in range(nreq):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in range(ws.num_kv_heads):
            place.head_pages(kc[lo:hi, h], vc[lo:hi, h], tier[lo:hi, h])
            kd, vd = place.head_dequantized(kc[lo:hi, h], vc[lo:hi, h], tier[lo:hi, h])
            oatt.decode_group(qc[b, h * G:(h + 1) * G], kd, vd, 1 / math.sqrt(128))
    dt = time.perf_counter() - t0
    return T * ws.num_kv_heads / dt, dt, (f"{nreq} request(s) x {ws.seqlens[0]} tokens x "
                                          f"{ws.num_kv_heads} KV heads: score, allocation, "
                                          f"page images, one decode step")


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; --gpus above 1 is not supported (the path would shard requests and KV heads across GPUs, each running this same single-GPU step)",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    from mixed_precision_paged_score_amd import kvc, pipeline, workloads
    dev = "cuda:0"
    torch.cuda.set_device(0)
    # the pool holds two layouts of the layer: every step's prompt-mode compaction returns the
    # previous step's pages to the ring tail and takes the new ones from the ring head, and
    # an all-or-nothing round may only hand out pages that are free when it starts
    w = workloads.workload(a.workload)
    w = dataclasses.replace(w, num_pages=2 * w.num_pages)
    nsteps_dec = a.decode_steps if a.decode_steps is not None else w.decode_steps
    k, v = workloads.make_kv(w, dev)
    acc = workloads.make_acc(w, k, dev)
    qs = [workloads.make_queries(w, dev, s) for s in range(nsteps_dec)]
    path = pipeline.PromptPath(w, dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if not a.eager:
        # the step's library calls are captured once into two HIP graphs (prompt round,
        # decode steps); every replay redoes all of the work on the resident inputs
        path.prompt(0, acc, k, v)
        torch.cuda.synchronize()
        g_prompt = path.capture_prompt(0, acc, k, v)
        g_dec = path.capture_decode(0, qs, out)
        torch.cuda.synchronize()

    spin = spin_cycles(stream)

    def step(record):
        e0, e1, e2 = ev(), ev(), ev()
        torch.cuda._sleep(spin)            # the host queues the step while the GPU spins
        e0.record(stream)
        if a.eager:
            path.prompt(0, acc, k, v)
        else:
            g_prompt.replay()
        e1.record(stream)
        if a.eager:
            for s in range(nsteps_dec):
                path.decode(0, qs[s], out)
        else:
            g_dec.replay()
        e2.record(stream)
        if record is not None:
            record.append((e0, e1, e2))

    for _ in range(a.warmup):
        step(None)
    torch.cuda.synchronize()
    status = path.pool.status()
    recs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    retier = None
    if "round_every" in w.extra and not a.no_retier:
        r_us, r_th, r_heads, r_bytes = time_retier_round(w, k, v, acc, ev, stream, spin)
        retier = {"us_per_round": r_us, "token_heads": r_th, "heads_rebuilt": r_heads,
                  "heads": w.batch * w.num_kv_heads, "round_every": w.extra["round_every"],
                  "token_heads_per_s": r_th / (r_us * 1e-6), "algorithmic_bytes": r_bytes,
                  "GBps": r_bytes / r_us / 1e3,
                  "frac_hbm": r_bytes / r_us / 1e3 / HBM_PEAK_GBPS}
    acc_us = None
    if not a.no_acc and nsteps_dec > 0:
        acc_us = time_decode_acc(a, path, qs, out, nsteps_dec, ev, stream)
    gen = None
    if a.gen_steps > 0:
        step_us, policy_us, gen_counts, gen_status = time_generation_loop(
            a, w, k, v, acc, ev, stream, a.gen_steps)
        gen = {"us_per_step": step_us, "policy_us_per_step": policy_us, "steps": a.gen_steps,
               "heads": w.batch * w.num_kv_heads, "decisions": gen_counts,
               "status": gen_status}
    schemes = None
    if not a.no_schemes and nsteps_dec > 0:
        schemes = time_schemes(a, w, k, v, acc, qs, ev, stream)
    pre = None
    if not a.no_prefill:
        pre_ms = time_prefill(a, w, k, v, ev, stream)
        fl_fwd, fl_cs = prefill_flops(w.seqlens, w.num_q_heads)
        pre = {"ms_per_call": pre_ms, "TFLOPs": (fl_fwd + fl_cs) / pre_ms / 1e9,
               "frac_mfma_fp16": (fl_fwd + fl_cs) / pre_ms / 1e9 / MFMA_FP16_PEAK_TFLOPS,
               "flops": fl_fwd + fl_cs, "flops_forward": fl_fwd, "flops_column_sums": fl_cs,
               "peak_TFLOPs": MFMA_FP16_PEAK_TFLOPS}
    comp_ms = [e0.elapsed_time(e1) for (e0, e1, e2) in recs]
    dec_ms = [e1.elapsed_time(e2) / max(nsteps_dec, 1) for (e0, e1, e2) in recs]
    count = path.new_count.cpu().numpy()
    T, Hkv, Hq, B = w.total_tokens, w.num_kv_heads, w.num_q_heads, w.batch
    token_heads = T * Hkv
    comp_s = float(np.mean(comp_ms)) / 1e3
    dec_s = float(np.mean(dec_ms)) / 1e3
    dbytes = decode_algorithmic_bytes(count, B, Hq)
    # the accumulating decode also reads and writes one fp32 accumulator per live token and
    # query head
    acc_bytes = int(count.sum()) * (Hq // Hkv) * 8
    cbytes = compaction_algorithmic_bytes(count, T, Hkv, Hq)
    dec_gbps = dbytes / dec_s / 1e9
    comp_gbps = cbytes / comp_s / 1e9
    ms_per_step = wall / a.steps * 1e3
    nh, nl = int(count[..., 0].sum()), int(count[..., 1].sum())
    traffic = traffic_record(w.name)
    dec_traffic, comp_traffic = traffic["decode"], traffic["compaction"]
    res = {
        "metric": "KV tokens compacted/s + paged decode attn GB/s (fraction of HBM peak)",
        "value": token_heads / comp_s,
        "unit": "KV token-heads compacted/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in, u8 codes, fp32 scale math",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.num_layers, "batch": B,
                   "seq_len": w.seqlens[0] if len(set(w.seqlens)) == 1 else "ragged",
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128, "pages": w.num_pages,
                   "decode_steps": nsteps_dec, "alpha_h": w.alpha_h, "alpha_l": w.alpha_l,
                   "window": w.window},
        "compaction": {"ms": comp_s * 1e3, "GBps": comp_gbps, "frac_hbm": comp_gbps / HBM_PEAK_GBPS,
                       "algorithmic_bytes": cbytes, "token_heads": token_heads,
                       "high": nh, "low": nl, "pruned": token_heads - nh - nl,
                       "traffic": comp_traffic},
        "decode_GBps": dec_gbps,
        "decode": {"us_per_call": dec_s * 1e6, "GBps": dec_gbps,
                   "frac_hbm": dec_gbps / HBM_PEAK_GBPS, "algorithmic_bytes": dbytes},
        "retier_round": retier,
        "decode_with_score_accumulation": None if acc_us is None else {
            "us_per_call": acc_us,
            "GBps": (dbytes + acc_bytes) / (acc_us / 1e6) / 1e9,
            "frac_hbm": (dbytes + acc_bytes) / (acc_us / 1e6) / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes": dbytes + acc_bytes, "traffic": traffic["decode_acc"]},
        "generation_loop": gen,
        "prefill": pre,
        "precision_schemes": schemes,
        "roofline": {"bound": "hbm", "kernel": "paged_decode_attention (main + combine)",
                     "achieved": dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dec_gbps / HBM_PEAK_GBPS, "traffic": dec_traffic},
        "pool_status": status,
        "ceilings": measure_ceilings(),
    }
    if not a.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            rate, secs, desc = cpu_baseline(w, k, v, acc, qs, a.cpu_sample_requests)
        res["cpu_baseline"] = {"value": rate, "unit": "KV token-heads compacted/s",
                               "cores": 1, "kind": "oracle", "sample": desc,
                               "seconds": secs}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
