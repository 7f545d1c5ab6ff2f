"""Benchmark of the DiffKV-style compaction + mixed-precision paged decode hot path on one
MI355X.

A step is one pass of the whole path over one batch of synthetic input resident in HBM: for
every layer, score_tokens -> compact_pages (prompt mode: the layer's previous pages go back to
the ring, new ones are assigned) -> quantize_and_place, then the workload's decode steps of
paged_decode_attention on every layer (fresh queries).  Default workload: the full-model
shape, 64 layers x 64 requests (lengths log-uniform in [1K, 32K]) x 64 query / 8 KV heads,
Zipf(1.1) accumulators, 3 key outlier channels x10 per layer, one decode step per layer; all
64 layers' K/V and accumulators (151 GB) are generated once and stay resident, the pool holds
2^24 pages (58 GB; the literal 2^20 holds only a few layers).  Calls are launched eagerly from
Python (single-layer workloads replay captured HIP graphs); HIP events on the stream bracket
the step's compaction phase (all layers' rounds) and its decode phase (all layers' calls), and
the per-call figures divide by the number of calls.  Each step starts with a short GPU spin
outside the timed region, so that the host has queued the step before the GPU reaches it.

Prints one JSON line.  `value` = KV token-heads compacted per second over the step's
compaction (all layers); `decode` = paged decode attention per call, with algorithmic bytes
per second; `roofline` is for the decode call (main + combine kernel), the metric's attention
half; `roofline_compaction` for the layer's compaction round.  `cold` repeats single calls
after a 1 GiB scratch read (which evicts the L2s and the 256 MB Infinity Cache) and reports
median and minimum over >= 20 reps.  `cpu_baseline` times the CPU oracle on layer 0 of the
same workload recipe on one core and on the host's cores (run before the GPU is touched).
Beside the step (skipped with --no-extras): `w3` the 16 x 32,768-token single-layer workload
(compaction round and 64 decode steps per step as graphs) with, on its data,
`decode_with_score_accumulation`, `generation_loop` (decode with score accumulation + the
per-step policy), `prefill` (causal prefill with the prompt accumulators, against the fp16
matrix-core peak) and `precision_schemes`; `w4` the chain-of-thought workload grown to
4,096 + 16,384 tokens through its full schedule (one appended token per head per step, a
re-tier round every 128 steps), with the decode and the last re-tier round timed at that
length.
"""
import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0      # dense fp16 matrix-core peak of MI355X
MAX_CPU_WORKERS = 16                # the host-core share of one GPU of an 8-GPU node
FLUSH_BYTES = 1 << 30               # scratch read before a cold rep


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="single calls after a 1 GiB scratch read, per kind (median, minimum)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the single-layer and chain-of-thought workloads beside the step")
    ap.add_argument("--no-acc", action="store_true",
                    help="skip the decode attention with score accumulation")
    ap.add_argument("--gen-steps", type=int, default=64,
                    help="steps of the generation loop timed on the single-layer workload")
    ap.add_argument("--no-schemes", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-w4", action="store_true",
                    help="skip the chain-of-thought workload")
    ap.add_argument("--eager", action="store_true",
                    help="launch every library call from Python instead of replaying HIP graphs")
    ap.add_argument("--group-sweep", action="store_true",
                    help="only time the decode at G = 1, 2, 4, 8, 16 query heads per KV head")
    ap.add_argument("--three-calls", action="store_true",
                    help="run each layer's round as the three calls (score, compact, quantize/place) "
                         "instead of kvc_compaction_round")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates HBM counters)")
    return ap.parse_args()


# ---- algorithmic bytes ----------------------------------------------------------------------
def decode_algorithmic_bytes(count, B, Hq):
    """Bytes the decode must move per call: per live token-head its codes and its scale/zero
    pairs, 200 B HIGH (128 + 64 code bytes + 8) or 104 B LOW (64 + 32 + 8) -- the positions
    stored in the pages are not read by the decode --, 4 per page id, the fp16 query and the
    fp32 output."""
    nh = count[..., 0].astype(np.int64)
    nl = count[..., 1].astype(np.int64)
    pages = -(-nh // 16) + -(-nl // 32)
    return int((nh * 200 + nl * 104 + pages * 4).sum() + B * Hq * 128 * (2 + 4))


def decode_acc_algorithmic_bytes(count, B, Hq, Hkv):
    """The accumulating decode also reads each live token's position (4 B) and reads and
    writes one fp32 accumulator per live token and query head."""
    live = int(count.sum())
    return decode_algorithmic_bytes(count, B, Hq) + live * 4 + live * (Hq // Hkv) * 8


def compaction_algorithmic_bytes(count, T, Hkv, Hq):
    """Per token-head: read the accumulators (4 B per query head) of every token and the K+V
    fp16 rows (512 B) of every kept token (a pruned token's rows are never needed); write
    204 B per HIGH and 108 B per LOW token-head (codes, scale/zero, position); 4 B per page of
    page-table, ring and reverse-map traffic."""
    nh = count[..., 0].astype(np.int64)
    nl = count[..., 1].astype(np.int64)
    pages = int((-(-nh // 16) + -(-nl // 32)).sum())
    kept = int(nh.sum() + nl.sum())
    return int(T * Hq * 4 + kept * 512 + nh.sum() * 204 + nl.sum() * 108 + pages * 4)


def pages_of(cnt):
    return int((-(-cnt[..., 0] // 16)).sum() + (-(-cnt[..., 1] // 32)).sum())


# ---- CPU baseline (the oracle as it stands), before the GPU is touched ----------------------
_CPU = {}
CPU_SAMPLE_REQUESTS = 64


def _cpu_head(bh):
    """Oracle work of one (request, KV head): score and tier its tokens from its query heads'
    accumulators, then the page images, the dequantized keys/values and one decode step.
    Returns its (#HIGH, #LOW) counts."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as oatt, place, score as osc
    b, h = bh
    d = _CPU
    lo, hi = int(d["cu"][b]), int(d["cu"][b + 1])
    n = hi - lo
    G = d["G"]
    with threadpool_limits(1):
        tier, count, _ = osc.score_tokens(d["acc"][lo:hi, h * G:(h + 1) * G], np.array([0, n]),
                                          1, d["ah"], d["al"], d["W"])
        k, v, t = d["k"][lo:hi, h], d["v"][lo:hi, h], tier[:, 0]
        place.head_pages(k, v, t)
        kd, vd = place.head_dequantized(k, v, t)
        oatt.decode_group(d["q"][b, h * G:(h + 1) * G], kd, vd, d["scale"])
    return count[0, 0]


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, nreq=CPU_SAMPLE_REQUESTS):
    """The oracle on a seeded sample of `nreq` requests of workload w (their lengths, inputs
    drawn on the CPU with the workload's recipe for layer 0): score, allocation, page images
    and one decode step of every (request, KV head), once on one core and once over a process
    pool of the host's cores (one (request, KV head) per task, longest first; allocation, a
    sequential prefix over the heads, in the parent).  Returns a dict."""
    import multiprocessing as mp
    from oracle import pool as opool
    from mixed_precision_paged_score_amd import workloads
    rng = np.random.default_rng(w.seed + 17)
    pick = sorted(rng.choice(w.batch, min(nreq, w.batch), replace=False).tolist())
    ws = dataclasses.replace(w, batch=len(pick), seqlens=[w.seqlens[b] for b in pick])
    k, v = workloads.make_kv(ws, "cpu", 0)
    acc = workloads.make_acc(ws, k, "cpu", 0)
    q = workloads.make_queries(ws, "cpu", 0, 0)
    _CPU.update(k=k.numpy(), v=v.numpy(), acc=acc.numpy(), q=q.numpy(), cu=ws.cu_seqlens(),
                G=ws.group, ah=ws.alpha_h, al=ws.alpha_l, W=ws.window,
                scale=1.0 / math.sqrt(128))
    del k, v, acc, q
    H = ws.num_kv_heads
    token_heads = ws.total_tokens * H
    tasks = sorted(((b, h) for b in range(ws.batch) for h in range(H)),
                   key=lambda x: -ws.seqlens[x[0]])

    def allocate(done):
        counts = np.zeros((ws.batch, H, 2), np.int64)
        for (b, h), c in done.items():
            counts[b, h] = c
        pl = opool.Pool(1, ws.batch, H, ws.row_capacity, 1 << 24)
        pl.compact(0, counts)

    t0 = time.perf_counter()
    allocate({bh: _cpu_head(bh) for bh in tasks})
    t1 = time.perf_counter() - t0
    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    nproc = max(1, min(MAX_CPU_WORKERS, ncpu, len(tasks)))
    ctx = mp.get_context("fork")
    with ctx.Pool(nproc) as pool:
        pool.map(_cpu_head, tasks[-nproc:])             # workers up, imports done
        t0 = time.perf_counter()
        allocate(dict(zip(tasks, pool.map(_cpu_head, tasks, chunksize=1))))
        tn = time.perf_counter() - t0
    _CPU.clear()
    sample = (f"{ws.batch} of the {w.batch} requests of {w.name} (seeded), {ws.total_tokens} "
              f"tokens x {H} KV heads, layer 0 inputs drawn on the CPU with the workload's "
              f"recipe; score, allocation, page images, one decode step")
    return {"value": token_heads / tn, "unit": "KV token-heads compacted/s", "cores": nproc,
            "kind": "oracle", "sample": sample, "seconds": tn, "cpu_model": cpu_model(),
            "nproc": ncpu,
            "single_core": {"value": token_heads / t1, "cores": 1, "seconds": t1}}


# ---- GPU helpers ---------------------------------------------------------------------------
def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch, 4 launches.
    Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its per-dispatch counters give the factor
    that turns those counters into bytes."""
    import torch
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
    import torch
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
    before a timed region, it lets the host submit the region's work first, so that the
    events time the GPU's work and not the host's submission."""
    import torch
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


class Timer:
    """HIP event pairs on one stream."""

    def __init__(self, stream):
        import torch
        self.torch, self.stream, self.pairs = torch, stream, []

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def us(self, e0, e1):
        return e0.elapsed_time(e1) * 1e3


def evict(flush):
    """Reads the 1 GiB scratch buffer (written once when it was made): afterwards the L2s and
    the 256 MB Infinity Cache hold only its clean lines and none of a timed call's data.  A
    write would leave ~260 MB of dirty lines that the next call pays to write back (measured:
    the 16 x 32K decode at 184 us after a 1 GiB fill against 136 us warm)."""
    import torch
    flush.view(torch.int32).sum()


def cold_reps(reps, flush, run, timer):
    """`reps` single calls run(r), each after a read of the 1 GiB scratch buffer that evicts
    the caches (evict()); microseconds per rep."""
    import torch
    out = []
    for r in range(reps):
        evict(flush)
        e0 = timer.ev()
        run(r)
        e1 = timer.ev()
        out.append((e0, e1))
    torch.cuda.synchronize()
    return [timer.us(a, b) for a, b in out]


def stats(us, nbytes):
    """Median and minimum of per-rep microseconds; GB/s and fraction of the HBM peak at each
    (nbytes: per rep)."""
    us = np.asarray(us, np.float64)
    nb = np.asarray(nbytes, np.float64) if np.ndim(nbytes) else np.full(len(us), float(nbytes))
    gbps = nb / us / 1e3
    return {"reps": int(len(us)), "us_median": float(np.median(us)), "us_min": float(us.min()),
            "GBps_median": float(np.median(gbps)), "GBps_max": float(gbps.max()),
            "frac_hbm_median": float(np.median(gbps)) / HBM_PEAK_GBPS,
            "frac_hbm_max": float(gbps.max()) / HBM_PEAK_GBPS}


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
    out = dict(none)
    if same(["attention.hip", "page_load.h", "workspace.h", "kvc_internal.h"]):
        out["decode"] = rec.get("decode_call_bytes", {}).get("total")
        out["decode_acc"] = rec.get("decode_acc_call_bytes", {}).get("total")
    if same(["score.hip", "compact.hip", "compact_dev.h", "quantize.hip", "quant_row.h",
             "page_io.h", "workspace.h", "kvc_internal.h"]):
        out["compaction"] = rec.get("compaction_round_bytes", {}).get("total")
    return out


# ---- the step --------------------------------------------------------------------------------
def run_step_workload(a, w, stream, spin, flush, steps, warmup, nsteps_dec, graphs):
    """The step on workload w: all layers' prompt rounds, then nsteps_dec decode calls per
    layer; inputs generated once per layer and kept resident.  Returns a result dict and the
    path (for extras on its data)."""
    import torch
    from mixed_precision_paged_score_amd import pipeline, workloads
    dev = "cuda:0"
    L = w.num_layers
    ins = []
    for layer in range(L):
        k, v = workloads.make_kv(w, dev, layer)
        acc = workloads.make_acc(w, k, dev, layer)
        qs = [workloads.make_queries(w, dev, s, layer) for s in range(nsteps_dec)]
        ins.append((k, v, acc, qs))
    torch.cuda.synchronize()
    path = pipeline.PromptPath(w, dev)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
    timer = Timer(stream)
    # a layer's round: kvc_compaction_round (up to 1024 KV heads), else the three calls
    fused = not a.three_calls and w.batch * w.num_kv_heads <= 1024
    round_fn = path.prompt_fused if fused else path.prompt
    # the first pass places every layer (and, in graph mode, makes the workspaces before capture)
    for layer in range(L):
        k, v, acc, _ = ins[layer]
        round_fn(layer, acc, k, v)
    torch.cuda.synchronize()
    counts = [path.pool.count[layer].cpu().numpy() for layer in range(L)]
    g_prompt = g_dec = None
    if graphs:
        g_prompt = path.capture_prompt(0, ins[0][2], ins[0][0], ins[0][1], fused=fused)
        g_dec = path.capture_decode(0, ins[0][3], out)
        torch.cuda.synchronize()

    # HIP events only at the phase boundaries: an event recorded between two calls leaves the
    # GPU idle for ~5 us before the next kernel (measured in a kernel trace), which the layers of
    # a model issued back to back do not pay
    def step(rec):
        torch.cuda._sleep(spin)            # the host queues the step while the GPU spins
        ev = [timer.ev()]
        for layer in range(L):
            if graphs:
                g_prompt.replay()
            else:
                k, v, acc, _ = ins[layer]
                round_fn(layer, acc, k, v)
        ev.append(timer.ev())
        for layer in range(L):
            if graphs:
                g_dec.replay()
            else:
                for q in ins[layer][3]:
                    path.decode(layer, q, out)
        ev.append(timer.ev())
        if rec is not None:
            rec.append(ev)

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    status = path.pool.status()
    recs = []
    t0 = time.perf_counter()
    for _ in range(steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    status |= path.pool.status()
    comp_us = np.array([timer.us(e[0], e[1]) / L for e in recs])          # per layer round
    dec_us = np.array([timer.us(e[1], e[2]) / (L * max(nsteps_dec, 1)) for e in recs])
    B, Hq, Hkv, T = w.batch, w.num_q_heads, w.num_kv_heads, w.total_tokens
    dbytes = np.array([decode_algorithmic_bytes(c, B, Hq) for c in counts])
    cbytes = np.array([compaction_algorithmic_bytes(c, T, Hkv, Hq) for c in counts])
    token_heads = L * T * Hkv
    comp_s = comp_us.mean() * L / 1e6                  # all layers' rounds per step
    dec_call_us = float(dec_us.mean())
    dec_gbps = float(dbytes.mean()) / dec_call_us / 1e3
    comp_round_us = float(comp_us.mean())
    comp_gbps = float(cbytes.mean()) / comp_round_us / 1e3
    nh = int(sum(c[..., 0].sum() for c in counts))
    nl = int(sum(c[..., 1].sum() for c in counts))
    res = {
        "value": token_heads / comp_s,
        "ms_per_step": wall / steps * 1e3,
        "compaction": {"path": "kvc_compaction_round" if fused else
                               "kvc_score_tokens + kvc_compact_pages + kvc_quantize_and_place",
                       "us_per_layer_round": comp_round_us, "ms_all_layers": comp_s * 1e3,
                       "GBps": comp_gbps, "frac_hbm": comp_gbps / HBM_PEAK_GBPS,
                       "algorithmic_bytes_per_layer": float(cbytes.mean()),
                       "token_heads": token_heads, "high": nh, "low": nl,
                       "pruned": token_heads - nh - nl},
        "decode": {"us_per_call": dec_call_us, "GBps": dec_gbps,
                   "frac_hbm": dec_gbps / HBM_PEAK_GBPS,
                   "algorithmic_bytes_per_call": float(dbytes.mean()),
                   "calls_per_step": L * nsteps_dec,
                   "us_per_call_min_step": float(dec_us.min()),
                   "us_per_call_max_step": float(dec_us.max())},
        "pool_status": status,
    }
    # cold: one call after a 1 GiB scratch read, layers taken in turn
    reps = max(a.cold_reps, 1)

    def dec_one(r):
        layer = (r * 37) % L
        path.decode(layer, ins[layer][3][0], out)

    def comp_one(r):
        layer = (r * 37) % L
        k, v, acc, _ = ins[layer]
        round_fn(layer, acc, k, v)

    def comp_three(r):
        layer = (r * 37) % L
        k, v, acc, _ = ins[layer]
        path.prompt(layer, acc, k, v)
    lay = [(r * 37) % L for r in range(reps)]
    res["cold"] = {
        "decode": stats(cold_reps(reps, flush, dec_one, timer), dbytes[lay]),
        "compaction_round": stats(cold_reps(reps, flush, comp_one, timer), cbytes[lay]),
        "protocol": "a 1 GiB scratch read before each rep (evicts the L2s and the Infinity "
                    "Cache, leaves no dirty lines); one call per rep, layers in turn",
    }
    if fused:
        # the same rounds as the three separate calls, for comparison
        res["cold"]["compaction_round_three_calls"] = stats(
            cold_reps(reps, flush, comp_three, timer), cbytes[lay])
    res["pool_status"] |= path.pool.status()
    return res, path, ins, counts


def time_decode_acc(a, path, qs, out, nsteps_dec, stream):
    """Decode attention with score accumulation (every cached token's weight added into fp32
    accumulators), the same decode steps, replayed as one graph; microseconds per call."""
    import torch
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
    timer = Timer(stream)
    e0 = timer.ev()
    for _ in range(a.steps):
        run()
    e1 = timer.ev()
    torch.cuda.synchronize()
    return timer.us(e0, e1) / (a.steps * nsteps_dec)


def time_generation_loop(a, w, k, v, acc, stream, nsteps):
    """The generation phase of one layer, `nsteps` steps after the workload's prompt: each step
    is a decode with score accumulation (a fresh query per request and query head) into one
    padded accumulator buffer [B][N + nsteps][Hq], then kvc_generation_step on the same buffer
    (append the new tokens, score the token leaving the window), captured as one graph; before
    each replay the pool, accumulators and positions are restored from a snapshot taken after
    the prompt (outside the timed region).  Returns us per step, the policy step alone per
    step, and the decisions of the last replay."""
    import torch
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
    timer = Timer(stream)

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
            e0 = timer.ev()
            run()
            e1 = timer.ev()
            torch.cuda.synchronize()
            times.append(timer.us(e0, e1) / nsteps)
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


def time_prefill(a, w, k, v, stream):
    """kvc_prefill_attention on the workload's prompts (fresh fp16 queries, fp16 output, the
    accumulators): milliseconds per call over a few calls after one warmup."""
    import torch
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
    timer = Timer(stream)
    e0 = timer.ev()
    for _ in range(reps):
        kvc.prefill_attention(geom, q, k, v, cu, ms, scale, out, acc, ws)
    e1 = timer.ev()
    torch.cuda.synchronize()
    t = timer.us(e0, e1) / 1e3 / reps
    del q, out, acc, ws
    torch.cuda.empty_cache()
    return t


SCHEME_PAIRS = [("K8V4", "K4V2"), ("K4V8", "K2V4"), ("K8V2", "K4V1"), ("K4V2", "K4V1")]


def time_schemes(w, k, v, acc, qs, stream):
    """Decode attention over pages in each precision scheme's slot-major layout (the prompt
    placed with kvc_quantize_and_place_scheme, then the workload's decode steps with
    kvc_paged_decode_attention_scheme): microseconds per call and algorithmic bytes, a live
    token costing 16 (k + v) code bytes and 8 parameter bytes."""
    import torch
    from mixed_precision_paged_score_amd import kvc, pipeline
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=k.device)
    res = {}
    path = pipeline.PromptPath(w, k.device)
    timer = Timer(stream)
    for high, low in SCHEME_PAIRS:
        sc = kvc.make_scheme(high, low)
        path.prompt_scheme(0, acc, k, v, sc)
        for q in qs[:2]:
            path.decode_scheme(0, q, out, sc)
        torch.cuda.synchronize()
        e0 = timer.ev()
        for q in qs:
            path.decode_scheme(0, q, out, sc)
        e1 = timer.ev()
        torch.cuda.synchronize()
        us = timer.us(e0, e1) / len(qs)
        count = path.new_count.cpu().numpy()
        nh, nl = int(count[..., 0].sum()), int(count[..., 1].sum())
        kh, vh = kvc.FORMATS[high]
        kl, vl = kvc.FORMATS[low]
        byts = (nh * (16 * (kh + vh) + 8) + nl * (16 * (kl + vl) + 8) + 4 * pages_of(count) +
                w.batch * w.num_q_heads * 128 * 6)
        res[f"{high}-{low}"] = {"us_per_call": us, "algorithmic_bytes": byts,
                                "GBps": byts / (us * 1e-6) / 1e9,
                                "frac_hbm": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                "status": path.pool.status()}
    del path
    torch.cuda.empty_cache()
    return res


def decode_by_group(a, stream, flush, groups=(1, 2, 4, 8, 16)):
    """The decode at G = 1, 2, 4, 8 and 16 query heads per KV head, on the 16 x 32,768-token
    shape with its 8 KV heads and the same keys and values.  The score product is one 16x16
    matrix-core tile per pair of 16-token tiles (G query heads of tile A and of tile B), so at
    G < 8 part of its columns are zero: per G, microseconds per call back to back (64 calls)
    and cold (a 1 GiB scratch read before each), against the algorithmic bytes."""
    import torch
    from mixed_precision_paged_score_amd import pipeline, workloads
    dev = "cuda:0"
    base = workloads.workload(3)
    k, v = workloads.make_kv(base, dev)
    timer = Timer(stream)
    res = {}
    for G in groups:
        w = dataclasses.replace(base, name=f"w3-16x32768-g{G}", num_q_heads=base.num_kv_heads * G)
        acc = workloads.make_acc(w, k, dev)
        path = pipeline.PromptPath(w, dev)
        path.prompt(0, acc, k, v)
        qs = [workloads.make_queries(w, dev, s) for s in range(8)]
        out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=dev)
        for q in qs[:2]:
            path.decode(0, q, out)
        torch.cuda.synchronize()
        e0 = timer.ev()
        for _ in range(8):
            for q in qs:
                path.decode(0, q, out)
        e1 = timer.ev()
        torch.cuda.synchronize()
        us = timer.us(e0, e1) / (8 * len(qs))
        cold = cold_reps(max(a.cold_reps // 2, 1), flush,
                         lambda r: path.decode(0, qs[r % len(qs)], out), timer)
        cnt = path.new_count.cpu().numpy()
        byts = decode_algorithmic_bytes(cnt, w.batch, w.num_q_heads)
        res[str(G)] = {"us_per_call": us, "GBps": byts / us / 1e3,
                       "frac_hbm": byts / us / 1e3 / HBM_PEAK_GBPS, "algorithmic_bytes": byts,
                       "cold": stats(cold, byts), "status": path.pool.status()}
        del path, acc, out
        torch.cuda.empty_cache()
    return res


def extras_w3(a, stream, spin, flush):
    """The 16 x 32,768-token single-layer workload: its step (compaction round + 64 decode
    steps, graphs) and, on its data, the accumulating decode, the generation loop, the prefill
    and the precision-scheme decodes."""
    import torch
    from mixed_precision_paged_score_amd import workloads
    w = workloads.workload(3)
    w = dataclasses.replace(w, num_pages=2 * w.num_pages)     # two layouts: repeated rounds
    res, path, ins, counts = run_step_workload(a, w, stream, spin, flush, a.steps, a.warmup,
                                               w.decode_steps, graphs=not a.eager)
    k, v, acc, qs = ins[0]
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device="cuda:0")
    traffic = traffic_record(w.name)
    res["decode"]["traffic"] = traffic["decode"]
    res["compaction"]["traffic"] = traffic["compaction"]
    res["config"] = {"workload": w.name, "layers": 1, "batch": w.batch, "seq_len": 32768,
                     "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                     "decode_steps": w.decode_steps, "pages": w.num_pages}
    if not a.no_acc:
        acc_us = time_decode_acc(a, path, qs, out, len(qs), stream)
        abytes = decode_acc_algorithmic_bytes(counts[0], w.batch, w.num_q_heads, w.num_kv_heads)
        res["decode_with_score_accumulation"] = {
            "us_per_call": acc_us, "GBps": abytes / acc_us / 1e3,
            "frac_hbm": abytes / acc_us / 1e3 / HBM_PEAK_GBPS, "algorithmic_bytes": abytes,
            "traffic": traffic["decode_acc"]}
    if a.gen_steps > 0:
        step_us, policy_us, gen_counts, gen_status = time_generation_loop(
            a, w, k, v, acc, stream, a.gen_steps)
        res["generation_loop"] = {"us_per_step": step_us, "policy_us_per_step": policy_us,
                                  "steps": a.gen_steps, "heads": w.batch * w.num_kv_heads,
                                  "decisions": gen_counts, "status": gen_status}
    if not a.no_schemes:
        res["precision_schemes"] = time_schemes(w, k, v, acc, qs, stream)
    if not a.no_prefill:
        pre_ms = time_prefill(a, w, k, v, stream)
        fl_fwd, fl_cs = prefill_flops(w.seqlens, w.num_q_heads)
        res["prefill"] = {"ms_per_call": pre_ms, "TFLOPs": (fl_fwd + fl_cs) / pre_ms / 1e9,
                          "frac_mfma_fp16": (fl_fwd + fl_cs) / pre_ms / 1e9 / MFMA_FP16_PEAK_TFLOPS,
                          "flops": fl_fwd + fl_cs, "flops_forward": fl_fwd,
                          "flops_column_sums": fl_cs, "peak_TFLOPs": MFMA_FP16_PEAK_TFLOPS}
    del path, ins
    torch.cuda.empty_cache()
    return res


def extras_w4(a, stream, flush):
    """The chain-of-thought workload through its full schedule: 16 x 4,096-token prompts, then
    16,384 steps each appending one token per (request, KV head), a re-tier round every 128
    steps whose accumulators add that round's Zipf weights to the sums of the rounds before.  Timed: the prompt's
    compaction round, the decode at the grown length (4,096 + 16,384 tokens) and the last
    re-tier round (rerun from a snapshot of the state before it), each after a 1 GiB scratch
    read, median and minimum over reps."""
    import torch
    from mixed_precision_paged_score_amd import kvc, pipeline, workloads
    dev = "cuda:0"
    w = workloads.workload(4)
    R, steps = int(w.extra["round_every"]), int(w.decode_steps)
    B, Hkv, Hq, T0 = w.batch, w.num_kv_heads, w.num_q_heads, w.total_tokens
    k, v = workloads.make_kv(w, dev)
    acc = workloads.make_acc(w, k, dev)
    timer = Timer(stream)
    reps = max(a.cold_reps, 1)
    # the prompt round (prompt mode: each rep returns the previous rep's pages to the ring)
    pp = pipeline.PromptPath(w, dev)
    pp.prompt(0, acc, k, v)
    pp.prompt_fused(0, acc, k, v)
    pr_us = cold_reps(reps, flush, lambda r: pp.prompt_fused(0, acc, k, v), timer)
    pr3_us = cold_reps(reps, flush, lambda r: pp.prompt(0, acc, k, v), timer)
    cnt0 = pp.new_count.cpu().numpy()
    pbytes = compaction_algorithmic_bytes(cnt0, T0, Hkv, Hq)
    res = {"prompt_round": stats(pr_us, pbytes),
           "prompt_round_three_calls": stats(pr3_us, pbytes)}
    res["prompt_round"]["path"] = "kvc_compaction_round"
    status = pp.pool.status()
    del pp
    path = pipeline.GenerationPath(w, max(w.seqlens) + steps, dev)
    path.prompt(0, acc, k, v)
    g = torch.Generator(device=dev).manual_seed(w.seed + 99)
    last = None
    acc_cur, lens_prev = acc, list(w.seqlens)
    for s in range(steps):
        kn = torch.randn((B, Hkv, 128), generator=g, device=dev).to(torch.float16)
        vn = torch.randn((B, Hkv, 128), generator=g, device=dev).to(torch.float16)
        path.append(0, kn, vn)
        if (s + 1) % R == 0:
            # each round's weights are added to the sums of the rounds before
            wr = dataclasses.replace(w, seqlens=list(path.lens), seed=w.seed + 1000 * (s + 1))
            acc_cur = workloads.make_acc_zipf_round(wr, acc_cur, lens_prev, dev, (s + 1) // R)
            lens_prev = list(path.lens)
            if s + 1 == steps:
                last = acc_cur
                break
            path.retier(0, acc_cur)
    torch.cuda.synchronize()
    status |= path.pool.status()
    # decode at the grown length
    q = workloads.make_queries(w, dev, 5)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    cnt = path.pool.count[0].cpu().numpy()
    d_us = cold_reps(reps, flush, lambda r: path.decode(0, q, out), timer)
    res["decode_grown"] = stats(d_us, decode_algorithmic_bytes(cnt, B, Hq))
    res["decode_grown"]["tokens_per_request"] = path.lens[0]
    # the last re-tier round from a snapshot of the state before it
    pool = path.pool
    state = [pool.pages, pool.page_table, pool.count, pool.owner, pool.free_ring, pool.ring_ctr,
             pool.dev_status, path.state]
    snap = [t.clone() for t in state]

    def round_one(r):
        for t, s0 in zip(state, snap):
            t.copy_(s0)
        evict(flush)

    ws_round = kvc.workspace(path.geom, kvc.OP_ROUND, path.seqlen_cap, device=dev)

    def timed_rounds(fused):
        us = []
        for r in range(reps + 1):             # the first round is a warm-up
            round_one(r)
            prev = path.packed_state()
            e0 = timer.ev()
            if fused:
                kvc.compaction_round(path.geom, 0, pool, last, path.cu, path.T, path.max_seqlen,
                                     w.alpha_h, w.alpha_l, w.window, None, None, path.tier,
                                     path.new_count, ws_round, prev_tier=prev,
                                     changed=path.changed)
            else:
                kvc.score_tokens(path.geom, last, path.cu, path.T, path.max_seqlen, w.alpha_h,
                                 w.alpha_l, w.window, path.tier, path.new_count, prev_tier=prev,
                                 changed=path.changed, dev_status=path.score_status)
                kvc.compact_pages(path.geom, 0, pool, path.new_count, path.ws_compact,
                                  changed=path.changed, old_rows=path.old_rows,
                                  old_count=path.old_count)
                kvc.quantize_and_place(path.geom, 0, pool, None, None, path.cu, path.T,
                                       path.max_seqlen, path.tier, path.ws_quant, prev_tier=prev,
                                       changed=path.changed, old_rows=path.old_rows,
                                       old_count=path.old_count)
            e1 = timer.ev()
            torch.cuda.synchronize()
            if r > 0:
                us.append(timer.us(e0, e1))
        return us
    rt3_us = timed_rounds(False)
    status |= pool.status()
    rt_us = timed_rounds(True)
    status |= pool.status()
    chg = path.changed.cpu().numpy().astype(bool)
    old_c = snap[2][0].cpu().numpy()[chg]               # the counts before the round
    new_c = path.new_count.cpu().numpy()[chg]
    T = path.T
    # algorithmic bytes of a round: the accumulators, previous and new tiers, and for every
    # rebuilt head its old pages read and its new pages written
    rbytes = T * Hq * 4 + 2 * T * Hkv + (pages_of(old_c) + pages_of(new_c)) * kvc.PAGE_BYTES
    res["retier_round"] = stats(rt_us, rbytes)
    res["retier_round"].update({"path": "kvc_compaction_round", "algorithmic_bytes": rbytes,
                                "heads_rebuilt": int(chg.sum()), "token_heads": T * Hkv,
                                "tokens_per_request": path.lens[0]})
    res["retier_round_three_calls"] = stats(rt3_us, rbytes)
    res["status"] = status
    res["config"] = {"workload": w.name, "batch": B, "prompt": max(w.seqlens),
                     "generated": steps, "round_every": R, "q_heads": Hq, "kv_heads": Hkv}
    del path, snap, k, v, acc
    torch.cuda.empty_cache()
    return res


def main():
    a = parse()
    if a.copy_calibration:
        copy_calibration()
        return
    if a.group_sweep:
        import torch
        torch.cuda.set_device(0)
        flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
        print(json.dumps({"decode_by_group": decode_by_group(a, torch.cuda.current_stream(),
                                                             flush)}))
        return
    if a.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; --gpus above 1 is not supported (the path would shard requests and KV heads across GPUs, each running this same single-GPU step)",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    from mixed_precision_paged_score_amd import workloads
    w = workloads.workload(a.workload)
    if w.num_layers > 1:
        w = dataclasses.replace(w, num_pages=1 << 24)        # 2^20 holds a few layers only
    else:
        w = dataclasses.replace(w, num_pages=2 * w.num_pages)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(w)                 # before anything touches the GPU (fork pool)
    import torch
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    spin = spin_cycles(stream)
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    nsteps_dec = a.decode_steps if a.decode_steps is not None else w.decode_steps
    graphs = w.num_layers == 1 and not a.eager
    res_main, path, ins, counts = run_step_workload(a, w, stream, spin, flush, a.steps,
                                                    a.warmup, nsteps_dec, graphs)
    del path, ins
    torch.cuda.empty_cache()
    traffic = traffic_record(w.name)
    dec, comp = res_main["decode"], res_main["compaction"]
    res = {
        "metric": "KV tokens compacted/s + paged decode attn GB/s (fraction of HBM peak)",
        "value": res_main["value"],
        "unit": "KV token-heads compacted/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": res_main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in, u8 codes, fp32 scale math",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.num_layers, "batch": w.batch,
                   "seq_len": w.seqlens[0] if len(set(w.seqlens)) == 1 else "ragged",
                   "mean_seq_len": w.total_tokens / w.batch,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": 128,
                   "pages": w.num_pages, "decode_steps_per_layer": nsteps_dec,
                   "alpha_h": w.alpha_h, "alpha_l": w.alpha_l, "window": w.window},
        "compaction": dict(comp, traffic=traffic["compaction"]),
        "decode_GBps": dec["GBps"],
        "decode": dict(dec, traffic=traffic["decode"]),
        "cold": res_main["cold"],
        "roofline": {"bound": "hbm", "kernel": "paged_decode_attention (main + combine), per call",
                     "achieved": dec["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dec["GBps"] / HBM_PEAK_GBPS, "traffic": traffic["decode"]},
        "roofline_compaction": {"bound": "hbm",
                                "kernel": "compaction round (score + compact + quantize/place), per layer",
                                "achieved": comp["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                "frac": comp["GBps"] / HBM_PEAK_GBPS,
                                "traffic": traffic["compaction"]},
        "pool_status": res_main["pool_status"],
    }
    print(json.dumps({"progress": "step timed", "value": res["value"],
                      "decode_frac": res["roofline"]["frac"]}), file=sys.stderr, flush=True)
    if not a.no_extras:
        res["w3"] = extras_w3(a, stream, spin, flush)
        print(json.dumps({"progress": "w3 done"}), file=sys.stderr, flush=True)
        if not a.no_w4:
            res["w4"] = extras_w4(a, stream, flush)
            print(json.dumps({"progress": "w4 done"}), file=sys.stderr, flush=True)
    res["ceilings"] = measure_ceilings()
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
