"""Seeded synthetic workloads (inputs only).

This module draws random inputs of the shapes and value distributions of the five
workloads below.  It computes none of the method's arithmetic (no scoring, tiering,
quantization or placement); both the HIP path and the CPU oracle receive exactly what it
produces.  The attention-score accumulators are the method's *input*: the sum of the
softmax weight each token received from strictly later queries, made either from a causal
softmax of random queries or from a Zipf law over positions.

Workloads (DiffKV review page: models and datasets are not available, so shaped random data
stands in for them):
  1  one layer, 1 request, 32 query / 8 KV heads, N = 512, K/V ~ N(0,1) fp16, accumulators
     from a causal softmax of random fp16 queries, alpha 1.0 / 0.2, 4096 pages.
  2  one layer, 8 requests, 32 / 8 heads, N ~ U{2048..4096}, 4 key channels x8 outliers,
     causal-softmax accumulators, alpha 1.0 / 0.25, 65,536 pages, one decode step.
  3  one layer, 16 requests, 64 / 8 heads, N = 32,768, Zipf(1.1) accumulators,
     alpha 1.0 / 0.2, 2^18 pages, 64 decode steps.
  4  chain-of-thought growth: 16 requests, 64 / 8 heads, 4096-token prompt, 16,384 decode
     steps, a re-tier round every 128 steps whose accumulators add the round's Zipf weights
     to the previous sums (make_acc_zipf_round), alpha 1.0 / 0.2, 2^18 pages.
  5  64 layers, 64 requests, 64 / 8 heads, N log-uniform in [1024, 32768], per-layer key
     outliers x10 on 3 channels, Zipf(1.1) accumulators, alpha 1.0 / 0.2.
"""
from dataclasses import dataclass, field, replace
import math

import numpy as np
import torch

D = 128


@dataclass
class Workload:
    name: str
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seqlens: list
    alpha_h: float
    alpha_l: float
    window: int
    num_pages: int
    acc_recipe: str               # "causal" or "zipf"
    k_outlier_channels: int = 0
    k_outlier_factor: float = 1.0
    decode_steps: int = 1
    seed: int = 20260000
    extra: dict = field(default_factory=dict)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self):
        return int(sum(self.seqlens))

    @property
    def row_capacity(self):
        # enough row slots for any HIGH/LOW split of the longest request
        return max(1, -(-max(self.seqlens + [1]) // 16) + 1)

    def cu_seqlens(self):
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)


def workload(i, **overrides):
    seed = 20260000 + i
    if i == 1:
        w = Workload("w1-1x512-g4", 1, 1, 32, 8, [512], 1.0, 0.2, 64, 4096, "causal", seed=seed)
    elif i == 2:
        rng = np.random.default_rng(seed)
        lens = [int(x) for x in rng.integers(2048, 4097, size=8)]
        w = Workload("w2-8xU[2048,4096]-g4", 1, 8, 32, 8, lens, 1.0, 0.25, 64, 65536,
                     "causal", k_outlier_channels=4, k_outlier_factor=8.0, seed=seed)
    elif i == 3:
        w = Workload("w3-16x32768-g8", 1, 16, 64, 8, [32768] * 16, 1.0, 0.2, 64, 1 << 18,
                     "zipf", decode_steps=64, seed=seed)
    elif i == 4:
        w = Workload("w4-16x(4096+16384)-g8", 1, 16, 64, 8, [4096] * 16, 1.0, 0.2, 64, 1 << 18,
                     "zipf", decode_steps=16384, seed=seed,
                     extra={"round_every": 128})
    elif i == 5:
        rng = np.random.default_rng(seed)
        lens = [int(round(math.exp(x))) for x in rng.uniform(math.log(1024), math.log(32768), 64)]
        w = Workload("w5-64L-64xlogU[1K,32K]-g8", 64, 64, 64, 8, lens, 1.0, 0.2, 64, 1 << 20,
                     "zipf", k_outlier_channels=3, k_outlier_factor=10.0, seed=seed)
    else:
        raise ValueError(i)
    return replace(w, **overrides) if overrides else w


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def make_kv(w, device="cpu", layer=0):
    """K and V, fp16 [T][Hkv][128], N(0,1) rounded to fp16; optional key outlier channels
    (one seeded set per layer shared by all heads and tokens, scaled before rounding)."""
    T, H = w.total_tokens, w.num_kv_heads
    g = _gen(device, w.seed * 1000 + 2 * layer)
    k = torch.randn((T, H, D), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((T, H, D), generator=g, device=device, dtype=torch.float32)
    if w.k_outlier_channels:
        rng = np.random.default_rng(w.seed * 1000 + 2 * layer + 1)
        ch = torch.as_tensor(rng.choice(D, size=w.k_outlier_channels, replace=False),
                             device=device)
        k[:, :, ch] *= float(w.k_outlier_factor)
    return k.to(torch.float16), v.to(torch.float16)


def make_queries(w, device="cpu", step=0, layer=0):
    """One decode query per request: fp16 [B][Hq][128] ~ N(0,1)."""
    g = _gen(device, w.seed * 1000 + 500 + 7919 * step + layer)
    q = torch.randn((w.batch, w.num_q_heads, D), generator=g, device=device,
                    dtype=torch.float32)
    return q.to(torch.float16)


def make_acc_causal(w, k, device="cpu", layer=0):
    """acc[t][hq] = sum over later positions i of softmax_j(q_i . k_j / sqrt(d))[t], with
    one random fp16 query per (position, query head).  float64 on the CPU, float32 on a
    GPU; rounded to float32."""
    dt = torch.float64 if str(device) == "cpu" else torch.float32
    G, Hkv = w.group, w.num_kv_heads
    cu = w.cu_seqlens()
    acc = torch.zeros((w.total_tokens, w.num_q_heads), dtype=torch.float32, device=device)
    g = _gen(device, w.seed * 1000 + 300 + layer)
    for b in range(w.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if n == 0:
            continue
        qp = torch.randn((n, w.num_q_heads, D), generator=g, device=device,
                         dtype=torch.float32).to(torch.float16)
        mask = torch.ones((n, n), dtype=torch.bool, device=device).tril()
        for h in range(Hkv):
            kh = k[lo:hi, h, :].to(dt)
            for gg in range(G):
                hq = h * G + gg
                logits = (qp[:, hq, :].to(dt) @ kh.T) / math.sqrt(D)   # [i][j]
                logits = logits.masked_fill(~mask, float("-inf"))
                p = torch.softmax(logits, dim=1)
                p = p - torch.diag(torch.diagonal(p))                  # strictly later only
                acc[lo:hi, hq] = p.sum(dim=0).to(torch.float32)
    return acc


def make_acc_zipf(w, device="cpu", layer=0, s=1.1):
    """Zipf(s) accumulators: per (request, query head) a seeded permutation pi of the
    positions; the mean attention token t receives is (pi(t)+1)^-s / H_{N,s}; the sum is
    that mean times the number of later positions (float64, rounded to float32)."""
    cu = w.cu_seqlens()
    acc = torch.zeros((w.total_tokens, w.num_q_heads), dtype=torch.float32, device=device)
    g = _gen(device, w.seed * 1000 + 700 + layer)
    for b in range(w.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if n == 0:
            continue
        ranks = torch.argsort(torch.rand((w.num_q_heads, n), generator=g, device=device),
                              dim=1)                                     # [hq][t] -> rank
        kk = torch.arange(1, n + 1, device=device, dtype=torch.float64)
        harm = torch.sum(kk ** (-s))
        mean = (ranks.to(torch.float64) + 1.0) ** (-s) / harm             # [hq][t]
        cnt = (n - 1 - torch.arange(n, device=device, dtype=torch.float64))
        acc[lo:hi, :] = (mean * cnt[None, :]).T.to(torch.float32)
    return acc


def make_acc_zipf_round(w, acc_prev, lens_prev, device="cpu", round_id=0, s=1.1):
    """Accumulators after a generation round: the previous sums plus the weight the round's
    new queries gave each earlier token.  w.seqlens are the lengths after the round,
    lens_prev the lengths before it (acc_prev over those, ragged rows).  Per (request, query
    head) one fresh seeded Zipf(s) permutation gives the mean weight m_t a new query puts on
    position t; token t gains m_t times the number of new queries strictly after it
    (N - N_prev for t < N_prev, N - 1 - t for a token added in the round).  The sums stay
    'weight received from strictly later queries' (float64 increments, float32 result)."""
    cu = w.cu_seqlens()
    cu_prev = np.concatenate([[0], np.cumsum(lens_prev)]).astype(np.int64)
    acc = torch.zeros((w.total_tokens, w.num_q_heads), dtype=torch.float32, device=device)
    g = _gen(device, w.seed * 1000 + 900 + 7 * round_id)
    for b in range(w.batch):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n, n0 = hi - lo, int(lens_prev[b])
        if n == 0:
            continue
        ranks = torch.argsort(torch.rand((w.num_q_heads, n), generator=g, device=device),
                              dim=1)
        kk = torch.arange(1, n + 1, device=device, dtype=torch.float64)
        harm = torch.sum(kk ** (-s))
        mean = (ranks.to(torch.float64) + 1.0) ** (-s) / harm             # [hq][t]
        t = torch.arange(n, device=device, dtype=torch.float64)
        later = torch.where(t < n0, torch.full_like(t, float(n - n0)), n - 1 - t)
        inc = (mean * later[None, :]).T                                   # [t][hq]
        if n0 > 0:
            inc[:n0] += acc_prev[int(cu_prev[b]):int(cu_prev[b]) + n0].to(torch.float64)
        acc[lo:hi, :] = inc.to(torch.float32)
    return acc


def make_acc(w, k=None, device="cpu", layer=0):
    if w.acc_recipe == "causal":
        return make_acc_causal(w, k, device, layer)
    return make_acc_zipf(w, device, layer)
