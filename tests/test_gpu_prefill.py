"""Causal prefill attention and the prompt accumulators on the GPU (kvc_prefill_attention) vs
the float64 oracle (MI355X only).  Output rows within the attention tolerance (2e-3 max-abs,
1e-3 relative L2); accumulators within 1e-4 relative + 1e-6 absolute (float32 scores and sums
against float64; the probabilities that weight V are fp16, the ones summed into the
accumulators float32).  Small ragged batches are compared in full; long requests on sampled
rows and columns."""
import math
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from oracle import prefill as op  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL_ACC, ATOL_ACC = 1e-4, 1e-6


def _inputs(lens, hq, hkv, seed, scale_q=1.0):
    g = torch.Generator().manual_seed(seed)
    T = sum(lens)
    q = (torch.randn((T, hq, 128), generator=g) * scale_q).to(torch.float16)
    k = torch.randn((T, hkv, 128), generator=g).to(torch.float16)
    v = torch.randn((T, hkv, 128), generator=g).to(torch.float16)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu


def _run(q, k, v, cu, hq, hkv, out_fp32=True, max_seqlen=None, with_acc=True):
    from mixed_precision_paged_score_amd import kvc
    B = len(cu) - 1
    lens = np.diff(cu)
    ms = int(lens.max()) if max_seqlen is None else max_seqlen
    geom = kvc.make_geom(1, B, hq, hkv, 1, 1)
    ws = kvc.workspace(geom, kvc.OP_PREFILL, ms, device=DEV)
    T = int(cu[-1])
    out = torch.empty((max(T, 1), hq, 128), dtype=torch.float32 if out_fp32 else torch.float16,
                      device=DEV)
    acc = torch.full((max(T, 1), hq), -7.0, dtype=torch.float32, device=DEV) if with_acc else None
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(128)
    print(f"[prefill] B={B} lens={list(lens[:6])} Hq={hq} Hkv={hkv} fp32={out_fp32}", flush=True)
    kvc.prefill_attention(geom, q.to(DEV), k.to(DEV), v.to(DEV),
                          torch.tensor(cu, device=DEV), ms, scale, out, acc, ws, dev_status=st)
    torch.cuda.synchronize()
    return out, acc, int(st.item()), scale


def _check_acc(got, want):
    err = np.abs(got - want)
    bad = err > RTOL_ACC * np.abs(want) + ATOL_ACC
    assert not bad.any(), f"{int(bad.sum())} accumulators off, worst {err.max():.3e}"


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (16, 2)])
def test_ragged_full(hq, hkv):
    lens = [1, 0, 63, 64, 65, 129, 300]
    q, k, v, cu = _inputs(lens, hq, hkv, seed=hq * 10 + hkv)
    out, acc, st, scale = _run(q, k, v, cu, hq, hkv)
    assert st == 0
    want_o, want_a = op.prefill(q.numpy(), k.numpy(), v.numpy(), cu, hkv, scale)
    T = int(cu[-1])
    for b in range(len(lens)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in range(hq):
            if hi > lo:
                parity.assert_close_attention(parity.np_(out[lo:hi, h]), want_o[lo:hi, h])
    _check_acc(parity.np_(acc[:T]).astype(np.float64), want_a)
    # the last token of every request gets nothing: exactly zero
    for b in range(len(lens)):
        if cu[b + 1] > cu[b]:
            assert np.all(parity.np_(acc[int(cu[b + 1]) - 1]) == 0.0)


def test_fp16_output_and_peaked_scores():
    # larger query norms make the softmax peaked: the lazy running max must rescale correctly
    lens = [200, 77]
    q, k, v, cu = _inputs(lens, 8, 2, seed=7, scale_q=4.0)
    out, acc, st, scale = _run(q, k, v, cu, 8, 2, out_fp32=False)
    assert st == 0
    want_o, want_a = op.prefill(q.numpy(), k.numpy(), v.numpy(), cu, 2, scale)
    got = parity.np_(out).astype(np.float64)
    for b in range(2):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in range(8):
            parity.assert_close_attention(got[lo:hi, h], want_o[lo:hi, h])
    _check_acc(parity.np_(acc).astype(np.float64), want_a)


def test_mass_invariant_and_identical_keys():
    # identical keys: uniform rows, so acc[t] = H_n - H_{t+1} and the output is the running
    # mean of v (closed forms at a size spanning 11 key blocks and 6 query blocks)
    n = 700
    g = torch.Generator().manual_seed(3)
    q = torch.randn((n, 4, 128), generator=g).to(torch.float16)
    k = torch.randn((1, 1, 128), generator=g).to(torch.float16).repeat(n, 1, 1)
    v = torch.randn((n, 1, 128), generator=g).to(torch.float16)
    cu = np.array([0, n], np.int32)
    out, acc, st, scale = _run(q, k, v, cu, 4, 1)
    assert st == 0
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    want = H[n] - H[1:n + 1]
    got = parity.np_(acc).astype(np.float64)
    for h in range(4):
        _check_acc(got[:, h], want)
    running = np.cumsum(v[:, 0].numpy().astype(np.float64), axis=0) / np.arange(1, n + 1)[:, None]
    for h in range(4):
        parity.assert_close_attention(parity.np_(out[:, h]), running)


def test_seqlen_bound_and_no_accumulators():
    # a request longer than max_seqlen is skipped with KVC_DEV_SEQLEN; acc_sum NULL skips the
    # column sums and leaves the output as with them
    from mixed_precision_paged_score_amd import kvc
    lens = [50, 90]
    q, k, v, cu = _inputs(lens, 4, 2, seed=11)
    out_a, acc_a, st, _ = _run(q, k, v, cu, 4, 2)
    out_b, _, st_b, _ = _run(q, k, v, cu, 4, 2, with_acc=False)
    assert st == 0 and st_b == 0
    assert torch.equal(out_a, out_b)
    _, acc_c, st_c, _ = _run(q, k, v, cu, 4, 2, max_seqlen=60)
    assert st_c & kvc.DEV_SEQLEN
    assert torch.all(acc_c[50:] == -7.0)            # request 1 (90 > 60) untouched
    assert torch.equal(acc_c[:50], acc_a[:50])


@pytest.mark.parametrize("n,hq,hkv", [(4096, 8, 2), (8192 + 37, 16, 2)])
def test_long_requests_sampled(n, hq, hkv):
    lens = [n, n // 3 + 5]
    q, k, v, cu = _inputs(lens, hq, hkv, seed=n % 97)
    out, acc, st, scale = _run(q, k, v, cu, hq, hkv)
    assert st == 0
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    rng = np.random.default_rng(n)
    for b in range(2):
        N = lens[b]
        for hh in rng.choice(hq, 2, replace=False):
            rows = sorted(set([0, 1, 63, 64, 127, 128, N - 1] + list(rng.integers(0, N, 6))))
            want = op.prefill_rows(qn, kn, vn, cu, hkv, scale, b, int(hh), rows)
            got = parity.np_(out[int(cu[b]) + np.array(rows), int(hh)])
            parity.assert_close_attention(got, want)
            cols = sorted(set([N - 1, N - 2, N - 65, N - 200] + list(rng.integers(N - 400, N, 4))))
            want_c = op.prefill_colsums(qn, kn, cu, hkv, scale, b, int(hh), cols)
            got_c = parity.np_(acc[int(cu[b]) + np.array(cols), int(hh)]).astype(np.float64)
            _check_acc(got_c, want_c)
        # one more head of the request in full: every row and every accumulator
        hh = int(rng.integers(0, hq))
        h = hh // (hq // hkv)
        lo, hi = int(cu[b]), int(cu[b + 1])
        want_o, want_a = op.prefill(qn[lo:hi, hh:hh + 1], kn[lo:hi, h:h + 1], vn[lo:hi, h:h + 1],
                                    [0, N], 1, scale)
        parity.assert_close_attention(parity.np_(out[lo:hi, hh]), want_o[:, 0])
        _check_acc(parity.np_(acc[lo:hi, hh]).astype(np.float64), want_a[:, 0])


def test_request_of_32768_tokens():
    # the prompt length the bench times: one 32,768-token request (and a short one), G = 8;
    # one query head checked in full (every output row and every accumulator) by the oracle's
    # row-blocked form, two more on sampled rows and columns
    n, hq, hkv = 32768, 8, 1
    lens = [n, 777]
    q, k, v, cu = _inputs(lens, hq, hkv, seed=3276)
    out, acc, st, scale = _run(q, k, v, cu, hq, hkv)
    assert st == 0
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    rng = np.random.default_rng(32768)
    hh = int(rng.integers(0, hq))
    want_o, want_a = op.prefill_head(qn[:n, hh], kn[:n, 0], vn[:n, 0], scale)
    parity.assert_close_attention(parity.np_(out[:n, hh]), want_o)
    _check_acc(parity.np_(acc[:n, hh]).astype(np.float64), want_a)
    print(f"[prefill] 32,768 tokens: head {hh} in full ok", flush=True)
    for h2 in rng.choice([x for x in range(hq) if x != hh], 2, replace=False):
        rows = sorted(set([0, 1, 4095, 4096, 16383, n - 1] + list(rng.integers(0, n, 8))))
        want = op.prefill_rows(qn, kn, vn, cu, hkv, scale, 0, int(h2), rows)
        parity.assert_close_attention(parity.np_(out[np.array(rows), int(h2)]), want)
        cols = sorted(set([n - 1, n - 2, n - 65, n - 300] + list(rng.integers(n - 600, n, 4))))
        want_c = op.prefill_colsums(qn, kn, cu, hkv, scale, 0, int(h2), cols)
        _check_acc(parity.np_(acc[np.array(cols), int(h2)]).astype(np.float64), want_c)
