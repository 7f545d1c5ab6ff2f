"""kvc_paged_decode_attention_static -- the decode for callers that cannot allocate, its split
partials in the library's own device array -- against kvc_paged_decode_attention with a
workspace, through the C ABI: bit-identical outputs on two calls in a row (the second on a
smaller batch, so it reuses the array the first one filled), one of them also against the
oracle; and the refusal, before any device work, of a geometry whose partials exceed the
array."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(__file__))
import parity  # noqa: E402
from mixed_precision_paged_score_amd import workloads  # noqa: E402

DEV = "cuda:0"


def _decode_both(w, out_dtype):
    from mixed_precision_paged_score_amd import kvc, pipeline
    k, v = workloads.make_kv(w)
    acc = workloads.make_acc(w, k)
    q = workloads.make_queries(w)
    path = pipeline.PromptPath(w, DEV)
    path.prompt(0, acc.to(DEV), k.to(DEV), v.to(DEV))
    qd = q.to(DEV)
    shape = (w.batch, w.num_q_heads, 128)
    out_ws = torch.full(shape, 7.0, dtype=out_dtype, device=DEV)
    out_st = torch.full(shape, -7.0, dtype=out_dtype, device=DEV)
    kvc.paged_decode_attention(path.geom, 0, path.pool, qd, path.scale, out_ws, path.ws_decode)
    kvc.paged_decode_attention_static(path.geom, 0, path.pool, qd, path.scale, out_st)
    torch.cuda.synchronize()
    assert path.pool.status() == 0
    return path, k, v, acc, q, out_ws, out_st


@pytest.mark.gpu
def test_static_decode_matches_workspace_decode_on_two_calls():
    # first call: 16 requests with long and empty heads, G = 8 (64 query / 8 KV heads, many
    # splits); second call: a smaller batch, G = 4, fp16 output, reusing the array
    big = workloads.Workload("noalloc-big", 1, 16, 64, 8,
                             [16384, 0, 1, 37, 300, 777, 2048, 9000, 5000, 100, 64, 65, 3000,
                              15, 900, 4000], 1.0, 0.2, 64, 1 << 16, "zipf", seed=91)
    small = workloads.Workload("noalloc-small", 1, 3, 16, 4, [129, 2000, 5], 1.0, 0.2, 16, 4096,
                               "zipf", seed=92)
    print("[noalloc] call 1: 16 requests, 64/8 heads, fp32 out", flush=True)
    path, k, v, acc, q, a, b = _decode_both(big, torch.float32)
    assert torch.equal(a, b)
    # the first call's output is also the oracle's (the tolerance of the path)
    tier, _, _ = parity.oracle_score(big, acc)
    G = big.group
    for bb in (0, 3, 7):
        for h in (0, 5):
            want = parity.oracle_attention(big, bb, h, k.numpy(), v.numpy(), tier, q.numpy(),
                                           path.scale)
            parity.assert_close_attention(parity.np_(b[bb, h * G:(h + 1) * G]), want)
    print("[noalloc] call 2: 3 requests, 16/4 heads, fp16 out", flush=True)
    _, _, _, _, _, a2, b2 = _decode_both(small, torch.float16)
    assert torch.equal(a2, b2)
    print("[noalloc] ok: bit-identical to the workspace decode on both calls", flush=True)


def test_static_decode_refuses_geometry_beyond_its_array():
    # 2,048 requests x 8 KV heads, G = 16: one split per head, 2,048 x 128 x 528 bytes of
    # partials (138 MB) > 64 MiB; refused on the host, so this needs no GPU
    from mixed_precision_paged_score_amd import kvc
    g = kvc.make_geom(1, 2048, 128, 8, 10, 1 << 16)
    assert kvc.workspace_bytes(g, kvc.OP_DECODE) > kvc.STATIC_SCRATCH_BYTES
    p = kvc.PoolPtrs(16, 16, 16, 16, 16, 16, 16)
    rc = kvc._lib.kvc_paged_decode_attention_static(ctypes.byref(g), 0, ctypes.byref(p), 16,
                                                    ctypes.c_float(1.0), 16, 1, None)
    assert rc == kvc.E_WORKSPACE
    # a geometry that fits is not refused on size (the null query is what fails here)
    g2 = kvc.make_geom(1, 64, 64, 8, 2049, 1 << 16)
    assert kvc.workspace_bytes(g2, kvc.OP_DECODE) <= kvc.STATIC_SCRATCH_BYTES
    rc = kvc._lib.kvc_paged_decode_attention_static(ctypes.byref(g2), 0, ctypes.byref(p), None,
                                                    ctypes.c_float(1.0), 16, 1, None)
    assert rc == kvc.E_NULL
