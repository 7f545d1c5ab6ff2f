"""The C ABI library loads without a GPU, exports every function include/kvc.h declares, and
rejects bad arguments synchronously (no device work is started by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", src)))


def test_exports_match_header():
    from mixed_precision_paged_score_amd import kvc
    lib = ctypes.CDLL(kvc.LIB_PATH)
    names = _declared()
    assert set(names) == set(kvc.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_workspace_sizes():
    from mixed_precision_paged_score_amd import kvc
    assert "gfx950" in kvc.version()
    g = kvc.make_geom(1, 16, 64, 8, 2049, 1 << 18)
    assert kvc.workspace_bytes(g, kvc.OP_COMPACT) > 0
    assert kvc.workspace_bytes(g, kvc.OP_QUANTIZE, 32768) >= 16 * 8 * 32768 * 4
    assert kvc.workspace_bytes(g, kvc.OP_DECODE) > 0
    # the accumulating decode also holds one logit per live token and query head
    assert kvc.workspace_bytes(g, kvc.OP_DECODE_ACC, 32768) >= \
        kvc.workspace_bytes(g, kvc.OP_DECODE) + 16 * 64 * 2 * 2049 * 16 * 4 + \
        16 * 8 * 2 * (32768 // 64 + 1) * 4
    assert kvc.workspace_bytes(g, kvc.OP_DECODE_ACC, -1) == 0
    assert kvc.workspace_bytes(g, kvc.OP_GENERATE) > kvc.workspace_bytes(g, kvc.OP_COMPACT)
    assert kvc.workspace_bytes(g, kvc.OP_PREFILL, 32768) >= 16 * 32768 * 64 * 8
    # the fused round holds the quantize workspace, the allocation scan and the old rows
    assert kvc.workspace_bytes(g, kvc.OP_ROUND, 32768) >= \
        kvc.workspace_bytes(g, kvc.OP_QUANTIZE, 32768) + kvc.workspace_bytes(g, kvc.OP_COMPACT) + \
        16 * 8 * 2049 * 4
    assert kvc.workspace_bytes(g, 99) == 0
    bad = kvc.make_geom(1, 16, 60, 8, 2049, 1 << 18)        # Hq % Hkv != 0
    assert kvc.workspace_bytes(bad, kvc.OP_COMPACT) == 0


def test_synchronous_errors_enqueue_nothing():
    from mixed_precision_paged_score_amd import kvc
    lib = kvc._lib
    g = kvc.make_geom(1, 2, 8, 2, 10, 100)
    assert lib.kvc_pool_init(ctypes.byref(g), None, None) == kvc.E_NULL
    bad = kvc.make_geom(1, 2, 8, 3, 10, 100)
    p = kvc.PoolPtrs(16, 16, 16, 16, 16, 16, 16)
    assert lib.kvc_pool_init(ctypes.byref(bad), ctypes.byref(p), None) == kvc.E_SHAPE
    huge = kvc.make_geom(1, 2, 8, 2, 10, 1 << 31)
    assert lib.kvc_pool_init(ctypes.byref(huge), ctypes.byref(p), None) == kvc.E_SHAPE
    p_unaligned = kvc.PoolPtrs(18, 16, 16, 16, 16, 16, 16)
    assert lib.kvc_pool_init(ctypes.byref(g), ctypes.byref(p_unaligned), None) == kvc.E_ALIGN
    # compact: layer out of range, workspace too small
    assert lib.kvc_compact_pages(ctypes.byref(g), 1, ctypes.byref(p), 16, None, None, None,
                                 256, 1 << 20, None) == kvc.E_SHAPE
    assert lib.kvc_compact_pages(ctypes.byref(g), 0, ctypes.byref(p), 16, None, None, None,
                                 256, 8, None) == kvc.E_WORKSPACE
    # quantize: re-tier mode needs all four of prev_tier, changed, old_rows, old_count
    assert lib.kvc_quantize_and_place(ctypes.byref(g), 0, ctypes.byref(p), 16, 16, 16, 10, 5,
                                      16, 16, None, None, None, 256, 1 << 20,
                                      None) == kvc.E_NULL
    assert lib.kvc_quantize_and_place(ctypes.byref(g), 0, ctypes.byref(p), 16, 16, 16, 10, 5,
                                      16, None, 16, None, None, 256, 1 << 20,
                                      None) == kvc.E_UNSUPPORTED
    # append: missing positions, misaligned keys
    assert lib.kvc_append_tokens(ctypes.byref(g), 0, ctypes.byref(p), 16, 16, None, 256,
                                 1 << 20, None) == kvc.E_NULL
    assert lib.kvc_append_tokens(ctypes.byref(g), 0, ctypes.byref(p), 18, 16, 16, 256,
                                 1 << 20, None) == kvc.E_ALIGN
    # decode: misaligned query
    assert lib.kvc_paged_decode_attention(ctypes.byref(g), 0, ctypes.byref(p), 18, 1.0, 16, 1,
                                          256, 1 << 20, None) == kvc.E_ALIGN
    # accumulating decode: accumulators without sequence offsets, then a small workspace
    assert lib.kvc_paged_decode_attention_acc(ctypes.byref(g), 0, ctypes.byref(p), 16, 1.0, 16,
                                              1, 256, None, 10, 256, 1 << 30, None) == kvc.E_NULL
    assert lib.kvc_paged_decode_attention_acc(ctypes.byref(g), 0, ctypes.byref(p), 16, 1.0, 16,
                                              1, 256, 256, 10, 256, 64, None) == kvc.E_WORKSPACE
    assert lib.kvc_paged_decode_attention_acc(ctypes.byref(g), 0, ctypes.byref(p), 16, 1.0, 16,
                                              1, 256, 256, -1, 256, 1 << 30, None) == kvc.E_SHAPE
    # generation step: no accumulators; window outside 1..KVC_GEN_MAX_WINDOW; small workspace
    f1, f0 = ctypes.c_float(1.0), ctypes.c_float(0.2)
    assert lib.kvc_generation_step(ctypes.byref(g), 0, ctypes.byref(p), 16, 16, 16, None, 16,
                                   f1, f0, 8, 16, 256, 1 << 20, None) == kvc.E_NULL
    for win in (0, kvc.GEN_MAX_WINDOW + 1):
        assert lib.kvc_generation_step(ctypes.byref(g), 0, ctypes.byref(p), 16, 16, 16, 16, 16,
                                       f1, f0, win, 16, 256, 1 << 20, None) == kvc.E_SHAPE
    assert lib.kvc_generation_step(ctypes.byref(g), 0, ctypes.byref(p), 16, 16, 16, 16, 16,
                                   f1, f0, 8, 16, 256, 64, None) == kvc.E_WORKSPACE
    assert lib.kvc_generation_step(ctypes.byref(g), 0, ctypes.byref(p), 16, 18, 16, 16, 16,
                                   f1, f0, 8, 16, 256, 1 << 20, None) == kvc.E_ALIGN
    # prefill: missing cu_seqlens, misaligned keys, negative max_seqlen, small workspace
    assert lib.kvc_prefill_attention(ctypes.byref(g), 16, 16, 16, None, 8, f1, 16, 1, 16, None,
                                     256, 1 << 20, None) == kvc.E_NULL
    assert lib.kvc_prefill_attention(ctypes.byref(g), 16, 18, 16, 16, 8, f1, 16, 1, 16, None,
                                     256, 1 << 20, None) == kvc.E_ALIGN
    assert lib.kvc_prefill_attention(ctypes.byref(g), 16, 16, 16, 16, -1, f1, 16, 1, 16, None,
                                     256, 1 << 20, None) == kvc.E_SHAPE
    assert lib.kvc_prefill_attention(ctypes.byref(g), 16, 16, 16, 16, 8, f1, 16, 1, 16, None,
                                     256, 8, None) == kvc.E_WORKSPACE
    # schemes: no scheme, bit widths that do not fit, small workspace
    sc_bad = kvc.Scheme(8, 8, 4, 2)
    sc_ok = kvc.make_scheme("K8V2", "K4V1")
    assert lib.kvc_paged_decode_attention_scheme(ctypes.byref(g), None, 0, ctypes.byref(p), 16,
                                                 1.0, 16, 1, 256, 1 << 20, None) == kvc.E_NULL
    assert lib.kvc_paged_decode_attention_scheme(ctypes.byref(g), ctypes.byref(sc_bad), 0,
                                                 ctypes.byref(p), 16, 1.0, 16, 1, 256, 1 << 20,
                                                 None) == kvc.E_SHAPE
    assert lib.kvc_paged_decode_attention_scheme(ctypes.byref(g), ctypes.byref(sc_ok), 0,
                                                 ctypes.byref(p), 16, 1.0, 16, 1, 256, 8,
                                                 None) == kvc.E_WORKSPACE
    assert lib.kvc_quantize_and_place_scheme(ctypes.byref(g), ctypes.byref(kvc.Scheme(8, 4, 4, 4)),
                                             0, ctypes.byref(p), 16, 16, 16, 10, 5, 16, None,
                                             None, None, None, 256, 1 << 20, None) == kvc.E_SHAPE
    assert lib.kvc_quantize_and_place_scheme(ctypes.byref(g), ctypes.byref(sc_ok), 0,
                                             ctypes.byref(p), 16, 18, 16, 10, 5, 16, None, None,
                                             None, None, 256, 1 << 20, None) == kvc.E_ALIGN
    # re-tier mode needs all four re-tier arguments; only some of them is refused
    assert lib.kvc_quantize_and_place_scheme(ctypes.byref(g), ctypes.byref(sc_ok), 0,
                                             ctypes.byref(p), 16, 16, 16, 10, 5, 16, 16, None,
                                             16, 16, 256, 1 << 20, None) == kvc.E_NULL
    assert lib.kvc_quantize_and_place_scheme(ctypes.byref(g), ctypes.byref(sc_ok), 0,
                                             ctypes.byref(p), 16, 16, 16, 10, 5, 16, None, 16,
                                             None, None, 256, 1 << 20, None) == kvc.E_UNSUPPORTED
    # scheme append: no scheme, a scheme that does not fit, misaligned rows, small workspace
    assert lib.kvc_append_tokens_scheme(ctypes.byref(g), None, 0, ctypes.byref(p), 16, 16, 16,
                                        256, 1 << 20, None) == kvc.E_NULL
    assert lib.kvc_append_tokens_scheme(ctypes.byref(g), ctypes.byref(sc_bad), 0, ctypes.byref(p),
                                        16, 16, 16, 256, 1 << 20, None) == kvc.E_SHAPE
    assert lib.kvc_append_tokens_scheme(ctypes.byref(g), ctypes.byref(sc_ok), 0, ctypes.byref(p),
                                        18, 16, 16, 256, 1 << 20, None) == kvc.E_ALIGN
    assert lib.kvc_append_tokens_scheme(ctypes.byref(g), ctypes.byref(sc_ok), 0, ctypes.byref(p),
                                        16, 16, 16, 256, 8, None) == kvc.E_WORKSPACE
    # score: negative window
    assert lib.kvc_score_tokens(ctypes.byref(g), 16, 16, 10, 5, ctypes.c_float(1.0),
                                ctypes.c_float(0.1), -1, None, 16, 16, None, None,
                                None) == kvc.E_SHAPE


def test_compaction_round_rejects_bad_arguments():
    import ctypes as ct
    from mixed_precision_paged_score_amd import kvc
    lib = kvc._lib                     # with the argument types (int64 and size_t arguments)
    f1 = ct.c_float(1.0)
    g = kvc.make_geom(1, 4, 16, 4, 64, 1 << 12)
    p = kvc.PoolPtrs(16, 16, 16, 16, 16, 16, 16)

    def call(geom, acc=16, cu=16, k=16, v=16, prev=None, tier=16, cnt=16, chg=None, ws=256,
             wsb=1 << 28, total=10, max_seqlen=5, window=4):
        return lib.kvc_compaction_round(ct.byref(geom), 0, ct.byref(p), acc, cu, total,
                                        max_seqlen, f1, f1, window, k, v, prev, tier, cnt, chg,
                                        ws, wsb, None)
    assert call(g, k=None) == kvc.E_NULL                 # prompt mode needs the rows
    assert call(g, prev=16) == kvc.E_NULL                # re-tier mode needs changed
    assert call(g, cnt=None) == kvc.E_NULL
    assert call(g, acc=18) == kvc.E_ALIGN
    assert call(g, window=-1) == kvc.E_SHAPE
    assert call(g, wsb=8) == kvc.E_WORKSPACE
    big = kvc.make_geom(1, 129, 64, 8, 64, 1 << 12)      # 1,032 KV heads
    assert call(big) == kvc.E_SHAPE
