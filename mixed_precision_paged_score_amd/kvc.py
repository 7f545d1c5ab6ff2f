"""Thin ctypes binding of libkvc (include/kvc.h).  Argument marshalling only: every step of
the path runs in the library's HIP kernels.  PyTorch provides device memory and the
current stream.  If libkvc.so is missing this module raises on import -- there is no
fallback implementation.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVC_LIB_PATH") or os.path.join(HERE, "libkvc.so")

OK, E_NULL, E_ALIGN, E_SHAPE, E_WORKSPACE, E_HIP, E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
DEV_POOL_EXHAUSTED, DEV_ROW_OVERFLOW, DEV_SHRINK, DEV_COUNT_MISMATCH, DEV_SEQLEN = 1, 2, 4, 8, 16
DEV_INTERNAL, DEV_BAD_TIER = 32, 64
PRUNE, LOW, HIGH, FRESH = 0, 1, 2, 3
OP_COMPACT, OP_QUANTIZE, OP_DECODE, OP_APPEND, OP_DECODE_ACC, OP_GENERATE = 1, 2, 3, 4, 5, 6
OP_ROUND = 8
OP_PREFILL = 7
HEAD_DIM, HIGH_SLOTS, LOW_SLOTS, PAGE_BYTES = 128, 16, 32, 3456
STATIC_SCRATCH_BYTES = 64 << 20     # the device array behind kvc_paged_decode_attention_static
GEN_MAX_WINDOW = 112
NO_TOKEN = 255      # generation step: no token left the window

EXPORTS = ["kvc_version", "kvc_last_error", "kvc_workspace_bytes", "kvc_pool_init",
           "kvc_score_tokens", "kvc_compact_pages", "kvc_quantize_and_place",
           "kvc_paged_decode_attention", "kvc_paged_decode_attention_acc", "kvc_append_tokens",
           "kvc_generation_step", "kvc_prefill_attention", "kvc_quantize_and_place_scheme",
           "kvc_paged_decode_attention_scheme", "kvc_paged_decode_attention_static",
           "kvc_append_tokens_scheme", "kvc_generation_step_scheme",
           "kvc_paged_decode_attention_scheme_acc", "kvc_compaction_round"]

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m mixed_precision_paged_score_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)


class Geom(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("row_capacity", ctypes.c_int32), ("num_pages", ctypes.c_int64)]


class Scheme(ctypes.Structure):
    """Key / value bits of the HIGH and LOW tiers (kvc_scheme)."""
    _fields_ = [("k_bits_high", ctypes.c_int32), ("v_bits_high", ctypes.c_int32),
                ("k_bits_low", ctypes.c_int32), ("v_bits_low", ctypes.c_int32)]


FORMATS = {"K8V4": (8, 4), "K4V8": (4, 8), "K8V2": (8, 2), "K4V2": (4, 2), "K2V4": (2, 4),
           "K4V1": (4, 1)}


def make_scheme(high="K8V4", low="K4V2"):
    return Scheme(*FORMATS[high], *FORMATS[low])


class PoolPtrs(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("owner", ctypes.c_void_p),
                ("free_ring", ctypes.c_void_p), ("ring_ctr", ctypes.c_void_p),
                ("dev_status", ctypes.c_void_p)]


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_G, _P = ctypes.POINTER(Geom), ctypes.POINTER(PoolPtrs)

_lib.kvc_version.restype = ctypes.c_char_p
_lib.kvc_last_error.restype = ctypes.c_char_p
_lib.kvc_workspace_bytes.argtypes = [_G, _i32, _i32]
_lib.kvc_workspace_bytes.restype = _sz
_lib.kvc_pool_init.argtypes = [_G, _P, _vp]
_lib.kvc_score_tokens.argtypes = [_G, _vp, _vp, _i64, _i32, _f32, _f32, _i32, _vp, _vp, _vp,
                                  _vp, _vp, _vp]
_lib.kvc_compact_pages.argtypes = [_G, _i32, _P, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.kvc_quantize_and_place.argtypes = [_G, _i32, _P, _vp, _vp, _vp, _i64, _i32, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _sz, _vp]
_lib.kvc_paged_decode_attention.argtypes = [_G, _i32, _P, _vp, _f32, _vp, _i32, _vp, _sz, _vp]
_lib.kvc_paged_decode_attention_static.argtypes = [_G, _i32, _P, _vp, _f32, _vp, _i32, _vp]
_lib.kvc_paged_decode_attention_acc.argtypes = [_G, _i32, _P, _vp, _f32, _vp, _i32, _vp, _vp,
                                                _i32, _vp, _sz, _vp]
_lib.kvc_append_tokens.argtypes = [_G, _i32, _P, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.kvc_generation_step.argtypes = [_G, _i32, _P, _vp, _vp, _vp, _vp, _vp, _f32, _f32, _i32,
                                     _vp, _vp, _sz, _vp]
_lib.kvc_prefill_attention.argtypes = [_G, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _i32, _vp, _vp,
                                       _vp, _sz, _vp]
_S = ctypes.POINTER(Scheme)
_lib.kvc_quantize_and_place_scheme.argtypes = [_G, _S, _i32, _P, _vp, _vp, _vp, _i64, _i32, _vp,
                                               _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.kvc_append_tokens_scheme.argtypes = [_G, _S, _i32, _P, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.kvc_generation_step_scheme.argtypes = [_G, _S, _i32, _P, _vp, _vp, _vp, _vp, _vp, _f32,
                                            _f32, _i32, _vp, _vp, _sz, _vp]
_lib.kvc_paged_decode_attention_scheme_acc.argtypes = [_G, _S, _i32, _P, _vp, _f32, _vp, _i32,
                                                       _vp, _vp, _i32, _vp, _sz, _vp]
_lib.kvc_compaction_round.argtypes = [_G, _i32, _P, _vp, _vp, _i64, _i32, _f32, _f32, _i32, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.kvc_paged_decode_attention_scheme.argtypes = [_G, _S, _i32, _P, _vp, _f32, _vp, _i32, _vp,
                                                   _sz, _vp]
for _f in ("kvc_pool_init", "kvc_score_tokens", "kvc_compact_pages", "kvc_quantize_and_place",
           "kvc_paged_decode_attention", "kvc_paged_decode_attention_acc", "kvc_append_tokens",
           "kvc_generation_step", "kvc_prefill_attention", "kvc_quantize_and_place_scheme",
           "kvc_paged_decode_attention_scheme", "kvc_paged_decode_attention_static",
           "kvc_append_tokens_scheme", "kvc_generation_step_scheme",
           "kvc_paged_decode_attention_scheme_acc", "kvc_compaction_round"):
    getattr(_lib, _f).restype = ctypes.c_int


class KvcError(RuntimeError):
    pass


def _check(rc, name):
    if rc != OK:
        msg = _lib.kvc_last_error().decode() if rc == E_HIP else ""
        raise KvcError(f"{name} returned {rc} {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def version():
    return _lib.kvc_version().decode()


def make_geom(num_layers, batch, num_q_heads, num_kv_heads, row_capacity, num_pages):
    return Geom(num_layers, batch, num_q_heads, num_kv_heads, row_capacity, num_pages)


def workspace_bytes(geom, op, max_seqlen=0):
    return int(_lib.kvc_workspace_bytes(ctypes.byref(geom), op, max_seqlen))


def workspace(geom, op, max_seqlen=0, device="cuda"):
    """Workspace for one call type (zero-filled; every call initialises what it reads)."""
    n = max(workspace_bytes(geom, op, max_seqlen), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


class Pool:
    """Device arrays of one page pool (torch tensors) and their C view."""

    def __init__(self, geom, device="cuda"):
        g = geom
        self.geom = g
        L, B, H, C, P = g.num_layers, g.batch, g.num_kv_heads, g.row_capacity, g.num_pages
        self.pages = torch.empty((P, PAGE_BYTES), dtype=torch.uint8, device=device)
        self.page_table = torch.empty((L, B, H, C), dtype=torch.int32, device=device)
        self.count = torch.empty((L, B, H, 2), dtype=torch.int32, device=device)
        self.owner = torch.empty((P,), dtype=torch.int32, device=device)
        self.free_ring = torch.empty((P,), dtype=torch.int32, device=device)
        self.ring_ctr = torch.empty((2,), dtype=torch.int64, device=device)
        self.dev_status = torch.empty((1,), dtype=torch.int32, device=device)
        self.c = PoolPtrs(*(t.data_ptr() for t in (self.pages, self.page_table, self.count,
                                                   self.owner, self.free_ring, self.ring_ctr,
                                                   self.dev_status)))

    def init(self, stream=None):
        _check(_lib.kvc_pool_init(ctypes.byref(self.geom), ctypes.byref(self.c), _stream(stream)),
               "kvc_pool_init")

    def status(self):
        return int(self.dev_status.item())

    def clear_status(self):
        self.dev_status.zero_()


def score_tokens(geom, acc_sum, cu_seqlens, total_tokens, max_seqlen, alpha_h, alpha_l,
                 window, tier, new_count, prev_tier=None, changed=None, dev_status=None,
                 stream=None):
    _check(_lib.kvc_score_tokens(ctypes.byref(geom), _ptr(acc_sum), _ptr(cu_seqlens),
                                 int(total_tokens), int(max_seqlen), float(alpha_h),
                                 float(alpha_l), int(window), _ptr(prev_tier), _ptr(tier),
                                 _ptr(new_count), _ptr(changed), _ptr(dev_status),
                                 _stream(stream)), "kvc_score_tokens")


def compact_pages(geom, layer, pool, new_count, ws, changed=None, old_rows=None,
                  old_count=None, stream=None):
    _check(_lib.kvc_compact_pages(ctypes.byref(geom), int(layer), ctypes.byref(pool.c),
                                  _ptr(new_count), _ptr(changed), _ptr(old_rows),
                                  _ptr(old_count), _ptr(ws), ws.numel(), _stream(stream)),
           "kvc_compact_pages")


def quantize_and_place(geom, layer, pool, k, v, cu_seqlens, total_tokens, max_seqlen, tier,
                       ws, prev_tier=None, changed=None, old_rows=None, old_count=None,
                       stream=None):
    _check(_lib.kvc_quantize_and_place(ctypes.byref(geom), int(layer), ctypes.byref(pool.c),
                                       _ptr(k), _ptr(v), _ptr(cu_seqlens), int(total_tokens),
                                       int(max_seqlen), _ptr(tier), _ptr(prev_tier),
                                       _ptr(changed), _ptr(old_rows), _ptr(old_count),
                                       _ptr(ws), ws.numel(), _stream(stream)),
           "kvc_quantize_and_place")


def paged_decode_attention(geom, layer, pool, q, softmax_scale, out, ws, stream=None):
    _check(_lib.kvc_paged_decode_attention(ctypes.byref(geom), int(layer), ctypes.byref(pool.c),
                                           _ptr(q), float(softmax_scale), _ptr(out),
                                           int(out.dtype == torch.float32), _ptr(ws), ws.numel(),
                                           _stream(stream)), "kvc_paged_decode_attention")


def paged_decode_attention_static(geom, layer, pool, q, softmax_scale, out, stream=None):
    """kvc_paged_decode_attention with its partials in the library's own device array (no
    workspace argument, no allocation)."""
    _check(_lib.kvc_paged_decode_attention_static(ctypes.byref(geom), int(layer),
                                                  ctypes.byref(pool.c), _ptr(q),
                                                  float(softmax_scale), _ptr(out),
                                                  int(out.dtype == torch.float32),
                                                  _stream(stream)),
           "kvc_paged_decode_attention_static")


def paged_decode_attention_acc(geom, layer, pool, q, softmax_scale, out, acc_sum, cu_seqlens,
                               max_seqlen, ws, stream=None):
    _check(_lib.kvc_paged_decode_attention_acc(ctypes.byref(geom), int(layer),
                                               ctypes.byref(pool.c), _ptr(q), float(softmax_scale),
                                               _ptr(out), int(out.dtype == torch.float32),
                                               _ptr(acc_sum), _ptr(cu_seqlens), int(max_seqlen),
                                               _ptr(ws), ws.numel(), _stream(stream)),
           "kvc_paged_decode_attention_acc")


def append_tokens(geom, layer, pool, k_new, v_new, positions, ws, stream=None):
    _check(_lib.kvc_append_tokens(ctypes.byref(geom), int(layer), ctypes.byref(pool.c),
                                  _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(ws),
                                  ws.numel(), _stream(stream)), "kvc_append_tokens")


def generation_step(geom, layer, pool, k_new, v_new, positions, acc_sum, cu_seqlens, alpha_h,
                    alpha_l, window, tier_out, ws, stream=None):
    _check(_lib.kvc_generation_step(ctypes.byref(geom), int(layer), ctypes.byref(pool.c),
                                    _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(acc_sum),
                                    _ptr(cu_seqlens), float(alpha_h), float(alpha_l),
                                    int(window), _ptr(tier_out), _ptr(ws), ws.numel(),
                                    _stream(stream)), "kvc_generation_step")


def generation_step_scheme(geom, scheme, layer, pool, k_new, v_new, positions, acc_sum,
                           cu_seqlens, alpha_h, alpha_l, window, tier_out, ws, stream=None):
    _check(_lib.kvc_generation_step_scheme(ctypes.byref(geom), ctypes.byref(scheme), int(layer),
                                           ctypes.byref(pool.c), _ptr(k_new), _ptr(v_new),
                                           _ptr(positions), _ptr(acc_sum), _ptr(cu_seqlens),
                                           float(alpha_h), float(alpha_l), int(window),
                                           _ptr(tier_out), _ptr(ws), ws.numel(),
                                           _stream(stream)), "kvc_generation_step_scheme")


def prefill_attention(geom, q, k, v, cu_seqlens, max_seqlen, softmax_scale, out, acc_sum, ws,
                      dev_status=None, stream=None):
    _check(_lib.kvc_prefill_attention(ctypes.byref(geom), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(cu_seqlens), int(max_seqlen), float(softmax_scale),
                                      _ptr(out), int(out.dtype == torch.float32),
                                      None if acc_sum is None else _ptr(acc_sum),
                                      None if dev_status is None else _ptr(dev_status),
                                      _ptr(ws), ws.numel(), _stream(stream)),
           "kvc_prefill_attention")


def quantize_and_place_scheme(geom, scheme, layer, pool, k, v, cu_seqlens, total_tokens,
                              max_seqlen, tier, ws, prev_tier=None, changed=None, old_rows=None,
                              old_count=None, stream=None):
    _check(_lib.kvc_quantize_and_place_scheme(ctypes.byref(geom), ctypes.byref(scheme),
                                              int(layer), ctypes.byref(pool.c), _ptr(k), _ptr(v),
                                              _ptr(cu_seqlens), int(total_tokens),
                                              int(max_seqlen), _ptr(tier), _ptr(prev_tier),
                                              _ptr(changed), _ptr(old_rows), _ptr(old_count),
                                              _ptr(ws), ws.numel(), _stream(stream)),
           "kvc_quantize_and_place_scheme")


def paged_decode_attention_scheme_acc(geom, scheme, layer, pool, q, softmax_scale, out, acc_sum,
                                      cu_seqlens, max_seqlen, ws, stream=None):
    _check(_lib.kvc_paged_decode_attention_scheme_acc(
        ctypes.byref(geom), ctypes.byref(scheme), int(layer), ctypes.byref(pool.c), _ptr(q),
        float(softmax_scale), _ptr(out), int(out.dtype == torch.float32), _ptr(acc_sum),
        _ptr(cu_seqlens), int(max_seqlen), _ptr(ws), ws.numel(), _stream(stream)),
        "kvc_paged_decode_attention_scheme_acc")


def compaction_round(geom, layer, pool, acc_sum, cu_seqlens, total_tokens, max_seqlen, alpha_h,
                     alpha_l, window, k, v, tier, new_count, ws, prev_tier=None, changed=None,
                     stream=None):
    _check(_lib.kvc_compaction_round(ctypes.byref(geom), int(layer), ctypes.byref(pool.c),
                                     _ptr(acc_sum), _ptr(cu_seqlens), int(total_tokens),
                                     int(max_seqlen), float(alpha_h), float(alpha_l), int(window),
                                     _ptr(k), _ptr(v), _ptr(prev_tier), _ptr(tier),
                                     _ptr(new_count), _ptr(changed), _ptr(ws), ws.numel(),
                                     _stream(stream)), "kvc_compaction_round")


def append_tokens_scheme(geom, scheme, layer, pool, k_new, v_new, positions, ws, stream=None):
    _check(_lib.kvc_append_tokens_scheme(ctypes.byref(geom), ctypes.byref(scheme), int(layer),
                                         ctypes.byref(pool.c), _ptr(k_new), _ptr(v_new),
                                         _ptr(positions), _ptr(ws), ws.numel(), _stream(stream)),
           "kvc_append_tokens_scheme")


def paged_decode_attention_scheme(geom, scheme, layer, pool, q, softmax_scale, out, ws,
                                  stream=None):
    _check(_lib.kvc_paged_decode_attention_scheme(ctypes.byref(geom), ctypes.byref(scheme),
                                                  int(layer), ctypes.byref(pool.c), _ptr(q),
                                                  float(softmax_scale), _ptr(out),
                                                  int(out.dtype == torch.float32), _ptr(ws),
                                                  ws.numel(), _stream(stream)),
           "kvc_paged_decode_attention_scheme")
