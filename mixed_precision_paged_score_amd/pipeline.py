"""Device-side driver of the hot path for one workload: buffers, and the four library calls
in order (score -> compact -> quantize/place for a layer's prompt, then decode attention).
Marshalling only; all arithmetic runs in libkvc's kernels."""
import math

import torch

from . import kvc


class PromptPath:
    def __init__(self, w, device="cuda", num_pages=None):
        self.w = w
        self.device = device
        P = int(num_pages if num_pages is not None else w.num_pages)
        self.geom = kvc.make_geom(w.num_layers, w.batch, w.num_q_heads, w.num_kv_heads,
                                  w.row_capacity, P)
        self.pool = kvc.Pool(self.geom, device)
        self.pool.init()
        self.T = w.total_tokens
        self.max_seqlen = max(w.seqlens) if w.seqlens else 0
        self.cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32, device=device)
        H = w.num_kv_heads
        self.tier = torch.empty((max(self.T, 1), H), dtype=torch.uint8, device=device)
        self.new_count = torch.empty((w.batch, H, 2), dtype=torch.int32, device=device)
        self.zero_count = torch.zeros((w.batch, H, 2), dtype=torch.int32, device=device)
        self.score_status = torch.zeros((1,), dtype=torch.int32, device=device)
        self.ws_compact = kvc.workspace(self.geom, kvc.OP_COMPACT, device=device)
        self.ws_quant = kvc.workspace(self.geom, kvc.OP_QUANTIZE, self.max_seqlen, device=device)
        self.ws_decode = kvc.workspace(self.geom, kvc.OP_DECODE, device=device)
        self.scale = 1.0 / math.sqrt(kvc.HEAD_DIM)

    # -- steps ----------------------------------------------------------------------------
    def score(self, acc):
        w = self.w
        kvc.score_tokens(self.geom, acc, self.cu, self.T, self.max_seqlen, w.alpha_h, w.alpha_l,
                         w.window, self.tier, self.new_count, dev_status=self.score_status)

    def compact(self, layer, new_count=None, old_rows=None, old_count=None):
        kvc.compact_pages(self.geom, layer, self.pool,
                          self.new_count if new_count is None else new_count, self.ws_compact,
                          old_rows=old_rows, old_count=old_count)

    def release(self, layer):
        """Return every page of the layer to the ring (prompt-mode round with zero counts)."""
        self.compact(layer, self.zero_count)

    def place(self, layer, k, v):
        kvc.quantize_and_place(self.geom, layer, self.pool, k, v, self.cu, self.T,
                               self.max_seqlen, self.tier, self.ws_quant)

    def prompt(self, layer, acc, k, v):
        self.score(acc)
        self.compact(layer)
        self.place(layer, k, v)

    def decode(self, layer, q, out):
        kvc.paged_decode_attention(self.geom, layer, self.pool, q, self.scale, out,
                                   self.ws_decode)
