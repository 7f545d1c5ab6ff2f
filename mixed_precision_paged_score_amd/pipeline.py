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
        self.ws_decode_acc = None           # made on first use (it holds every live logit)
        self.ws_round = None                # made on first use of the fused round
        self.seqlen_cap = self.max_seqlen   # longest request the workspaces are sized for
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

    def prompt_fused(self, layer, acc, k, v):
        """The same round as prompt() through kvc_compaction_round (up to 1024 KV heads)."""
        w = self.w
        if self.ws_round is None:
            self.ws_round = kvc.workspace(self.geom, kvc.OP_ROUND, self.max_seqlen,
                                          device=self.device)
        kvc.compaction_round(self.geom, layer, self.pool, acc, self.cu, self.T, self.max_seqlen,
                             w.alpha_h, w.alpha_l, w.window, k, v, self.tier, self.new_count,
                             self.ws_round)

    def prompt_scheme(self, layer, acc, k, v, scheme):
        """A prompt round whose pages use a precision scheme (kvc.make_scheme): score,
        compact, then the scheme's page writer."""
        self.score(acc)
        self.compact(layer)
        kvc.quantize_and_place_scheme(self.geom, scheme, layer, self.pool, k, v, self.cu, self.T,
                                      self.max_seqlen, self.tier, self.ws_quant)

    def decode_scheme(self, layer, q, out, scheme):
        kvc.paged_decode_attention_scheme(self.geom, scheme, layer, self.pool, q, self.scale, out,
                                          self.ws_decode)

    def decode(self, layer, q, out):
        kvc.paged_decode_attention(self.geom, layer, self.pool, q, self.scale, out,
                                   self.ws_decode)

    def decode_acc(self, layer, q, out, acc, cu=None):
        """Decode attention that also adds every cached token's attention weight into
        `acc` ([T][Hq] float32 over this path's current requests, or rows laid out by `cu`,
        e.g. a padded [B][seqlen_cap][Hq] buffer with cu = b * seqlen_cap)."""
        if self.ws_decode_acc is None:
            self.ws_decode_acc = kvc.workspace(self.geom, kvc.OP_DECODE_ACC, self.seqlen_cap,
                                               device=self.device)
        scheme = getattr(self, "scheme", None)
        if scheme is None:
            kvc.paged_decode_attention_acc(self.geom, layer, self.pool, q, self.scale, out, acc,
                                           self.cu if cu is None else cu,
                                           self.max_seqlen if cu is None else self.seqlen_cap,
                                           self.ws_decode_acc)
        else:
            kvc.paged_decode_attention_scheme_acc(
                self.geom, scheme, layer, self.pool, q, self.scale, out, acc,
                self.cu if cu is None else cu,
                self.max_seqlen if cu is None else self.seqlen_cap, self.ws_decode_acc)

    # -- HIP graphs -------------------------------------------------------------------------
    # Every library call is asynchronous on the current stream, reads its sizes from device
    # memory and clears its own scratch with kernels (no memset nodes), so a sequence of calls
    # can be captured once and replayed; each replay redoes all the work on the current data.
    def capture_prompt(self, layer, acc, k, v, fused=False):
        """Graph of one prompt round of a layer: score, compact (prompt mode: the layer's
        current pages go back to the ring, new ones are assigned) and quantize/place, as the
        three calls or (fused) as kvc_compaction_round."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if fused:
                self.prompt_fused(layer, acc, k, v)
            else:
                self.prompt(layer, acc, k, v)
        return g

    def capture_decode(self, layer, qs, out):
        """Graph of len(qs) decode steps (one per query tensor, all writing `out`)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for q in qs:
                self.decode(layer, q, out)
        return g


class GenerationPath(PromptPath):
    """Prompt, then per decode step one appended token per (request, KV head), and every
    `round` steps a re-tier round: score with the previous tiers as ceiling, compact with the
    rebuilt heads' flags, quantize/place in re-tier mode.  The per-position tier state is the
    caller's bookkeeping: it is kept here as [B][max_len][Hkv] and packed to the ragged layout
    the library reads (a device copy, outside the library calls)."""

    def __init__(self, w, max_len, device="cuda", num_pages=None, scheme=None):
        import dataclasses
        # size workspaces and row capacity for the longest sequence the run reaches
        wl = dataclasses.replace(w, seqlens=[max_len] * w.batch)
        super().__init__(wl, device, num_pages)
        self.w = w
        self.scheme = scheme        # a kvc.Scheme: every page of the run in its layout
        self.lens = list(w.seqlens)
        H = w.num_kv_heads
        self.state = torch.full((w.batch, max_len, H), kvc.PRUNE, dtype=torch.uint8, device=device)
        self.ws_append = kvc.workspace(self.geom, kvc.OP_APPEND, device=device)
        self.ws_gen = None
        self.decided = torch.empty((w.batch, H), dtype=torch.uint8, device=device)
        self.changed = torch.empty((w.batch, H), dtype=torch.uint8, device=device)
        self.old_rows = torch.empty((w.batch, H, self.geom.row_capacity), dtype=torch.int32,
                                    device=device)
        self.old_count = torch.empty((w.batch, H, 2), dtype=torch.int32, device=device)
        self._set_layout()

    def _set_layout(self):
        import numpy as np
        cu = np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)
        self.cu = torch.tensor(cu, dtype=torch.int32, device=self.device)
        self.T = int(cu[-1])
        self.max_seqlen = max(self.lens)
        self.lens_dev = torch.tensor(self.lens, dtype=torch.int32, device=self.device)
        self._bidx = torch.arange(self.w.batch, device=self.device)
        self._cu_step = torch.arange(self.w.batch + 1, dtype=torch.int32, device=self.device)

    def packed_state(self):
        return torch.cat([self.state[b, :n] for b, n in enumerate(self.lens)]).contiguous()

    def unpack_state(self, tier):
        o = 0
        for b, n in enumerate(self.lens):
            self.state[b, :n] = tier[o:o + n]
            o += n

    def prompt(self, layer, acc, k, v):
        self._set_layout()
        if self.scheme is None:
            super().prompt(layer, acc, k, v)
        else:
            self.prompt_scheme(layer, acc, k, v, self.scheme)
        self.unpack_state(self.tier[:self.T])

    def decode(self, layer, q, out):
        if self.scheme is None:
            super().decode(layer, q, out)
        else:
            self.decode_scheme(layer, q, out, self.scheme)

    def append(self, layer, k_new, v_new):
        if self.scheme is None:
            kvc.append_tokens(self.geom, layer, self.pool, k_new, v_new, self.lens_dev,
                              self.ws_append)
        else:
            kvc.append_tokens_scheme(self.geom, self.scheme, layer, self.pool, k_new, v_new,
                                     self.lens_dev, self.ws_append)
        # bookkeeping: the new positions are HIGH, every request is one token longer
        self.state[self._bidx, self.lens_dev.long()] = kvc.HIGH
        self.lens_dev.add_(1)
        self.cu.add_(self._cu_step)
        self.lens = [n + 1 for n in self.lens]
        self.T += self.w.batch
        self.max_seqlen += 1

    def padded_cu(self):
        """Row offsets of a padded accumulator buffer [B][seqlen_cap][Hq]: the layout both
        accumulating calls accept for every step of a generation run."""
        return torch.arange(self.w.batch + 1, dtype=torch.int32,
                            device=self.device) * self.seqlen_cap

    def step(self, layer, k_new, v_new, acc, cu=None):
        """One decode step under the per-step policy: append the new tokens and give the
        token leaving the window its tier.  acc float32 [T + B][Hq] over the lengths after
        the new tokens (the layout of cu_next), or rows laid out by `cu` (padded_cu())."""
        w = self.w
        if self.ws_gen is None:
            self.ws_gen = kvc.workspace(self.geom, kvc.OP_GENERATE, device=self.device)
        cu_next = self.cu + self._cu_step
        if self.scheme is None:
            kvc.generation_step(self.geom, layer, self.pool, k_new, v_new, self.lens_dev, acc,
                                cu_next if cu is None else cu, w.alpha_h, w.alpha_l, w.window,
                                self.decided, self.ws_gen)
        else:
            kvc.generation_step_scheme(self.geom, self.scheme, layer, self.pool, k_new, v_new,
                                       self.lens_dev, acc, cu_next if cu is None else cu,
                                       w.alpha_h, w.alpha_l, w.window, self.decided,
                                       self.ws_gen)
        # bookkeeping: the new positions are HIGH, the leaving token takes its tier
        pos = self.lens_dev.long()
        self.state[self._bidx, pos] = kvc.HIGH
        t_c = (pos - w.window).clamp(min=0)
        left = self.decided != kvc.NO_TOKEN
        cur = self.state[self._bidx, t_c]
        self.state[self._bidx, t_c] = torch.where(left, self.decided, cur)
        self.lens_dev.add_(1)
        self.cu = cu_next
        self.lens = [n + 1 for n in self.lens]
        self.T += self.w.batch
        self.max_seqlen += 1

    def retier_fused(self, layer, acc):
        """The same round as retier() through kvc_compaction_round (up to 1024 KV heads)."""
        w = self.w
        if self.ws_round is None:
            self.ws_round = kvc.workspace(self.geom, kvc.OP_ROUND, self.seqlen_cap,
                                          device=self.device)
        prev = self.packed_state()
        kvc.compaction_round(self.geom, layer, self.pool, acc, self.cu, self.T, self.max_seqlen,
                             w.alpha_h, w.alpha_l, w.window, None, None, self.tier,
                             self.new_count, self.ws_round, prev_tier=prev, changed=self.changed)
        self.unpack_state(self.tier[:self.T])

    def retier(self, layer, acc):
        w = self.w
        prev = self.packed_state()
        kvc.score_tokens(self.geom, acc, self.cu, self.T, self.max_seqlen, w.alpha_h, w.alpha_l,
                         w.window, self.tier, self.new_count, prev_tier=prev,
                         changed=self.changed, dev_status=self.score_status)
        kvc.compact_pages(self.geom, layer, self.pool, self.new_count, self.ws_compact,
                          changed=self.changed, old_rows=self.old_rows, old_count=self.old_count)
        if self.scheme is None:
            kvc.quantize_and_place(self.geom, layer, self.pool, None, None, self.cu, self.T,
                                   self.max_seqlen, self.tier, self.ws_quant, prev_tier=prev,
                                   changed=self.changed, old_rows=self.old_rows,
                                   old_count=self.old_count)
        else:
            kvc.quantize_and_place_scheme(self.geom, self.scheme, layer, self.pool, None, None,
                                          self.cu, self.T, self.max_seqlen, self.tier,
                                          self.ws_quant, prev_tier=prev, changed=self.changed,
                                          old_rows=self.old_rows, old_count=self.old_count)
        self.unpack_state(self.tier[:self.T])
