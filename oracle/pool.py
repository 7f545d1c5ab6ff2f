"""Oracle: circular free-page ring, bidirectional page table, prefix-sum allocator.

Test infrastructure only.

Source: DiffKV review page, "What carries the argument" -- after each attention head has
decided how many high- and low-precision pages it needs, a parallel prefix sum over the
circular free page list gives every head a disjoint contiguous region of page IDs, so
allocation and recycling happen on the GPU in one coordinated step.  "Core claim": unified
pages, a circular free page list and a bidirectional page table.

Readings taken:
  * the ring holds page ids; the free pages are ring[(head + k) mod P] for k < tail - head;
    head and tail only grow.  Pages are taken at head and returned at tail.
  * one row of C slots per (layer, request, KV head): HIGH pages fill positions 0,1,2,...
    from the left, LOW pages positions C-1, C-2, ... from the right.  The reverse map
    owner[page] = gid*C + position (gid = (layer*B + b)*Hkv + h) is the other direction of
    the bidirectional table; -1 marks a free page.
  * per head i (b-major, then KV head) in one call for one layer:
        pH = ceil(n_high/16), pL = ceil(n_low/32) before, pH', pL' after;
        rebuilt head (prompt mode, or its `changed` flag): takes pH'+pL' fresh pages and
            returns all pH+pL old ones;
        other heads grow in place by (pH'-pH) + (pL'-pL) pages; a shrink there is an error.
    alloc offsets and free offsets are exclusive prefix sums over heads in that order; head
    i takes ring slots head+off_i .. head+off_i+alloc_i-1 (HIGH positions first, ascending,
    then LOW positions from the right) and writes its old pages (HIGH in row order, then
    LOW from the right end) to ring slots tail+foff_i ...
  * only pages free when the call starts are handed out; pages returned by the call become
    usable by the next call, so a rebuilt head's old pages stay readable until then.
  * all or nothing: if the total demand exceeds the free pages, or a row would exceed C
    slots, or a non-rebuilt head shrinks, a status bit is set and no state changes; once a
    status bit is set, later calls change nothing until the caller clears it.
"""
import numpy as np

HIGH_SLOTS, LOW_SLOTS = 16, 32
ST_POOL_EXHAUSTED, ST_ROW_OVERFLOW, ST_SHRINK, ST_COUNT_MISMATCH = 1, 2, 4, 8


def pages_needed(n_high, n_low):
    return -(-int(n_high) // HIGH_SLOTS), -(-int(n_low) // LOW_SLOTS)


class Pool:
    def __init__(self, num_layers, batch, num_kv_heads, row_capacity, num_pages):
        self.L, self.B, self.Hkv, self.C, self.P = (num_layers, batch, num_kv_heads,
                                                     row_capacity, num_pages)
        self.rows = np.full((self.L, self.B, self.Hkv, self.C), -1, np.int32)
        self.count = np.zeros((self.L, self.B, self.Hkv, 2), np.int32)
        self.owner = np.full(self.P, -1, np.int32)
        self.ring = np.arange(self.P, dtype=np.int32)
        self.head = 0
        self.tail = self.P
        self.status = 0

    def copy(self):
        o = Pool.__new__(Pool)
        o.__dict__ = {k: (v.copy() if isinstance(v, np.ndarray) else v)
                      for k, v in self.__dict__.items()}
        return o

    def gid(self, layer, b, h):
        return (layer * self.B + b) * self.Hkv + h

    def compact(self, layer, new_count, changed=None):
        """One allocation round for one layer.  Returns (old_rows, old_count) snapshots
        ([B][Hkv][C], [B][Hkv][2]) of the layer as it was before the call."""
        new_count = np.asarray(new_count, np.int64).reshape(self.B, self.Hkv, 2)
        old_rows = self.rows[layer].copy()
        old_count = self.count[layer].copy()
        if self.status:
            return old_rows, old_count
        C, P = self.C, self.P
        nheads = self.B * self.Hkv
        alloc = np.zeros(nheads, np.int64)
        free = np.zeros(nheads, np.int64)
        rebuilt = np.zeros(nheads, bool)
        shape = []
        err = 0
        for i in range(nheads):
            b, h = divmod(i, self.Hkv)
            pH, pL = pages_needed(*old_count[b, h])
            qH, qL = pages_needed(*new_count[b, h])
            rebuilt[i] = changed is None or bool(np.asarray(changed).reshape(-1)[i])
            if rebuilt[i]:
                alloc[i] = qH + qL
                free[i] = pH + pL
            else:
                if qH < pH or qL < pL:
                    err |= ST_SHRINK
                alloc[i] = max(qH - pH, 0) + max(qL - pL, 0)
            if qH + qL > C:
                err |= ST_ROW_OVERFLOW
            shape.append((pH, pL, qH, qL))
        if alloc.sum() > self.tail - self.head:
            err |= ST_POOL_EXHAUSTED
        if err:
            self.status |= err
            return old_rows, old_count
        off = np.concatenate([[0], np.cumsum(alloc)[:-1]])     # exclusive prefix sums
        foff = np.concatenate([[0], np.cumsum(free)[:-1]])
        for i in range(nheads):
            b, h = divmod(i, self.Hkv)
            pH, pL, qH, qL = shape[i]
            row = self.rows[layer, b, h]
            g = self.gid(layer, b, h)
            taken = [int(self.ring[(self.head + off[i] + k) % P]) for k in range(alloc[i])]
            if rebuilt[i]:
                old = [int(row[k]) for k in range(pH)] + [int(row[C - 1 - k]) for k in range(pL)]
                for k, page in enumerate(old):
                    self.ring[(self.tail + foff[i] + k) % P] = page
                    self.owner[page] = -1
                row[:] = -1
                positions = list(range(qH)) + [C - 1 - k for k in range(qL)]
            else:
                positions = list(range(pH, qH)) + [C - 1 - k for k in range(pL, qL)]
            for page, p in zip(taken, positions):
                row[p] = page
                self.owner[page] = g * C + p
            self.count[layer, b, h] = new_count[b, h]
        self.head += int(alloc.sum())
        self.tail += int(free.sum())
        return old_rows, old_count

    # ---- invariant checks (I1..I6) used by tests -------------------------------------
    def check_invariants(self):
        P, C = self.P, self.C
        assert 0 <= self.tail - self.head <= P
        free_ids = [int(self.ring[(self.head + k) % P]) for k in range(self.tail - self.head)]
        live = {}
        for l in range(self.L):
            for b in range(self.B):
                for h in range(self.Hkv):
                    row = self.rows[l, b, h]
                    nh, nl = self.count[l, b, h]
                    pH, pL = pages_needed(nh, nl)
                    assert pH + pL <= C
                    # I5 row shape and I6 page counts
                    assert np.all(row[:pH] >= 0)
                    if pL:
                        assert np.all(row[C - pL:] >= 0)
                    assert np.all(row[pH:C - pL] == -1)
                    g = self.gid(l, b, h)
                    for p in list(range(pH)) + list(range(C - pL, C)):
                        page = int(row[p])
                        assert page not in live, "page in two rows"
                        live[page] = g * C + p
        # I1 every page is either free (exactly once) or live (exactly once)
        assert len(set(free_ids)) == len(free_ids)
        assert not (set(free_ids) & set(live))
        # I2 conservation
        assert len(free_ids) + len(live) == P
        # I4 reverse map agrees with the rows
        for page in free_ids:
            assert self.owner[page] == -1
        for page, o in live.items():
            assert self.owner[page] == o
        return True
