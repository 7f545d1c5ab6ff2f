"""Pins of the oracle allocator: closed form on a fresh ring, invariants I1-I6 across random
rounds, all-or-nothing failures (DiffKV review page, 'What carries the argument': disjoint
contiguous region of page ids per head from a prefix sum over the circular free list)."""
import numpy as np
import pytest

from oracle import pool as opool


def _counts(rng, B, H, nmax):
    return rng.integers(0, nmax + 1, size=(B, H, 2))


def test_fresh_ring_closed_form():
    B, H, C, P = 3, 4, 40, 2000
    pl = opool.Pool(1, B, H, C, P)
    rng = np.random.default_rng(0)
    cnt = _counts(rng, B, H, 300)
    pl.compact(0, cnt)
    off = 0
    for b in range(B):
        for h in range(H):
            qH, qL = opool.pages_needed(*cnt[b, h])
            row = pl.rows[0, b, h]
            # HIGH pages first (ascending row positions), then LOW from the right end
            assert row[:qH].tolist() == list(range(off, off + qH))
            assert [row[C - 1 - k] for k in range(qL)] == list(range(off + qH, off + qH + qL))
            off += qH + qL
    assert pl.head == off and pl.tail == P
    pl.check_invariants()


def test_pages_needed():
    assert opool.pages_needed(0, 0) == (0, 0)
    assert opool.pages_needed(1, 1) == (1, 1)
    assert opool.pages_needed(16, 32) == (1, 1)
    assert opool.pages_needed(17, 33) == (2, 2)


def test_random_rounds_keep_invariants_and_contiguity():
    rng = np.random.default_rng(1)
    L, B, H, C, P = 2, 3, 2, 30, 400
    pl = opool.Pool(L, B, H, C, P)
    cur = np.zeros((L, B, H, 2), np.int64)
    for it in range(60):
        layer = int(rng.integers(0, L))
        mode = rng.integers(0, 3)
        if mode == 0:           # prompt: everything rebuilt
            new = _counts(rng, B, H, 150)
            changed = None
        else:                   # round: some heads shrink (changed), others grow
            new = cur[layer].copy()
            changed = rng.integers(0, 2, size=(B, H)).astype(np.uint8)
            grow = rng.integers(0, 40, size=(B, H, 2))
            shrink = np.minimum(new, rng.integers(0, 60, size=(B, H, 2)))
            new = np.where(changed[..., None] == 1, new - shrink, new + grow)
        before = pl.copy()
        head0 = pl.head
        pl.compact(layer, new, changed)
        if pl.status:
            # all or nothing: nothing but the status changed
            assert np.array_equal(pl.rows, before.rows) and np.array_equal(pl.ring, before.ring)
            assert np.array_equal(pl.owner, before.owner) and pl.head == before.head
            pl.status = 0
            continue
        cur[layer] = new
        pl.check_invariants()
        # I3: the pages handed out form one contiguous ring segment, in head order
        taken = [int(before.ring[(head0 + k) % P]) for k in range(pl.head - head0)]
        got = []
        for b in range(B):
            for h in range(H):
                r1 = pl.rows[layer, b, h]
                pH, pL = opool.pages_needed(*before.count[layer, b, h])
                qH, qL = opool.pages_needed(*new[b, h])
                if changed is None or changed[b, h]:
                    pH, pL = 0, 0
                got += [int(r1[p]) for p in range(pH, qH)]
                got += [int(r1[C - 1 - k]) for k in range(pL, qL)]
        assert got == taken


def test_exhaustion_is_all_or_nothing_and_sticky():
    pl = opool.Pool(1, 2, 2, 100, 50)
    cnt = np.full((2, 2, 2), 16 * 10)    # 10 HIGH pages + 5 LOW pages per head = 60 > 50
    before = pl.copy()
    pl.compact(0, cnt)
    assert pl.status & opool.ST_POOL_EXHAUSTED
    assert np.array_equal(pl.rows, before.rows) and pl.head == 0 and pl.tail == 50
    # sticky: a call that would fit changes nothing while the bit is set
    pl.compact(0, np.ones((2, 2, 2)))
    assert np.all(pl.rows == -1)
    pl.status = 0
    pl.compact(0, np.ones((2, 2, 2)))
    assert pl.head == 8
    pl.check_invariants()


def test_row_overflow_and_shrink_errors():
    pl = opool.Pool(1, 1, 2, 3, 100)
    pl.compact(0, [[[16 * 3, 1], [1, 1]]])          # 3 + 1 pages > C = 3
    assert pl.status == opool.ST_ROW_OVERFLOW
    pl.status = 0
    pl.compact(0, [[[20, 0], [1, 1]]])
    assert pl.status == 0
    before = pl.copy()
    pl.compact(0, [[[1, 0], [1, 1]]], changed=np.zeros((1, 2), np.uint8))   # shrink, not rebuilt
    assert pl.status == opool.ST_SHRINK
    assert np.array_equal(pl.rows, before.rows)


def test_rebuilt_pages_go_to_tail_in_row_order_and_wrap():
    B, H, C, P = 1, 2, 10, 12
    pl = opool.Pool(1, B, H, C, P)
    pl.compact(0, [[[40, 40], [20, 0]]])            # head0: 3 H + 2 L, head1: 2 H
    r0 = pl.rows[0, 0].copy()       # [h][row position] of request 0
    assert pl.head == 7
    pl.compact(0, [[[16, 0], [0, 33]]])             # rebuild both: 1 + 2 pages
    # freed: head0 H(row 0,1,2) then L(row C-1, C-2); head1 H(row 0,1); tail was 12
    freed = [r0[0, 0], r0[0, 1], r0[0, 2], r0[0, C - 1], r0[0, C - 2], r0[1, 0], r0[1, 1]]
    assert [pl.ring[(12 + k) % P] for k in range(7)] == [int(x) for x in freed]
    assert pl.head == 10 and pl.tail == 19
    pl.check_invariants()
    # the next prompt round reuses the freed pages across the ring's end
    pl.compact(0, [[[16 * 5, 0], [0, 0]]])
    assert pl.head == 15
    pl.check_invariants()
