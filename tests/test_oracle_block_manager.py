"""Pins of the Python block-manager model against the invariants the pages fix.

* A sequence of n tokens holds exactly ceil(n / B) blocks: at most B - 1 slots
  of its last block are unused ("KV Cache 原理与 PagedAttention", §三 收益
  table; bjdmk.com.cn article, §3.1: at most 15 tokens wasted at B = 16).
* Reference counts equal the number of table entries naming each block.
* Freeing every sequence returns every block.
* Running out of blocks fails without changing any state (the pages' cue for
  preemption, "KV Cache 原理与 PagedAttention", §六).
* Copy-on-write: a write into a shared block copies it first (bjdmk.com.cn
  article, §3.2).  For the 1500-token prefix shared by 200 sequences the first
  step copies 199 times (the last holder writes in place).
"""

import copy
import math

import numpy as np
import pytest

from oracle.block_manager import (ERR_INVALID, ERR_OUT_OF_BLOCKS, OK,
                                  BlockManagerModel)


def _check_invariants(bm):
    counts = [0] * bm.num_blocks
    for s, tab in bm.tables.items():
        assert len(tab) == math.ceil(bm.ctx[s] / bm.B)
        assert len(tab) * bm.B - bm.ctx[s] <= bm.B - 1
        for b in tab:
            counts[b] += 1
    assert counts == bm.ref
    free = set(bm.free)
    assert len(free) == len(bm.free)
    for b in range(bm.num_blocks):
        assert (b in free) == (bm.ref[b] == 0)


def test_random_workload_invariants():
    rng = np.random.default_rng(21)
    bm = BlockManagerModel(64, 8, rng.permutation(64))
    live = []
    nxt = 0
    for step in range(400):
        op = rng.integers(0, 4)
        if op == 0:
            st = bm.add_seq(nxt, int(rng.integers(0, 30)))
            if st == OK:
                live.append(nxt)
            nxt += 1
        elif op == 1 and live:
            st = bm.fork(int(rng.choice(live)), nxt)
            assert st == OK
            live.append(nxt)
            nxt += 1
        elif op == 2 and live:
            k = int(rng.integers(1, len(live) + 1))
            batch = list(rng.choice(live, size=k, replace=False))
            snap = copy.deepcopy(bm.__dict__)
            st, slots, pairs = bm.append_batch(batch)
            if st == ERR_OUT_OF_BLOCKS:
                snap["failed_allocs"] += 1
                assert bm.__dict__ == snap
            else:
                assert st == OK and len(slots) == k
                assert len(set(slots)) == k
                # every slot lies in its sequence's table at the written position
                for s, sl in zip(batch, slots):
                    pos = bm.ctx[s] - 1
                    assert sl == bm.tables[s][pos // bm.B] * bm.B + pos % bm.B
                    assert bm.ref[bm.tables[s][pos // bm.B]] == 1
                for src, dst in pairs:
                    assert src != dst
        elif op == 3 and live:
            s = int(rng.choice(live))
            assert bm.free_seq(s) == OK
            live.remove(s)
        _check_invariants(bm)
    for s in list(live):
        bm.free_seq(s)
    assert bm.stats()[0] == 0 and len(bm.free) == 64


def test_exhaustion_leaves_state_unchanged():
    bm = BlockManagerModel(4, 16, [3, 1, 0, 2])
    assert bm.add_seq(0, 48) == OK
    snap = copy.deepcopy(bm.__dict__)
    assert bm.add_seq(1, 40) == ERR_OUT_OF_BLOCKS
    snap["failed_allocs"] += 1
    assert bm.__dict__ == snap
    assert bm.tables[0] == [3, 1, 0]
    assert bm.add_seq(1, 16) == OK and bm.tables[1] == [2]
    st, _, _ = bm.append_batch([0, 1])      # both need a fresh block, none left
    assert st == ERR_OUT_OF_BLOCKS
    assert bm.stats() == (4, 4, 2)


def test_fifo_order_and_release():
    bm = BlockManagerModel(6, 4, [5, 4, 3, 2, 1, 0])
    bm.add_seq(0, 5)          # [5, 4]
    bm.add_seq(1, 4)          # [3]
    bm.free_seq(0)            # 5, 4 go to the back
    bm.add_seq(2, 12)         # [2, 1, 0]
    bm.add_seq(3, 8)          # [5, 4]
    assert bm.tables[2] == [2, 1, 0] and bm.tables[3] == [5, 4]


def test_invalid_calls():
    bm = BlockManagerModel(4, 16)
    assert bm.add_seq(0, 3) == OK
    assert bm.add_seq(0, 3) == ERR_INVALID
    assert bm.fork(9, 1) == ERR_INVALID
    assert bm.fork(0, 0) == ERR_INVALID
    assert bm.append_batch([0, 0])[0] == ERR_INVALID
    assert bm.append_batch([7])[0] == ERR_INVALID
    assert bm.free_seq(3) == ERR_INVALID
    with pytest.raises(ValueError):
        BlockManagerModel(4, 16, [0, 1, 1, 2])


def test_shared_prefix_first_step_copies_199_times():
    n = 200
    prefix = 1500
    nb = 94 + 2 * n
    bm = BlockManagerModel(nb, 16)
    bm.add_seq(0, prefix)
    for c in range(1, n):
        bm.fork(0, c)
    shared_last = bm.tables[0][93]
    assert bm.ref[shared_last] == n
    st, slots, pairs = bm.append_batch(list(range(n)))
    assert st == OK
    assert len(pairs) == n - 1
    assert all(src == shared_last for src, _ in pairs)
    assert bm.tables[n - 1][93] == shared_last       # last holder writes in place
    assert slots[n - 1] == shared_last * 16 + 1500 % 16
    # the 93 full prefix blocks stay shared by all
    assert all(bm.ref[b] == n for b in bm.tables[0][:93])
    # three more steps fill block 93 of every sequence, the next opens block 94
    for _ in range(3):
        st, _, pairs = bm.append_batch(list(range(n)))
        assert st == OK and pairs == []
    used_before = bm.stats()[0]
    st, slots, pairs = bm.append_batch(list(range(n)))
    assert st == OK and pairs == [] and bm.stats()[0] == used_before + n
    assert all(len(bm.tables[s]) == 95 for s in range(n))
    assert all(sl % 16 == 0 for sl in slots)
    _check_invariants(bm)
