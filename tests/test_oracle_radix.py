"""Pins of the radix-tree prefix cache in the block-manager model
(oracle/block_manager.py), against what the bjdmk.com.cn article, §4.2,
fixes: the longest shared prefix is reused, also one that ends inside a
block; unmatched tokens are computed; least recently used leaves are evicted
first, so a shared prefix outlives its branches.

The central pin simulates the pool's memory: every slot holds the id of the
token whose K/V it stores.  A request writes its tokens from its cached count
on (after copying the pair it was given), an append writes one token (after
its copy-on-write pairs); every live sequence must then read back exactly its
own tokens.  A reused block holding other tokens, a partial match without its
copy, or an eviction of a block still in use shows up as a wrong token."""

import json
import os
import random

import pytest

from oracle.block_manager import (ERR_OUT_OF_BLOCKS, ERR_UNSUPPORTED, OK, BlockManagerModel)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "radix_partial_match.json"),
                      encoding="utf-8"))


class Memory:
    """Token ids per (block, slot), driven by the model's outputs."""

    def __init__(self, bm: BlockManagerModel):
        self.bm = bm
        self.mem = [[None] * bm.B for _ in range(bm.num_blocks)]
        self.history = {}

    def slot(self, seq, pos):
        b = self.bm.tables[seq][pos // self.bm.B]
        return b, pos % self.bm.B

    def add(self, seq, tokens):
        st, cached, pair = self.bm.add_seq_radix(seq, tokens)
        if st != OK:
            return st, cached, pair
        if pair is not None:
            src, dst = pair
            self.mem[dst] = list(self.mem[src])
        for p, t in enumerate(tokens):
            b, o = self.slot(seq, p)
            if p < cached:
                assert self.mem[b][o] == t, (seq, p)      # reused K/V must be this token's
            else:
                self.mem[b][o] = t                        # computed by the prefill
        self.history[seq] = list(tokens)
        return st, cached, pair

    def append(self, seqs, tokens):
        st, slots, pairs = self.bm.append_batch(seqs)
        if st != OK:
            return st
        for src, dst in pairs:
            self.mem[dst] = list(self.mem[src])
        for s, sl, t in zip(seqs, slots, tokens):
            self.mem[sl // self.bm.B][sl % self.bm.B] = t
            self.history[s].append(t)
        return st

    def fork(self, parent, child):
        assert self.bm.fork(parent, child) == OK
        self.history[child] = list(self.history[parent])

    def free(self, seq):
        assert self.bm.free_seq(seq) == OK
        del self.history[seq]

    def check(self):
        for s, toks in self.history.items():
            for p, t in enumerate(toks):
                b, o = self.slot(s, p)
                assert self.mem[b][o] == t, (s, p)
        check_invariants(self.bm)


def check_invariants(bm: BlockManagerModel):
    refs = [0] * bm.num_blocks
    for tab in bm.tables.values():
        for b in tab:
            refs[b] += 1
    assert refs == bm.ref
    idle = [b for b in bm.node_parent if bm.ref[b] == 0]
    assert not set(bm.free) & set(bm.node_parent)
    assert len(bm.free) + len(idle) + sum(1 for r in bm.ref if r > 0) == bm.num_blocks
    for b, par in bm.node_parent.items():
        assert par == bm.ROOT or par in bm.node_parent
        assert b in bm.children[par]
        if bm.ref[b] > 0:                        # a referenced node's ancestors are referenced
            a = par
            while a != bm.ROOT:
                assert bm.ref[a] > 0
                a = bm.node_parent[a]


def lcp(a, b):
    k = 0
    while k < len(a) and k < len(b) and a[k] == b[k]:
        k += 1
    return k


@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_pages_example_shares_six_tokens(B):
    a = [ord(c) for c in GOLD["prompt_a"]]
    b = [ord(c) for c in GOLD["prompt_b"]]
    bm = BlockManagerModel(16, B)
    m = Memory(bm)
    assert m.add(0, a)[:2] == (OK, 0)
    st, cached, pair = m.add(1, b)
    assert st == OK and cached == GOLD["shared_tokens"]
    # whole blocks of the shared part are the same physical blocks
    assert bm.tables[1][:cached // B] == bm.tables[0][:cached // B]
    if cached % B:
        assert pair == (bm.tables[0][cached // B], bm.tables[1][cached // B])
    else:
        assert pair is None
    m.check()
    # the hash chain reuses only whole blocks of the shared part
    h = BlockManagerModel(16, B)
    h.add_seq_tokens(0, a)
    assert h.add_seq_tokens(1, b) == (OK, GOLD["shared_tokens"] // B * B)


@pytest.mark.parametrize("B", [1, 2, 4, 5])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_longest_prefix_by_brute_force(B, seed):
    """No eviction (a pool larger than every prompt together): a request
    reuses the longest prefix it shares with the full blocks of any earlier
    prompt, capped before its own last token."""
    rng = random.Random(seed)
    bm = BlockManagerModel(4000, B)
    m = Memory(bm)
    stems = [[rng.randrange(4) for _ in range(rng.randrange(0, 30))] for _ in range(5)]
    earlier = []
    live = []
    for seq in range(120):
        base = rng.choice(stems + [p for p in earlier[-10:]] + [[]])
        toks = base[:rng.randrange(0, len(base) + 1)] + [rng.randrange(4) for _ in range(rng.randrange(0, 12))]
        want = 0
        if toks:
            for p in earlier:
                want = max(want, lcp(toks, p[:len(p) // B * B]))
            want = min(want, len(toks) - 1)
        st, cached, pair = m.add(seq, toks)
        assert st == OK and cached == want, (seq, toks)
        assert (pair is not None) == (cached % B != 0)
        earlier.append(toks)
        live.append(seq)
        if rng.random() < 0.3:
            m.free(live.pop(rng.randrange(len(live))))
        m.check()


def test_lru_leaves_go_first_and_shared_prefix_survives():
    B = 2
    bm = BlockManagerModel(6, B)
    m = Memory(bm)
    p1 = [1, 2, 3, 4, 5, 6, 7]                 # blocks [1 2] [3 4] [5 6] cached, [7] not
    p2 = [1, 2, 3, 4, 8, 9, 10]                # shares [1 2] [3 4]
    assert m.add(1, p1)[:2] == (OK, 0)
    m.free(1)                                   # tick 2: p1's blocks idle
    assert m.add(2, p2)[:2] == (OK, 4)          # tick 3: [1 2] [3 4] used again
    t2 = list(bm.tables[2])
    a12, a34 = t2[0], t2[1]
    m.free(2)                                   # tick 4: p2's blocks idle
    # tree: [1 2] -> [3 4] -> {[5 6] last used at tick 2, [8 9] at tick 4}
    assert bm.radix_stats()[2:] == (4, 4)
    a56 = next(c for c in bm.children[a34] if bm.node_tokens[c] == (5, 6))
    a89 = next(c for c in bm.children[a34] if bm.node_tokens[c] == (8, 9))
    # 3 fresh blocks: the 2 uncached free ones, then the leaf used longest
    # ago, [5 6] - not [8 9], and never [1 2] or [3 4], which have children
    st, cached, _ = m.add(3, [20, 21, 22, 23, 24])
    assert (st, cached) == (OK, 0)
    assert a56 in bm.tables[3] and a56 not in bm.node_parent
    assert a89 in bm.node_parent and a12 in bm.node_parent and a34 in bm.node_parent
    m.free(3)
    # the surviving branch, with its shared prefix, is found whole
    assert m.add(4, [1, 2, 3, 4, 8, 9, 11])[:2] == (OK, 6)
    m.check()


def test_all_or_nothing_and_pinned_blocks_are_not_counted():
    B = 2
    bm = BlockManagerModel(4, B)
    m = Memory(bm)
    assert m.add(0, [1, 2, 3, 4, 5])[:2] == (OK, 0)      # 3 blocks
    m.free(0)                                            # [1 2] [3 4] idle, [5] free
    before = (dict(bm.node_parent), list(bm.free), list(bm.ref), bm.stats())
    # reuses [1 2] [3 4]; needs 3 fresh blocks, only 2 obtainable once the
    # matched blocks are held
    st, _, _ = bm.add_seq_radix(1, [1, 2, 3, 4, 6, 7, 8, 9, 10])
    assert st == ERR_OUT_OF_BLOCKS
    assert (dict(bm.node_parent), list(bm.free), list(bm.ref)) == before[:3]
    assert bm.stats()[2] == before[3][2] + 1
    assert m.add(1, [1, 2, 3, 4, 6, 7])[:2] == (OK, 4)
    m.check()


def test_one_prefix_cache_per_manager():
    bm = BlockManagerModel(8, 2)
    assert bm.add_seq_radix(0, [1, 2, 3])[0] == OK
    assert bm.add_seq_tokens(1, [1, 2, 3]) == (ERR_UNSUPPORTED, 0)
    h = BlockManagerModel(8, 2)
    assert h.add_seq_tokens(0, [1, 2, 3])[0] == OK
    assert h.add_seq_radix(1, [1, 2, 3])[0] == ERR_UNSUPPORTED


@pytest.mark.parametrize("B", [1, 2, 4])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_walk_under_eviction(B, seed):
    """Requests, appends, forks and frees on a small pool: eviction runs often,
    and every live sequence keeps reading its own tokens."""
    rng = random.Random(100 + seed)
    nb = 24
    bm = BlockManagerModel(nb, B, rng.sample(range(nb), nb))
    m = Memory(bm)
    stems = [[rng.randrange(3) for _ in range(rng.randrange(1, 14))] for _ in range(4)]
    nxt = 0
    for _ in range(400):
        live = sorted(m.history)
        r = rng.random()
        if r < 0.4:
            base = rng.choice(stems)
            toks = base[:rng.randrange(len(base) + 1)] + [rng.randrange(3) for _ in range(rng.randrange(0, 6))]
            st, _, _ = m.add(nxt, toks)
            assert st in (OK, ERR_OUT_OF_BLOCKS)
            nxt += 1
        elif r < 0.6 and live:
            seqs = rng.sample(live, rng.randrange(1, len(live) + 1))
            assert m.append(seqs, [rng.randrange(3) for _ in seqs]) in (OK, ERR_OUT_OF_BLOCKS)
        elif r < 0.7 and live:
            m.fork(rng.choice(live), nxt)
            nxt += 1
        elif live:
            m.free(rng.choice(live))
        m.check()
