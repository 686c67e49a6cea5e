"""Python model of the host block manager (test infrastructure only).

What it models:

* A pool of ``num_blocks`` preallocated physical blocks of ``block_size``
  token slots, handed to sequences on demand and returned when a sequence
  ends ("KV Cache 原理与 PagedAttention", §三 工作方式 steps 1-3; aiworkagent.org
  Q17, PagedAttention 的关键数据结构: KV Memory Pool).
* A per-sequence block table: entry i is the physical block of logical block i
  (same sources).  A sequence of n tokens holds exactly ceil(n / B) blocks, so
  at most one block, its last, is partly empty (§三 收益 table).
* Sharing: a forked sequence points at its parent's physical blocks; before a
  sequence writes into a block that someone else also references, the block is
  copied, the writer's table is repointed at the copy, then the write happens
  (bjdmk.com.cn article, §3.1 and §3.2 Copy-on-Write).

Rules that the pages leave open, fixed here (and in the C++ manager) so that
tables, slots and copy pairs are unique and comparable bit for bit:

* Free blocks form a FIFO queue.  Its initial order is supplied by the caller
  (an explicit permutation of all block ids); allocation pops the front, a
  block whose reference count drops to zero is pushed to the back.
* Appending to a sequence of current length n writes position n.  If n % B == 0
  a fresh block is appended to the table.  Otherwise, if the last block's
  reference count exceeds one, a fresh block ``dst`` is taken, the pair
  (src=last, dst) is reported for copying, the count of ``src`` drops by one,
  ``dst`` starts at one and replaces ``src`` in the writer's table; the last
  remaining holder writes in place.  The slot is table[n // B] * B + n % B.
* A batch append processes sequences in the order given and is all or
  nothing: if the pool cannot serve every block the batch needs, it fails,
  the failed-allocation counter rises by one and nothing else changes.
* Freeing a sequence releases its blocks in table order.
* Table rows are padded with 0 past the sequence's blocks.

Prefix caching (bjdmk.com.cn article, §4.1: a prompt that starts like an
earlier one reuses that prompt's KV blocks; §4.3: only an exact prefix at the
same positions qualifies):

* The key of full prompt block i is SHA-256(key(i-1) + its B token ids as
  little-endian int32), key(-1) = 32 zero bytes - a chain, so a key names the
  whole prefix up to the block.
* A new prompt reuses the longest run of leading full blocks whose keys are
  cached (their counts rise, also from zero); all other blocks are fresh, and
  each fresh full block becomes the holder of its key.  The partial last
  block and blocks filled by later appends are not cached.
* A cached block freed to count zero keeps its key on the free queue and
  leaves the cache when the queue hands it out again (least recently freed
  first).  A reused free block is taken out of the queue.

Radix-tree prefix cache, the alternative to the hash chain (bjdmk.com.cn
article, §4.2: cached KV organised as a tree over token sequences, a new
request takes the longest matching prefix - also one that ends inside a block
- and the least recently used leaves are evicted first, so shared prefixes
outlive the branches that use them).  A manager uses one of the two; a call
of the other kind is refused (ERR_UNSUPPORTED).  With paged storage a tree
node is one full prompt block: the B token ids it holds, under the node of
the block before it (the root for block 0).  The rules fixed here:

* Matching walks from the root through children whose B tokens equal the
  prompt's next block, while the whole block lies before the last prompt
  token (that token is always computed, as above).  In the first block not
  matched whole, the child sharing the longest run of leading tokens with the
  prompt (capped at the last prompt token; the earliest inserted child among
  equals) gives a partial match of l tokens: the new sequence takes a fresh
  block and reports the pair (that child, fresh block) for the caller to
  copy before it computes the rest, so the copy carries the l matched
  tokens' K/V.  Cached tokens = B * (blocks matched whole) + l.
* Capacity: the free queue plus every cached block nobody references (all
  of them can be evicted, leaves first); the blocks matched (and the partial
  source, held during the call) are not counted.  All or nothing, as above.
* Fresh blocks come from the free queue (uncached blocks only) while it has
  any, else by evicting the cached, unreferenced leaf used longest ago (then
  the deeper, then the lower block id).  Using a block = being matched, or
  dropping to count zero in free_seq; each free_seq and each radix call is
  one tick of the clock.
* The prompt's full fresh blocks are inserted in order as a chain under the
  last matched block; a block whose tokens a sibling already holds (only the
  last full block, when the last token cut its match short) and the blocks
  after it are not inserted.
"""

from __future__ import annotations

import hashlib
from collections import deque

import numpy as np

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_OUT_OF_BLOCKS = 0, -1, -2, -3


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, initial_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("bad sizes")
        order = list(range(num_blocks)) if initial_order is None else [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial order must be a permutation of all block ids")
        self.num_blocks = num_blocks
        self.B = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.ctx: dict[int, int] = {}
        self.failed_allocs = 0
        self.cache: dict[bytes, int] = {}        # prefix key -> block
        self.block_key: dict[int, bytes] = {}    # block -> its key
        self.lookups = 0
        self.hits = 0
        # radix tree: 0 no prefix cache used yet, 1 hash chain, 2 radix tree
        self.mode = 0
        self.node_parent: dict[int, int] = {}    # cached block -> block before it (ROOT for block 0)
        self.node_tokens: dict[int, tuple] = {}
        self.node_depth: dict[int, int] = {}
        self.children: dict[int, list] = {self.ROOT: []}
        self.last_use: dict[int, int] = {}
        self.clock = 0
        self.radix_lookups = 0
        self.radix_hits = 0

    ROOT = -1

    # ------------------------------------------------------------ helpers
    def _available(self) -> int:
        """Blocks a request may obtain: the free queue, and in radix mode the
        cached blocks nobody references."""
        extra = sum(1 for b in self.node_parent if self.ref[b] == 0) if self.mode == 2 else 0
        return len(self.free) + extra

    def _evict(self) -> int:
        leaves = [b for b in self.node_parent if self.ref[b] == 0 and not self.children[b]]
        b = min(leaves, key=lambda x: (self.last_use[x], -self.node_depth[x], x))
        self.children[self.node_parent[b]].remove(b)
        for d in (self.node_parent, self.node_tokens, self.node_depth, self.children, self.last_use):
            del d[b]
        return b

    def _take(self) -> int:
        if self.mode == 2 and not self.free:
            b = self._evict()
            self.ref[b] = 1
            return b
        b = self.free.popleft()
        self.ref[b] = 1
        if b in self.block_key:                  # evicted: its content is about to change
            del self.cache[self.block_key.pop(b)]
        return b

    # ------------------------------------------------------------ API
    def add_seq(self, seq: int, ctx_len: int) -> int:
        if seq in self.tables or ctx_len < 0:
            return ERR_INVALID
        need = -(-ctx_len // self.B)
        if need > self._available():
            self.failed_allocs += 1
            return ERR_OUT_OF_BLOCKS
        self.tables[seq] = [self._take() for _ in range(need)]
        self.ctx[seq] = ctx_len
        return OK

    @staticmethod
    def key(parent: bytes | None, tokens) -> bytes:
        data = (parent if parent is not None else bytes(32)) + np.asarray(tokens, dtype="<i4").tobytes()
        return hashlib.sha256(data).digest()

    def add_seq_tokens(self, seq: int, tokens):
        """Returns (status, cached tokens)."""
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            return ERR_INVALID, 0
        if self.mode == 2:
            return ERR_UNSUPPORTED, 0
        B = self.B
        n = len(tokens)
        full, total = n // B, -(-n // B)
        # only blocks wholly before the last prompt token can be reused: that
        # token is always computed, since its forward pass gives the first
        # generated token (bjdmk.com.cn article, section 4.1: reuse the
        # cached prefix, compute the rest)
        eligible = (n - 1) // B if n > 0 else 0
        keys = []
        for i in range(full):
            keys.append(self.key(keys[-1] if keys else None, tokens[i * B:(i + 1) * B]))
        matched = 0
        while matched < eligible and keys[matched] in self.cache:
            matched += 1
        matched_free = sum(1 for i in range(matched) if self.ref[self.cache[keys[i]]] == 0)
        if total - matched > len(self.free) - matched_free:
            self.failed_allocs += 1
            return ERR_OUT_OF_BLOCKS, 0
        self.mode = 1
        self.lookups += eligible
        self.hits += matched
        table = []
        for i in range(matched):
            b = self.cache[keys[i]]
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            table.append(b)
        for i in range(matched, total):
            b = self._take()
            table.append(b)
            if i < full:
                old = self.cache.get(keys[i])
                if old is not None:
                    del self.block_key[old]
                self.cache[keys[i]] = b
                self.block_key[b] = keys[i]
        self.tables[seq] = table
        self.ctx[seq] = n
        return OK, matched * B

    def prefix_stats(self):
        return self.lookups, self.hits, len(self.cache)

    def add_seq_radix(self, seq: int, tokens):
        """Returns (status, cached tokens, copy pair (src, dst) or None)."""
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            return ERR_INVALID, 0, None
        if self.mode == 1:
            return ERR_UNSUPPORTED, 0, None
        B = self.B
        n = len(tokens)
        full, total = n // B, -(-n // B)
        last = n - 1 if n > 0 else 0            # tokens that may be reused
        node, path = self.ROOT, []
        while (len(path) + 1) * B <= last:
            blk = tuple(tokens[len(path) * B:(len(path) + 1) * B])
            nxt = next((c for c in self.children[node] if self.node_tokens[c] == blk), None)
            if nxt is None:
                break
            path.append(nxt)
            node = nxt
        i = len(path)
        lim = min(B, last - i * B)
        src, l = -1, 0
        for c in self.children[node] if lim > 0 else []:
            t = self.node_tokens[c]
            k = 0
            while k < lim and t[k] == tokens[i * B + k]:
                k += 1
            if k > l:
                src, l = c, k
        pinned = sum(1 for b in path if self.ref[b] == 0) + (1 if src >= 0 and self.ref[src] == 0 else 0)
        if total - i > self._available() - pinned:
            self.failed_allocs += 1
            return ERR_OUT_OF_BLOCKS, 0, None
        self.mode = 2
        self.clock += 1
        for b in path + ([src] if src >= 0 else []):
            self.ref[b] += 1
            self.last_use[b] = self.clock
        table = list(path)
        parent, insert = node, True
        for k in range(i, total):
            b = self._take()
            table.append(b)
            if insert and k < full:
                blk = tuple(tokens[k * B:(k + 1) * B])
                if any(self.node_tokens[c] == blk for c in self.children[parent]):
                    insert = False
                    continue
                self.node_parent[b] = parent
                self.node_tokens[b] = blk
                self.node_depth[b] = k
                self.children[parent].append(b)
                self.children[b] = []
                self.last_use[b] = self.clock
                parent = b
        if src >= 0:
            self.ref[src] -= 1                    # held only while the call took blocks
        self.tables[seq] = table
        self.ctx[seq] = n
        self.radix_lookups += last
        self.radix_hits += i * B + l
        return OK, i * B + l, ((src, table[i]) if src >= 0 else None)

    def radix_stats(self):
        """(lookup tokens, hit tokens, cached blocks, cached blocks nobody references)."""
        idle = sum(1 for b in self.node_parent if self.ref[b] == 0)
        return self.radix_lookups, self.radix_hits, len(self.node_parent), idle

    def fork(self, parent: int, child: int) -> int:
        if parent not in self.tables or child in self.tables:
            return ERR_INVALID
        self.tables[child] = list(self.tables[parent])
        self.ctx[child] = self.ctx[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return OK

    def append_batch(self, seqs):
        """Returns (status, slots list, cow pairs list)."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs) or any(s not in self.tables for s in seqs):
            return ERR_INVALID, [], []
        # dry run: count the fresh blocks the batch needs
        need = 0
        ref_delta: dict[int, int] = {}
        for s in seqs:
            pos = self.ctx[s]
            if pos % self.B == 0:
                need += 1
            else:
                last = self.tables[s][pos // self.B]
                if self.ref[last] + ref_delta.get(last, 0) > 1:
                    need += 1
                    ref_delta[last] = ref_delta.get(last, 0) - 1
        if need > self._available():
            self.failed_allocs += 1
            return ERR_OUT_OF_BLOCKS, [], []
        slots, pairs = [], []
        for s in seqs:
            pos = self.ctx[s]
            tab = self.tables[s]
            if pos % self.B == 0:
                tab.append(self._take())
            else:
                last = tab[pos // self.B]
                if self.ref[last] > 1:
                    dst = self._take()
                    self.ref[last] -= 1
                    tab[pos // self.B] = dst
                    pairs.append((last, dst))
            slots.append(tab[pos // self.B] * self.B + pos % self.B)
            self.ctx[s] = pos + 1
        return OK, slots, pairs

    def free_seq(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_INVALID
        self.clock += 1
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if b in self.node_parent:           # stays cached: evictable from now on
                    self.last_use[b] = self.clock
                else:
                    self.free.append(b)
        del self.ctx[seq]
        return OK

    def block_table(self, seq: int, width: int):
        tab = self.tables[seq]
        if len(tab) > width:
            raise ValueError("table wider than width")
        return tab + [0] * (width - len(tab))

    def stats(self):
        return self.num_blocks - self._available(), self.num_blocks, self.failed_allocs
