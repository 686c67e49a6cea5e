"""Seeded synthetic inputs shared by the tests, the oracle checks and bench.py.

This module holds *no* arithmetic of the method (no slot mapping, no
quantisation, no attention): only the random draws and the shapes of the
workloads.  Both the HIP path and the oracle receive what it produces.

Shapes follow the pages' worked examples:

* ``tiny``        - 4 sequences (contexts 1, 15, 16, 33), 4 query / 2 KV heads,
                    head_dim 64, 16-token blocks, a 16-block pool.
* ``llama8b``     - one Llama-3-8B-shaped layer: 64 sequences, contexts uniform
                    in [512, 4096], 32 query / 8 KV heads, head_dim 128.
* ``llama70b``    - the 70B shape used for the pages' size example
                    ("KV Cache 原理与 PagedAttention", §一: 80 layers, 8 KV heads,
                    head_dim 128, BF16; 100 concurrent requests of ~4K tokens),
                    64 query heads, contexts ~N(4096, 256) clipped to
                    [3072, 5120].
* ``cow_prefix``  - 200 sequences sharing a 1500-token prefix, 13B-shaped MHA
                    (40 heads, head_dim 128; bjdmk.com.cn article §2.2 and
                    §3.2), each generating 64..512 further tokens.
* ``long_quant``  - 8 sequences of 32768 tokens, 64 query / 8 KV heads,
                    32-token blocks, FP8-e5m2 or INT8 storage.
* ``prefix_prefill`` - 200 requests = a 1500-token system prompt (bjdmk.com.cn
                    article §3.2) + 64..512 private tokens, 70B-shaped heads;
                    the prompt's 93 full blocks come from the prefix cache
                    and are shared, the rest of every prompt is prefilled.
* ``full_prefill`` - 16 whole 4096-token prompts (no cache hit), 70B-shaped
                    heads, blocks placed by a seeded permutation.

Values are fp32 N(0, 1) draws rounded to bf16 (round-to-nearest-even via
torch), carried as uint16 bit patterns.  Seeds: numpy SeedSequence(436000 +
config id), spawned into independent streams.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KV_BF16, KV_FP8_E5M2, KV_INT8 = 0, 1, 2


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even, torch) and return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclass
class Workload:
    name: str
    config_id: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_layers: int
    kv_dtype: int
    context_lens: np.ndarray             # int32 [S]: lengths *including* the decoded token
    num_blocks: int                      # physical blocks per layer
    block_order: np.ndarray              # int32 [num_blocks]: initial free-list order
    table_width: int                     # W
    partition_size: int = 0              # 0 = single pass
    k_scale: float = 1.0
    v_scale: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))

    def streams(self, n: int = 8):
        ss = np.random.SeedSequence(436000 + self.config_id)
        return [np.random.default_rng(s) for s in ss.spawn(n)]


# ------------------------------------------------------------------ configs
def tiny() -> Workload:
    ctx = np.array([1, 15, 16, 33], dtype=np.int32)
    w = Workload("tiny", 1, 4, 4, 2, 64, 16, 1, KV_BF16, ctx, 16,
                 np.zeros(16, np.int32), 3)
    r = w.streams()
    w.block_order = r[1].permutation(16).astype(np.int32)
    return w


def llama8b(seed_offset: int = 0) -> Workload:
    ss = np.random.SeedSequence(436000 + 2 + seed_offset)
    r0 = np.random.default_rng(ss.spawn(1)[0])
    S = 64
    ctx = r0.integers(512, 4096, size=S, endpoint=True).astype(np.int32)
    need = int(sum(math.ceil(c / 16) for c in ctx))
    nb = math.ceil(1.2 * need)
    w = Workload("llama8b", 2, S, 32, 8, 128, 16, 1, KV_BF16, ctx, nb,
                 np.zeros(nb, np.int32), math.ceil(4096 / 16))
    r = w.streams()
    w.block_order = r[1].permutation(nb).astype(np.int32)
    return w


def llama70b(num_layers: int = 80, extra_steps: int = 64, block_size: int = 16) -> Workload:
    """extra_steps: tokens each sequence may still append (bench growth).
    block_size: tokens per block (16 by default; 8 and 32 are the other sizes
    the pages' engine offers)."""
    ss = np.random.SeedSequence(436000 + 3)
    r0 = np.random.default_rng(ss.spawn(1)[0])
    S = 100
    B = block_size
    ctx = np.clip(np.rint(r0.normal(4096.0, 256.0, size=S)), 3072, 5120).astype(np.int32)
    need = int(sum(math.ceil(c / B) for c in ctx))
    grow = S * math.ceil(extra_steps / B + 1)
    nb = math.ceil(1.02 * need) + grow
    W = math.ceil((5120 + extra_steps) / B)
    w = Workload("llama70b", 3, S, 64, 8, 128, B, num_layers, KV_BF16, ctx, nb,
                 np.zeros(nb, np.int32), W, partition_size=512)
    r = w.streams()
    w.block_order = r[1].permutation(nb).astype(np.int32)
    w.extra["extra_steps"] = extra_steps
    return w


def cow_prefix(num_seqs: int = 200, prefix: int = 1500, lo: int = 64,
               hi: int = 512) -> Workload:
    ss = np.random.SeedSequence(436000 + 4)
    r0 = np.random.default_rng(ss.spawn(1)[0])
    steps = r0.integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int32)
    B = 16
    pre_blocks = math.ceil(prefix / B)
    # shared prefix blocks + every sequence's own blocks for its generated
    # suffix (+1 for the copy of the shared partial block)
    nb = pre_blocks + int(sum(math.ceil((prefix + s) / B) - pre_blocks + 1 for s in steps))
    ctx = np.full(num_seqs, prefix, dtype=np.int32)
    w = Workload("cow_prefix", 4, num_seqs, 40, 40, 128, B, 1, KV_BF16, ctx, nb,
                 np.zeros(nb, np.int32), math.ceil((prefix + hi) / B))
    r = w.streams()
    w.block_order = r[1].permutation(nb).astype(np.int32)
    w.extra["gen_steps"] = steps
    w.extra["prefix"] = prefix
    return w


def long_quant(kv_dtype: int = KV_FP8_E5M2, num_seqs: int = 8,
               ctx_len: int = 32768) -> Workload:
    B = 32
    S = num_seqs
    ctx = np.full(S, ctx_len, dtype=np.int32)
    nb = S * math.ceil(ctx_len / B)
    w = Workload("long_quant", 5, S, 64, 8, 128, B, 1, kv_dtype, ctx, nb,
                 np.zeros(nb, np.int32), math.ceil(ctx_len / B), partition_size=512)
    r = w.streams()
    w.block_order = r[1].permutation(nb).astype(np.int32)
    return w


def prefix_prefill(num_seqs: int = 200, prefix: int = 1500, lo: int = 64, hi: int = 512,
                   num_q_heads: int = 64, num_kv_heads: int = 8, head_dim: int = 128) -> Workload:
    """Prefill after a prefix-cache hit: every prompt is the shared system
    prompt plus its own tokens; the prompt's full blocks are cached and shared
    (one physical copy, the first ``prefix // 16`` table entries of every
    sequence), and each sequence's chunk is everything after them.
    ``context_lens`` = prompt lengths; ``extra['chunk']`` = tokens to prefill;
    ``extra['tables']`` = int32 [S, W] block tables."""
    B = 16
    ss = np.random.SeedSequence(436000 + 6)
    r0 = np.random.default_rng(ss.spawn(1)[0])
    own = r0.integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int32)
    ctx = (prefix + own).astype(np.int32)
    shared = prefix // B
    private = [math.ceil(int(c) / B) - shared for c in ctx]
    nb = shared + int(sum(private))
    W = math.ceil((prefix + hi) / B)
    w = Workload("prefix_prefill", 6, num_seqs, num_q_heads, num_kv_heads, head_dim, B, 1, KV_BF16, ctx, nb,
                 np.zeros(nb, np.int32), W)
    r = w.streams()
    w.block_order = r[1].permutation(nb).astype(np.int32)
    tables = np.zeros((num_seqs, W), dtype=np.int32)
    tables[:, :shared] = w.block_order[:shared]
    pos = shared
    for s, n in enumerate(private):
        tables[s, shared:shared + n] = w.block_order[pos:pos + n]
        pos += n
    w.extra["tables"] = tables
    w.extra["chunk"] = (ctx - shared * B).astype(np.int32)
    w.extra["prefix"] = prefix
    return w


def full_prefill(num_seqs: int = 16, prompt: int = 4096, num_q_heads: int = 64, num_kv_heads: int = 8,
                 head_dim: int = 128) -> Workload:
    """Whole-prompt prefill: every sequence's chunk is its whole prompt.
    ``extra['chunk']`` = tokens to prefill; ``extra['tables']`` = int32
    [S, W] block tables."""
    B = 16
    ctx = np.full(num_seqs, prompt, dtype=np.int32)
    W = math.ceil(prompt / B)
    nb = num_seqs * W
    w = Workload("full_prefill", 7, num_seqs, num_q_heads, num_kv_heads, head_dim, B, 1, KV_BF16, ctx, nb,
                 np.zeros(nb, np.int32), W)
    r = w.streams()
    w.block_order = r[1].permutation(nb).astype(np.int32)
    w.extra["tables"] = static_tables(w)
    w.extra["chunk"] = ctx.copy()
    return w


def static_tables(w: Workload) -> np.ndarray:
    """Tables for the no-sharing configs: each sequence takes its blocks, in
    sequence order, from the front of ``block_order`` (the allocation a FIFO
    free list seeded with that order produces).  int32 [S, W], padded with 0.
    """
    bt = np.zeros((w.num_seqs, w.table_width), dtype=np.int32)
    pos = 0
    for s in range(w.num_seqs):
        n = math.ceil(int(w.context_lens[s]) / w.block_size)
        bt[s, :n] = w.block_order[pos:pos + n]
        pos += n
    return bt


# ------------------------------------------------------------------ tensors
def queries(w: Workload, rng_index: int = 2) -> np.ndarray:
    """bf16 bits [S, Hq, D]."""
    r = w.streams()[rng_index]
    return normal_bf16(r, (w.num_seqs, w.num_q_heads, w.head_dim))


def token_kv(w: Workload, num_tokens: int, stream: int = 3):
    """bf16 bits K and V, each [num_tokens, Hkv, D]."""
    r = w.streams()[stream]
    k = normal_bf16(r, (num_tokens, w.num_kv_heads, w.head_dim))
    v = normal_bf16(r, (num_tokens, w.num_kv_heads, w.head_dim))
    return k, v


def sequence_kv(w: Workload, seq: int, num_tokens: int):
    """bf16 bits K and V, each [num_tokens, Hkv, D], drawn from a stream of
    their own for sequence ``seq`` (for workloads written one sequence at a
    time)."""
    r = np.random.default_rng(np.random.SeedSequence([436000 + w.config_id, 1000 + seq]))
    k = normal_bf16(r, (num_tokens, w.num_kv_heads, w.head_dim))
    v = normal_bf16(r, (num_tokens, w.num_kv_heads, w.head_dim))
    return k, v


def plant_needles(w: Workload, q_bits: np.ndarray, k_tok: np.ndarray,
                  token_seq: np.ndarray, token_pos: np.ndarray,
                  per_seq: int = 8, stream: int = 5) -> np.ndarray:
    """Peaked inputs: in each sequence, overwrite the K of ``per_seq`` random
    positions (for every KV head) with 4 * sqrt(D) * q/|q| of the first query
    head of that KV head's group, so that a few tokens carry most of the
    softmax mass and reading a wrong block moves the output by O(1).

    k_tok: [N, Hkv, D] bf16 bits of all tokens, token_seq/token_pos: [N] the
    sequence and logical position of each token.  Returns a modified copy.
    """
    import torch
    r = w.streams()[stream]
    k = k_tok.copy()
    qf = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    for s in range(w.num_seqs):
        idx = np.nonzero(token_seq == s)[0]
        if idx.size == 0:
            continue
        pick = r.choice(idx, size=min(per_seq, idx.size), replace=False)
        for g in range(w.num_kv_heads):
            qh = qf[s, g * w.group]
            nv = qh / max(np.linalg.norm(qh), 1e-6) * 4.0 * math.sqrt(w.head_dim)
            k[pick, g, :] = to_bf16_bits(np.tile(nv.astype(np.float32), (pick.size, 1)))
    return k
