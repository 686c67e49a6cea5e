"""Slot mapping, block-table gather and decode attention in fp64
(test infrastructure only; see package docstring).

Definitions followed:

* Attention output is softmax(q K^T / sqrt(d)) V (bjdmk.com.cn article,
  §2.1 从注意力公式推导KV Cache为什么必须存在).  In decode the query is the
  single newest token and it attends over every cached position, its own
  included ("KV Cache 原理与 PagedAttention", §一: generating token t needs
  K_1..K_t and V_1..V_t).  So ``context_len`` counts the token being decoded;
  no mask other than the context length applies.
* The cache is split into fixed-size blocks; a sequence's table maps logical
  block i to a physical block, and attention gathers the scattered physical
  blocks through that table ("KV Cache 原理与 PagedAttention", §三 工作方式
  steps 1, 2 and 4).  Logical position t lives in logical block t // B at
  offset t % B, i.e. in slot table[t // B] * B + t % B.
* Sliding window ("Transformer 架构", aiworkagent.org, question 17, 进阶
  item 3: keep only the most recent N tokens): with a window of w > 0
  positions the query attends to positions [max(0, ctx - w), ctx) only - the
  same softmax over that shorter range.  Blocks wholly before the range are
  not read at all (their table entries may name anything).
* Grouped-query attention: with Hq query heads sharing Hkv < Hq KV heads
  (same page, §一 GQA / MQA 为什么省 KV Cache), query head h reads KV head
  h // G, G = Hq / Hkv (contiguous groups; the pages only count heads, the
  grouping order is this library's reading).

The oracle resolves the table into contiguous fp64 K/V and applies the
textbook formula with an explicit max subtraction.  It never splits contexts
and never uses a streaming softmax.
"""

from __future__ import annotations

import numpy as np

from . import codecs
from .layout import (KV_BF16, KV_FP8_E5M2, KV_INT4, KV_INT8, KV_INT8_CHANNEL, KV_INT8_KCHANNEL_VTENSOR,
                     KV_INT8_TENSOR, PoolImage,
                     channel_scale_offset, int4_k_nibble, int4_v_nibble, k_offset, read_nibbles,
                     scale_offset, v_offset)
from .layout import k_tiles_as_tokens as layout_k_tokens
from .layout import scales_as_tokens as layout_scale_tokens
from .layout import v_tiles_as_tokens as layout_v_tokens


def slot_of(block_table_row: np.ndarray, pos, block_size: int):
    """Physical slot of logical position(s) ``pos`` of one sequence."""
    pos = np.asarray(pos, dtype=np.int64)
    row = np.asarray(block_table_row, dtype=np.int64)
    return row[pos // block_size] * block_size + pos % block_size


def gather_kv(img: PoolImage, layer: int, block_table_row: np.ndarray,
              ctx: int, k_scale: float = 1.0, v_scale: float = 1.0, start: int = 0):
    """Contiguous dequantised K and V of positions [start, ctx), each
    [ctx - start, Hkv, D] float64.

    Reads whole tiles of the blocks the table names from block start // B on
    (layout.*_as_tokens); ``gather_kv_by_slot`` reads the same values one
    element at a time through the slot mapping and the layout's index
    functions, and the two agree exactly (tests/test_oracle_paging.py)."""
    p = img.shape
    if ctx <= start:
        z = np.zeros((0, p.num_kv_heads, p.head_dim))
        return z, z.copy()
    b0 = start // p.block_size
    nblk = -(-ctx // p.block_size)
    blocks = np.asarray(block_table_row, dtype=np.int64)[b0:nblk]
    cut = slice(start - b0 * p.block_size, ctx - b0 * p.block_size)
    kraw = layout_k_tokens(p, img.k, layer, blocks)[cut]
    vraw = layout_v_tokens(p, img.v, layer, blocks)[cut]
    if p.kv_dtype == KV_BF16:
        return codecs.bf16_bits_to_f64(kraw), codecs.bf16_bits_to_f64(vraw)
    if p.kv_dtype == KV_FP8_E5M2:
        ks = np.float64(np.float32(k_scale))
        vs = np.float64(np.float32(v_scale))
        return codecs.e5m2_decode(kraw) * ks, codecs.e5m2_decode(vraw) * vs
    if p.kv_dtype == KV_INT8:
        ksc = layout_scale_tokens(p, img.k_scale, layer, blocks)[cut]
        vsc = layout_scale_tokens(p, img.v_scale, layer, blocks)[cut]
        return codecs.int8_dequant(kraw, ksc), codecs.int8_dequant(vraw, vsc)
    return _dequant_fixed_scales(p, img, layer, kraw, vraw, k_scale, v_scale)


def _dequant_fixed_scales(p, img, layer, kraw, vraw, k_scale, v_scale):
    """INT8 codes [n, Hkv, D] under per-tensor scales (the call's) or per-
    channel scales (the pool's, for this layer): code * scale in float64."""
    if p.kv_dtype == KV_INT8_TENSOR:
        ks = np.float64(np.float32(k_scale))
        vs = np.float64(np.float32(v_scale))
        return kraw.astype(np.float64) * ks, vraw.astype(np.float64) * vs
    if p.kv_dtype == KV_INT4:                # stored nibble = code + 8
        kraw = kraw.astype(np.int64) - 8
        vraw = vraw.astype(np.int64) - 8
    if p.kv_dtype in (KV_INT8_CHANNEL, KV_INT4, KV_INT8_KCHANNEL_VTENSOR):
        co = channel_scale_offset(p, layer, np.arange(p.num_kv_heads)[:, None], np.arange(p.head_dim)[None, :])
        ks = img.k_scale[co].astype(np.float64)[None]      # [1, Hkv, D]
        if p.kv_dtype == KV_INT8_KCHANNEL_VTENSOR:       # V under the call's one scale
            vs = np.float64(np.float32(v_scale))
        else:
            vs = img.v_scale[co].astype(np.float64)[None]
        return kraw.astype(np.float64) * ks, vraw.astype(np.float64) * vs
    raise ValueError(p.kv_dtype)


def gather_kv_by_slot(img: PoolImage, layer: int, block_table_row: np.ndarray,
                      ctx: int, k_scale: float = 1.0, v_scale: float = 1.0, start: int = 0):
    """``gather_kv`` element by element: token t (start <= t < ctx) of the
    sequence is read at slot table[t // B] * B + t % B through the layout's
    index functions."""
    p = img.shape
    if ctx <= start:
        z = np.zeros((0, p.num_kv_heads, p.head_dim))
        return z, z.copy()
    pos = np.arange(start, ctx, dtype=np.int64)
    slots = slot_of(block_table_row, pos, p.block_size)
    blk = (slots // p.block_size)[:, None, None]
    t = (slots % p.block_size)[:, None, None]
    h = np.arange(p.num_kv_heads)[None, :, None]
    d = np.arange(p.head_dim)[None, None, :]
    if p.kv_dtype == KV_INT4:
        kc = read_nibbles(img.k, int4_k_nibble(p, layer, blk, h, t, d)) - 8
        vc = read_nibbles(img.v, int4_v_nibble(p, layer, blk, h, t, d)) - 8
        co = channel_scale_offset(p, layer, h + 0 * t, d + 0 * t)
        return (kc.astype(np.float64) * img.k_scale[co].astype(np.float64),
                vc.astype(np.float64) * img.v_scale[co].astype(np.float64))
    kraw = img.k[k_offset(p, layer, blk, h, t, d)]
    vraw = img.v[v_offset(p, layer, blk, h, t, d)]
    if p.kv_dtype == KV_BF16:
        return codecs.bf16_bits_to_f64(kraw), codecs.bf16_bits_to_f64(vraw)
    if p.kv_dtype == KV_FP8_E5M2:
        ks = np.float64(np.float32(k_scale))
        vs = np.float64(np.float32(v_scale))
        return codecs.e5m2_decode(kraw) * ks, codecs.e5m2_decode(vraw) * vs
    if p.kv_dtype == KV_INT8:
        so = scale_offset(p, layer, blk[:, :, 0], h[:, :, 0], t[:, :, 0])
        return (codecs.int8_dequant(kraw, img.k_scale[so]),
                codecs.int8_dequant(vraw, img.v_scale[so]))
    if p.kv_dtype == KV_INT8_CHANNEL:         # element by element, as for the codes
        co = channel_scale_offset(p, layer, h + 0 * t, d + 0 * t)
        return (kraw.astype(np.float64) * img.k_scale[co].astype(np.float64),
                vraw.astype(np.float64) * img.v_scale[co].astype(np.float64))
    if p.kv_dtype == KV_INT8_KCHANNEL_VTENSOR:
        co = channel_scale_offset(p, layer, h + 0 * t, d + 0 * t)
        return (kraw.astype(np.float64) * img.k_scale[co].astype(np.float64),
                vraw.astype(np.float64) * np.float64(np.float32(v_scale)))
    if p.kv_dtype == KV_INT8_TENSOR:
        return (kraw.astype(np.float64) * np.float64(np.float32(k_scale)),
                vraw.astype(np.float64) * np.float64(np.float32(v_scale)))
    raise ValueError(p.kv_dtype)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Decode attention of one sequence on contiguous fp64 K/V.

    q: [Hq, D] float64; K, V: [ctx, Hkv, D] float64; scale: the fp32 softmax
    scale (used as its exact float64 value).  Returns [Hq, D] float64.
    """
    hq, dim = q.shape
    ctx, hkv, _ = K.shape
    out = np.zeros((hq, dim), dtype=np.float64)
    if ctx == 0:
        return out
    group = hq // hkv
    sc = np.float64(np.float32(scale))
    for h in range(hq):
        g = h // group
        z = sc * (K[:, g, :] @ q[h])                     # [ctx]
        w = np.exp(z - np.max(z))
        p = w / np.sum(w)
        out[h] = p @ V[:, g, :]
    return out


def window_start(ctx: int, window: int) -> int:
    """First position a window of ``window`` positions keeps (0 = no window)."""
    return ctx - window if 0 < window < ctx else 0


def paged_decode(q_bits: np.ndarray, img: PoolImage, layer: int,
                 block_tables: np.ndarray, context_lens: np.ndarray,
                 scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs=None, window: int = 0) -> np.ndarray:
    """Paged decode for every sequence (or the listed ``seqs``), attending to
    the last ``window`` positions only when ``window`` > 0.

    q_bits: [S, Hq, D] bf16 bit patterns.  Returns [S, Hq, D] float64 (rows
    of sequences not in ``seqs`` are left zero).
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    S, hq, dim = q_bits.shape
    out = np.zeros((S, hq, dim), dtype=np.float64)
    idx = range(S) if seqs is None else seqs
    for s in idx:
        ctx = int(context_lens[s])
        K, V = gather_kv(img, layer, block_tables[s], ctx, k_scale, v_scale, window_start(ctx, window))
        out[s] = attend(codecs.bf16_bits_to_f64(q_bits[s]), K, V, scale)
    return out


def shared_prefix_bounds(ctx: int, prefix_len: int):
    """How a sequence of ``ctx`` positions splits against a shared prefix of
    ``prefix_len`` positions: (positions read through the shared table, the
    first position read through the sequence's own table)."""
    return min(ctx, prefix_len), prefix_len


def paged_decode_shared_prefix(q_bits: np.ndarray, img: PoolImage, layer: int,
                               block_tables: np.ndarray, context_lens: np.ndarray,
                               prefix_table: np.ndarray, prefix_len: int, scale: float,
                               k_scale: float = 1.0, v_scale: float = 1.0, seqs=None) -> np.ndarray:
    """Paged decode of sequences that share a cached prompt prefix.

    Requests that start with the same prompt have block tables naming the
    same physical blocks for it (bjdmk.com.cn article, §3.1; §3.2: a
    1500-token system prompt held once for 200 concurrent requests).
    Reading of a decode over such a batch: the shared blocks are named once, by
    ``prefix_table`` (physical blocks of positions [0, prefix_len),
    prefix_len a multiple of the block size); sequence s reads positions
    [0, min(ctx_s, prefix_len)) through it and positions [prefix_len, ctx_s)
    through its own table row, whose entries below prefix_len / B are not
    read.  The attention is ``attend`` over those positions in order - the
    same decode as ``paged_decode`` with the shared blocks written into
    every sequence's table.

    Returns [S, Hq, D] float64 (rows of sequences not in ``seqs`` are zero).
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    S, hq, dim = q_bits.shape
    out = np.zeros((S, hq, dim), dtype=np.float64)
    idx = range(S) if seqs is None else seqs
    for s in idx:
        ctx = int(context_lens[s])
        n_shared, own_from = shared_prefix_bounds(ctx, int(prefix_len))
        Kp, Vp = gather_kv(img, layer, prefix_table, n_shared, k_scale, v_scale)
        Ko, Vo = gather_kv(img, layer, block_tables[s], ctx, k_scale, v_scale, own_from)
        out[s] = attend(codecs.bf16_bits_to_f64(q_bits[s]), np.concatenate([Kp, Ko]),
                        np.concatenate([Vp, Vo]), scale)
    return out


def paged_prefill(q_bits: np.ndarray, img: PoolImage, layer: int, block_tables: np.ndarray,
                  context_lens: np.ndarray, query_start: np.ndarray, scale: float,
                  k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Paged prefill of a chunk of new tokens per sequence, causal.

    Prefix caching keeps the KV of a cached prompt prefix and computes only
    the rest of the prompt (bjdmk.com.cn article, §4.1: the prefill of the
    prefix is skipped; "KV Cache 原理与 PagedAttention", §五).  Reading of that
    step: sequence s brings n_s = query_start[s+1] - query_start[s] new
    tokens, the last n_s of its context_lens[s] positions, whose K/V are
    already in the cache; new token k sits at position ctx_s - n_s + k and
    attends to positions 0 .. ctx_s - n_s + k (itself included, nothing
    after), the decode formula of ``attend`` over that shorter context.

    q_bits: [T, Hq, D] bf16 bits, sequence s's queries in rows
    query_start[s] .. query_start[s+1] - 1.  Returns [T, Hq, D] float64; a
    query whose position would be negative (n_s > ctx_s) gets a zero row.
    """
    q_bits = np.asarray(q_bits, dtype=np.uint16)
    T, hq, dim = q_bits.shape
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((T, hq, dim), dtype=np.float64)
    for s in range(len(context_lens)):
        ctx = int(context_lens[s])
        n = int(qs[s + 1] - qs[s])
        if n == 0:
            continue
        K, V = gather_kv(img, layer, block_tables[s], ctx, k_scale, v_scale)
        q = codecs.bf16_bits_to_f64(q_bits[qs[s]:qs[s + 1]])
        for k in range(n):
            pos = ctx - n + k
            if pos < 0:
                continue
            out[qs[s] + k] = attend(q[k], K[:pos + 1], V[:pos + 1], scale)
    return out
