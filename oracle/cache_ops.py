"""Expected pool contents after the two write operations (test infrastructure only).

* ``reshape_and_cache``: when token t is generated its K_t and V_t are computed
  once and appended to the end of the sequence's cache
  ("KV Cache 原理与 PagedAttention", §一, the decode-step box); in a paged cache
  "the end" is the slot that the block table gives for position t (§三 工作方式
  steps 2-3).  Each new token's K/V for every KV head lands in its slot,
  quantised on the way in for 8-bit storage; every other byte of the pool is
  left unchanged.  A negative slot means "no token" and writes nothing.

* ``copy_blocks``: copy-on-write splitting of a shared block copies the whole
  physical block before the writer's table is repointed (bjdmk.com.cn article,
  §3.2 Copy-on-Write).  Every layer's K tile, V tile and (INT8) scale rows of
  ``src`` are copied to ``dst``; all copies read the state before the call.
"""

from __future__ import annotations

import numpy as np

from . import codecs
from .layout import (KV_BF16, KV_FP8_E5M2, KV_INT4, KV_INT8, KV_INT8_CHANNEL, KV_INT8_KCHANNEL_VTENSOR,
                     KV_INT8_TENSOR, PoolImage,
                     channel_scale_offset, int4_k_nibble, int4_v_nibble, k_offset,
                     scale_offset, tile_base, v_offset, write_nibbles)


def reshape_and_cache(img: PoolImage, layer: int, key_bits: np.ndarray,
                      value_bits: np.ndarray, slots: np.ndarray,
                      k_scale: float = 1.0, v_scale: float = 1.0,
                      inplace: bool = False) -> PoolImage:
    """Return a pool image with tokens ``key_bits/value_bits`` [N, Hkv, D]
    (bf16 bit patterns) written at ``slots`` [N] of ``layer``: a new image,
    or ``img`` itself updated when ``inplace`` (for multi-GB images)."""
    p = img.shape
    out = img if inplace else img.copy()
    key_bits = np.asarray(key_bits, dtype=np.uint16)
    value_bits = np.asarray(value_bits, dtype=np.uint16)
    slots = np.asarray(slots, dtype=np.int64)
    n_tok, hkv, d = key_bits.shape
    assert hkv == p.num_kv_heads and d == p.head_dim

    keep = np.nonzero(slots >= 0)[0]
    if keep.size == 0:
        return out
    blk = slots[keep] // p.block_size
    t = slots[keep] % p.block_size
    # broadcast to [n, Hkv, D]
    blk3 = blk[:, None, None]
    t3 = t[:, None, None]
    h3 = np.arange(hkv)[None, :, None]
    d3 = np.arange(d)[None, None, :]
    kx = key_bits[keep]
    vx = value_bits[keep]
    if p.kv_dtype == KV_INT4:
        # the layer's calibrated channel scales, [1, Hkv, D]; stored nibble = code + 8
        co = channel_scale_offset(p, layer, h3, d3)
        kc = codecs.int4_encode(codecs.bf16_bits_to_f32(kx), img.k_scale[co]).astype(np.int64) + 8
        vc = codecs.int4_encode(codecs.bf16_bits_to_f32(vx), img.v_scale[co]).astype(np.int64) + 8
        write_nibbles(out.k, int4_k_nibble(p, layer, blk3, h3, t3, d3), kc)
        write_nibbles(out.v, int4_v_nibble(p, layer, blk3, h3, t3, d3), vc)
        return out
    ko = k_offset(p, layer, blk3, h3, t3, d3)
    vo = v_offset(p, layer, blk3, h3, t3, d3)

    if p.kv_dtype == KV_BF16:
        out.k[ko] = kx
        out.v[vo] = vx
    elif p.kv_dtype == KV_FP8_E5M2:
        out.k[ko] = codecs.e5m2_encode(codecs.bf16_bits_to_f32(kx), k_scale)
        out.v[vo] = codecs.e5m2_encode(codecs.bf16_bits_to_f32(vx), v_scale)
    elif p.kv_dtype == KV_INT8:
        kc, ks = codecs.int8_quantize(codecs.bf16_bits_to_f32(kx))
        vc, vs = codecs.int8_quantize(codecs.bf16_bits_to_f32(vx))
        out.k[ko] = kc
        out.v[vo] = vc
        so = scale_offset(p, layer, blk[:, None], np.arange(hkv)[None, :], t[:, None])
        out.k_scale[so] = ks
        out.v_scale[so] = vs
    elif p.kv_dtype == KV_INT8_TENSOR:
        out.k[ko] = codecs.int8_encode(codecs.bf16_bits_to_f32(kx), k_scale)
        out.v[vo] = codecs.int8_encode(codecs.bf16_bits_to_f32(vx), v_scale)
    elif p.kv_dtype == KV_INT8_CHANNEL:
        co = channel_scale_offset(p, layer, h3, d3)       # [1, Hkv, D]: the layer's calibrated scales
        out.k[ko] = codecs.int8_encode(codecs.bf16_bits_to_f32(kx), img.k_scale[co])
        out.v[vo] = codecs.int8_encode(codecs.bf16_bits_to_f32(vx), img.v_scale[co])
    elif p.kv_dtype == KV_INT8_KCHANNEL_VTENSOR:
        # K and V at different granularities (bjdmk.com.cn article, §5.2: K,
        # the more sensitive, per channel; V coarser, one scale per tensor)
        co = channel_scale_offset(p, layer, h3, d3)
        out.k[ko] = codecs.int8_encode(codecs.bf16_bits_to_f32(kx), img.k_scale[co])
        out.v[vo] = codecs.int8_encode(codecs.bf16_bits_to_f32(vx), v_scale)
    else:
        raise ValueError(p.kv_dtype)
    return out


def copy_blocks(img: PoolImage, pairs: np.ndarray, inplace: bool = False) -> PoolImage:
    """Return an image where, in every layer, block dst holds a byte copy of
    block src for each (src, dst) row of ``pairs``.  All copies read the state
    before the call: with ``inplace`` the sources are snapshotted first, so a
    block that is both a source and a destination still reads its old bytes."""
    p = img.shape
    src_img = img
    if inplace:
        pairs_ = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
        src_img = _snapshot_blocks(img, np.unique(pairs_[:, 0]))
    out = img if inplace else img.copy()
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    te = p.tile_units
    for layer in range(p.num_layers):
        for src, dst in pairs:
            for h in range(p.num_kv_heads):
                s0 = int(tile_base(p, layer, src, h))
                d0 = int(tile_base(p, layer, dst, h))
                out.k[d0:d0 + te] = src_img.k[s0:s0 + te]
                out.v[d0:d0 + te] = src_img.v[s0:s0 + te]
                if p.has_scales:
                    ss = int(scale_offset(p, layer, src, h, 0))
                    ds = int(scale_offset(p, layer, dst, h, 0))
                    out.k_scale[ds:ds + p.block_size] = src_img.k_scale[ss:ss + p.block_size]
                    out.v_scale[ds:ds + p.block_size] = src_img.v_scale[ss:ss + p.block_size]
    return out


def swap_blocks(src_img: PoolImage, dst_img: PoolImage, pairs: np.ndarray) -> PoolImage:
    """Offload / restore (bjdmk.com.cn article, §6.1: blocks move to CPU
    memory and back).  Return a copy of ``dst_img`` where, in every layer,
    block dst holds a byte copy of block src of ``src_img`` for each (src,
    dst) row of ``pairs``; the two images have the same shape apart from
    num_blocks.  A row with src or dst outside its image's blocks is
    skipped."""
    ps, pd = src_img.shape, dst_img.shape
    assert (ps.num_layers, ps.block_size, ps.num_kv_heads, ps.head_dim, ps.kv_dtype) == \
        (pd.num_layers, pd.block_size, pd.num_kv_heads, pd.head_dim, pd.kv_dtype)
    out = dst_img.copy()
    te = ps.tile_units
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < ps.num_blocks and 0 <= dst < pd.num_blocks):
            continue
        for layer in range(ps.num_layers):
            for h in range(ps.num_kv_heads):
                s0 = int(tile_base(ps, layer, src, h))
                d0 = int(tile_base(pd, layer, dst, h))
                out.k[d0:d0 + te] = src_img.k[s0:s0 + te]
                out.v[d0:d0 + te] = src_img.v[s0:s0 + te]
                if ps.has_scales:
                    ss = int(scale_offset(ps, layer, src, h, 0))
                    ds = int(scale_offset(pd, layer, dst, h, 0))
                    out.k_scale[ds:ds + ps.block_size] = src_img.k_scale[ss:ss + ps.block_size]
                    out.v_scale[ds:ds + ps.block_size] = src_img.v_scale[ss:ss + ps.block_size]
    return out


def _snapshot_blocks(img: PoolImage, blocks: np.ndarray) -> PoolImage:
    """An image holding copies of the listed blocks' tiles and scale rows (in
    every layer) at their own positions; other positions are never read."""
    p = img.shape
    snap = PoolImage(p, np.empty_like(img.k), np.empty_like(img.v),
                     None if img.k_scale is None else np.empty_like(img.k_scale),
                     None if img.v_scale is None else np.empty_like(img.v_scale))
    te = p.tile_units
    for layer in range(p.num_layers):
        for b in blocks:
            for h in range(p.num_kv_heads):
                o = int(tile_base(p, layer, int(b), h))
                snap.k[o:o + te] = img.k[o:o + te]
                snap.v[o:o + te] = img.v[o:o + te]
                if p.has_scales:
                    so = int(scale_offset(p, layer, int(b), h, 0))
                    snap.k_scale[so:so + p.block_size] = img.k_scale[so:so + p.block_size]
                    snap.v_scale[so:so + p.block_size] = img.v_scale[so:so + p.block_size]
    return snap
