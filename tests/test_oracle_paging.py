"""Pins of the oracle's layout, gather, cache ops and copy-on-write.

* Layout: the documented index functions are bijections onto their regions,
  and each (layer, block, head) tile is one contiguous range.
* Write-then-gather returns exactly what was written.
* Permutation invariance: moving physical blocks and mapping the table to
  match leaves the decode output bit-identical.
* The aliasing example of aiworkagent.org Q17 (PagedAttention 的关键数据结构):
  tables A = [0, 2, 5, 7] and B = [1, 0, 3] share physical block 0 at
  different logical positions; the result equals that of unshared copies.
* Copy-on-write (bjdmk.com.cn article, §3.2): copying a shared block and
  repointing the writer's table changes no decode output; a write by one
  sharer leaves the others' outputs bit-identical.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import attention, cache_ops, codecs, layout
from oracle.block_manager import BlockManagerModel
from tests.helpers import expanded_slots, fill_pool, random_tables


def test_slot_mapping_matches_expanded_table():
    rng = np.random.default_rng(10)
    for B in (4, 8, 16, 32):
        row = rng.permutation(40)[:9]
        n = 9 * B - int(rng.integers(0, B))
        got = attention.slot_of(row, np.arange(n), B)
        assert np.array_equal(got, expanded_slots(row, n, B))


@pytest.mark.parametrize("dt", [layout.KV_BF16, layout.KV_FP8_E5M2, layout.KV_INT8])
@pytest.mark.parametrize("B,D", [(16, 64), (32, 128), (8, 32), (4, 16)])
def test_layout_is_a_bijection(dt, B, D):
    p = layout.PoolShape(2, 3, B, 2, D, dt)
    L, NB, H, T, DD = np.meshgrid(np.arange(2), np.arange(3), np.arange(2), np.arange(B),
                                  np.arange(D), indexing="ij")
    for fn in (layout.k_offset, layout.v_offset):
        off = fn(p, L, NB, H, T, DD).ravel()
        assert np.array_equal(np.sort(off), np.arange(p.region_elems))
        # one tile = one contiguous range
        tile = fn(p, 1, 2, 1, T[0, 0, 0], DD[0, 0, 0])
        base = layout.tile_base(p, 1, 2, 1)
        assert tile.min() == base and tile.max() == base + p.tile_elems - 1
    s = layout.scale_offset(p, L[..., 0], NB[..., 0], H[..., 0], T[..., 0]).ravel()
    assert np.array_equal(np.sort(s), np.arange(2 * 3 * 2 * B))
    k, v, ks, vs, total = layout.region_offsets(p)
    assert k == 0 and v % 256 == 0 and total % 256 == 0
    assert v >= p.region_elems * p.elem_bytes


def test_k_tile_rows_are_16_byte_pieces():
    # in a bf16 K tile, the 16 tokens' values of dims 8c..8c+7 are 256
    # consecutive bytes (so one wavefront reads a 16-token block in 1 KB runs)
    p = layout.PoolShape(1, 1, 16, 1, 128)
    for c in range(16):
        offs = np.array([[layout.k_offset(p, 0, 0, 0, t, 8 * c + i) for i in range(8)] for t in range(16)])
        assert np.array_equal(np.sort(offs.ravel()), np.arange(128 * c, 128 * c + 128))


def test_write_then_gather_round_trip():
    rng = np.random.default_rng(11)
    ctx = np.array([5, 16, 40, 1], np.int32)
    B, hkv, D = 16, 2, 32
    nb = 12
    p = layout.PoolShape(2, nb, B, hkv, D)
    bt = random_tables(rng, nb, ctx, B)
    k_tok = [workloads.to_bf16_bits(rng.standard_normal((c, hkv, D), dtype=np.float32)) for c in ctx]
    v_tok = [workloads.to_bf16_bits(rng.standard_normal((c, hkv, D), dtype=np.float32)) for c in ctx]
    img = fill_pool(p, bt, ctx, k_tok, v_tok, layer=1)
    for s in range(4):
        K, V = attention.gather_kv(img, 1, bt[s], int(ctx[s]))
        assert np.array_equal(K, codecs.bf16_bits_to_f64(k_tok[s]))
        assert np.array_equal(V, codecs.bf16_bits_to_f64(v_tok[s]))
    # layer 0 untouched
    K0, _ = attention.gather_kv(img, 0, bt[2], int(ctx[2]))
    assert not K0.any()


def test_negative_slots_write_nothing():
    p = layout.PoolShape(1, 2, 16, 1, 16)
    img = layout.empty_image(p)
    k = np.full((3, 1, 16), 0x3F80, np.uint16)
    out = cache_ops.reshape_and_cache(img, 0, k, k, np.array([-1, 5, -7]))
    assert np.count_nonzero(out.k) == 16 and np.count_nonzero(out.v) == 16


@pytest.mark.parametrize("dt", [layout.KV_BF16, layout.KV_FP8_E5M2, layout.KV_INT8])
def test_permutation_invariance(dt):
    rng = np.random.default_rng(12)
    ctx = np.array([33, 70, 16, 2], np.int32)
    B, hkv, D, G = 16, 2, 32, 3
    nb = 20
    p = layout.PoolShape(1, nb, B, hkv, D, dt)
    bt = random_tables(rng, nb, ctx, B)
    k_tok = [workloads.to_bf16_bits(rng.standard_normal((c, hkv, D), dtype=np.float32)) for c in ctx]
    v_tok = [workloads.to_bf16_bits(rng.standard_normal((c, hkv, D), dtype=np.float32)) for c in ctx]
    q = workloads.to_bf16_bits(rng.standard_normal((4, hkv * G, D), dtype=np.float32))
    img = fill_pool(p, bt, ctx, k_tok, v_tok, k_scale=0.5, v_scale=2.0)
    out = attention.paged_decode(q, img, 0, bt, ctx, 0.17, 0.5, 2.0)
    # move block b to pi[b] (tile bytes and scales) and remap the tables
    pi = rng.permutation(nb)
    moved = layout.empty_image(p)
    te = p.tile_elems
    for b in range(nb):
        for h in range(hkv):
            s0, d0 = int(layout.tile_base(p, 0, b, h)), int(layout.tile_base(p, 0, pi[b], h))
            moved.k[d0:d0 + te] = img.k[s0:s0 + te]
            moved.v[d0:d0 + te] = img.v[s0:s0 + te]
            if p.has_scales:
                a, c = int(layout.scale_offset(p, 0, b, h, 0)), int(layout.scale_offset(p, 0, pi[b], h, 0))
                moved.k_scale[c:c + B] = img.k_scale[a:a + B]
                moved.v_scale[c:c + B] = img.v_scale[a:a + B]
    bt2 = pi[bt].astype(np.int32)
    out2 = attention.paged_decode(q, moved, 0, bt2, ctx, 0.17, 0.5, 2.0)
    assert np.array_equal(out, out2)


def test_aliasing_example_from_block_table_notes():
    # Sequence A: [0, 2, 5, 7]; Sequence B: [1, 0, 3].  Block 0 is A's first
    # logical block and B's second.
    rng = np.random.default_rng(13)
    B, hkv, D = 16, 1, 16
    p = layout.PoolShape(1, 9, B, hkv, D)
    img = layout.empty_image(p)
    for blk in range(8):
        kb = workloads.to_bf16_bits(rng.standard_normal((B, hkv, D), dtype=np.float32))
        vb = workloads.to_bf16_bits(rng.standard_normal((B, hkv, D), dtype=np.float32))
        img = cache_ops.reshape_and_cache(img, 0, kb, vb, blk * B + np.arange(B))
    bt = np.array([[0, 2, 5, 7], [1, 0, 3, 0]], np.int32)
    ctx = np.array([60, 40], np.int32)
    q = workloads.to_bf16_bits(rng.standard_normal((2, 2, D), dtype=np.float32))
    shared = attention.paged_decode(q, img, 0, bt, ctx, 0.25)
    # unshared: B gets its own copy of block 0 in block 8
    img2 = cache_ops.copy_blocks(img, np.array([[0, 8]]))
    bt2 = np.array([[0, 2, 5, 7], [1, 8, 3, 0]], np.int32)
    unshared = attention.paged_decode(q, img2, 0, bt2, ctx, 0.25)
    assert np.array_equal(shared, unshared)
    # and the gathered K of B is block 1, then block 0, then block 3's first 8 tokens
    K, _ = attention.gather_kv(img, 0, bt[1], 40)
    KA, _ = attention.gather_kv(img, 0, bt[0], 64)
    assert np.array_equal(K[16:32], KA[0:16])


def test_copy_on_write_keeps_outputs():
    rng = np.random.default_rng(14)
    B, hkv, D, G = 16, 2, 32, 2
    nb = 16
    p = layout.PoolShape(2, nb, B, hkv, D)
    bm = BlockManagerModel(nb, B, rng.permutation(nb))
    assert bm.add_seq(0, 20) == 0                    # 2 blocks, second holds 4 tokens
    for c in (1, 2):
        assert bm.fork(0, c) == 0
    tables = np.array([bm.block_table(s, 4) for s in range(3)], np.int32)
    ctx = np.array([20, 20, 20], np.int32)
    k0 = workloads.to_bf16_bits(rng.standard_normal((20, hkv, D), dtype=np.float32))
    v0 = workloads.to_bf16_bits(rng.standard_normal((20, hkv, D), dtype=np.float32))
    img = layout.empty_image(p)
    for layer in range(2):
        img = fill_pool(p, tables[:1], ctx[:1], [k0], [v0], layer=layer, img=img)
    q = workloads.to_bf16_bits(rng.standard_normal((3, hkv * G, D), dtype=np.float32))
    before = [attention.paged_decode(q, img, l, tables, ctx, 0.2) for l in range(2)]

    st, slots, pairs = bm.append_batch([0, 1, 2])
    assert st == 0 and len(pairs) == 2              # seqs 0 and 1 copy; seq 2 writes in place
    img2 = cache_ops.copy_blocks(img, np.array(pairs))
    tables2 = np.array([bm.block_table(s, 4) for s in range(3)], np.int32)
    assert not np.array_equal(tables2, tables)
    # after the split and before the write: bit-identical outputs in every layer
    for l in range(2):
        assert np.array_equal(attention.paged_decode(q, img2, l, tables2, ctx, 0.2), before[l])

    # sequence 0 writes its new token; sequences 1 and 2 must not see it
    kn = workloads.to_bf16_bits(rng.standard_normal((1, hkv, D), dtype=np.float32))
    img3 = cache_ops.reshape_and_cache(img2, 0, kn, kn, np.array(slots[:1]))
    after = attention.paged_decode(q, img3, 0, tables2, ctx, 0.2)
    assert np.array_equal(after[1:], before[0][1:])
    ctx3 = np.array([21, 20, 20], np.int32)
    after0 = attention.paged_decode(q, img3, 0, tables2, ctx3, 0.2)
    K, _ = attention.gather_kv(img3, 0, tables2[0], 21)
    assert np.array_equal(K[20], codecs.bf16_bits_to_f64(kn[0]))
    assert np.array_equal(after0[1:], before[0][1:])


@pytest.mark.parametrize("dt", [layout.KV_BF16, layout.KV_INT8])
def test_inplace_cache_ops_equal_copying_ones(dt):
    # the in-place forms (used on multi-GB images) give byte-identical images,
    # including a copy whose destination is also another pair's source: every
    # copy reads the state before the call
    rng = np.random.default_rng(77)
    p = layout.PoolShape(2, 6, 16, 2, 64, dt)
    img = layout.empty_image(p)
    img.k[:] = rng.integers(0, 2**8 if dt else 2**16, size=img.k.size).astype(img.k.dtype)
    img.v[:] = rng.integers(0, 2**8 if dt else 2**16, size=img.v.size).astype(img.v.dtype)
    if p.has_scales:
        img.k_scale[:] = rng.random(img.k_scale.size).astype(np.float32)
        img.v_scale[:] = rng.random(img.v_scale.size).astype(np.float32)
    pairs = np.array([[0, 3], [3, 4], [5, 1]], np.int64)
    want = cache_ops.copy_blocks(img, pairs)
    got = cache_ops.copy_blocks(img.copy(), pairs, inplace=True)
    for name in ("k", "v", "k_scale", "v_scale"):
        a, b = getattr(want, name), getattr(got, name)
        assert (a is None and b is None) or np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # block 4 holds block 3's old bytes, not block 0's
    t3 = int(layout.tile_base(p, 1, 3, 1))
    t4 = int(layout.tile_base(p, 1, 4, 1))
    assert np.array_equal(got.k[t4:t4 + p.tile_elems], img.k[t3:t3 + p.tile_elems])
    kb = workloads.to_bf16_bits(rng.standard_normal((5, 2, 64), dtype=np.float32))
    slots = np.array([3, 17, -1, 40, 95], np.int64)
    want = cache_ops.reshape_and_cache(img, 1, kb, kb, slots)
    got = cache_ops.reshape_and_cache(img.copy(), 1, kb, kb, slots, inplace=True)
    for name in ("k", "v", "k_scale", "v_scale"):
        a, b = getattr(want, name), getattr(got, name)
        assert (a is None and b is None) or np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dt", [layout.KV_BF16, layout.KV_FP8_E5M2, layout.KV_INT8])
@pytest.mark.parametrize("B,D", [(16, 64), (32, 128), (8, 32)])
def test_tile_gather_equals_slot_gather(dt, B, D):
    # the whole-tile read used by the oracle's decode equals the definition
    # (slot mapping + element index functions), bit for bit
    rng = np.random.default_rng(91 + dt + B + D)
    p = layout.PoolShape(2, 7, B, 3, D, dt)
    img = layout.empty_image(p)
    if dt == layout.KV_BF16:
        img.k[:] = rng.integers(0, 2**16, size=img.k.size, dtype=np.uint16) & np.uint16(0x3FFF)
        img.v[:] = rng.integers(0, 2**16, size=img.v.size, dtype=np.uint16) & np.uint16(0x3FFF)
    else:
        img.k[:] = rng.integers(0, 256, size=img.k.size).astype(img.k.dtype)
        img.v[:] = rng.integers(0, 256, size=img.v.size).astype(img.v.dtype)
        if dt == layout.KV_FP8_E5M2:   # keep the codes finite (exponent < 31)
            img.k[:] = img.k & np.uint8(0xBB)
            img.v[:] = img.v & np.uint8(0xBB)
    if p.has_scales:
        img.k_scale[:] = rng.random(img.k_scale.size).astype(np.float32)
        img.v_scale[:] = rng.random(img.v_scale.size).astype(np.float32)
    row = rng.permutation(7).astype(np.int32)
    for ctx in (0, 1, B - 1, B, B + 1, 7 * B):
        for layer in (0, 1):
            a = attention.gather_kv(img, layer, row, ctx, 0.5, 1.5)
            b = attention.gather_kv_by_slot(img, layer, row, ctx, 0.5, 1.5)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
