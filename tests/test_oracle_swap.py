"""Pins of the oracle's swap_blocks (offload to host memory and back; CPU).

The definition is a byte move of whole blocks (every layer, K, V and int8
scales) between two pools of the same shape.  Pinned by what a swap must
preserve: decoding a sequence from the other pool through its remapped table
gives the same bits as before (first and last layer, through a swap out and
back in), every moved token reads the same values element by element through
the slot mapping, bytes outside the destination blocks are untouched, and
pairs outside either pool do nothing.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import attention, cache_ops, layout
from tests.helpers import fill_pool, random_tables


def _pool(rng, dt, L=3, B=8, hkv=2, D=32, ctx=(5, 17, 30)):
    ctx = np.asarray(ctx, np.int32)
    nb = sum(math.ceil(int(c) / B) for c in ctx) + 3
    shape = layout.PoolShape(L, nb, B, hkv, D, dt)
    bt = random_tables(rng, nb, ctx, B)
    img = layout.empty_image(shape)
    for layer in range(L):
        k_tok = [workloads.to_bf16_bits(rng.standard_normal((int(c), hkv, D), dtype=np.float32)) for c in ctx]
        v_tok = [workloads.to_bf16_bits(rng.standard_normal((int(c), hkv, D), dtype=np.float32)) for c in ctx]
        img = fill_pool(shape, bt, ctx, k_tok, v_tok, layer=layer, k_scale=0.5, v_scale=2.0, img=img)
    q = workloads.to_bf16_bits(rng.standard_normal((len(ctx), hkv * 2, D), dtype=np.float32))
    return shape, bt, ctx, img, q


@pytest.mark.parametrize("dt", [layout.KV_BF16, layout.KV_FP8_E5M2, layout.KV_INT8])
def test_swap_out_and_back_keeps_every_decode(dt):
    rng = np.random.default_rng(8800 + dt)
    shape, bt, ctx, img, q = _pool(rng, dt)
    B = shape.block_size
    host_shape = layout.PoolShape(shape.num_layers, 11, B, shape.num_kv_heads, shape.head_dim, dt)
    host = layout.empty_image(host_shape)
    s = 2
    n = math.ceil(int(ctx[s]) / B)
    host_ids = rng.permutation(11)[:n]
    out_pairs = np.stack([bt[s, :n], host_ids], axis=1)
    host = cache_ops.swap_blocks(img, host, out_pairs)
    host_bt = bt.copy()
    host_bt[s, :n] = host_ids
    # back into the device pool at other blocks (the originals were reused)
    back = layout.empty_image(shape)
    new_ids = rng.permutation(shape.num_blocks)[:n]
    back = cache_ops.swap_blocks(host, back, np.stack([host_ids, new_ids], axis=1))
    back_bt = bt.copy()
    back_bt[s, :n] = new_ids
    for layer in (0, shape.num_layers - 1):
        want = attention.paged_decode(q, img, layer, bt, ctx, 0.3, 0.5, 2.0, seqs=[s])
        got_h = attention.paged_decode(q, host, layer, host_bt, ctx, 0.3, 0.5, 2.0, seqs=[s])
        got_b = attention.paged_decode(q, back, layer, back_bt, ctx, 0.3, 0.5, 2.0, seqs=[s])
        assert np.array_equal(got_h, want) and np.array_equal(got_b, want)
        # element by element through the slot mapping
        a = attention.gather_kv_by_slot(img, layer, bt[s], int(ctx[s]), 0.5, 2.0)
        b = attention.gather_kv_by_slot(host, layer, host_bt[s], int(ctx[s]), 0.5, 2.0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bytes_outside_destination_blocks_are_untouched():
    rng = np.random.default_rng(8900)
    shape, bt, ctx, img, q = _pool(rng, layout.KV_INT8)
    dst = layout.empty_image(shape)
    dst.k[:] = 0x5a
    dst.v[:] = 0x3c
    dst.k_scale[:] = 7.0
    dst.v_scale[:] = 9.0
    pairs = np.array([[bt[0, 0], 4], [bt[1, 1], 0]])
    out = cache_ops.swap_blocks(img, dst, pairs)
    te = shape.tile_elems
    touched_k = np.zeros(out.k.size, bool)
    touched_s = np.zeros(out.k_scale.size, bool)
    for layer in range(shape.num_layers):
        for _, d in pairs:
            for h in range(shape.num_kv_heads):
                b0 = int(layout.tile_base(shape, layer, d, h))
                touched_k[b0:b0 + te] = True
                s0 = int(layout.scale_offset(shape, layer, d, h, 0))
                touched_s[s0:s0 + shape.block_size] = True
    assert np.all(out.k[~touched_k] == 0x5a) and np.all(out.v[~touched_k] == 0x3c)
    assert np.all(out.k_scale[~touched_s] == 7.0) and np.all(out.v_scale[~touched_s] == 9.0)
    assert not np.array_equal(out.k[touched_k], dst.k[touched_k])


def test_pairs_outside_either_pool_do_nothing():
    rng = np.random.default_rng(9000)
    shape, bt, ctx, img, q = _pool(rng, layout.KV_BF16)
    dst = layout.empty_image(layout.PoolShape(shape.num_layers, 4, shape.block_size, shape.num_kv_heads,
                                              shape.head_dim))
    out = cache_ops.swap_blocks(img, dst, np.array([[-1, 0], [0, 4], [shape.num_blocks, 1], [0, -2]]))
    assert np.array_equal(out.k, dst.k) and np.array_equal(out.v, dst.v)
