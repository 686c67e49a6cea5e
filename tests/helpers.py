"""Shared test helpers: build oracle pool images from per-token K/V."""

import math

import numpy as np

from oracle import attention, cache_ops, layout


def expanded_slots(table_row, n, block_size):
    """Slots of positions 0..n-1 by expanding the table block by block:
    physical block p contributes slots p*B .. p*B+B-1 in order."""
    runs = [np.arange(int(p) * block_size, (int(p) + 1) * block_size) for p in table_row]
    return np.concatenate(runs)[:n] if runs else np.zeros(0, np.int64)


def fill_pool(shape: layout.PoolShape, tables: np.ndarray, ctx: np.ndarray,
              k_tok, v_tok, layer: int = 0, k_scale=1.0, v_scale=1.0, img=None):
    """Write K/V of every position < ctx[s] of every sequence through the
    oracle's cache write.  k_tok[s] / v_tok[s]: [ctx_s, Hkv, D] bf16 bits."""
    if img is None:
        img = layout.empty_image(shape)
    keys, vals, slots = [], [], []
    for s in range(len(ctx)):
        n = int(ctx[s])
        if n == 0:
            continue
        slots.append(expanded_slots(tables[s], n, shape.block_size))
        keys.append(k_tok[s][:n])
        vals.append(v_tok[s][:n])
    if not slots:
        return img
    return cache_ops.reshape_and_cache(img, layer, np.concatenate(keys), np.concatenate(vals),
                                       np.concatenate(slots), k_scale, v_scale)


def random_tables(rng, num_blocks, ctx, block_size, width=None):
    need = [math.ceil(int(c) / block_size) for c in ctx]
    width = width or max(1, max(need))
    perm = rng.permutation(num_blocks)
    bt = np.zeros((len(ctx), width), dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[pos:pos + n]
        pos += n
    assert pos <= num_blocks
    return bt
