"""Pins of the oracle's sliding-window decode (CPU only).

The window keeps the last w positions, [max(0, ctx - w), ctx) ("Transformer
架构", aiworkagent.org, question 17, 进阶 item 3: keep only the most recent N
tokens).  Pinned by: torch's scaled_dot_product_attention in float64 with an
explicit boolean mask (a library routine given the mask, not the slicing),
the closed form for w = 1 (the newest token's V), identity when w >= ctx,
independence from the table entries of blocks wholly before the window, and
the tile gather agreeing with the element-wise slot gather from a start
position.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, layout
from tests.helpers import fill_pool, random_tables


def _bits_to_t64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _masked_sdpa(q_bits, k_tok, v_tok, ctx, group, scale, window):
    """Window through an attention mask over the whole context."""
    out = []
    for s in range(len(ctx)):
        n = int(ctx[s])
        q = _bits_to_t64(q_bits[s])
        if n == 0:
            out.append(torch.zeros_like(q))
            continue
        k = _bits_to_t64(k_tok[s][:n]).permute(1, 0, 2).repeat_interleave(group, dim=0).contiguous()
        v = _bits_to_t64(v_tok[s][:n]).permute(1, 0, 2).repeat_interleave(group, dim=0).contiguous()
        pos = torch.arange(n)
        keep = pos >= (n - window) if window > 0 else torch.ones(n, dtype=torch.bool)
        mask = keep[None, None, :].expand(q.shape[0], 1, n)
        o = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], k, v, attn_mask=mask,
                                                             scale=float(np.float32(scale)))
        out.append(o[:, 0, :])
    return torch.stack(out).numpy()


def _case(rng, S, hkv, group, D, B, max_ctx):
    ctx = rng.integers(1, max_ctx + 1, size=S).astype(np.int32)
    need = sum(math.ceil(int(c) / B) for c in ctx)
    nb = need + 2
    shape = layout.PoolShape(1, nb, B, hkv, D)
    bt = random_tables(rng, nb, ctx, B)
    q = workloads.to_bf16_bits(rng.standard_normal((S, hkv * group, D), dtype=np.float32))
    k_tok = [workloads.to_bf16_bits(rng.standard_normal((int(c), hkv, D), dtype=np.float32)) for c in ctx]
    v_tok = [workloads.to_bf16_bits(rng.standard_normal((int(c), hkv, D), dtype=np.float32)) for c in ctx]
    img = fill_pool(shape, bt, ctx, k_tok, v_tok)
    return shape, bt, ctx, q, k_tok, v_tok, img


@pytest.mark.parametrize("seed", range(24))
def test_window_matches_masked_sdpa(seed):
    rng = np.random.default_rng(7300 + seed)
    hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 3, 4]))
    D = int(rng.choice([16, 32]))
    B = int(rng.choice([4, 8, 16]))
    shape, bt, ctx, q, k_tok, v_tok, img = _case(rng, 3, hkv, group, D, B, 80)
    scale = 1.0 / math.sqrt(D)
    for window in (1, 2, 5, B, B + 1, 33, 200):
        got = attention.paged_decode(q, img, 0, bt, ctx, scale, window=window)
        ref = _masked_sdpa(q, k_tok, v_tok, ctx, group, scale, window)
        assert np.max(np.abs(got - ref)) < 1e-12, window


def test_window_one_is_the_newest_value():
    rng = np.random.default_rng(7400)
    shape, bt, ctx, q, k_tok, v_tok, img = _case(rng, 5, 2, 4, 32, 8, 60)
    got = attention.paged_decode(q, img, 0, bt, ctx, 0.17, window=1)
    for s in range(len(ctx)):
        v = _bits_to_t64(v_tok[s][int(ctx[s]) - 1]).numpy()
        for h in range(8):
            assert np.array_equal(got[s, h], v[h // 4])


def test_window_covering_the_context_changes_nothing():
    rng = np.random.default_rng(7500)
    shape, bt, ctx, q, k_tok, v_tok, img = _case(rng, 4, 2, 2, 32, 16, 90)
    full = attention.paged_decode(q, img, 0, bt, ctx, 0.2)
    for window in (int(ctx.max()), int(ctx.max()) + 1, 10 ** 6):
        assert np.array_equal(attention.paged_decode(q, img, 0, bt, ctx, 0.2, window=window), full)


def test_blocks_before_the_window_are_never_read():
    rng = np.random.default_rng(7600)
    B = 8
    shape, bt, ctx, q, k_tok, v_tok, img = _case(rng, 4, 2, 2, 32, B, 90)
    window = 13
    want = attention.paged_decode(q, img, 0, bt, ctx, 0.2, window=window)
    bad = bt.copy()
    for s in range(len(ctx)):
        first = attention.window_start(int(ctx[s]), window) // B
        bad[s, :first] = -987654   # not a block at all
    assert np.array_equal(attention.paged_decode(q, img, 0, bad, ctx, 0.2, window=window), want)


@pytest.mark.parametrize("dtype", [layout.KV_BF16, layout.KV_FP8_E5M2, layout.KV_INT8])
def test_tile_gather_from_a_start_equals_slot_gather(dtype):
    rng = np.random.default_rng(7700 + dtype)
    B, hkv, D = 8, 2, 32
    ctx = np.array([1, 9, 30, 57], np.int32)
    nb = sum(math.ceil(int(c) / B) for c in ctx) + 1
    shape = layout.PoolShape(1, nb, B, hkv, D, dtype)
    bt = random_tables(rng, nb, ctx, B)
    k_tok = [workloads.to_bf16_bits(rng.standard_normal((int(c), hkv, D), dtype=np.float32)) for c in ctx]
    v_tok = [workloads.to_bf16_bits(rng.standard_normal((int(c), hkv, D), dtype=np.float32)) for c in ctx]
    img = fill_pool(shape, bt, ctx, k_tok, v_tok, k_scale=0.5, v_scale=2.0)
    for s in range(len(ctx)):
        for start in range(0, int(ctx[s]) + 1, 3):
            a = attention.gather_kv(img, 0, bt[s], int(ctx[s]), 0.5, 2.0, start)
            b = attention.gather_kv_by_slot(img, 0, bt[s], int(ctx[s]), 0.5, 2.0, start)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            assert a[0].shape[0] == int(ctx[s]) - start
