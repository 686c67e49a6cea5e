"""Pins of the oracle's paged prefill (a chunk of new tokens per sequence,
causal over the cache): the whole-prompt case against a matrix-form causal
softmax attention written independently here, chunks at the end of each
context against torch's scaled_dot_product_attention with an explicit
boolean causal mask (a library routine), the chunk's last token against the
decode oracle, chunking invariance (one chunk or two give the same rows),
and zero rows for queries with no position.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import attention, cache_ops, codecs, layout
from tests.helpers import expanded_slots, random_tables


def _pool(rng, ctx, B=8, H=2, D=32, dt=layout.KV_BF16):
    nb = sum(math.ceil(int(c) / B) for c in ctx) + 2
    p = layout.PoolShape(1, nb, B, H, D, dt)
    img = layout.empty_image(p)
    bt = random_tables(rng, nb, np.asarray(ctx), B)
    k = workloads.to_bf16_bits(rng.standard_normal((int(sum(ctx)), H, D), dtype=np.float32))
    v = workloads.to_bf16_bits(rng.standard_normal((int(sum(ctx)), H, D), dtype=np.float32))
    slots = np.concatenate([expanded_slots(bt[s], int(ctx[s]), B) for s in range(len(ctx))])
    img = cache_ops.reshape_and_cache(img, 0, k, v, slots)
    return img, bt, k, v


def _causal_sdpa(q, k, v, scale, G):
    """q [n, Hq, D], k/v [n, Hkv, D] (float64): softmax(q k^T * scale + causal
    mask) v, as matrices."""
    n, hq, _ = q.shape
    out = np.zeros_like(q)
    mask = np.triu(np.ones((n, n), bool), 1)            # key j > query i is hidden
    for h in range(hq):
        s = (q[:, h, :] @ k[:, h // G, :].T) * scale
        s[mask] = -np.inf
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ v[:, h // G, :]
    return out


@pytest.mark.parametrize("G", [1, 3])
def test_whole_prompt_equals_matrix_causal_attention(G):
    rng = np.random.default_rng(14000 + G)
    ctx = [1, 9, 23]
    H, D = 2, 32
    img, bt, k, v = _pool(rng, ctx, H=H, D=D)
    qs = np.concatenate([[0], np.cumsum(ctx)])
    q = workloads.to_bf16_bits(rng.standard_normal((int(qs[-1]), H * G, D), dtype=np.float32))
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    got = attention.paged_prefill(q, img, 0, bt, np.asarray(ctx), qs, scale)
    for s in range(len(ctx)):
        a, b = int(qs[s]), int(qs[s + 1])
        want = _causal_sdpa(codecs.bf16_bits_to_f64(q[a:b]), codecs.bf16_bits_to_f64(k[a:b]),
                            codecs.bf16_bits_to_f64(v[a:b]), np.float64(np.float32(scale)), G)
        assert np.allclose(got[a:b], want, atol=1e-12, rtol=1e-12)


def test_last_token_of_a_chunk_is_the_decode():
    rng = np.random.default_rng(14100)
    ctx = np.array([5, 17, 40, 33])
    n = np.array([5, 3, 1, 16])                      # whole prompt, chunks, a single token
    img, bt, _, _ = _pool(rng, ctx)
    qs = np.concatenate([[0], np.cumsum(n)])
    q = workloads.to_bf16_bits(rng.standard_normal((int(qs[-1]), 4, 32), dtype=np.float32))
    got = attention.paged_prefill(q, img, 0, bt, ctx, qs, 0.17)
    last = q[qs[1:] - 1]
    want = attention.paged_decode(last, img, 0, bt, ctx, 0.17)
    assert np.array_equal(got[qs[1:] - 1], want)


def test_two_chunks_give_the_rows_of_one():
    # prefilling positions [0, 12) then [12, 30) equals prefilling [0, 30)
    rng = np.random.default_rng(14200)
    img, bt, _, _ = _pool(rng, [30])
    q = workloads.to_bf16_bits(rng.standard_normal((30, 2, 32), dtype=np.float32))
    whole = attention.paged_prefill(q, img, 0, bt, np.array([30]), np.array([0, 30]), 0.2)
    first = attention.paged_prefill(q[:12], img, 0, bt, np.array([12]), np.array([0, 12]), 0.2)
    second = attention.paged_prefill(q[12:], img, 0, bt, np.array([30]), np.array([0, 18]), 0.2)
    assert np.array_equal(np.concatenate([first, second]), whole)


def test_queries_without_a_position_are_zero():
    rng = np.random.default_rng(14300)
    img, bt, _, _ = _pool(rng, [4])
    q = workloads.to_bf16_bits(rng.standard_normal((6, 2, 32), dtype=np.float32))
    got = attention.paged_prefill(q, img, 0, bt, np.array([4]), np.array([0, 6]), 0.2)
    assert not got[:2].any() and np.all(np.abs(got[2:]).sum(axis=(1, 2)) > 0)


@pytest.mark.parametrize("seed", range(6))
def test_chunks_match_torch_sdpa_with_a_causal_mask(seed):
    """Chunks of new tokens at the end of each context (some longer than
    the context, whose extra queries get zero rows) against torch's
    scaled_dot_product_attention in float64 with an explicit boolean mask
    over the whole context (a library routine given the mask)."""
    import torch
    rng = np.random.default_rng(14100 + seed)
    G = int(rng.choice([1, 2, 4]))
    H, D, B = 2, 16, int(rng.choice([4, 8]))
    ctx = [int(x) for x in rng.integers(1, 40, size=4)]
    n = [int(rng.integers(0, c + 3)) for c in ctx]            # up to 2 past the context
    img, bt, k, v = _pool(rng, ctx, B=B, H=H, D=D)
    qs = np.concatenate([[0], np.cumsum(n)])
    q = workloads.to_bf16_bits(rng.standard_normal((int(qs[-1]), H * G, D), dtype=np.float32))
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    got = attention.paged_prefill(q, img, 0, bt, np.asarray(ctx), qs, scale)
    off = np.concatenate([[0], np.cumsum(ctx)])
    for s in range(len(ctx)):
        if n[s] == 0:
            continue
        c = ctx[s]
        kk = torch.from_numpy(codecs.bf16_bits_to_f64(k[off[s]:off[s] + c])).permute(1, 0, 2)
        vv = torch.from_numpy(codecs.bf16_bits_to_f64(v[off[s]:off[s] + c])).permute(1, 0, 2)
        kk = kk.repeat_interleave(G, dim=0).contiguous()
        vv = vv.repeat_interleave(G, dim=0).contiguous()
        qq = torch.from_numpy(codecs.bf16_bits_to_f64(q[qs[s]:qs[s + 1]])).permute(1, 0, 2).contiguous()
        pos = c - n[s] + torch.arange(n[s])                  # each query's position
        mask = torch.arange(c)[None, :] <= pos[:, None]      # [n, c]: keys at or before the position
        valid = pos >= 0
        want = torch.zeros_like(qq)
        if valid.any():
            o = torch.nn.functional.scaled_dot_product_attention(qq[:, valid], kk, vv, attn_mask=mask[valid],
                                                                 scale=float(np.float32(scale)))
            want[:, valid] = o
        want = want.permute(1, 0, 2).numpy()
        assert np.max(np.abs(got[qs[s]:qs[s + 1]] - want)) < 1e-12, s
