"""Prefix caching end to end on the GPU: a second request whose prompt starts
with the first one's reuses its cached blocks, writes KV only past the
reused prefix, and decodes to the oracle's output over the full prompt; the radix-tree
form also reuses a prefix that ends inside a block, through a block copy."""

import numpy as np
import pytest

import paged_kv_cache_436_amd as pkv
import workloads
from oracle import attention, cache_ops, codecs
from tests.gpu_helpers import bf16_dev, dev, errors, first_diff, images_equal, read_pool, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P", [0, 64])
def test_reused_prefix_blocks_decode_like_a_full_prefill(P):
    import torch
    rng = np.random.default_rng(13500 + P)
    B, H, G, D, NB = 16, 2, 4, 128, 64
    cfg = pkv.make_config(1, NB, B, H, D, pkv.PKV_KV_BF16)
    pool = pkv.Pool(cfg)
    pool.memory.fill_(255)
    bm = pkv.BlockManager(NB, B, rng.permutation(NB))
    prefix = rng.integers(0, 1000, size=256).tolist()
    prompts = [prefix + rng.integers(0, 1000, size=44).tolist(), prefix + rng.integers(0, 1000, size=7).tolist()]
    # K/V of a token depend on the whole prefix; here: a fixed function of (position, token) for the
    # shared part and fresh values per request after it
    kv = {}
    img = read_pool(pool)
    for s, pr in enumerate(prompts):
        cached = bm.add_seq_tokens(s, pr)
        say(f"request {s}: {len(pr)} tokens, {cached} reused")
        assert cached == (256 if s else 0)
        n = len(pr)
        k = workloads.to_bf16_bits(rng.standard_normal((n, H, D), dtype=np.float32))
        v = workloads.to_bf16_bits(rng.standard_normal((n, H, D), dtype=np.float32))
        if s:
            k[:256], v[:256] = kv[0][0][:256], kv[0][1][:256]   # the reused prefix is request 0's
        kv[s] = (k, v)
        tab, _ = bm.block_tables([s], 32)
        pos = np.arange(cached, n)
        slots = (tab[0][pos // B].astype(np.int64) * B + pos % B)
        pkv.reshape_and_cache(pool, 0, bf16_dev(k[cached:]), bf16_dev(v[cached:]), dev(slots))
        img = cache_ops.reshape_and_cache(img, 0, k[cached:], v[cached:], slots)
    tables, ctx = bm.block_tables([0, 1], 32)
    assert (tables[0][:16] == tables[1][:16]).all()
    q = workloads.to_bf16_bits(rng.standard_normal((2, H * G, D), dtype=np.float32))
    out = torch.empty((2, H * G, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, pkv.paged_attn_workspace_bytes(2, H * G, D, 32, B, P)), dtype=torch.uint8,
                     device="cuda")
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    pkv.paged_attn_decode(out, bf16_dev(q), pool, 0, dev(tables), dev(ctx), scale, partition_size=P,
                          workspace=ws if P else None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = attention.paged_decode(q, img, 0, tables, ctx, scale)
    # and the same as contiguous attention over each request's full K/V
    for s in range(2):
        K = np.asarray(kv[s][0]).view(np.uint16)
        ref = attention.attend(codecs.bf16_bits_to_f64(q[s]), codecs.bf16_bits_to_f64(K),
                               codecs.bf16_bits_to_f64(kv[s][1]), scale)
        assert np.max(np.abs(ref - want[s])) < 1e-12
    mx, rel = errors(got, want)
    assert mx <= 1e-2 and rel <= 1e-3


def test_whole_prompt_hit_leaves_last_block_to_prefill_then_decodes():
    """A second request with the very same 64-token prompt (a multiple of the
    block size) reuses every block before the last prompt token and prefills
    the last block into a fresh one of its own; the shared blocks are never
    written.  Prefill and a following appending decode step of both requests
    match the oracle (bjdmk.com.cn article, §4.1: reuse the cached prefix,
    compute the rest; "KV Cache 原理与 PagedAttention", §一: a decode step
    appends K_t, V_t and attends)."""
    import torch
    rng = np.random.default_rng(13600)
    B, H, G, D, NB, W = 16, 2, 4, 128, 32, 8
    hq = H * G
    cfg = pkv.make_config(1, NB, B, H, D, pkv.PKV_KV_BF16)
    pool = pkv.Pool(cfg)
    pool.memory.fill_(255)
    bm = pkv.BlockManager(NB, B, rng.permutation(NB))
    prompt = rng.integers(0, 1000, size=64).tolist()
    # the same tokens at the same positions have the same K/V
    k = workloads.to_bf16_bits(rng.standard_normal((64, H, D), dtype=np.float32))
    v = workloads.to_bf16_bits(rng.standard_normal((64, H, D), dtype=np.float32))
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    img = read_pool(pool)
    for s in range(2):
        cached = bm.add_seq_tokens(s, prompt)
        say(f"request {s}: 64 tokens, {cached} reused")
        assert cached == (48 if s else 0)
        tab, ctx = bm.block_tables([s], W)
        pos = np.arange(cached, 64)
        slots = tab[0][pos // B].astype(np.int64) * B + pos % B
        before = read_pool(pool)
        pkv.reshape_and_cache(pool, 0, bf16_dev(k[cached:]), bf16_dev(v[cached:]), dev(slots))
        img = cache_ops.reshape_and_cache(img, 0, k[cached:], v[cached:], slots)
        after = read_pool(pool)
        assert images_equal(after, img), first_diff(after, img)
        if s:
            # the blocks request 0 holds are unchanged by request 1's prefill
            t0, _ = bm.block_tables([0], W)
            per_block = H * B * D                  # elements of one block's tiles (one layer)
            for blk in t0[0][:4]:
                r = slice(int(blk) * per_block, (int(blk) + 1) * per_block)
                assert np.array_equal(after.k[r], before.k[r]) and np.array_equal(after.v[r], before.v[r])
        n = 64 - cached
        q = workloads.to_bf16_bits(rng.standard_normal((n, hq, D), dtype=np.float32))
        qs = np.array([0, n], np.int32)
        out = torch.full((n, hq, D), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attn_prefill(out, bf16_dev(q), pool, 0, dev(tab), dev(ctx), dev(qs), scale, n)
        torch.cuda.synchronize()
        want = attention.paged_prefill(q, img, 0, tab, ctx, qs, scale)
        mx, rel = errors(out.cpu().numpy(), want)
        say(f"  prefill of {n} tokens: max_abs={mx:.3e} rel={rel:.3e}")
        assert mx <= 1e-2 and rel <= 1e-3
    t_both, _ = bm.block_tables([0, 1], W)
    assert (t_both[0][:3] == t_both[1][:3]).all() and t_both[0][3] != t_both[1][3]
    # one appending decode step of both requests (position 64 opens block 4)
    slots, pairs = bm.append([0, 1])
    assert pairs.shape[0] == 0
    tables, ctx = bm.block_tables([0, 1], W)
    nk = workloads.to_bf16_bits(rng.standard_normal((2, H, D), dtype=np.float32))
    nv = workloads.to_bf16_bits(rng.standard_normal((2, H, D), dtype=np.float32))
    q = workloads.to_bf16_bits(rng.standard_normal((2, hq, D), dtype=np.float32))
    out = torch.empty((2, hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pkv.paged_attn_workspace_bytes(2, hq, D, W, B, 64), dtype=torch.uint8, device="cuda")
    pkv.paged_attn_decode_append(out, bf16_dev(q), pool, 0, bf16_dev(nk), bf16_dev(nv), dev(tables), dev(ctx),
                                 scale, partition_size=64, workspace=ws)
    torch.cuda.synchronize()
    img = cache_ops.reshape_and_cache(img, 0, nk, nv, slots)
    got_img = read_pool(pool)
    assert images_equal(got_img, img), first_diff(got_img, img)
    want = attention.paged_decode(q, img, 0, tables, ctx, scale)
    mx, rel = errors(out.cpu().numpy(), want)
    say(f"  decode: max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= 1e-2 and rel <= 1e-3


def test_radix_partial_block_hit_copies_then_prefills_the_rest():
    """Radix-tree reuse that ends inside a block (bjdmk.com.cn article,
    §4.2): the second prompt shares 263 tokens with the first (16 whole
    blocks + 7 tokens of the 17th); it reuses the 16 blocks, copies the
    first prompt's 17th block into its own fresh block (copy_blocks with the
    pair the manager returned), writes K/V from position 263 on, and its
    prefill of the remaining tokens and a decode step match the oracle, and
    attention over its own full K/V."""
    import torch
    rng = np.random.default_rng(13700)
    B, H, G, D, NB, W = 16, 2, 4, 128, 64, 24
    hq = H * G
    cfg = pkv.make_config(1, NB, B, H, D, pkv.PKV_KV_BF16)
    pool = pkv.Pool(cfg)
    pool.memory.fill_(255)
    bm = pkv.BlockManager(NB, B, rng.permutation(NB))
    shared = rng.integers(0, 1000, size=263).tolist()
    prompts = [shared + [1001] + rng.integers(0, 1000, size=40).tolist(),
               shared + [1002] + rng.integers(0, 1000, size=20).tolist()]
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    img = read_pool(pool)
    kv = {}
    for s, pr in enumerate(prompts):
        cached, pair = bm.add_seq_radix(s, pr)
        say(f"request {s}: {len(pr)} tokens, {cached} reused, copy {pair}")
        n = len(pr)
        tab, ctx = bm.block_tables([s], W)
        if s:
            assert cached == 263 and pair == (int(kv[0][2][16]), int(tab[0][16]))
            assert (tab[0][:16] == kv[0][2][:16]).all()
            pk = dev(np.asarray([pair], dtype=np.int64))
            pkv.copy_blocks(pool, pk)
            img = cache_ops.copy_blocks(img, np.asarray([pair], dtype=np.int64))
        else:
            assert (cached, pair) == (0, None)
        k = workloads.to_bf16_bits(rng.standard_normal((n, H, D), dtype=np.float32))
        v = workloads.to_bf16_bits(rng.standard_normal((n, H, D), dtype=np.float32))
        if s:
            k[:263], v[:263] = kv[0][0][:263], kv[0][1][:263]     # the shared tokens' K/V are request 0's
        kv[s] = (k, v, tab[0].copy())
        pos = np.arange(cached, n)
        slots = tab[0][pos // B].astype(np.int64) * B + pos % B
        pkv.reshape_and_cache(pool, 0, bf16_dev(k[cached:]), bf16_dev(v[cached:]), dev(slots))
        img = cache_ops.reshape_and_cache(img, 0, k[cached:], v[cached:], slots)
        got_img = read_pool(pool)
        assert images_equal(got_img, img), first_diff(got_img, img)
        m = n - cached
        q = workloads.to_bf16_bits(rng.standard_normal((m, hq, D), dtype=np.float32))
        qs = np.array([0, m], np.int32)
        out = torch.full((m, hq, D), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attn_prefill(out, bf16_dev(q), pool, 0, dev(tab), dev(ctx), dev(qs), scale, m)
        torch.cuda.synchronize()
        want = attention.paged_prefill(q, img, 0, tab, ctx, qs, scale)
        mx, rel = errors(out.cpu().numpy(), want)
        say(f"  prefill of {m} tokens: max_abs={mx:.3e} rel={rel:.3e}")
        assert mx <= 1e-2 and rel <= 1e-3
    # decode of both over the pool equals attention over each one's own K/V
    tables, ctx = bm.block_tables([0, 1], W)
    q = workloads.to_bf16_bits(rng.standard_normal((2, hq, D), dtype=np.float32))
    out = torch.empty((2, hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pkv.paged_attn_workspace_bytes(2, hq, D, W, B, 64), dtype=torch.uint8, device="cuda")
    pkv.paged_attn_decode(out, bf16_dev(q), pool, 0, dev(tables), dev(ctx), scale, partition_size=64, workspace=ws)
    torch.cuda.synchronize()
    want = attention.paged_decode(q, img, 0, tables, ctx, scale)
    for s in range(2):
        ref = attention.attend(codecs.bf16_bits_to_f64(q[s]), codecs.bf16_bits_to_f64(kv[s][0]),
                               codecs.bf16_bits_to_f64(kv[s][1]), scale)
        assert np.max(np.abs(ref - want[s])) < 1e-12
    mx, rel = errors(out.cpu().numpy(), want)
    say(f"  decode: max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= 1e-2 and rel <= 1e-3
