"""Pins of the oracle's shared-prefix decode (CPU only).

Requests that start with the same prompt name the same physical blocks for
it (bjdmk.com.cn article, §3.1, §3.2).  The oracle reads positions below
min(ctx, prefix_len) through the one shared table and the rest through each
sequence's own row.  Pinned by: torch's scaled_dot_product_attention in
float64 on each sequence's tokens in order (a library routine on the token
lists the test builds, not on the oracle's gather); bit-identity with the
plain paged decode of a second pool in which every sequence holds its own
written copy of the prefix; identity with the plain decode when the tables
already name the shared blocks; prefix_len = 0.  The own rows' entries
below the prefix point to decoy blocks holding other tokens, so a read
through the wrong table changes the values.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, layout
from tests.helpers import fill_pool


def _bits_to_t64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _case(rng, S, hkv, group, D, B, prefix_blocks, max_own, dtype=layout.KV_BF16, short=True):
    """A pool with one shared prefix of prefix_blocks blocks and S sequences.

    Sequence s has context ctx_s: most run past the prefix by 1..max_own
    tokens; with ``short`` some stop inside it (or at 0).  Returns the
    shared image, the tables (own rows with decoy blocks below the prefix),
    the prefix table, per-sequence token lists (prefix tokens then own), and
    the materialised image + tables in which each sequence's first blocks
    hold its own copy of the prefix."""
    P = prefix_blocks * B
    ctx = P + rng.integers(1, max_own + 1, size=S)
    if short and S >= 3:
        ctx[0] = 0
        ctx[1] = int(rng.integers(1, max(2, P)))
        ctx[2] = P
    ctx = ctx.astype(np.int32)
    width = max(1, max(math.ceil(int(c) / B) for c in ctx))
    own_blocks = [max(0, math.ceil(int(c) / B) - prefix_blocks) for c in ctx]
    # blocks: prefix, decoys (one per own-row entry below the prefix), own suffixes
    n_dec = S * prefix_blocks
    nb = prefix_blocks + n_dec + sum(own_blocks) + 1
    perm = rng.permutation(nb)
    prefix_table = perm[:prefix_blocks].astype(np.int32)
    bt = np.zeros((S, width), np.int32)
    pos = prefix_blocks
    for s in range(S):
        bt[s, :prefix_blocks] = perm[pos:pos + prefix_blocks]
        pos += prefix_blocks
    for s in range(S):
        bt[s, prefix_blocks:prefix_blocks + own_blocks[s]] = perm[pos:pos + own_blocks[s]]
        pos += own_blocks[s]
    shape = layout.PoolShape(1, nb, B, hkv, D, dtype)
    pk = workloads.to_bf16_bits(rng.standard_normal((P, hkv, D), dtype=np.float32))
    pv = workloads.to_bf16_bits(rng.standard_normal((P, hkv, D), dtype=np.float32))
    k_tok, v_tok, dk, dv = [], [], [], []
    for s in range(S):
        n_own = max(0, int(ctx[s]) - P)
        ok = workloads.to_bf16_bits(rng.standard_normal((n_own, hkv, D), dtype=np.float32))
        ov = workloads.to_bf16_bits(rng.standard_normal((n_own, hkv, D), dtype=np.float32))
        k_tok.append(np.concatenate([pk[:min(int(ctx[s]), P)], ok]))
        v_tok.append(np.concatenate([pv[:min(int(ctx[s]), P)], ov]))
        # decoys: other tokens in the own row's blocks below the prefix
        dk.append(np.concatenate([workloads.to_bf16_bits(rng.standard_normal((P, hkv, D), dtype=np.float32)), ok]))
        dv.append(np.concatenate([workloads.to_bf16_bits(rng.standard_normal((P, hkv, D), dtype=np.float32)), ov]))
    ks, vs = (0.5, 1.5) if dtype != layout.KV_BF16 else (1.0, 1.0)
    full = np.maximum(ctx, P)      # the decoys fill every own-row block below the prefix
    img = fill_pool(shape, bt, full, dk, dv, k_scale=ks, v_scale=vs)
    img = fill_pool(shape, prefix_table[None, :], np.array([P]), [pk], [pv], k_scale=ks, v_scale=vs, img=img)
    # materialised: each sequence's first blocks hold its copy of the prefix
    mat = fill_pool(shape, bt, ctx, k_tok, v_tok, k_scale=ks, v_scale=vs)
    return dict(shape=shape, img=img, bt=bt, ctx=ctx, prefix_table=prefix_table, P=P, k_tok=k_tok,
                v_tok=v_tok, mat=mat, ks=ks, vs=vs)


def _sdpa(q_bits, k_tok, v_tok, group, scale):
    out = []
    for s in range(len(k_tok)):
        q = _bits_to_t64(q_bits[s])
        n = k_tok[s].shape[0]
        if n == 0:
            out.append(torch.zeros_like(q))
            continue
        k = _bits_to_t64(k_tok[s]).permute(1, 0, 2).repeat_interleave(group, dim=0).contiguous()
        v = _bits_to_t64(v_tok[s]).permute(1, 0, 2).repeat_interleave(group, dim=0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], k, v, scale=float(np.float32(scale)))
        out.append(o[:, 0, :])
    return torch.stack(out).numpy()


@pytest.mark.parametrize("seed", range(12))
def test_shared_prefix_matches_sdpa_on_the_token_lists(seed):
    rng = np.random.default_rng(8100 + seed)
    hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([16, 32]))
    B = int(rng.choice([4, 8, 16]))
    c = _case(rng, 5, hkv, group, D, B, int(rng.integers(1, 4)), 40)
    q = workloads.to_bf16_bits(rng.standard_normal((5, hkv * group, D), dtype=np.float32))
    scale = 1.0 / math.sqrt(D)
    got = attention.paged_decode_shared_prefix(q, c["img"], 0, c["bt"], c["ctx"], c["prefix_table"], c["P"], scale)
    ref = _sdpa(q, c["k_tok"], c["v_tok"], group, scale)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("dtype", [layout.KV_BF16, layout.KV_FP8_E5M2, layout.KV_INT8, layout.KV_INT8_TENSOR])
def test_shared_prefix_equals_decode_of_materialised_copies(dtype):
    rng = np.random.default_rng(8200 + dtype)
    c = _case(rng, 6, 2, 3, 32, 8, 3, 30, dtype)
    q = workloads.to_bf16_bits(rng.standard_normal((6, 6, 32), dtype=np.float32))
    got = attention.paged_decode_shared_prefix(q, c["img"], 0, c["bt"], c["ctx"], c["prefix_table"], c["P"], 0.2,
                                               c["ks"], c["vs"])
    want = attention.paged_decode(q, c["mat"], 0, c["bt"], c["ctx"], 0.2, c["ks"], c["vs"])
    assert np.array_equal(got, want)


def test_tables_naming_the_shared_blocks_give_the_plain_decode():
    rng = np.random.default_rng(8300)
    c = _case(rng, 5, 2, 2, 32, 8, 2, 25)
    bt = c["bt"].copy()
    bt[:, :2] = c["prefix_table"]          # the tables as a block manager holds them
    q = workloads.to_bf16_bits(rng.standard_normal((5, 4, 32), dtype=np.float32))
    got = attention.paged_decode_shared_prefix(q, c["img"], 0, bt, c["ctx"], c["prefix_table"], c["P"], 0.3)
    assert np.array_equal(got, attention.paged_decode(q, c["img"], 0, bt, c["ctx"], 0.3))


def test_empty_prefix_is_the_plain_decode():
    rng = np.random.default_rng(8400)
    c = _case(rng, 4, 1, 4, 16, 4, 2, 20)
    q = workloads.to_bf16_bits(rng.standard_normal((4, 4, 16), dtype=np.float32))
    got = attention.paged_decode_shared_prefix(q, c["img"], 0, c["bt"], c["ctx"], np.zeros(0, np.int32), 0, 0.25)
    assert np.array_equal(got, attention.paged_decode(q, c["img"], 0, c["bt"], c["ctx"], 0.25))
