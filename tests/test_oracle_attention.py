"""Pins of the oracle's decode attention.

* Library routine: torch's scaled_dot_product_attention in float64 on CPU,
  fed the contiguous K/V (widened by torch) with each KV head repeated over
  its query group.  Any slip in slot mapping, gather, grouping, scaling or
  softmax fails this.
* Closed forms: one token gives its V exactly; q = 0 gives the mean of V;
  a dominant key returns its value; huge logits stay finite.
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


def _sdpa_reference(q_bits, k_tok, v_tok, ctx, group, scale):
    out = []
    for s in range(len(ctx)):
        n = int(ctx[s])
        q = _bits_to_t64(q_bits[s])                      # [Hq, D]
        if n == 0:
            out.append(torch.zeros_like(q))
            continue
        k = _bits_to_t64(k_tok[s][:n]).permute(1, 0, 2)  # [Hkv, n, D]
        v = _bits_to_t64(v_tok[s][:n]).permute(1, 0, 2)
        k = k.repeat_interleave(group, dim=0).contiguous()
        v = v.repeat_interleave(group, dim=0).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(
            q[:, None, :], k, v, scale=float(np.float32(scale)))
        out.append(o[:, 0, :])
    return torch.stack(out).numpy()


def _case(rng, S, hkv, group, D, B, max_ctx, zero_ok=False):
    lo = 0 if zero_ok else 1
    ctx = rng.integers(lo, max_ctx + 1, size=S).astype(np.int32)
    need = sum(math.ceil(int(c) / B) for c in ctx)
    nb = need + int(rng.integers(0, 5)) + 1
    shape = layout.PoolShape(1, nb, B, hkv, D)
    bt = random_tables(rng, nb, ctx, B)
    hq = hkv * group
    q = workloads.to_bf16_bits(rng.standard_normal((S, hq, D), dtype=np.float32))
    k_tok = [workloads.to_bf16_bits(rng.standard_normal((max(int(c), 1), hkv, D), dtype=np.float32)) for c in ctx]
    v_tok = [workloads.to_bf16_bits(rng.standard_normal((max(int(c), 1), hkv, D), dtype=np.float32)) for c in ctx]
    return shape, bt, ctx, q, k_tok, v_tok


def test_tiny_config_matches_sdpa():
    w = workloads.tiny()
    bt = workloads.static_tables(w)
    shape = layout.PoolShape(1, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    q = workloads.queries(w)
    total = int(w.context_lens.sum())
    k_all, v_all = workloads.token_kv(w, total)
    offs = np.concatenate([[0], np.cumsum(w.context_lens)])
    k_tok = [k_all[offs[s]:offs[s + 1]] for s in range(w.num_seqs)]
    v_tok = [v_all[offs[s]:offs[s + 1]] for s in range(w.num_seqs)]
    img = fill_pool(shape, bt, w.context_lens, k_tok, v_tok)
    got = attention.paged_decode(q, img, 0, bt, w.context_lens, w.scale)
    ref = _sdpa_reference(q, k_tok, v_tok, w.context_lens, w.group, w.scale)
    assert np.max(np.abs(got - ref)) < 1e-12
    # context 1: the output is that token's V exactly
    v0 = _bits_to_t64(v_tok[0][0]).numpy()
    for h in range(w.num_q_heads):
        assert np.array_equal(got[0, h], v0[h // w.group])


@pytest.mark.parametrize("seed", range(50))
def test_random_small_cases_match_sdpa(seed):
    rng = np.random.default_rng(1000 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([16, 32, 64]))
    B = int(rng.choice([4, 8, 16, 32]))
    shape, bt, ctx, q, k_tok, v_tok = _case(rng, int(rng.integers(1, 5)), hkv, group, D, B, 70,
                                            zero_ok=True)
    img = fill_pool(shape, bt, ctx, k_tok, v_tok)
    got = attention.paged_decode(q, img, 0, bt, ctx, 1.0 / math.sqrt(D))
    ref = _sdpa_reference(q, k_tok, v_tok, ctx, group, 1.0 / math.sqrt(D))
    assert np.max(np.abs(got - ref)) < 1e-12
    # empty contexts give zeros
    for s in np.nonzero(ctx == 0)[0]:
        assert not got[s].any()


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((37, 2, 16))
    V = rng.standard_normal((37, 2, 16))
    out = attention.attend(np.zeros((4, 16)), K, V, 0.25)
    for h in range(4):
        assert np.allclose(out[h], V[:, h // 2, :].mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_key_returns_its_value():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((50, 1, 32))
    V = rng.standard_normal((50, 1, 32))
    t_star = 17
    q = 50.0 * K[t_star, 0][None, :]
    out = attention.attend(q, K, V, 1.0)
    z = K[:, 0, :] @ q[0]
    gap = z[t_star] - np.max(np.delete(z, t_star))
    assert gap > 100
    assert np.max(np.abs(out[0] - V[t_star, 0])) <= 50 * math.exp(-gap) * np.max(np.abs(V)) + 1e-15


def test_huge_logits_do_not_overflow():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((20, 1, 8)) * 300
    V = rng.standard_normal((20, 1, 8))
    q = rng.standard_normal((1, 8)) * 300          # logits ~ 1e5
    out = attention.attend(q, K, V, 1.0)
    assert np.all(np.isfinite(out))
    t = np.argmax(K[:, 0, :] @ q[0])
    assert np.allclose(out[0], V[t, 0])
