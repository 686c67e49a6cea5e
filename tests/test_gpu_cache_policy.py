"""The split form's K/V cache policy (PKV_DECODE_KEEP_KV_CACHED) changes how
lines are kept in the caches, never the arithmetic: streamed and cached
loads give the same output bits, in the plain, appending and shared-prefix
decodes, for every storage type; and the cached form matches the oracle on
tables that share blocks (the case it is for).
"""

import numpy as np
import pytest

import paged_kv_cache_436_amd as pkv
import workloads
from oracle import attention
from tests.gpu_helpers import bf16_dev, dev, errors, say
from tests.test_gpu_shared_prefix import ALL, _bar, _case, _ctx_mix

pytestmark = pytest.mark.gpu


def _ex(c, keep, key=None, value=None):
    import torch
    S, D = len(c.ctx), c.cfg.head_dim
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    out = torch.full((S, c.hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(pkv.paged_attn_workspace_bytes(S, c.hq, D, c.width, c.cfg.block_size, 512), dtype=torch.uint8,
                     device="cuda")
    pkv.paged_attn_decode_ex(out, c.d_q, c.pool, 1, c.d_tables, c.d_ctx, scale, c.cfg.kv_dtype, c.ks, c.vs, 512, ws,
                             key=key, value=value, keep_kv_cached=keep)
    torch.cuda.synchronize()
    return out.cpu().numpy(), scale


@pytest.mark.parametrize("dt", ALL)
def test_cached_and_streamed_loads_give_the_same_bits(dt):
    rng = np.random.default_rng(15000 + dt)
    c = _case(rng, dt, 6, _ctx_mix(96, rng, 12), 2, 4, 128, 16)
    c.tables[:, :6] = c.prefix_table            # the tables name the shared blocks themselves
    c.d_tables = dev(c.tables)
    say(f"cache policy dt={dt}")
    a, scale = _ex(c, False)
    b, _ = _ex(c, True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    want = attention.paged_decode(c.q, c.img, 1, c.tables, c.ctx, scale, c.ks, c.vs)
    mx, rel = errors(b, want)
    say(f"  cached: max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= _bar(dt)[0] and rel <= _bar(dt)[1]


@pytest.mark.parametrize("dt", [pkv.PKV_KV_BF16, pkv.PKV_KV_INT8])
def test_cache_policy_in_the_appending_and_shared_prefix_forms(dt):
    import torch
    rng = np.random.default_rng(15100 + dt)
    c = _case(rng, dt, 6, [96 + int(x) for x in rng.integers(1, 200, size=10)], 2, 4, 128, 16, spare=12)
    c.tables[:, :6] = c.prefix_table
    c.d_tables = dev(c.tables)
    # the appending form, each new token at ctx - 1 (a slot the case wrote)
    kn = bf16_dev(workloads.to_bf16_bits(rng.standard_normal((10, 2, 128), dtype=np.float32)))
    vn = bf16_dev(workloads.to_bf16_bits(rng.standard_normal((10, 2, 128), dtype=np.float32)))
    before = c.pool.memory.clone()
    a, _ = _ex(c, False, kn, vn)
    pool_a = c.pool.memory.clone()
    c.pool.memory.copy_(before)
    b, _ = _ex(c, True, kn, vn)
    assert torch.equal(pool_a, c.pool.memory)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # the shared-prefix form
    S, D = len(c.ctx), 128
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    ws = torch.empty(pkv.paged_attn_shared_prefix_workspace_bytes(S, c.hq, 2, D, c.width, 16, dt, c.P),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for keep in (False, True):
        out = torch.full((S, c.hq, D), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attn_decode_shared_prefix(out, c.d_q, c.pool, 1, c.d_tables, c.d_ctx, scale, c.d_prefix, c.P,
                                            dt, c.ks, c.vs, workspace=ws, keep_kv_cached=keep)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
