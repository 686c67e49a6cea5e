"""Shared-prefix decode on the GPU (paged_attn_decode_shared_prefix) against
the oracle's paged_decode_shared_prefix.

Every sequence's own table row points its first prefix_len / B entries at a
block of 0xFF bytes (NaN bf16 / NaN e5m2 / -1 codes with NaN scales) that
is never written: a read of the own row below the prefix would reach the
output.  Contexts cover the empty sequence, contexts that end inside the
prefix or exactly at its end, and ones running past it; sizes cover several
column groups per KV head in the prefix pass and prefixes split over its
waves, every storage type, block sizes 8 / 16 / 32, head dims 64 / 128 and
GQA groups of 1, 3 and 4 heads.
"""

import math

import numpy as np
import pytest

import paged_kv_cache_436_amd as pkv
import workloads
from oracle import attention, cache_ops
from tests.gpu_helpers import bf16_dev, dev, errors, read_pool, say
from tests.helpers import expanded_slots

pytestmark = pytest.mark.gpu

SCALES = {pkv.PKV_KV_FP8_E5M2: (0.75, 1.25), pkv.PKV_KV_INT8_TENSOR: (0.035, 0.03),
          pkv.PKV_KV_INT8_KCHANNEL_VTENSOR: (1.0, 0.03)}
ALL = [pkv.PKV_KV_BF16, pkv.PKV_KV_FP8_E5M2, pkv.PKV_KV_INT8, pkv.PKV_KV_INT8_TENSOR, pkv.PKV_KV_INT8_CHANNEL,
       pkv.PKV_KV_INT4, pkv.PKV_KV_INT8_KCHANNEL_VTENSOR]


def _bar(dt):
    return (1e-2, 1e-3) if dt == pkv.PKV_KV_BF16 else (2e-2, 5e-3)


class Case:
    pass


def _case(rng, dt, prefix_blocks, ctx, hkv, G, D, B, width_extra=0, spare=1):
    """Pool (layer 1 of 2) with one shared prefix and per-sequence suffixes;
    K/V written through the library's cache write and the oracle's."""
    import torch
    c = Case()
    P = prefix_blocks * B
    c.P = P
    c.ctx = np.asarray(ctx, np.int32)
    S = len(ctx)
    own = [max(0, math.ceil(int(x) / B) - prefix_blocks) for x in c.ctx]
    c.width = max(prefix_blocks, max(prefix_blocks + n for n in own)) + width_extra
    nb = prefix_blocks + sum(own) + 1 + spare
    perm = rng.permutation(nb)
    c.prefix_table = perm[:prefix_blocks].astype(np.int32)
    poison = int(perm[prefix_blocks])                       # never written: 0xFF bytes
    c.tables = np.zeros((S, c.width), np.int32)
    pos = prefix_blocks + 1
    for s in range(S):
        c.tables[s, :prefix_blocks] = poison
        c.tables[s, prefix_blocks:prefix_blocks + own[s]] = perm[pos:pos + own[s]]
        c.tables[s, prefix_blocks + own[s]:] = rng.integers(0, 2**31 - 1, size=c.width - prefix_blocks - own[s])
        pos += own[s]
    c.cfg = pkv.make_config(2, nb, B, hkv, D, dt)
    c.pool = pkv.Pool(c.cfg)
    c.pool.memory.fill_(255)
    _, _, ks_off, vs_off = c.pool.region_offsets()
    n = 2 * hkv * D
    if dt in (pkv.PKV_KV_INT8_CHANNEL, pkv.PKV_KV_INT4, pkv.PKV_KV_INT8_KCHANNEL_VTENSOR):
        lo, hi = (0.25, 0.6) if dt == pkv.PKV_KV_INT4 else (0.02, 0.05)
        if ks_off is not None:
            c.pool.memory[ks_off:ks_off + 4 * n].view(torch.float32).copy_(
                torch.from_numpy(rng.uniform(lo, hi, n).astype(np.float32)))
        if vs_off is not None:
            c.pool.memory[vs_off:vs_off + 4 * n].view(torch.float32).copy_(
                torch.from_numpy(rng.uniform(lo, hi, n).astype(np.float32)))
    c.ks, c.vs = SCALES.get(dt, (1.0, 1.0))
    c.hq = hkv * G
    c.q = workloads.to_bf16_bits(rng.standard_normal((S, c.hq, D), dtype=np.float32))
    # the prefix's tokens, then each sequence's own tokens [P, ctx)
    pk = workloads.to_bf16_bits(rng.standard_normal((P, hkv, D), dtype=np.float32))
    pv = workloads.to_bf16_bits(rng.standard_normal((P, hkv, D), dtype=np.float32))
    keys, vals, slots = [pk], [pv], [expanded_slots(c.prefix_table, P, B)]
    for s in range(S):
        m = max(0, int(c.ctx[s]) - P)
        if m:
            keys.append(workloads.to_bf16_bits(rng.standard_normal((m, hkv, D), dtype=np.float32)))
            vals.append(workloads.to_bf16_bits(rng.standard_normal((m, hkv, D), dtype=np.float32)))
            slots.append(expanded_slots(c.tables[s], int(c.ctx[s]), B)[P:])
    k, v, sl = np.concatenate(keys), np.concatenate(vals), np.concatenate(slots).astype(np.int64)
    img0 = read_pool(c.pool)
    pkv.reshape_and_cache(c.pool, 1, bf16_dev(k), bf16_dev(v), dev(sl), k_scale=c.ks, v_scale=c.vs)
    c.img = cache_ops.reshape_and_cache(img0, 1, k, v, sl, c.ks, c.vs)
    c.d_tables, c.d_ctx, c.d_q = dev(c.tables), dev(c.ctx), bf16_dev(c.q)
    c.d_prefix = dev(c.prefix_table)
    torch.cuda.synchronize()
    return c


def _run(c, key=None, value=None, P_part=512, prefix_len=None, ws=None):
    import torch
    D = c.cfg.head_dim
    S = len(c.ctx)
    pl = c.P if prefix_len is None else prefix_len
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    out = torch.full((S, c.hq, D), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = pkv.paged_attn_shared_prefix_workspace_bytes(S, c.hq, c.cfg.num_kv_heads, D, c.width,
                                                           c.cfg.block_size, c.cfg.kv_dtype, pl)
    assert nbytes > 0
    if ws is None:
        ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")   # scratch: any contents
    pkv.paged_attn_decode_shared_prefix(out, c.d_q, c.pool, 1, c.d_tables, c.d_ctx, scale, c.d_prefix, pl,
                                        c.cfg.kv_dtype, c.ks, c.vs, P_part, ws, key=key, value=value)
    torch.cuda.synchronize()
    return out.cpu().numpy(), scale


def _want(c, scale, img=None):
    return attention.paged_decode_shared_prefix(c.q, c.img if img is None else img, 1, c.tables, c.ctx,
                                                c.prefix_table, c.P, scale, c.ks, c.vs)


def _ctx_mix(P, rng, S):
    base = [0, 3, P - 1, P, P + 1, P + 17, P + 100, P + 600, P + 33, P + 250, 1]
    more = list(P + rng.integers(1, 400, size=max(0, S - len(base))))
    return (base + more)[:S]


@pytest.mark.parametrize("dt", ALL)
@pytest.mark.parametrize("D,B,hkv,G", [(128, 16, 2, 4), (64, 32, 2, 3), (128, 8, 3, 1)])
def test_shared_prefix_matches_oracle(dt, D, B, hkv, G):
    rng = np.random.default_rng(14000 + 11 * dt + D + B + G)
    blocks = {8: 25, 16: 13, 32: 7}[B]
    c = _case(rng, dt, blocks, _ctx_mix(blocks * B, rng, 14), hkv, G, D, B)
    say(f"shared prefix dt={dt} D={D} B={B} hkv={hkv} G={G} P={c.P}")
    got, scale = _run(c)
    want = _want(c, scale)
    assert np.all(np.isfinite(got)), "non-finite output: a block below the prefix was read through an own table?"
    mx, rel = errors(got, want)
    say(f"  max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= _bar(dt)[0] and rel <= _bar(dt)[1]
    assert not got[c.ctx == 0].any()


@pytest.mark.parametrize("hkv,G", [(2, 8), (1, 20)])
@pytest.mark.parametrize("dt", [pkv.PKV_KV_BF16, pkv.PKV_KV_INT8])
def test_wide_query_groups(dt, hkv, G):
    """Query groups of 8 (the 70B shape) and 20 (more than one 16-head tile
    per KV head in the split pass; columns of one sequence spread over two
    tiles in the prefix pass)."""
    rng = np.random.default_rng(14400 + 3 * dt + G)
    c = _case(rng, dt, 10, _ctx_mix(160, rng, 12), hkv, G, 128, 16)
    say(f"shared prefix wide groups dt={dt} hkv={hkv} G={G}")
    got, scale = _run(c)
    want = _want(c, scale)
    assert np.all(np.isfinite(got))
    mx, rel = errors(got, want)
    say(f"  max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= _bar(dt)[0] and rel <= _bar(dt)[1]


@pytest.mark.parametrize("dt", [pkv.PKV_KV_BF16, pkv.PKV_KV_FP8_E5M2, pkv.PKV_KV_INT4])
def test_many_sequences_span_several_column_groups(dt):
    """200 sequences with one query head per KV head (the shared-prompt
    batch's shape, fewer heads): the prefix pass takes several column groups
    per KV head, each splitting the 1488-position prefix over its waves."""
    rng = np.random.default_rng(14500 + dt)
    B = 16
    ctx = [1488 + int(x) for x in rng.integers(1, 96, size=200)]
    ctx[7] = 1488
    ctx[11] = 700
    c = _case(rng, dt, 93, ctx, 4, 1, 128, B)
    say(f"shared prefix 200 seqs dt={dt}")
    got, scale = _run(c)
    want = _want(c, scale)
    mx, rel = errors(got, want)
    say(f"  max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= _bar(dt)[0] and rel <= _bar(dt)[1]


@pytest.mark.parametrize("dt", [pkv.PKV_KV_BF16, pkv.PKV_KV_INT8, pkv.PKV_KV_INT4])
def test_appending_form_equals_cache_write_then_decode(dt):
    """The appending form writes each sequence's new token at ctx - 1 (past
    the prefix) and attends it: the same pool bytes and output bits as
    reshape_and_cache followed by the shared-prefix decode."""
    import torch
    rng = np.random.default_rng(14600 + dt)
    B, D, hkv, G = 16, 128, 2, 4
    blocks = 9
    P = blocks * B
    ctx = [P + 1, P + 2, P + 16, P + 17, P + 300, P + 33]
    c = _case(rng, dt, blocks, [x - 1 for x in ctx], hkv, G, D, B, width_extra=2, spare=4)
    # blocks for the new tokens that open one
    used = set(c.prefix_table.tolist()) | set(int(b) for s in range(len(ctx))
                                              for b in c.tables[s, :math.ceil((ctx[s] - 1) / B)])
    spare = [b for b in range(c.cfg.num_blocks) if b not in used]
    need = [s for s in range(len(ctx)) if (ctx[s] - 1) % B == 0]
    assert len(need) <= len(spare)
    for s in need:
        c.tables[s, (ctx[s] - 1) // B] = spare.pop()
    c.ctx = np.asarray(ctx, np.int32)
    c.d_ctx, c.d_tables = dev(c.ctx), dev(c.tables)
    kn = workloads.to_bf16_bits(rng.standard_normal((len(ctx), hkv, D), dtype=np.float32))
    vn = workloads.to_bf16_bits(rng.standard_normal((len(ctx), hkv, D), dtype=np.float32))
    slots = np.array([attention.slot_of(c.tables[s], ctx[s] - 1, B) for s in range(len(ctx))], np.int64)
    before = c.pool.memory.clone()
    pkv.reshape_and_cache(c.pool, 1, bf16_dev(kn), bf16_dev(vn), dev(slots), k_scale=c.ks, v_scale=c.vs)
    got_a, scale = _run(c)
    pool_a = c.pool.memory.clone()
    c.pool.memory.copy_(before)
    got_b, _ = _run(c, key=bf16_dev(kn), value=bf16_dev(vn))
    assert torch.equal(pool_a, c.pool.memory)
    assert np.array_equal(got_a.view(np.uint32), got_b.view(np.uint32))
    img = cache_ops.reshape_and_cache(c.img, 1, kn, vn, slots, c.ks, c.vs)
    mx, rel = errors(got_b, _want(c, scale, img))
    say(f"shared prefix append dt={dt}: max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= _bar(dt)[0] and rel <= _bar(dt)[1]


def test_empty_prefix_is_the_plain_decode():
    import torch
    rng = np.random.default_rng(14700)
    c = _case(rng, pkv.PKV_KV_BF16, 2, [40, 77, 5, 0, 130], 2, 4, 128, 16)
    # own rows that name real blocks below the "prefix": the plain decode reads them
    c.tables[:, :2] = c.prefix_table
    c.d_tables = dev(c.tables)
    got, scale = _run(c, prefix_len=0)
    ws = torch.empty(pkv.paged_attn_workspace_bytes(5, c.hq, 128, c.width, 16, 512), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((5, c.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode_ex(out, c.d_q, c.pool, 1, c.d_tables, c.d_ctx, scale, pkv.PKV_KV_BF16, 1.0, 1.0, 512, ws)
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), out.cpu().numpy().view(np.uint32))


def test_shared_prefix_repeats_bit_for_bit():
    """Two calls on one workspace (epoch-tagged counters left by the first)
    give the same bits."""
    import torch
    rng = np.random.default_rng(14800)
    c = _case(rng, pkv.PKV_KV_BF16, 20, _ctx_mix(320, rng, 40), 2, 2, 128, 16)
    ws = torch.randint(0, 256, (pkv.paged_attn_shared_prefix_workspace_bytes(40, 4, 2, 128, c.width, 16,
                                                                             pkv.PKV_KV_BF16, 320),),
                       dtype=torch.uint8, device="cuda")
    a, _ = _run(c, ws=ws)
    b, _ = _run(c, ws=ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_workspace_sized_for_a_batch_serves_every_smaller_batch():
    """The workspace for 200 sequences also serves a call over the first n
    of them."""
    import torch
    rng = np.random.default_rng(14900)
    ctx = [1488 + int(x) for x in rng.integers(1, 64, size=200)]
    c = _case(rng, pkv.PKV_KV_BF16, 93, ctx, 4, 1, 128, 16)
    nbytes = pkv.paged_attn_shared_prefix_workspace_bytes(200, 4, 4, 128, c.width, 16, pkv.PKV_KV_BF16, c.P)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    scale = float(np.float32(1.0) / np.sqrt(np.float32(128)))
    want = _want(c, scale)
    for n in (200, 191, 150, 97, 48, 1):
        assert pkv.paged_attn_shared_prefix_workspace_bytes(n, 4, 4, 128, c.width, 16, pkv.PKV_KV_BF16, c.P) <= nbytes
        out = torch.full((n, 4, 128), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_attn_decode_shared_prefix(out, c.d_q[:n], c.pool, 1, c.d_tables[:n], c.d_ctx[:n], scale,
                                            c.d_prefix, c.P, workspace=ws)
        torch.cuda.synchronize()
        mx, rel = errors(out.cpu().numpy(), want[:n])
        say(f"shared prefix n={n}: max_abs={mx:.3e} rel={rel:.3e}")
        assert mx <= 1e-2 and rel <= 1e-3, n
