"""INT8 storage with per-tensor and per-channel scales, and with K per
channel and V per tensor, on the GPU, against the oracle: the cache write
bit for bit (codes; channel scales untouched), decode in both forms and the
appending form (same bits as the two calls).
"""

import math

import numpy as np
import pytest

import paged_kv_cache_436_amd as pkv
import workloads
from oracle import attention, cache_ops
from tests.gpu_helpers import bf16_dev, dev, errors, first_diff, images_equal, read_pool, say
from tests.helpers import expanded_slots

pytestmark = pytest.mark.gpu

KS, VS = 0.035, 0.03            # per-tensor scales (|x| up to ~4.4 and ~3.8 before saturation)
BAR = (2e-2, 1e-3)     # the split form meets the codes with p as one fp16 (rounding <= 2^-11 relative)


class Case:
    pass


def _case(rng, dt, ctx, hkv=2, G=4, D=128, B=16, spare=3):
    import torch
    c = Case()
    c.ctx = np.asarray(ctx, np.int32)
    need = [math.ceil(int(x) / B) for x in ctx]
    nb = sum(need) + spare
    c.width = max(1, max(need))
    perm = rng.permutation(nb)
    c.tables = np.zeros((len(ctx), c.width), np.int32)
    pos = 0
    for s, n in enumerate(need):
        c.tables[s, :n] = perm[pos:pos + n]
        pos += n
    c.cfg = pkv.make_config(2, nb, B, hkv, D, dt)
    c.pool = pkv.Pool(c.cfg)
    c.pool.memory.fill_(255)                      # unwritten codes: -1
    _, _, ks, vs = c.pool.region_offsets()
    n = 2 * hkv * D                                # calibrated channel scales, both layers
    if ks is not None:
        c.ch_k = rng.uniform(0.02, 0.05, n).astype(np.float32)
        c.pool.memory[ks:ks + 4 * n].view(torch.float32).copy_(torch.from_numpy(c.ch_k))
    if vs is not None:                             # (none when V has one scale per tensor)
        c.ch_v = rng.uniform(0.02, 0.05, n).astype(np.float32)
        c.pool.memory[vs:vs + 4 * n].view(torch.float32).copy_(torch.from_numpy(c.ch_v))
    c.hq = hkv * G
    c.q = workloads.to_bf16_bits(rng.standard_normal((len(ctx), c.hq, D), dtype=np.float32))
    total = int(c.ctx.sum())
    c.k = workloads.to_bf16_bits(rng.standard_normal((total, hkv, D), dtype=np.float32))
    c.v = workloads.to_bf16_bits(rng.standard_normal((total, hkv, D), dtype=np.float32))
    c.slots = np.concatenate([expanded_slots(c.tables[s], int(c.ctx[s]), B) for s in range(len(ctx))])
    img0 = read_pool(c.pool)
    pkv.reshape_and_cache(c.pool, 1, bf16_dev(c.k), bf16_dev(c.v), dev(c.slots.astype(np.int64)),
                          k_scale=KS, v_scale=VS)
    c.img = cache_ops.reshape_and_cache(img0, 1, c.k, c.v, c.slots, KS, VS)
    c.d_tables, c.d_ctx, c.d_q = dev(c.tables), dev(c.ctx), bf16_dev(c.q)
    return c


def _decode(c, P, window=0, key=None, value=None):
    import torch
    D = c.cfg.head_dim
    S = len(c.ctx)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    out = torch.full((S, c.hq, D), float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    if P:
        ws = torch.empty(pkv.paged_attn_workspace_bytes(S, c.hq, D, c.width, c.cfg.block_size, P),
                         dtype=torch.uint8, device="cuda")
    pkv.paged_attn_decode_ex(out, c.d_q, c.pool, 1, c.d_tables, c.d_ctx, scale, c.cfg.kv_dtype, KS, VS, P, ws,
                             key=key, value=value, sliding_window=window)
    torch.cuda.synchronize()
    return out.cpu().numpy(), scale


@pytest.mark.parametrize("dt", [pkv.PKV_KV_INT8_TENSOR, pkv.PKV_KV_INT8_CHANNEL, pkv.PKV_KV_INT8_KCHANNEL_VTENSOR])
@pytest.mark.parametrize("D,B", [(128, 16), (64, 32)])
def test_cache_write_is_bit_exact(dt, D, B):
    rng = np.random.default_rng(12000 + dt + D + B)
    c = _case(rng, dt, [1, 7, 40, 65], D=D, B=B)
    got = read_pool(c.pool)
    assert images_equal(got, c.img), first_diff(got, c.img)


@pytest.mark.parametrize("dt", [pkv.PKV_KV_INT8_TENSOR, pkv.PKV_KV_INT8_CHANNEL, pkv.PKV_KV_INT8_KCHANNEL_VTENSOR])
@pytest.mark.parametrize("D,B", [(128, 16), (64, 32), (128, 32), (128, 8)])
@pytest.mark.parametrize("P", [0, 32, 512])
def test_decode_matches_oracle(dt, D, B, P):
    say(f"int8 scales dt={dt} D={D} B={B} P={P}")
    rng = np.random.default_rng(12100 + dt + D + B + P)
    hkv, G = (2, 4) if D == 128 else (1, 3)
    c = _case(rng, dt, [1, 15, 16, 17, 100, 0, 333, 700], hkv=hkv, G=G, D=D, B=B)
    got, scale = _decode(c, P)
    want = attention.paged_decode(c.q, c.img, 1, c.tables, c.ctx, scale, KS, VS)
    assert np.all(np.isfinite(got))
    mx, rel = errors(got, want)
    say(f"  max_abs={mx:.3e} rel={rel:.3e}")
    assert mx <= BAR[0] and rel <= BAR[1]
    assert not got[c.ctx == 0].any()
    if P:   # with a window too
        got_w, _ = _decode(c, P, window=40)
        want_w = attention.paged_decode(c.q, c.img, 1, c.tables, c.ctx, scale, KS, VS, window=40)
        mx, rel = errors(got_w, want_w)
        assert mx <= BAR[0] and rel <= BAR[1]


@pytest.mark.parametrize("dt", [pkv.PKV_KV_INT8_TENSOR, pkv.PKV_KV_INT8_CHANNEL, pkv.PKV_KV_INT8_KCHANNEL_VTENSOR])
def test_appending_decode_equals_two_calls(dt):
    import torch
    rng = np.random.default_rng(12200 + dt)
    ctx = [1, 16, 17, 50, 300]
    B, D, hkv = 16, 128, 2
    hist = [x - 1 for x in ctx]
    c = _case(rng, dt, hist, spare=len(ctx) + 2)
    c.width = math.ceil(max(ctx) / B)
    t = np.zeros((len(ctx), c.width), np.int32)
    t[:, :c.tables.shape[1]] = c.tables
    used = set(int(b) for s in range(len(ctx)) for b in t[s, :math.ceil(hist[s] / B)])
    free = [b for b in range(c.cfg.num_blocks) if b not in used]
    for s in range(len(ctx)):
        for i in range(math.ceil(hist[s] / B), math.ceil(ctx[s] / B)):
            t[s, i] = free.pop()
    c.tables, c.ctx = t, np.asarray(ctx, np.int32)
    c.d_tables, c.d_ctx = dev(c.tables), dev(c.ctx)
    kn = workloads.to_bf16_bits(rng.standard_normal((len(ctx), hkv, D), dtype=np.float32))
    vn = workloads.to_bf16_bits(rng.standard_normal((len(ctx), hkv, D), dtype=np.float32))
    slots = np.array([attention.slot_of(c.tables[s], ctx[s] - 1, B) for s in range(len(ctx))], np.int64)
    before = c.pool.memory.clone()
    pkv.reshape_and_cache(c.pool, 1, bf16_dev(kn), bf16_dev(vn), dev(slots), k_scale=KS, v_scale=VS)
    got_a, scale = _decode(c, 64)
    pool_a = c.pool.memory.clone()
    c.pool.memory.copy_(before)
    got_b, _ = _decode(c, 64, key=bf16_dev(kn), value=bf16_dev(vn))
    assert torch.equal(pool_a, c.pool.memory)
    assert np.array_equal(got_a.view(np.uint32), got_b.view(np.uint32))
    img = cache_ops.reshape_and_cache(c.img, 1, kn, vn, slots, KS, VS)
    want = attention.paged_decode(c.q, img, 1, c.tables, c.ctx, scale, KS, VS)
    mx, rel = errors(got_b, want)
    assert mx <= BAR[0] and rel <= BAR[1]
