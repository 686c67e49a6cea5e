"""Pins of the oracle's INT8 storage with per-tensor and per-channel scales
(bjdmk.com.cn article, §5.2: one scale for the whole cache, or one per
channel; "KV Cache 原理与 PagedAttention", §四: INT8 per-tensor/per-channel),
and with K and V at different granularities (same article, §5.2: K, the
more sensitive, per channel; V coarser, one scale per tensor).

code = clamp(rint_even(fp32(x / s)), -127, 127), 0 where s == 0, with s the
caller's calibrated scale (per tensor: one for K, one for V; per channel: one
per (layer, KV head, dim), kept in the pool).  Pinned by a brute-force search
over all 255 codes, the half-way ties, saturation, the error bound s / 2,
per-channel with equal scales giving the per-tensor codes, and the cache
write followed by element-wise and tile gathers reading code * scale with
the right (head, dim) scale.  The mixed granularity is pinned to the two
uniform ones: with all its K channel scales equal it is INT8 per tensor, and
INT8 per channel with all V channel scales equal to its V scale is it, codes
and decode outputs alike; a one-token context returns that token's V code
times the V scale exactly.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import attention, cache_ops, codecs, layout
from tests.helpers import expanded_slots, random_tables


def _brute(x, s):
    """Nearest code to fp32(x / s) by exact search over -127..127 (ties to
    the even code)."""
    if s == 0:
        return 0
    y = Fraction(float(np.float32(np.float32(x) / np.float32(s))))
    dist = [(abs(Fraction(c) - y), c % 2, c) for c in range(-127, 128)]
    return min(dist)[2]


def test_encode_matches_brute_force_search():
    rng = np.random.default_rng(11000)
    for s in (np.float32(0.013), np.float32(1.0), np.float32(0.5), np.float32(3.75)):
        x = np.concatenate([rng.standard_normal(400).astype(np.float32) * s * 60,
                            (np.arange(-130, 131) + np.float32(0.5)).astype(np.float32) * s,   # ties
                            np.array([0.0, -0.0, 1e30, -1e30], np.float32) * s])
        codes = codecs.int8_encode(x, s)
        want = np.array([_brute(v, s) for v in x])
        assert np.array_equal(codes.astype(np.int64), want), s


def test_zero_scale_gives_zero_codes_and_bound_holds():
    x = np.linspace(-5, 5, 101, dtype=np.float32)
    assert not codecs.int8_encode(x, 0.0).any()
    s = np.float32(0.04)
    inside = x[np.abs(x) <= 127 * s]
    err = np.abs(codecs.int8_encode(inside, s).astype(np.float64) * np.float64(s) - inside.astype(np.float64))
    # half a step, plus the rounding of the fp32 division (|x / s| <= 127)
    assert np.all(err <= np.float64(s) / 2 + 127 * np.float64(s) * 2.0 ** -23)


def test_channel_scales_that_are_all_equal_give_the_tensor_codes():
    rng = np.random.default_rng(11100)
    x = rng.standard_normal((9, 2, 32)).astype(np.float32) * 3
    s = np.full((2, 32), 0.07, np.float32)
    assert np.array_equal(codecs.int8_encode(x, s[None]), codecs.int8_encode(x, np.float32(0.07)))


def _write_and_read(dt, rng, B=8, H=2, D=32, L=2, layer=1):
    ctx = np.array([3, 17, 26], np.int32)
    nb = sum(math.ceil(int(c) / B) for c in ctx) + 2
    p = layout.PoolShape(L, nb, B, H, D, dt)
    img = layout.empty_image(p)
    ch_k = rng.uniform(0.005, 0.05, size=(L, H, D)).astype(np.float32)
    ch_v = rng.uniform(0.005, 0.05, size=(L, H, D)).astype(np.float32)
    if p.has_k_channel_scales:
        img.k_scale[:] = ch_k.reshape(-1)
    if p.has_channel_scales:
        img.v_scale[:] = ch_v.reshape(-1)
    bt = random_tables(rng, nb, ctx, B)
    toks = [(workloads.to_bf16_bits(rng.standard_normal((int(c), H, D), dtype=np.float32)),
             workloads.to_bf16_bits(rng.standard_normal((int(c), H, D), dtype=np.float32))) for c in ctx]
    slots = np.concatenate([expanded_slots(bt[s], int(ctx[s]), B) for s in range(3)])
    kx = np.concatenate([t[0] for t in toks])
    vx = np.concatenate([t[1] for t in toks])
    img = cache_ops.reshape_and_cache(img, layer, kx, vx, slots, 0.021, 0.034)
    return p, img, bt, ctx, toks, ch_k[layer], ch_v[layer]


@pytest.mark.parametrize("dt", [layout.KV_INT8_TENSOR, layout.KV_INT8_CHANNEL, layout.KV_INT8_KCHANNEL_VTENSOR])
def test_cache_write_then_gathers_read_code_times_scale(dt):
    rng = np.random.default_rng(11200 + dt)
    p, img, bt, ctx, toks, ck, cv = _write_and_read(dt, rng)
    for s in range(3):
        n = int(ctx[s])
        k, v = attention.gather_kv_by_slot(img, 1, bt[s], n, 0.021, 0.034)
        kt, vt = attention.gather_kv(img, 1, bt[s], n, 0.021, 0.034)
        assert np.array_equal(k, kt) and np.array_equal(v, vt)
        xk = codecs.bf16_bits_to_f32(toks[s][0])
        xv = codecs.bf16_bits_to_f32(toks[s][1])
        sk = np.float32(0.021) if dt == layout.KV_INT8_TENSOR else ck[None]
        sv = cv[None] if dt == layout.KV_INT8_CHANNEL else np.float32(0.034)
        # exactly code * scale, with the code of the written input
        codes_k = codecs.int8_encode(xk, sk)
        assert np.array_equal(k, codes_k.astype(np.float64) * np.broadcast_to(sk, k.shape).astype(np.float64))
        codes_v = codecs.int8_encode(xv, sv)
        assert np.array_equal(v, codes_v.astype(np.float64) * np.broadcast_to(sv, v.shape).astype(np.float64))


def test_channel_scales_are_layer_constants_kept_by_block_copies():
    rng = np.random.default_rng(11300)
    p, img, bt, ctx, toks, ck, cv = _write_and_read(layout.KV_INT8_CHANNEL, rng)
    out = cache_ops.copy_blocks(img, np.array([[bt[0, 0], p.num_blocks - 1]]))
    assert np.array_equal(out.k_scale, img.k_scale) and np.array_equal(out.v_scale, img.v_scale)
    other = layout.empty_image(p)
    other.k_scale[:] = img.k_scale
    other.v_scale[:] = img.v_scale
    sw = cache_ops.swap_blocks(img, other, np.array([[bt[1, 0], 0]]))
    assert np.array_equal(sw.k_scale, img.k_scale)


def test_channel_byte_layout_round_trips():
    rng = np.random.default_rng(11400)
    p, img, *_ = _write_and_read(layout.KV_INT8_CHANNEL, rng)
    back = layout.image_from_bytes(p, layout.image_to_bytes(img))
    assert np.array_equal(back.k_scale, img.k_scale) and np.array_equal(back.k, img.k)
    k_off, v_off, ks_off, vs_off, total = layout.region_offsets(p)
    assert ks_off % 256 == 0 and vs_off - ks_off >= p.num_layers * p.num_kv_heads * p.head_dim * 4


# ------------------------------------------------ K per channel, V per tensor
def _mixed_case(rng, H=2, D=32, B=8, L=2, layer=1):
    ctx = np.array([1, 9, 30], np.int32)
    nb = sum(math.ceil(int(c) / B) for c in ctx) + 1
    bt = random_tables(rng, nb, ctx, B)
    slots = np.concatenate([expanded_slots(bt[s], int(ctx[s]), B) for s in range(len(ctx))])
    n = int(ctx.sum())
    kx = workloads.to_bf16_bits(rng.standard_normal((n, H, D), dtype=np.float32) * 2)
    vx = workloads.to_bf16_bits(rng.standard_normal((n, H, D), dtype=np.float32) * 2)
    q = workloads.to_bf16_bits(rng.standard_normal((len(ctx), 3 * H, D), dtype=np.float32))
    return (L, nb, B, H, D), layer, bt, ctx, slots, kx, vx, q


def test_mixed_region_layout_has_k_channel_scales_only():
    p = layout.PoolShape(3, 5, 16, 2, 64, layout.KV_INT8_KCHANNEL_VTENSOR)
    k_off, v_off, ks_off, vs_off, total = layout.region_offsets(p)
    assert vs_off is None and ks_off % 256 == 0
    assert total == ks_off + -(-(3 * 2 * 64 * 4) // 256) * 256
    img = layout.empty_image(p)
    assert img.v_scale is None and img.k_scale.size == 3 * 2 * 64
    img.k_scale[:] = np.arange(img.k_scale.size, dtype=np.float32)
    back = layout.image_from_bytes(p, layout.image_to_bytes(img))
    assert back.v_scale is None and np.array_equal(back.k_scale, img.k_scale)


def test_mixed_with_equal_k_channel_scales_is_int8_per_tensor():
    rng = np.random.default_rng(11500)
    shp, layer, bt, ctx, slots, kx, vx, q = _mixed_case(rng)
    mixed = layout.empty_image(layout.PoolShape(*shp, layout.KV_INT8_KCHANNEL_VTENSOR))
    mixed.k_scale[:] = np.float32(0.03)
    tensor = layout.empty_image(layout.PoolShape(*shp, layout.KV_INT8_TENSOR))
    mixed = cache_ops.reshape_and_cache(mixed, layer, kx, vx, slots, 0.5, 0.027)   # its K scale is the pool's
    tensor = cache_ops.reshape_and_cache(tensor, layer, kx, vx, slots, 0.03, 0.027)
    assert np.array_equal(mixed.k, tensor.k) and np.array_equal(mixed.v, tensor.v)
    a = attention.paged_decode(q, mixed, layer, bt, ctx, 0.125, 0.5, 0.027)
    b = attention.paged_decode(q, tensor, layer, bt, ctx, 0.125, 0.03, 0.027)
    assert np.array_equal(a, b)


def test_int8_per_channel_with_equal_v_scales_is_the_mixed_granularity():
    rng = np.random.default_rng(11600)
    shp, layer, bt, ctx, slots, kx, vx, q = _mixed_case(rng)
    L, nb, B, H, D = shp
    ck = rng.uniform(0.01, 0.06, size=L * H * D).astype(np.float32)
    mixed = layout.empty_image(layout.PoolShape(*shp, layout.KV_INT8_KCHANNEL_VTENSOR))
    mixed.k_scale[:] = ck
    chan = layout.empty_image(layout.PoolShape(*shp, layout.KV_INT8_CHANNEL))
    chan.k_scale[:] = ck
    chan.v_scale[:] = np.float32(0.041)
    mixed = cache_ops.reshape_and_cache(mixed, layer, kx, vx, slots, 1.0, 0.041)
    chan = cache_ops.reshape_and_cache(chan, layer, kx, vx, slots)
    assert np.array_equal(mixed.k, chan.k) and np.array_equal(mixed.v, chan.v)
    a = attention.paged_decode(q, mixed, layer, bt, ctx, 0.125, 1.0, 0.041)
    b = attention.paged_decode(q, chan, layer, bt, ctx, 0.125)
    assert np.array_equal(a, b)
    # the K codes follow the channel scales, the V codes the one V scale:
    # another V scale changes V codes only
    other = layout.empty_image(layout.PoolShape(*shp, layout.KV_INT8_KCHANNEL_VTENSOR))
    other.k_scale[:] = ck
    other = cache_ops.reshape_and_cache(other, layer, kx, vx, slots, 1.0, 0.02)
    assert np.array_equal(other.k, mixed.k) and not np.array_equal(other.v, mixed.v)


def test_mixed_one_token_context_returns_v_code_times_v_scale():
    rng = np.random.default_rng(11700)
    shp, layer, bt, ctx, slots, kx, vx, q = _mixed_case(rng)
    L, nb, B, H, D = shp
    img = layout.empty_image(layout.PoolShape(*shp, layout.KV_INT8_KCHANNEL_VTENSOR))
    img.k_scale[:] = rng.uniform(0.01, 0.06, size=L * H * D).astype(np.float32)
    img = cache_ops.reshape_and_cache(img, layer, kx, vx, slots, 1.0, 0.037)
    out = attention.paged_decode(q, img, layer, bt, ctx, 0.125, 1.0, 0.037)
    # sequence 0 has one token (the first written): softmax over one key is 1
    v0 = codecs.int8_encode(codecs.bf16_bits_to_f32(vx[0]), np.float32(0.037)).astype(np.float64)
    want = v0 * np.float64(np.float32(0.037))                     # [H, D]
    group = q.shape[1] // H
    assert np.array_equal(out[0], np.repeat(want, group, axis=0))
