"""Pins of the oracle's INT8 storage with per-tensor and per-channel scales
(bjdmk.com.cn article, §5.2: one scale for the whole cache, or one per
channel; "KV Cache 原理与 PagedAttention", §四: INT8 per-tensor/per-channel).

code = clamp(rint_even(fp32(x / s)), -127, 127), 0 where s == 0, with s the
caller's calibrated scale (per tensor: one for K, one for V; per channel: one
per (layer, KV head, dim), kept in the pool).  Pinned by a brute-force search
over all 255 codes, the half-way ties, saturation, the error bound s / 2,
per-channel with equal scales giving the per-tensor codes, and the cache
write followed by element-wise and tile gathers reading code * scale with
the right (head, dim) scale.
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
    if p.has_channel_scales:
        img.k_scale[:] = ch_k.reshape(-1)
        img.v_scale[:] = ch_v.reshape(-1)
    bt = random_tables(rng, nb, ctx, B)
    toks = [(workloads.to_bf16_bits(rng.standard_normal((int(c), H, D), dtype=np.float32)),
             workloads.to_bf16_bits(rng.standard_normal((int(c), H, D), dtype=np.float32))) for c in ctx]
    slots = np.concatenate([expanded_slots(bt[s], int(ctx[s]), B) for s in range(3)])
    kx = np.concatenate([t[0] for t in toks])
    vx = np.concatenate([t[1] for t in toks])
    img = cache_ops.reshape_and_cache(img, layer, kx, vx, slots, 0.021, 0.034)
    return p, img, bt, ctx, toks, ch_k[layer], ch_v[layer]


@pytest.mark.parametrize("dt", [layout.KV_INT8_TENSOR, layout.KV_INT8_CHANNEL])
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
        sv = np.float32(0.034) if dt == layout.KV_INT8_TENSOR else cv[None]
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
