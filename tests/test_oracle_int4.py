"""Pins of the oracle's INT4 storage ("KV Cache 原理与 PagedAttention", §四:
INT4 KV, more aggressive than INT8, needs calibration, a quarter of the
memory; bjdmk.com.cn article, §5.2: per-channel scales).

This library's reading: symmetric codes clamp(rint_even(fp32(x / s)), -7, 7)
under calibrated per-(layer, KV head, dim) scales s, two codes per byte,
stored as code + 8.  Pinned by a brute-force nearest-code search, the error
bound s / 2, saturation, the nibble index functions being a bijection onto
each tile, V bytes each holding a single token, the tile-wise unpack agreeing
with the element-wise index functions, and the cache write read back as code *
scale by both gathers.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import attention, cache_ops, codecs, layout
from tests.helpers import expanded_slots, random_tables


def _brute(x, s):
    """Nearest code in -7..7 to fp32(x / s) by exact search (ties to the
    even code)."""
    if s == 0:
        return 0
    y = Fraction(float(np.float32(np.float32(x) / np.float32(s))))
    return min((abs(Fraction(c) - y), c % 2, c) for c in range(-7, 8))[2]


def test_encode_matches_brute_force_search():
    rng = np.random.default_rng(12000)
    for s in (np.float32(0.013), np.float32(1.0), np.float32(0.37)):
        x = np.concatenate([rng.standard_normal(300).astype(np.float32) * s * 5,
                            (np.arange(-9, 9) + np.float32(0.5)).astype(np.float32) * s,   # ties
                            np.array([0.0, -0.0, 1e30, -1e30], np.float32) * s])
        codes = codecs.int4_encode(x, s)
        want = np.array([_brute(v, s) for v in x])
        assert np.array_equal(codes.astype(np.int64), want), s


def test_bound_saturation_and_zero_scale():
    s = np.float32(0.25)
    x = np.linspace(-3, 3, 241, dtype=np.float32)
    c = codecs.int4_encode(x, s).astype(np.int64)
    assert c.min() == -7 and c.max() == 7
    inside = np.abs(x) <= 7 * s
    err = np.abs(c[inside] * np.float64(s) - x[inside].astype(np.float64))
    assert np.all(err <= np.float64(s) / 2 + 7 * np.float64(s) * 2.0 ** -23)
    assert np.all(c[x > 7.5 * s] == 7) and np.all(c[x < -7.5 * s] == -7)
    assert not codecs.int4_encode(x, 0.0).any()


@pytest.mark.parametrize("B,D", [(8, 64), (16, 128), (32, 64)])
def test_nibble_functions_are_a_bijection_onto_each_tile(B, D):
    p = layout.PoolShape(2, 3, B, 2, D, layout.KV_INT4)
    t = np.arange(B)[:, None]
    d = np.arange(D)[None, :]
    for fn in (layout.int4_k_nibble, layout.int4_v_nibble):
        nib = fn(p, 1, 2, 1, t, d).ravel()
        base = 2 * int(layout.tile_base(p, 1, 2, 1))
        assert np.array_equal(np.sort(nib), np.arange(base, base + B * D)), fn.__name__
    assert p.tile_units * 2 == B * D and layout.region_offsets(p)[1] >= p.region_elems // 2


@pytest.mark.parametrize("B,D", [(8, 64), (16, 128)])
def test_each_v_byte_holds_one_token_and_each_k_word_one_mfma_slot(B, D):
    p = layout.PoolShape(1, 1, B, 1, D, layout.KV_INT4)
    t = np.arange(B)[:, None] + 0 * np.arange(D)[None, :]
    d = np.arange(D)[None, :] + 0 * t
    vbyte = layout.int4_v_nibble(p, 0, 0, 0, t, d) >> 1
    for b in np.unique(vbyte):
        assert np.unique(t[vbyte == b]).size == 1
    # a K word (4 bytes) holds the 8 dims 32 kk + 8 j .. + 7 of one token
    kword = layout.int4_k_nibble(p, 0, 0, 0, t, d) >> 3
    for w in np.unique(kword):
        tt, dd = t[kword == w], d[kword == w]
        assert np.unique(tt).size == 1 and dd.size == 8
        assert dd.min() % 8 == 0 and dd.max() == dd.min() + 7


@pytest.mark.parametrize("B,D", [(8, 64), (16, 128), (32, 64)])
def test_tile_unpack_equals_element_reads(B, D):
    rng = np.random.default_rng(12100 + B + D)
    p = layout.PoolShape(2, 5, B, 3, D, layout.KV_INT4)
    region = rng.integers(0, 256, size=p.region_units).astype(np.uint8)
    blocks = np.array([4, 0, 2])
    kt = layout.k_tiles_as_tokens(p, region, 1, blocks)
    vt = layout.v_tiles_as_tokens(p, region, 1, blocks)
    blk = np.repeat(blocks, B)[:, None, None]
    t = np.tile(np.arange(B), blocks.size)[:, None, None]
    h = np.arange(3)[None, :, None]
    d = np.arange(D)[None, None, :]
    assert np.array_equal(kt, layout.read_nibbles(region, layout.int4_k_nibble(p, 1, blk, h, t, d)))
    assert np.array_equal(vt, layout.read_nibbles(region, layout.int4_v_nibble(p, 1, blk, h, t, d)))


def _write(rng, B=8, H=2, D=64, L=2, layer=1):
    ctx = np.array([3, 17, 26], np.int32)
    nb = sum(math.ceil(int(c) / B) for c in ctx) + 2
    p = layout.PoolShape(L, nb, B, H, D, layout.KV_INT4)
    img = layout.empty_image(p)
    ck = rng.uniform(0.1, 0.5, size=(L, H, D)).astype(np.float32)
    cv = rng.uniform(0.1, 0.5, size=(L, H, D)).astype(np.float32)
    img.k_scale[:] = ck.reshape(-1)
    img.v_scale[:] = cv.reshape(-1)
    bt = random_tables(rng, nb, ctx, B)
    toks = [(workloads.to_bf16_bits(rng.standard_normal((int(c), H, D), dtype=np.float32)),
             workloads.to_bf16_bits(rng.standard_normal((int(c), H, D), dtype=np.float32))) for c in ctx]
    slots = np.concatenate([expanded_slots(bt[s], int(ctx[s]), B) for s in range(3)])
    img = cache_ops.reshape_and_cache(img, layer, np.concatenate([t[0] for t in toks]),
                                      np.concatenate([t[1] for t in toks]), slots)
    return p, img, bt, ctx, toks, ck[layer], cv[layer]


@pytest.mark.parametrize("B,D", [(8, 64), (16, 128)])
def test_cache_write_then_gathers_read_code_times_scale(B, D):
    rng = np.random.default_rng(12200 + B + D)
    p, img, bt, ctx, toks, ck, cv = _write(rng, B=B, D=D)
    for s in range(3):
        n = int(ctx[s])
        k, v = attention.gather_kv_by_slot(img, 1, bt[s], n)
        kt, vt = attention.gather_kv(img, 1, bt[s], n)
        assert np.array_equal(k, kt) and np.array_equal(v, vt)
        ck_ = codecs.int4_encode(codecs.bf16_bits_to_f32(toks[s][0]), ck[None]).astype(np.float64)
        cv_ = codecs.int4_encode(codecs.bf16_bits_to_f32(toks[s][1]), cv[None]).astype(np.float64)
        assert np.array_equal(k, ck_ * np.broadcast_to(ck, k.shape).astype(np.float64))
        assert np.array_equal(v, cv_ * np.broadcast_to(cv, v.shape).astype(np.float64))
    # layer 0 was not written: nibbles 0, i.e. code -8 everywhere
    k0, _ = attention.gather_kv_by_slot(img, 0, bt[0], 3)
    assert np.array_equal(k0, -8 * np.broadcast_to(img.k_scale[:p.num_kv_heads * p.head_dim].reshape(
        p.num_kv_heads, p.head_dim), k0.shape).astype(np.float64))


def test_a_quarter_of_the_bf16_bytes():
    # [KVP] §四: INT4 stores a quarter of FP16's KV bytes (channel scales aside)
    b16 = layout.PoolShape(80, 256, 16, 8, 128, layout.KV_BF16)
    b4 = layout.PoolShape(80, 256, 16, 8, 128, layout.KV_INT4)
    k16, v16, _, _, _ = layout.region_offsets(b16)
    k4, v4, ks, vs, total = layout.region_offsets(b4)
    assert (v4 - k4) * 4 == v16 - k16
    assert total - 2 * (v4 - k4) <= 2 * (80 * 8 * 128 * 4 + 256)
