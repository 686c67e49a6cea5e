"""GPU parity of the cache write and the copy-on-write block copy: every byte
of the pool must equal the oracle's expectation (bit-exact)."""

import numpy as np
import pytest

import paged_kv_cache_436_amd as pkv
import workloads
from oracle import cache_ops
from tests.gpu_helpers import (bf16_dev, dev, first_diff, images_equal, read_pool, say,
                               write_pool)

pytestmark = pytest.mark.gpu


def _random_pool(cfg, rng):
    import torch
    pool = pkv.Pool(cfg)
    raw = rng.integers(0, 256, size=pool.memory.numel(), dtype=np.uint8)
    if cfg.kv_dtype == pkv.PKV_KV_BF16:
        # keep the background finite so that nothing depends on NaN payloads
        raw = raw & np.uint8(0x3F)
    pool.memory.copy_(torch.from_numpy(raw))
    torch.cuda.synchronize()
    return pool


def _special_values(D):
    v = [0.0, -0.0, 1.0, -1.5, 57344.0, 60000.0, 1e30, -1e30, float("inf"), float("-inf"), float("nan"),
         2.0 ** -16, 2.0 ** -17, 3 * 2.0 ** -17, 2.0 ** -15 * 1.25, 1.75, 1.875, 2.5, -3.5, 0.1]
    out = np.zeros(D, np.float32)
    out[: len(v)] = v
    return out


@pytest.mark.parametrize("dt", [pkv.PKV_KV_BF16, pkv.PKV_KV_FP8_E5M2, pkv.PKV_KV_INT8])
@pytest.mark.parametrize("B,D", [(16, 64), (16, 128), (32, 128), (32, 64), (8, 128), (8, 64)])
@pytest.mark.parametrize("kscale", [1.0, 0.37])
def test_reshape_and_cache_bit_exact(dt, B, D, kscale):
    if dt != pkv.PKV_KV_FP8_E5M2 and kscale != 1.0:
        pytest.skip("per-tensor scales apply to fp8 only")
    say(f"reshape_and_cache dt={dt} B={B} D={D} kscale={kscale}")
    rng = np.random.default_rng(700 + 10 * dt + B + D)
    L, NB, H = 2, 9, 3
    cfg = pkv.make_config(L, NB, B, H, D, dt)
    pool = _random_pool(cfg, rng)
    before = read_pool(pool)
    N = 40
    slots = rng.choice(NB * B, size=N, replace=False).astype(np.int64)
    slots[3] = -1
    slots[7] = NB * B + 5            # outside the pool: skipped
    x = rng.standard_normal((N, H, D), dtype=np.float32) * 3
    x[0, 0] = _special_values(D)
    if dt == pkv.PKV_KV_INT8:   # int8 storage expects finite inputs
        x[0, 0] = np.nan_to_num(x[0, 0], nan=0.0, posinf=1e30, neginf=-1e30)
    x[1, 1, :] = 0.0                 # int8: absmax 0
    x[2, 2, :] = 0.0
    x[2, 2, 5] = -7.25               # int8: a single nonzero
    kb = workloads.to_bf16_bits(x)
    vb = workloads.to_bf16_bits(x[::-1].copy() * 0.5)
    layer = 1
    pkv.reshape_and_cache(pool, layer, bf16_dev(kb), bf16_dev(vb), dev(slots), k_scale=kscale,
                          v_scale=kscale * 2)
    got = read_pool(pool)
    keep = (slots >= 0) & (slots < NB * B)
    want = cache_ops.reshape_and_cache(before, layer, kb[keep], vb[keep], slots[keep], kscale, kscale * 2)
    assert images_equal(got, want), first_diff(got, want)


@pytest.mark.parametrize("dt", [pkv.PKV_KV_BF16, pkv.PKV_KV_INT8])
def test_copy_blocks_bit_exact(dt):
    say(f"copy_blocks dt={dt}")
    rng = np.random.default_rng(800 + dt)
    cfg = pkv.make_config(3, 12, 16, 2, 128, dt)
    pool = _random_pool(cfg, rng)
    before = read_pool(pool)
    pairs = np.array([[0, 5], [3, 7], [3, 8], [11, 2], [4, 40]], np.int64)  # last one is skipped
    pkv.copy_blocks(pool, dev(pairs))
    got = read_pool(pool)
    want = cache_ops.copy_blocks(before, pairs[:4])
    assert images_equal(got, want), first_diff(got, want)


def test_write_pool_round_trip():
    say("pool upload/readback")
    rng = np.random.default_rng(9)
    cfg = pkv.make_config(1, 4, 16, 1, 64, pkv.PKV_KV_INT8)
    pool = _random_pool(cfg, rng)
    img = read_pool(pool)
    img.k[:] = 1
    write_pool(pool, img)
    assert images_equal(read_pool(pool), img)
