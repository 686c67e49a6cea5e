"""Paged prefill with PKV_PREFILL_P_ONE_PART (the softmax weights meet V
rounded once) against the exact oracle, under the bound that rounding
gives: with unit roundoff u (2^-8 for bf16 weights, 2^-11 where V enters
as fp16: INT8 per tensor and per channel) each weight p_i becomes
p_i (1 + d_i), |d_i| <= u.  Normalised by the sum of the rounded weights,
the weights w_i = p_i / sum p and their rounded forms both sum to 1, so the
output moves by sum (w~_i - w_i)(v_i - c) for any c, at most
2u / (1 - u) * (max v - min v) / 2 over the positions attended (c the
midpoint).  INT8 per token-head normalises by the unrounded sum (its
weights carry the V scale): at most u * max |v|.  On top comes the default
form's own error (its bars in test_gpu_prefill.py).  The bound here takes
max and min over all of a sequence's positions, a superset of every
query's.
"""

import numpy as np
import pytest

import paged_kv_cache_436_amd as pkv
from oracle import attention
from tests.gpu_helpers import say
from tests.test_gpu_prefill import BAR, BAR8, _run

pytestmark = pytest.mark.gpu

ALL = [pkv.PKV_KV_BF16, pkv.PKV_KV_FP8_E5M2, pkv.PKV_KV_INT8, pkv.PKV_KV_INT8_TENSOR, pkv.PKV_KV_INT8_CHANNEL,
       pkv.PKV_KV_INT4, pkv.PKV_KV_INT8_KCHANNEL_VTENSOR]


def _unit_roundoff(dt):
    return 2.0**-11 if dt in (pkv.PKV_KV_INT8_TENSOR, pkv.PKV_KV_INT8_CHANNEL) else 2.0**-8


def _bound(dt, info, T, hq):
    """Per-element bound [T, Hq, D] of the one-part rounding (module text)."""
    u = _unit_roundoff(dt)
    img, tables, ctx, qs, G = info["img"], info["tables"], info["ctx"], info["qs"], info["G"]
    out = None
    for s in range(len(ctx)):
        if qs[s + 1] == qs[s] or ctx[s] == 0:
            continue
        _, V = attention.gather_kv(img, 0, tables[s], int(ctx[s]), info["ks"], info["vs"])   # [ctx, Hkv, D]
        if out is None:
            out = np.zeros((T, hq, V.shape[2]))
        if dt == pkv.PKV_KV_INT8:
            b = u * np.abs(V).max(axis=0)                                   # [Hkv, D]
        else:
            b = 2 * u / (1 - u) * (V.max(axis=0) - V.min(axis=0)) / 2
        out[qs[s]:qs[s + 1]] = np.repeat(b, G, axis=0)[None]
    return out if out is not None else np.zeros((T, hq, 1))


def _check(dt, got, want, default, info):
    T, hq, _ = want.shape
    bar = BAR.get(dt, BAR8)
    slack = bar[1] * max(np.max(np.abs(want)), 1e-30)     # the default form's relative bar
    err = np.abs(got - want)
    bound = _bound(dt, info, T, hq)
    worst = np.max(err - bound)
    say(f"  max_abs={err.max():.3e}  max(err - bound)={worst:.3e}  slack={slack:.3e}")
    assert np.all(np.isfinite(got))
    assert worst <= slack
    assert not np.array_equal(got, default)               # the flag takes effect


@pytest.mark.parametrize("dt", ALL)
@pytest.mark.parametrize("D,B", [(128, 16), (64, 32), (128, 8)])
def test_one_part_prefill_within_its_bound(dt, D, B):
    say(f"prefill one part dt={dt} D={D} B={B}")
    hkv, G = (2, 4) if D == 128 else (1, 3)
    ctx = [1, 40, 100, 257, 33, 64, 300]
    chunk = [1, 40, 37, 30, 1, 0, 300]
    seed = 16000 + 10 * dt + D + B
    default, _ = _run(np.random.default_rng(seed), dt, ctx, chunk, hkv=hkv, G=G, D=D, B=B)
    info = {}
    got, want = _run(np.random.default_rng(seed), dt, ctx, chunk, hkv=hkv, G=G, D=D, B=B, p_one_part=True,
                     info=info)
    _check(dt, got, want, default, info)


@pytest.mark.parametrize("dt", ALL)
def test_one_part_prefill_peaked_needles(dt):
    """Peaked softmax: a few planted keys carry most of the weight, where a
    weight's rounding matters most."""
    say(f"prefill one part needles dt={dt}")
    seed = 16400 + dt
    ctx, chunk = [400, 130, 65, 1000], [400, 50, 17, 300]
    default, _ = _run(np.random.default_rng(seed), dt, ctx, chunk, hkv=2, G=4, needles=8)
    info = {}
    got, want = _run(np.random.default_rng(seed), dt, ctx, chunk, hkv=2, G=4, needles=8, p_one_part=True, info=info)
    assert np.max(np.abs(want)) > 0.5
    _check(dt, got, want, default, info)


def test_one_part_prefill_group_sizes():
    say("prefill one part group sizes")
    for G, hkv in ((1, 3), (8, 1), (24, 1)):
        seed = 16500 + G
        default, _ = _run(np.random.default_rng(seed), pkv.PKV_KV_BF16, [50, 130], [50, 31], hkv=hkv, G=G)
        info = {}
        got, want = _run(np.random.default_rng(seed), pkv.PKV_KV_BF16, [50, 130], [50, 31], hkv=hkv, G=G,
                         p_one_part=True, info=info)
        _check(pkv.PKV_KV_BF16, got, want, default, info)
