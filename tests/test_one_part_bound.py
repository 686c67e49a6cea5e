"""The error bound that the GPU tests of PKV_PREFILL_P_ONE_PART apply,
checked on the CPU against a simulation of the one-part arithmetic.

The simulation takes each softmax weight p_i = exp(s_i - max s) in fp64,
rounds it once (to bf16 with torch's round-to-nearest-even, or to fp16 with
numpy's), and forms sum p~_i v_i / sum p~_i (or / sum p_i for INT8 per
token-head, whose weights carry the V scale).  With unit roundoff u the
bound is u / (1 - u) * (max v - min v) per output dim (normalised by the
rounded sum) and u * max |v| (by the exact sum).  These tests show that the
bound holds on random and peaked weights, and that constructed weights
reach a quarter of it (half of the exact-sum one), so it is not vacuous.
"""

import numpy as np
import pytest
import torch


def _round(p, kind):
    if kind == "bf16":
        return torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    return p.astype(np.float16).astype(np.float64)


U = {"bf16": 2.0**-8, "fp16": 2.0**-11}


def _outputs(s, v, kind, exact_sum=False):
    """Exact and one-part attention outputs for logits s [n] and values v [n, d]."""
    p = np.exp(s - s.max())
    exact = p @ v / p.sum()
    pr = _round(p, kind)
    one = pr @ v / (p.sum() if exact_sum else pr.sum())
    return exact, one


def _bound(v, kind, exact_sum=False):
    u = U[kind]
    if exact_sum:
        return u * np.abs(v).max(axis=0)
    return u / (1 - u) * (v.max(axis=0) - v.min(axis=0))


@pytest.mark.parametrize("kind", ["bf16", "fp16"])
@pytest.mark.parametrize("exact_sum", [False, True])
def test_bound_holds_on_random_and_peaked_weights(kind, exact_sum):
    rng = np.random.default_rng(7100 + (kind == "fp16") + 2 * exact_sum)
    for trial in range(200):
        n = int(rng.integers(1, 400))
        spread = [0.5, 2.0, 8.0, 30.0][trial % 4]            # flat to sharply peaked
        s = rng.standard_normal(n) * spread
        v = rng.standard_normal((n, 16)) * rng.uniform(0.1, 10.0)
        exact, one = _outputs(s, v, kind, exact_sum)
        assert np.all(np.abs(one - exact) <= _bound(v, kind, exact_sum) * (1 + 1e-9) + 1e-15)


@pytest.mark.parametrize("kind", ["bf16", "fp16"])
def test_bound_is_nearly_reached(kind):
    """One key of weight 1 (exact) with value +1 and two keys of weight just
    below the rounding midpoint above 1/2 (they round down by ~u relative)
    with value -1: the rounded weights move mass towards the first key, by
    w0 (1 - w0) u on each side with w0 ~ 1/2, a quarter of the bound."""
    u = U[kind]
    q = 0.5 + (u / 2) * (1 - 1e-3)
    assert _round(np.array([q]), kind)[0] == 0.5          # rounds down, relative error ~u
    s = np.log(np.array([1.0, q, q]))
    v = np.array([[1.0], [-1.0], [-1.0]])
    exact, one = _outputs(s, v, kind)
    ratio = float(abs(one - exact)[0] / _bound(v, kind)[0])
    assert 0.2 < ratio <= 1.0
    # by the exact sum (the two rounded weights lose ~u/2 each of a total
    # of ~2): about half of u * max |v|
    exact, one = _outputs(s, v, kind, exact_sum=True)
    ratio = float(abs(one - exact)[0] / _bound(v, kind, exact_sum=True)[0])
    assert 0.4 < ratio <= 1.0
