"""Pins of the oracle's element codecs.

e5m2: decoding is checked against numpy's IEEE binary16 (an e5m2 byte is the
high byte of a binary16); encoding is checked against a brute-force nearest
search over every finite code, on every bf16 bit pattern.
INT8: brute-force nearest integer, the half-step error bound, edge cases.
"""

import numpy as np
import pytest

from oracle import codecs


def _all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    return bits.view(np.float32)


def test_e5m2_decode_matches_binary16_high_byte():
    codes = np.arange(256, dtype=np.uint8)
    ref = (codes.astype(np.uint16) << np.uint16(8)).view(np.float16).astype(np.float64)
    got = codecs.e5m2_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros preserved
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])


def _brute_force_encode(y32):
    """Nearest finite e5m2 value, ties to the even code; saturate finite
    overflow; inf -> inf code; NaN -> 0x7F | sign."""
    codes = np.arange(0, 0x7C, dtype=np.uint8)              # non-negative finite
    vals = codecs.e5m2_decode(codes)
    out = np.empty(y32.shape, dtype=np.uint8)
    for i, y in enumerate(y32.astype(np.float64)):
        s = 0x80 if np.signbit(y) else 0
        if np.isnan(y):
            out[i] = 0x7F | s
            continue
        a = abs(y)
        if np.isinf(a):
            out[i] = 0x7C | s
            continue
        if a >= vals[-1]:
            out[i] = 0x7B | s
            continue
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        if best.size == 2:                  # tie: even mantissa bit wins
            best = best[(codes[best] & 1) == 0]
        out[i] = codes[best[0]] | s
    return out


@pytest.mark.parametrize("scale", [1.0, 0.5, 3.0, 0.0078125])
def test_e5m2_encode_matches_brute_force_on_all_bf16(scale):
    x = _all_bf16_as_f32()
    if scale != 1.0:
        x = x[::7]          # keep the sweep quick for the extra scales
    y = (x / np.float32(scale)).astype(np.float32)
    got = codecs.e5m2_encode(x, scale)
    ref = _brute_force_encode(y)
    assert np.array_equal(got, ref)


def test_e5m2_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)
    vals = codecs.e5m2_decode(codes).astype(np.float32)
    assert np.array_equal(codecs.e5m2_encode(vals, 1.0), codes)


def test_e5m2_special_values():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 1e9, -1e9, 57344.0, 61440.0,
                  0.0, -0.0, 2.0 ** -17, 2.0 ** -16 * 1.5, 2.0 ** -16 * 2.5], dtype=np.float32)
    c = codecs.e5m2_encode(x, 1.0)
    assert list(c[:10]) == [0x7F, 0xFF, 0x7C, 0xFC, 0x7B, 0xFB, 0x7B, 0x7B, 0x00, 0x80]
    # 2^-17 is half the smallest subnormal: tie -> even (zero)
    assert c[10] == 0x00
    # 1.5 * 2^-16 -> tie between codes 1 and 2 -> 2; 2.5 * 2^-16 -> 2
    assert c[11] == 0x02 and c[12] == 0x02


def _int8_brute(x32):
    absmax = np.float32(np.max(np.abs(x32)))
    scale = np.float32(absmax / np.float32(127.0))
    if scale == 0:
        return np.zeros(x32.shape, np.int8), scale
    cand = np.arange(-127, 128, dtype=np.float64)
    out = []
    for v in x32:
        q = np.float64(np.float32(v / scale))
        d = np.abs(cand - q)
        best = np.flatnonzero(d == d.min())
        if best.size == 2:
            best = best[(cand[best].astype(np.int64) % 2) == 0]
        out.append(int(cand[best[0]]))
    return np.array(out, dtype=np.int8), scale


def test_int8_matches_brute_force_random():
    rng = np.random.default_rng(7)
    for _ in range(40):
        d = int(rng.choice([16, 64, 128]))
        x = (rng.standard_normal(d) * rng.choice([1e-3, 1.0, 40.0])).astype(np.float32)
        codes, scale = codecs.int8_quantize(x[None, :])
        bc, bs = _int8_brute(x)
        assert scale[0] == bs
        assert np.array_equal(codes[0], bc)
        # half-step error bound (plus the fp32 rounding of x / scale)
        err = np.abs(codes[0].astype(np.float64) * np.float64(bs) - x.astype(np.float64))
        assert np.all(err <= np.float64(bs) * (0.5 + 1e-6))
        assert np.max(np.abs(codes)) == 127


def test_int8_edge_cases():
    z, s = codecs.int8_quantize(np.zeros((1, 8), np.float32))
    assert s[0] == 0 and not z.any()
    one = np.zeros((1, 8), np.float32)
    one[0, 3] = -0.3
    c, s = codecs.int8_quantize(one)
    assert c[0, 3] == -127 and np.count_nonzero(c) == 1
    assert s[0] == np.float32(np.float32(0.3) / np.float32(127.0))
    # absmax 127 -> scale exactly 1: half-way values round to even
    x = np.array([[127.0, -127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5]], np.float32)
    c, s = codecs.int8_quantize(x)
    assert s[0] == 1.0
    assert list(c[0]) == [127, -127, 2, 4, -2, -4, 0, 2]
    # dequant is code * scale
    assert np.array_equal(codecs.int8_dequant(c, s)[0], c[0].astype(np.float64))


def test_bf16_widening_matches_torch():
    import torch
    bits = np.arange(0, 65536, 3, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
