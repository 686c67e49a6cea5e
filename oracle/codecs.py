"""Element codecs for KV storage (test infrastructure only; see package docstring).

The pages store the cache in 16-bit floats and, to halve memory and bandwidth,
in 8-bit codes that are widened back before the attention arithmetic
("KV Cache 原理与 PagedAttention", §四 KV Cache 量化 table: the FP8 row stores
FP8 and de-quantises before compute, the INT8 row quantises per tensor or per
channel; the vLLM launch example there selects ``fp8_e5m2``).  The bjdmk.com.cn
article, §5.2 量化粒度, names per-token-head scales (one scale for each token's
each attention head) as the usual, most accurate INT8 choice.

Readings taken where the pages stop short:

* bf16 is the storage type of unquantised K/V; widening is exact.
* FP8 is the OCP e5m2 format: 1 sign, 5 exponent bits (bias 15), 2 mantissa
  bits, subnormals, exponent 31 = inf (mantissa 0) / NaN.  Encoding divides
  by the per-tensor fp32 scale in fp32, rounds to nearest with ties to even,
  saturates finite overflow to +-57344, keeps +-inf, maps NaN to the NaN code
  with all mantissa bits set and the input's sign.
* INT8 is symmetric per (token, kv head) over the head_dim values:
  scale = fp32(absmax) / 127 in fp32; code = clamp(round_half_even(fp32(x /
  scale)), -127, 127); absmax == 0 gives scale 0 and all-zero codes;
  dequantisation is code * scale.
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------- bf16
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64: a bf16 is the
    high half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).copy()


# --------------------------------------------------------------------- e5m2
E5M2_MAX = 57344.0          # largest finite e5m2 magnitude: 2**15 * 1.75
E5M2_MAX_CODE = 0x7B
E5M2_INF_CODE = 0x7C
E5M2_NAN_CODE = 0x7F


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e5m2 byte as float64: sign * 2**(E-15) * (1 + M/4) for
    E in 1..30, sign * 2**-14 * (M/4) for E == 0, inf / NaN for E == 31."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = c & 0x3
    normal = np.ldexp(1.0 + m / 4.0, (e - 15).astype(np.int64))
    sub = np.ldexp(m / 4.0, -14)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 31) & (m == 0), np.inf, mag)
    mag = np.where((e == 31) & (m != 0), np.nan, mag)
    return sign * mag


def e5m2_encode(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Encode fp32 values to e5m2 bytes after dividing by ``scale`` in fp32.

    Round to nearest, ties to even, by exponent/mantissa arithmetic: within a
    binade [2**e, 2**(e+1)) the e5m2 grid step is 2**(e-2); below 2**-14 the
    (subnormal) step is 2**-16.  Scaling by a power of two is exact in
    float64, so ``np.rint`` (half-to-even) performs the rounding exactly.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y32 = (x / np.float32(scale)).astype(np.float32)     # IEEE fp32 division
    y = y32.astype(np.float64)
    neg = np.signbit(y32)
    a = np.abs(y)
    out = np.zeros(a.shape, dtype=np.int64)

    finite = np.isfinite(a)
    sub = finite & (a < 2.0 ** -14)
    # subnormal range (and zero): step 2**-16; n == 4 is the smallest normal
    n_sub = np.rint(np.where(sub, a, 0.0) * 2.0 ** 16).astype(np.int64)
    out = np.where(sub, n_sub, out)

    nrm = finite & ~sub
    a_n = np.where(nrm, a, 1.0)
    _, ex = np.frexp(a_n)                 # a = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1           # a in [2**e, 2**(e+1))
    n = np.rint(np.ldexp(a_n, (2 - e))).astype(np.int64)   # in [4, 8]
    carry = n == 8
    e = np.where(carry, e + 1, e)
    n = np.where(carry, 4, n)
    biased = e + 15
    code_n = (biased << 2) | (n - 4)
    code_n = np.where(biased >= 31, E5M2_MAX_CODE, code_n)   # saturate
    out = np.where(nrm, code_n, out)

    out = np.where(np.isinf(a), E5M2_INF_CODE, out)
    out = np.where(np.isnan(a), E5M2_NAN_CODE, out)
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8)


# --------------------------------------------------------------------- int8
def int8_quantize(x_f32: np.ndarray):
    """Symmetric INT8 over the last axis (one scale per leading index).

    Returns (codes int8 [..., D], scales float32 [...]).
    """
    x = np.asarray(x_f32, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=-1).astype(np.float32)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (x / safe[..., None]).astype(np.float32)            # fp32 division
    code = np.clip(np.rint(q), -127, 127)
    code = np.where(scale[..., None] > 0, code, 0)
    return code.astype(np.int8), scale


def int8_encode(x_f32: np.ndarray, scale) -> np.ndarray:
    """INT8 codes under a given (calibrated) scale, elementwise: clamp(
    rint_even(fp32(x / scale)), -127, 127), and 0 where the scale is 0 - the
    per-tensor and per-channel granularities of the bjdmk.com.cn article,
    §5.2 (one scale for the whole cache, or one per channel); ``scale``
    broadcasts against x."""
    x = np.asarray(x_f32, dtype=np.float32)
    s = np.broadcast_to(np.asarray(scale, dtype=np.float32), x.shape)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = (x / safe).astype(np.float32)                       # fp32 division
    code = np.where(s > 0, np.clip(np.rint(q), -127, 127), 0)
    return code.astype(np.int8)


def int4_encode(x_f32: np.ndarray, scale) -> np.ndarray:
    """INT4 codes under a given (calibrated) scale: clamp(rint_even(fp32(x /
    scale)), -7, 7), and 0 where the scale is 0.  The pages list INT4 KV as
    the more aggressive step after INT8 that needs calibration and stores a
    quarter of FP16's bytes ("KV Cache 原理与 PagedAttention", §四); this
    library reads that as the INT8 per-channel scheme with symmetric 4-bit
    codes (calibrated channel scales keep the size at a quarter)."""
    x = np.asarray(x_f32, dtype=np.float32)
    s = np.broadcast_to(np.asarray(scale, dtype=np.float32), x.shape)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = (x / safe).astype(np.float32)                       # fp32 division
    code = np.where(s > 0, np.clip(np.rint(q), -7, 7), 0)
    return code.astype(np.int8)


def int8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * scale in float64 (scales broadcast over the last axis)."""
    return (np.asarray(codes, dtype=np.int8).astype(np.float64)
            * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None])
