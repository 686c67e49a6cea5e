// Element codecs of the cache write, shared by the kernels that quantise a
// new token on its way into the pool (reshape_and_cache and the appending
// decode), so both store exactly the same bytes.
//
// FP8 storage is OCP e5m2 ("KV Cache 原理与 PagedAttention", §四 量化 table and
// its fp8_e5m2 example): stored = e5m2(fp32(x / scale)), rounded to nearest
// even, finite overflow saturating to +-57344, +-inf kept, NaN -> 0x7F | sign.
// INT8 storage is symmetric per (token, KV head) (bjdmk.com.cn article, §5.2):
// scale = fp32(absmax) / 127, code = clamp(rint_even(fp32(x / scale)), -127,
// 127), and absmax 0 gives scale 0 with all codes 0.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> e5m2 byte.
__device__ __forceinline__ uint32_t encode_e5m2(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu | sign;
  if (a == 0x7f800000u) return 0x7cu | sign;
  if (a >= 0x38800000u) {  // |y| >= 2^-14: e5m2 normal range before rounding
    // keep 2 of the 23 mantissa bits, ties to even; a carry bumps the exponent
    const uint32_t r = (a + 0x000fffffu + ((a >> 21) & 1u)) >> 21;
    uint32_t code = r - (112u << 2);  // rebias the exponent from 127 to 15
    if (code > 0x7bu) code = 0x7bu;   // saturate
    return code | sign;
  }
  // subnormal range: a multiple of 2^-16; 4 * 2^-16 is the smallest normal
  const float n = __builtin_rintf(__uint_as_float(a) * 65536.0f);
  return (uint32_t)n | sign;
}

// Stored e5m2 byte of a bf16 value under a per-tensor scale.
__device__ __forceinline__ uint32_t fp8_store(uint32_t bf16_bits, float scale) {
  return encode_e5m2(__fdiv_rn(bf16_bits_to_float(bf16_bits), scale));
}

// INT8 scale of a (token, head) from the absolute maximum of its values.
__device__ __forceinline__ float int8_scale(float absmax) { return __fdiv_rn(absmax, 127.0f); }

// INT8 code (as a byte) of a bf16 value under its token-head scale.
__device__ __forceinline__ uint32_t int8_store(uint32_t bf16_bits, float scale) {
  if (!(scale > 0.f)) return 0u;
  const float c = fminf(fmaxf(__builtin_rintf(__fdiv_rn(bf16_bits_to_float(bf16_bits), scale)), -127.f), 127.f);
  return (uint32_t)(int32_t)c & 0xffu;
}

// INT4 nibble (code + 8) of a bf16 value under its calibrated channel scale:
// code = clamp(rint(x / scale), -7, 7), 0 when the scale is not positive.
__device__ __forceinline__ uint32_t int4_store(uint32_t bf16_bits, float scale) {
  if (!(scale > 0.f)) return 8u;
  const float c = fminf(fmaxf(__builtin_rintf(__fdiv_rn(bf16_bits_to_float(bf16_bits), scale)), -7.f), 7.f);
  return (uint32_t)((int32_t)c + 8);
}

// Element i (0..7) of the 8 dims one INT4 K word holds sits in nibble
// 4 (i % 2) + i / 2, so byte b of the word holds elements
// int4_k_lo_elem(b) (low nibble) and int4_k_lo_elem(b) + 2 (high nibble).
__device__ __forceinline__ int int4_k_lo_elem(int b) { return (b & 1) * 4 + (b >> 1); }

}  // namespace pkv
