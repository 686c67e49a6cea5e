// Compute-only probe: the two ways to form one GQA group's q.K^T and P.V on
// gfx950, timed without HBM traffic, to decide which the decode kernels use.
//
// Per 16-token chunk of one KV head with bf16 K/V (head dim 128, 16 query
// heads in the group's tile), each wave computes the chunk's logits for its
// heads, the streaming-softmax update and P.V:
//   variant 1, matrix cores: q.K^T as four v_mfma_f32_16x16x32_bf16 (A = the
//       16 tokens' K, B = the 16 heads' q), P.V as sixteen
//       v_mfma_f32_16x16x16_bf16 (eight 16-dim tiles, p as bf16 hi + lo),
//       the logits' accumulator layout being P's operand layout - what
//       pa_split_kernel does;
//   variant 2, vector ALU: every lane holds its token's 32 dims of K and the
//       matching dims of all heads' q, forms the dot products with
//       v_dot2_f32_bf16 (two products per instruction), sums the four lanes
//       of a token, gathers the p of its four tokens from the lanes that
//       hold them and accumulates P.V with v_dot2_f32_bf16 (p as bf16 hi + lo);
//   variant 0, the loop and operand changes both variants carry, alone.
// K and V change every chunk (a few xor-ed bits), so nothing is hoisted out
// of the loop; the results are summed into `out` so nothing is dropped.
// The grid is the decode kernel's: one workgroup of four waves per CU, one
// wave per SIMD.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkvp {
namespace {

constexpr int kWave = 64;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
// sums / maxima over lanes 16 and 32 apart (the four lanes of one token or
// head in the 16 x 64 layouts), with gfx950's row and half swaps
__device__ __forceinline__ float swap16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                                    __builtin_bit_cast(uint32_t, x), false, false)[0]);
}
__device__ __forceinline__ float swap32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                                    __builtin_bit_cast(uint32_t, x), false, false)[0]);
}

constexpr float kScale = 0.08838835f * 1.44269504f;   // softmax scale in log2 units (head dim 128)
constexpr float kSlack = 8.0f;                       // lazy rescale threshold, as in the decode kernel

template <int V, int kHeads>
__global__ __launch_bounds__(kWave * 4) __attribute__((amdgpu_waves_per_eu(1, 1))) void probe_kernel(
    const uint32_t* __restrict__ seed, float* __restrict__ out, int chunks) {
  const int lane = threadIdx.x % kWave;
  const int j = lane >> 4;
  const uint32_t* sd = seed + (threadIdx.x % kWave) * 64;
  // this lane's K (token row, dims 32 u + 8 j .. + 7) and V (tokens 4 j ..
  // 4 j + 3, dims 32 u + 2 row, + 1) words, as the decode kernel loads them
  u32x4 k[4], v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    k[u] = u32x4{sd[4 * u], sd[4 * u + 1], sd[4 * u + 2], sd[4 * u + 3]};
    v[u] = u32x4{sd[16 + 4 * u], sd[17 + 4 * u], sd[18 + 4 * u], sd[19 + 4 * u]};
  }
  float sink = 0.f;
  if constexpr (V == 0) {
    for (int ch = 0; ch < chunks; ++ch) {
      const uint32_t x = (uint32_t)ch & 0x00030003u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        k[u] ^= x;
        v[u] ^= x;
      }
      sink += __uint_as_float((k[ch & 3][0] ^ v[ch & 3][1]) & 0x3f7f0000u);
    }
  } else if constexpr (V == 1) {
    bf16x8 q[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      q[kk] = __builtin_bit_cast(bf16x8, u32x4{sd[32 + 4 * kk], sd[33 + 4 * kk], sd[34 + 4 * kk], sd[35 + 4 * kk]});
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    for (int ch = 0; ch < chunks; ++ch) {
      const uint32_t x = (uint32_t)ch & 0x00030003u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        k[u] ^= x;
        v[u] ^= x;
      }
      f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[kk]),
                                                                                 q[kk], z, 0, 0, 0);
      float ml = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      ml = fmaxf(ml, swap16(ml));
      ml = fmaxf(ml, swap32(ml));
      const float ms = ml * kScale;
      const bool bump = ms > m_run + kSlack;
      const float m_ref = bump ? ms : m_run;
      const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.f;
      if (__builtin_amdgcn_ballot_w64(bump && m_run > -INFINITY)) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = acc[c] * alpha;
      }
      m_run = m_ref;
      float pv[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], kScale, -m_ref));
        ps += pv[i];
      }
      l_run = l_run * alpha + ps;
      const uint32_t h0 = pack_bf16x2(pv[0], pv[1]), h1 = pack_bf16x2(pv[2], pv[3]);
      const uint32_t l0 = pack_bf16x2(pv[0] - bf16_lo(h0), pv[1] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16x2(pv[2] - bf16_lo(h1), pv[3] - bf16_hi(h1));
      const s16x4 pop = __builtin_bit_cast(s16x4, u32x2{h0, h1});
      const s16x4 pop_lo = __builtin_bit_cast(s16x4, u32x2{l0, l1});
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int u = c >> 1, e = c & 1;
        const s16x4 aop = __builtin_bit_cast(s16x4, u32x2{v[u][2 * e], v[u][2 * e + 1]});
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, pop, acc[c], 0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, pop_lo, acc[c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sink += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    sink += l_run + m_run;
  } else {
    // the group's kHeads query heads (the matrix cores compute 16 columns
    // whatever the group), q at this lane's K dims
    uint32_t q[kHeads][16];
#pragma unroll
    for (int h = 0; h < kHeads; ++h)
#pragma unroll
      for (int pr = 0; pr < 16; ++pr) q[h][pr] = sd[(h * 16 + pr) & 63] ^ (uint32_t)h;
    float o[kHeads][8];   // P.V over this lane's 4 tokens: head h, dim 16 d + row
#pragma unroll
    for (int h = 0; h < kHeads; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) o[h][d] = 0.f;
    float m_run[kHeads], l_run[kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      m_run[h] = -INFINITY;
      l_run[h] = 0.f;
    }
    for (int ch = 0; ch < chunks; ++ch) {
      const uint32_t x = (uint32_t)ch & 0x00030003u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        k[u] ^= x;
        v[u] ^= x;
      }
      // logit of token `row` for every head: this lane's 32 dims, then the
      // four lanes of the token (16 apart) summed
      float p[kHeads];
      bool any_bump = false;
      float alpha[kHeads];
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int w = 0; w < 4; ++w) a = dot2(q[h][4 * u + w], k[u][w], a);
        a += swap16(a);
        a += swap32(a);
        // the head's max over the chunk's 16 tokens (the 16 lanes of a row group)
        float ml = a;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) ml = fmaxf(ml, __shfl_xor(ml, off, kWave));
        const float ms = ml * kScale;
        const bool bump = ms > m_run[h] + kSlack;
        const float m_ref = bump ? ms : m_run[h];
        alpha[h] = bump ? __builtin_amdgcn_exp2f(m_run[h] - m_ref) : 1.f;
        any_bump |= bump && m_run[h] > -INFINITY;
        m_run[h] = m_ref;
        p[h] = __builtin_amdgcn_exp2f(__builtin_fmaf(a, kScale, -m_ref));
        float ps = p[h];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) ps += __shfl_xor(ps, off, kWave);
        l_run[h] = l_run[h] * alpha[h] + ps;
      }
      if (__builtin_amdgcn_ballot_w64(any_bump)) {
#pragma unroll
        for (int h = 0; h < kHeads; ++h)
#pragma unroll
          for (int d = 0; d < 8; ++d) o[h][d] *= alpha[h];
      }
      // P.V: the p of this lane's tokens 4 j .. 4 j + 3, from the lanes of
      // those tokens, as bf16 hi + lo pairs, against the V pairs of its dims
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        float pt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pt[i] = __shfl(p[h], (lane & 48) | (4 * j + i), kWave);
        const uint32_t h0 = pack_bf16x2(pt[0], pt[1]), h1 = pack_bf16x2(pt[2], pt[3]);
        const uint32_t l0 = pack_bf16x2(pt[0] - bf16_lo(h0), pt[1] - bf16_hi(h0));
        const uint32_t l1 = pack_bf16x2(pt[2] - bf16_lo(h1), pt[3] - bf16_hi(h1));
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const int u = d >> 1, e = d & 1;            // V words of dim 16 d + row: tokens (0, 1), (2, 3)
          float a = o[h][d];
          a = dot2(h0, v[u][2 * e], a);
          a = dot2(h1, v[u][2 * e + 1], a);
          a = dot2(l0, v[u][2 * e], a);
          a = dot2(l1, v[u][2 * e + 1], a);
          o[h][d] = a;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
#pragma unroll
      for (int d = 0; d < 8; ++d) sink += o[h][d];
      sink += l_run[h] + m_run[h];
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = sink;
}

template <int V, int H>
int launch(const uint32_t* seed, float* out, int chunks, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL((probe_kernel<V, H>), dim3(workgroups), dim3(kWave * 4), 0, stream, seed, out, chunks);
  return (int)hipGetLastError();
}

}  // namespace
}  // namespace pkvp

extern "C" int pkv_probe_compute(int variant, const uint32_t* seed, float* out, int chunks, int workgroups,
                                 hipStream_t stream) {
  if (!seed || !out || chunks < 0 || workgroups <= 0 || workgroups > 65536) return (int)hipErrorInvalidValue;
  switch (variant) {
    case 0: return pkvp::launch<0, 16>(seed, out, chunks, workgroups, stream);
    case 1: return pkvp::launch<1, 16>(seed, out, chunks, workgroups, stream);
    case 2: return pkvp::launch<2, 8>(seed, out, chunks, workgroups, stream);
    case 3: return pkvp::launch<2, 4>(seed, out, chunks, workgroups, stream);
    default: return (int)hipErrorInvalidValue;
  }
}
