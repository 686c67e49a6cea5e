// Device helpers shared by the decode and prefill kernels: vector types,
// exact widening of stored K/V elements to bf16, lane-swap reductions, the
// single-pass parameter block and its K/V step loads, the query fold for
// per-channel scales, and the variant dispatcher.  Everything sits in an
// anonymous namespace: each translation unit that includes it gets its own
// copy.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "pkv_codecs.h"
#include "pkv_internal.h"

namespace pkv {
namespace {


constexpr int kWave = 64;
constexpr int kNW = 4;            // wavefronts per workgroup
constexpr int kStep = 32;         // tokens per step of the single-pass kernel
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// Two e5m2 bytes (16-bit half HI of w) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2_to_bf16x2(uint32_t w) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Two floats -> packed bf16x2 (round to nearest even; exact for int8 codes).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// The bf16 in the low / high half of a packed pair, as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four bytes of w (byte i = token or dim i) -> 4 bf16 in 2 dwords.
template <int KVT>
__device__ __forceinline__ void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (KVT == PKV_KV_FP8_E5M2) {
    lo = e5m2x2_to_bf16x2<false>(w);
    hi = e5m2x2_to_bf16x2<true>(w);
  } else {
    const float c0 = (float)(int8_t)(w & 0xff);
    const float c1 = (float)(int8_t)((w >> 8) & 0xff);
    const float c2 = (float)(int8_t)((w >> 16) & 0xff);
    const float c3 = (float)(int8_t)(w >> 24);
    lo = pack_bf16x2(c0, c1);
    hi = pack_bf16x2(c2, c3);
  }
}

// 8 bytes (two dwords) -> 8 bf16 operand (dims d..d+7 of one token).
template <int KVT>
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  uint32_t a, b, c, d;
  widen4<KVT>(w0, a, b);
  widen4<KVT>(w1, c, d);
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

// Wave-uniform read of memory that no kernel of this launch writes (block
// tables, context lengths): through the constant address space it becomes a
// scalar load, which does not occupy the vector-memory counter that the K/V
// prefetch pipeline waits on.
__device__ __forceinline__ int32_t uniform_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Combine each lane's value with that of lane ^ 16 / lane ^ 32 (the other
// token groups of the same head in the MFMA accumulator layout).  gfx950's
// row / half swaps do this in the VALU, without an LDS round trip.
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N), N <= 63 (vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maximum): wait until at most N vector memory operations of
// the wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait_at_most() {
  static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int clamp_ctx(int c, int max_ctx) { return c < 0 ? 0 : (c > max_ctx ? max_ctx : c); }

// Sliding window: a row of context ctx attends to positions [lo, ctx),
// lo = ctx - win when a window of win > 0 positions is set and shorter than
// the context, else 0.  The row's steps of TS tokens start at the step that
// holds lo (token base = floor(lo / TS) * TS); blocks before it are not read.
__device__ __forceinline__ int window_lo(int ctx, int win) { return (win > 0 && ctx > win) ? ctx - win : 0; }
template <int TS>
__device__ __forceinline__ int row_base(int ctx, int win) { return window_lo(ctx, win) / TS * TS; }
template <int TS>
__device__ __forceinline__ int row_steps(int ctx, int win) { return (ctx - row_base<TS>(ctx, win) + TS - 1) / TS; }

// Byte / half-word masks keeping the tokens of lane slot j that lie in
// [t_lo, t_end): token tb + i owns byte i (8-bit) or half-word i (bf16 pairs).
__device__ __forceinline__ bool tok_in(int t, int t_lo, int t_end) { return t < t_end && t >= t_lo; }
__device__ __forceinline__ uint32_t tok_mask8(int tb, int t_lo, int t_end) {
  return (tok_in(tb + 0, t_lo, t_end) ? 0x000000ffu : 0u) | (tok_in(tb + 1, t_lo, t_end) ? 0x0000ff00u : 0u) |
         (tok_in(tb + 2, t_lo, t_end) ? 0x00ff0000u : 0u) | (tok_in(tb + 3, t_lo, t_end) ? 0xff000000u : 0u);
}
__device__ __forceinline__ uint32_t tok_mask16(int tb, int t_lo, int t_end) {
  return (tok_in(tb, t_lo, t_end) ? 0x0000ffffu : 0u) | (tok_in(tb + 1, t_lo, t_end) ? 0xffff0000u : 0u);
}

// Query dims held by lane slot j of q.K MFMA kk (the same dims the K operand
// of that slot holds).
template <int E>
__device__ __forceinline__ int q_dim0(int kk, int j) {
  return (E == 2) ? (32 * kk + 8 * j) : (64 * (kk >> 1) + 16 * j + 8 * (kk & 1));
}

// Output dim of accumulator element i of tile c in lane slot j, by the
// accumulator layout AL of the storage type (its bytes per element, 0 for INT4):
//   bf16: 32u + 8j + 2i + e  (c = 2u + e)   8-bit: 64u + 16j + 4i + e (c = 4u + e)
//   INT4: 16c + 4j + i
template <int AL>
__device__ __forceinline__ int acc_dim(int c, int j, int i) {
  if constexpr (AL == 0) return 16 * c + 4 * j + i;
  return (AL == 2) ? (32 * (c >> 1) + 8 * j + 2 * i + (c & 1)) : (64 * (c >> 2) + 16 * j + 4 * i + (c & 3));
}

// ---- INT4: a stored nibble u = code + 8 becomes the bf16 of 128 + u =
// 136 + code (exact: bf16 has 8 significant bits) by OR-ing it into the
// mantissa of 128.0 (0x4300).  Word nibbles are placed so that pair k of a
// word - bits 4k .. 4k+3 and 16 + 4k .. 16 + 4k + 3 - is one bf16x2.  The
// kernels subtract the constant 136 after the products: 136 * sum(q) from
// each logit, 136 * sum(p) from each accumulator.
constexpr float kInt4Bias = 136.0f;
// The mask and the OR constant pass through an empty asm statement that
// makes them register values the compiler cannot fold back into literals
// (it is pure, so it is computed once and shared): (w & mask) | or then
// compiles to one v_and_or_b32 instead of an AND and an OR with literal
// operands, and the compiler still sees every instruction it schedules.
__device__ __forceinline__ uint32_t int4_pair(uint32_t w, int k) {
  uint32_t mask = 0x000F000Fu, orv = 0x43004300u;
  asm("" : "+v"(mask));
  asm("" : "+s"(orv));
  return ((k ? w >> (4 * k) : w) & mask) | orv;
}

// =====================================================================
// Single-pass kernel (partition_size == 0)
// =====================================================================
struct DecodeParams {
  const uint16_t* q;          // [S][Hq][D] bf16
  float* out;                 // [S][Hq][D]
  const char* k;              // this layer's K region
  const char* v;              // this layer's V region
  const float* ks;            // this layer's K scales (int8) or null
  const float* vs;            // this layer's V scales (int8) or null
  const int32_t* bt;          // [S][W]
  const int32_t* ctx;         // [S]
  int32_t W, S, Hq, Hkv, G, QT, num_blocks;
  int32_t num_items;          // S * Hkv * QT
  int32_t win;                // sliding window (positions), 0 = whole context
  float qk_scale;             // softmax scale * log2(e) (* fp8 k scale)
  float out_scale;            // fp8 / int8 per-tensor v scale, else 1
  const float* vs_ch;         // int8 per channel: this layer's V scales [Hkv][D] (output scale per dim), else null
  int32_t q_stride;           // elements between q rows: D, or 2 D for the folded q of int8 per channel
};

template <int D, int KVT>
struct Tile {
  static constexpr int E = KVT == PKV_KV_BF16 ? 2 : 1;        // bytes per element
  static constexpr int KLOADS = D * E / 64;                   // 16-B K loads per chunk per lane
  static constexpr int VLOADS = D * E / 64;                   // 16-B V loads per chunk per lane
  static constexpr int KK = D / 32;                           // q.K MFMAs per chunk
  static constexpr int NC = D / 16;                           // P.V MFMAs per step
};

// Registers of one step (two chunks).
template <int D, int KVT>
struct StepRegs {
  u32x4 k[2][Tile<D, KVT>::KLOADS];
  u32x4 v[2][Tile<D, KVT>::VLOADS];
  f32x4 ksc[2];   // int8: K scales of this lane's 4 tokens per chunk
  f32x4 vsc[2];
};

template <int D, int KVT, int B>
__device__ __forceinline__ void issue_step(StepRegs<D, KVT>& r, const DecodeParams& p, const int32_t* bt_row,
                                           int g, int tok0, int t_lo, int lane) {
  using T = Tile<D, KVT>;
  constexpr int E = T::E;
  const int row = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = tok0 + 16 * h;                   // first token of the chunk (multiple of 16)
    // a chunk wholly before the window does not use its table entries (block
    // 0 instead; its tokens are masked).  With B = 8 the chunk spans two blocks.
    const bool used = t + 16 > t_lo;
    int ph[2];
#pragma unroll
    for (int b = 0; b < (B < 16 ? 2 : 1); ++b) {
      int lb = (int)((uint32_t)t / B) + b;         // tokens are never negative
      lb = lb < p.W ? lb : p.W - 1;                // never index past the table row
      const int e = used ? bt_row[lb] : 0;
      ph[b] = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);  // stay inside the pool
    }
    if (B >= 16) ph[1] = ph[0];
    // K: lane row reads token t + row; V and the int8 scales: lane j reads
    // tokens t + 4j .. t + 4j + 3
    const int phk = row < 8 ? ph[0] : ph[1];
    const int phv = j < 2 ? ph[0] : ph[1];
    // chunks start at multiples of 16 tokens: with B >= 16 the chunk sits at
    // offset t % B of one block, with B = 8 it starts both of its blocks
    constexpr int TM = (B < 16 ? B : 16) - 1;
    const int toff = B < 16 ? 0 : (int)((uint32_t)t % B);
    const int tk = toff + (row & TM);              // token of lane row inside its block
    const int tv = toff + ((4 * j) & TM);          // first token of lane j's group inside its block
    // tile numbers are below num_blocks * Hkv < 2^31: unsigned 32-bit
    // products widened once keep the address arithmetic short
    const uint32_t tilek = (uint32_t)phk * (uint32_t)p.Hkv + (uint32_t)g;
    const uint32_t tilev = (uint32_t)phv * (uint32_t)p.Hkv + (uint32_t)g;
    const char* kt = p.k + (uint64_t)tilek * (uint32_t)(B * D * E);
    const char* vt = p.v + (uint64_t)tilev * (uint32_t)(B * D * E);
    // K: piece c holds dims [X*c, X*c+X) of all B tokens, 16 bytes per token
#pragma unroll
    for (int u = 0; u < T::KLOADS; ++u) r.k[h][u] = ld16(kt + (uint32_t)((4 * u + j) * B + tk) * 16u);
    // V: token group tv / 4, 4 tokens x dims as 4E-byte words
    const int grp = tv >> 2;
#pragma unroll
    for (int u = 0; u < T::VLOADS; ++u) {
      const int d = (E == 2) ? (32 * u + 2 * row) : (64 * u + 4 * row);
      r.v[h][u] = ld16(vt + (uint32_t)(grp * D + d) * (uint32_t)(4 * E));
    }
    if constexpr (KVT == PKV_KV_INT8) {
      const uint64_t so = (uint64_t)tilev * B + tv;
      r.ksc[h] = *reinterpret_cast<const f32x4*>(p.ks + so);
      r.vsc[h] = *reinterpret_cast<const f32x4*>(p.vs + so);
    }
  }
}

// INT8 with per-channel scales (and INT4): the K scale of (KV head, dim) is
// folded into the query, z = sum_d (q_d * s_d) * code_d, so the kernels see
// plain codes.  q'[s][h][d] = fp32(q) * s_k[h / G][d] is written as two bf16
// parts, hi = bf16(q') and lo = bf16(q' - hi) (round to nearest even; hi + lo
// carries ~16 significant bits of q'), over the output row out[s][h], which
// only that row's final store writes, after every read of q': hi in the first
// D bf16 slots of the row, lo in the next D (row stride 2 D bf16 elements).
// The kernels multiply both parts with the same K operand.
__global__ __launch_bounds__(256) void fold_q_kernel(const uint16_t* __restrict__ q, uint16_t* __restrict__ qf,
                                                     const float* __restrict__ ks_ch, int64_t n, int32_t Hq,
                                                     int32_t G, int32_t D) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int d = (int)(i % D);
  const int64_t row = i / D;
  const int h = (int)(row % Hq);
  const float x = bf16_bits_to_float(q[i]) * ks_ch[(h / G) * D + d];
  const uint32_t hi = pack_bf16x2(x, 0.f) & 0xffffu;
  const uint32_t lo = pack_bf16x2(x - bf16_bits_to_float(hi), 0.f) & 0xffffu;
  qf[row * 2 * D + d] = (uint16_t)hi;
  qf[row * 2 * D + D + d] = (uint16_t)lo;
}

// Partials cross from the waves that write them to the wave that merges them,
// which may sit on another XCD, whose L2 is not coherent with the writer's.
// They are therefore stored and loaded with the cache policy of an
// agent-scope atomic (the sc1 scope bit), which goes to the coherent level
// instead of a per-XCD L2; this avoids device-scope fences, which write back
// or invalidate a whole L2 each time.  Every access goes through a buffer
// resource whose size bounds it to its workspace region.
constexpr int kCoherentScope = 16;     // raw buffer access aux: sc1

__device__ __forceinline__ void st_agent2(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(a), __float_as_uint(b)}, r, off, 0, kCoherentScope);
}
__device__ __forceinline__ f32x2 ld_agent2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherentScope));
}

// 16-byte loads / stores of partials with the coherent-level cache policy.
__device__ __forceinline__ f32x4 ld_agent4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentScope));
}
__device__ __forceinline__ void st_agent4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherentScope);
}

// Add `mine` steps to an epoch-tagged row counter, in two parts so that the
// first can be issued well before its result is needed.  One lane of a wave
// makes the calls: the atomics are per lane, and a wave-wide call would add
// `mine` once per active lane.  Epochs increase
// from call to call, so raising the counter to (epoch << 32) first turns a
// counter of an earlier call into a zero count of this one and leaves a
// counter of this call alone; the add that follows, issued right behind it,
// takes effect after it (one wave's atomics on one address keep their
// order).  That costs a single round trip however many waves report at
// once.  report_steps issues both and returns the counter's value before the
// add; report_total gives the row's total for this epoch after the
// addition.  A counter with a larger tag (memory this library never wrote,
// or epochs that wrapped around) is instead replaced by compare-and-swap; an
// add that went to such a value is wiped by that replacement and redone by
// the wave that made it.
__device__ __forceinline__ unsigned long long report_steps(uint64_t* ctr, uint32_t epoch, int mine) {
  unsigned long long* c = reinterpret_cast<unsigned long long*>(ctr);
  const unsigned long long tag = (unsigned long long)epoch << 32;
  __hip_atomic_fetch_max(c, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __hip_atomic_fetch_add(c, (unsigned long long)(uint32_t)mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int report_total(uint64_t* ctr, uint32_t epoch, int mine, unsigned long long old) {
  if ((uint32_t)(old >> 32) == epoch) return (int)((uint32_t)old + (uint32_t)mine);
  unsigned long long* c = reinterpret_cast<unsigned long long*>(ctr);
  const unsigned long long tag = (unsigned long long)epoch << 32;
  unsigned long long expect = old + (uint32_t)mine;
  while (true) {
    const uint32_t base = (uint32_t)(expect >> 32) == epoch ? (uint32_t)expect : 0u;
    const unsigned long long want = tag | (base + (uint32_t)mine);
    unsigned long long prev = expect;
    if (__hip_atomic_compare_exchange_strong(c, &prev, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return (int)(base + (uint32_t)mine);
    expect = prev;
  }
}

// ---------------------------------------------------------------- launches
template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<D>, IC<KVT>, IC<B>) for the kernel variant of head dim D (64, 128),
// storage kv_dtype and block size B (8, 16, 32).  INT8 with per-channel
// K scales has its own variant: plain codes whose K channel scales are folded
// into the query (read as its bf16 hi and lo parts) and whose V scales (per
// channel, or one per tensor) are applied to the output.
template <bool kInt4, class F>
auto with_variant(int D, int kvt, int B, F&& f) {
  auto by_b = [&](auto dc, auto kc) {
    if (B == 8) return f(dc, kc, IC<8>{});
    if (B == 16) return f(dc, kc, IC<16>{});
    return f(dc, kc, IC<32>{});
  };
  auto by_kv = [&](auto dc) {
    switch (kvt) {
      case PKV_KV_BF16: return by_b(dc, IC<PKV_KV_BF16>{});
      case PKV_KV_FP8_E5M2: return by_b(dc, IC<PKV_KV_FP8_E5M2>{});
      case PKV_KV_INT8_TENSOR: return by_b(dc, IC<PKV_KV_INT8_TENSOR>{});
      case PKV_KV_INT8_CHANNEL:
      case PKV_KV_INT8_KCHANNEL_VTENSOR: return by_b(dc, IC<PKV_KV_INT8_CHANNEL>{});
      case PKV_KV_INT4:
        if constexpr (kInt4) return by_b(dc, IC<PKV_KV_INT4>{});
        [[fallthrough]];
      default: return by_b(dc, IC<PKV_KV_INT8>{});
    }
  };
  return D == 64 ? by_kv(IC<64>{}) : by_kv(IC<128>{});
}

}  // namespace
}  // namespace pkv
