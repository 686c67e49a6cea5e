// Paged prefill attention for gfx950 (CDNA4): causal attention of a chunk
// of new tokens per sequence over its paged KV cache, the prefill that a
// prefix-cache hit leaves to do (bjdmk.com.cn article, §4.1: the cached
// prefix is reused and only the rest is computed; "KV Cache 原理与
// PagedAttention", §五).  The K/V of every position, the new tokens included,
// are in the pool before the call (reshape_and_cache).
#include <algorithm>

#include "decode_common.h"

namespace pkv {
namespace {

// =====================================================================
// Paged prefill (a chunk of new tokens per sequence, causal)
// =====================================================================
// The decode matrix-core step with its 16 columns taken by (query token,
// query head) pairs of one KV head instead of by query heads: column c of a
// sequence's chunk is token c / G of the chunk and head g G + c % G.  Token k
// of a chunk of n sits at position ctx - n + k and sees positions 0 .. ctx -
// n + k, so each column masks the keys at or past its own limit.
// Every wave owns prefill_nt() tiles of 16 columns and streams all of their
// keys itself: each K/V step it loads is widened once and feeds the products
// of all its tiles, and the wave writes its columns' outputs from registers
// (no cross-wave merge).  The four waves of a workgroup take consecutive
// column spans of one (sequence, KV head), so they read the same keys at
// about the same time and share them through L2.  A wave holds one step of
// K/V: its load latency, and the serial q.K -> softmax -> P.V chain of a
// step, are covered by the other tiles' work and by a second wave on the
// SIMD (the kernel is built for two waves per SIMD: at most 256 registers),
// which measured faster than keeping a step in flight at fewer tiles.  The
// streaming softmax keeps a reference max per column that is raised only
// when a logit exceeds it by kPrefillSlack (log2 units), so the accumulators
// are rescaled a few times per column instead of at every step.
constexpr int kPrefillBuf = 1;         // K/V steps held per wave
constexpr float kPrefillSlack = 8.0f;  // p < 2^8 between rescales
constexpr int kPrefillWavesPerSimd = 2;

// 16-column tiles per wave: three where they fit the register budget of two
// waves per SIMD without spilling, else two.
template <int D, int KVT, int B>
constexpr int prefill_nt() {
  return D == 64 || (KVT == PKV_KV_BF16 && B < 32) || KVT == PKV_KV_FP8_E5M2 ? 3 : 2;
}

// INT4 step loads: per 16-token chunk one K piece (lane slot j, token row)
// and one V piece (token group of lane slot j, dim row) of D / 8 bytes each,
// in the INT4 tile layout (the split decode kernel reads the same pieces).
template <int D, int B>
__device__ __forceinline__ void issue_step_int4(StepRegs<D, PKV_KV_INT4>& r, const DecodeParams& p,
                                                const int32_t* bt_row, int g, int tok0, int lane) {
  constexpr int P = D / 8;
  const int row = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = tok0 + 16 * h;
    int ph[2];
#pragma unroll
    for (int b = 0; b < (B < 16 ? 2 : 1); ++b) {
      int lb = (int)((uint32_t)t / B) + b;
      lb = lb < p.W ? lb : p.W - 1;                // never index past the table row
      const int e = bt_row[lb];
      ph[b] = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);  // stay inside the pool
    }
    if (B >= 16) ph[1] = ph[0];
    const int phk = row < 8 ? ph[0] : ph[1];
    const int phv = j < 2 ? ph[0] : ph[1];
    constexpr int TM = (B < 16 ? B : 16) - 1;
    const int toff = B < 16 ? 0 : (int)((uint32_t)t % B);
    const int tk = toff + (row & TM);
    const int tv = toff + ((4 * j) & TM);
    const uint32_t tilek = (uint32_t)phk * (uint32_t)p.Hkv + (uint32_t)g;
    const uint32_t tilev = (uint32_t)phv * (uint32_t)p.Hkv + (uint32_t)g;
    const char* ka = p.k + (uint64_t)tilek * (uint32_t)(B * D / 2) + (uint32_t)(j * B + tk) * P;
    const char* va = p.v + (uint64_t)tilev * (uint32_t)(B * D / 2) + (uint32_t)((tv >> 2) * 16 + row) * P;
    if constexpr (P == 16) {
      r.k[h][0] = ld16(ka);
      r.v[h][0] = ld16(va);
    } else {
      const u32x2 k2 = *reinterpret_cast<const u32x2*>(ka);
      const u32x2 v2 = *reinterpret_cast<const u32x2*>(va);
      r.k[h][0] = u32x4{k2[0], k2[1], 0u, 0u};
      r.v[h][0] = u32x4{v2[0], v2[1], 0u, 0u};
    }
  }
}

// ---- INT8 codes as fp16: a signed byte c becomes u = c + 128 by flipping
// its top bit, and the fp16 with bits 0x64uu is 1024 + u = 1152 + c exactly
// (fp16 steps by 1 in [1024, 2048)); one byte permute places two bytes and
// the constant 0x64.  Three instructions widen four codes where the bf16
// route takes six, which matters in this vector-ALU-bound kernel.  The
// constant comes back out after the products: 1152 * sum(q) from each
// logit, 1152 * sum(p) from each accumulator.  The query enters as
// fp16(q * 2^-8) (exact for |q| in [2^-6, 2^23]), the 2^8 going back into
// the softmax scale.
constexpr float kInt8Bias = 1152.0f;
constexpr float kInt8QShift = 1.0f / 256.0f;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool HI>
__device__ __forceinline__ uint32_t int8x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, HI ? 0x04030402u : 0x05010400u);
}
__device__ __forceinline__ bf16x8 int8x8_to_f16x8(uint32_t w0, uint32_t w1) {
  return __builtin_bit_cast(bf16x8, u32x4{int8x2_to_f16x2<false>(w0), int8x2_to_f16x2<true>(w0),
                                          int8x2_to_f16x2<false>(w1), int8x2_to_f16x2<true>(w1)});
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// bf16 step loads: K as in issue_step; V as 8-byte pieces (4 tokens of one
// dim) placed so that the P.V operand of 16-dim tile cc is one register
// quad, words {chunk 0: tokens 4j, 4j+1 | 4j+2, 4j+3; chunk 1: the same} of
// dim 32 (cc / 2) + 2 row + cc % 2, kept at flat index cc of r.v - so the
// operand needs no assembly from two 16-byte loads.
template <int D, int B>
__device__ __forceinline__ void issue_step_bf16(StepRegs<D, PKV_KV_BF16>& r, const DecodeParams& p,
                                               const int32_t* bt_row, int g, int tok0, int lane) {
  using T = Tile<D, PKV_KV_BF16>;
  constexpr int NC = D / 16;
  constexpr int VL = T::VLOADS;
  const int row = lane & 15;
  const int j = lane >> 4;
  u32x2 vv[2][NC];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = tok0 + 16 * h;
    int ph[2];
#pragma unroll
    for (int b = 0; b < (B < 16 ? 2 : 1); ++b) {
      int lb = (int)((uint32_t)t / B) + b;
      lb = lb < p.W ? lb : p.W - 1;                // never index past the table row
      const int e = bt_row[lb];
      ph[b] = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);  // stay inside the pool
    }
    if (B >= 16) ph[1] = ph[0];
    const int phk = row < 8 ? ph[0] : ph[1];
    const int phv = j < 2 ? ph[0] : ph[1];
    constexpr int TM = (B < 16 ? B : 16) - 1;
    const int toff = B < 16 ? 0 : (int)((uint32_t)t % B);
    const int tk = toff + (row & TM);
    const int tv = toff + ((4 * j) & TM);
    const uint32_t tilek = (uint32_t)phk * (uint32_t)p.Hkv + (uint32_t)g;
    const uint32_t tilev = (uint32_t)phv * (uint32_t)p.Hkv + (uint32_t)g;
    const char* kt = p.k + (uint64_t)tilek * (uint32_t)(B * D * 2);
    const char* vt = p.v + (uint64_t)tilev * (uint32_t)(B * D * 2);
#pragma unroll
    for (int u = 0; u < T::KLOADS; ++u) r.k[h][u] = ld16(kt + (uint32_t)((4 * u + j) * B + tk) * 16u);
    const int grp = tv >> 2;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int d = 32 * (cc >> 1) + 2 * row + (cc & 1);
      vv[h][cc] = *reinterpret_cast<const u32x2*>(vt + (uint32_t)(grp * D + d) * 8u);
    }
  }
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) r.v[cc / VL][cc % VL] = u32x4{vv[0][cc][0], vv[0][cc][1], vv[1][cc][0], vv[1][cc][1]};
}

struct PrefillParams {
  DecodeParams d;             // q [T][Hq][D] (or the folded q), out [T][Hq][D], pool layer, tables, lengths
  const int32_t* qstart;      // [S + 1]: sequence s's queries are rows qstart[s] .. qstart[s+1] - 1;
                              // null: one query per sequence, row s (a decode step)
  int32_t tiles;              // workgroup column spans per (sequence, KV head):
                              // ceil(max_query_len * G / (16 prefill_nt() kNW))
  int32_t T;                  // rows of q and out
  int32_t maxq;               // queries per sequence served (later ones are left unwritten)
  // The shared-prefix pass of a decode (pa_prefix_kernel only): the columns
  // of KV head g are the (sequence, head) pairs of all T sequences; column
  // (s, h) attends positions [0, min(ctx_s, prefix_len)) of the shared
  // prefix, whose blocks are row 0 of d.bt (width d.W).  The four waves of a
  // workgroup take the same 16 prefill_nt() columns and split the prefix
  // into key ranges of chunk_len positions (a multiple of kStep); their
  // partial results meet in LDS, where they are merged with the result of
  // the other positions already in out (its (m, l) in merge_ml) into out.
  const float* merge_ml;      // [T][Hq] (m, l) of out's rows
  int32_t prefix_len, chunk_len;
};

constexpr int kPrefixBuf = 3;              // K/V steps held per wave in the shared-prefix pass

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, kWave));
  return v;
}

// The body of both kernels: SH selects the shared-prefix pass (columns
// across sequences, the prefix's keys split over a workgroup's waves and
// merged in LDS) over the prefill (columns of one sequence's chunk, causal).
// P1: p meets V as one rounded part (bf16, or fp16 where V enters as fp16)
// instead of hi + lo parts, one matrix-core product per tile instead of two;
// the softmax denominator is then the sum of the rounded p (per-token INT8,
// whose p carries the V scale: the sum of the unrounded p).
template <int D, int KVT, int B, int NT, int NB, bool SH, bool P1>
__device__ __forceinline__ void prefill_body(const PrefillParams& pp) {
  const DecodeParams& p = pp.d;
  using T = Tile<D, KVT>;
  constexpr int E = T::E;
  // INT4: the K and V operands hold 136 + code (bf16, exact), taken back
  // after the products; the query dims follow the bf16 slot layout and the
  // accumulator dims that of the INT4 V pieces
  constexpr bool I4 = KVT == PKV_KV_INT4;
  // INT8 codes through fp16 (1152 + code) in q.K where the query is plain
  // (per-token and per-tensor scales; the per-channel folded query takes the
  // exact bf16 route with its hi and lo parts, whose magnitudes the fixed
  // fp16 shift could not hold), and in P.V where the V scale is per tensor or
  // per channel (p <= 2^8 then; per-token V scales are folded into p, whose
  // range fp16 could not hold, so that V stays bf16)
  constexpr bool I8K = KVT == PKV_KV_INT8 || KVT == PKV_KV_INT8_TENSOR;
  constexpr bool I8V = KVT == PKV_KV_INT8_TENSOR || KVT == PKV_KV_INT8_CHANNEL;
  const float qks = I8K ? p.qk_scale * (1.0f / kInt8QShift) : p.qk_scale;   // the softmax scale of z
  constexpr int QL = I4 ? 2 : E;
  constexpr int AL = I4 ? 0 : E;

  const int nwg = (int)gridDim.x;
  const int xcd = (int)blockIdx.x % 8;
  const int per_xcd = (nwg + 7) / 8;
  const int item = xcd * per_xcd + (int)blockIdx.x / 8;
  if (item >= p.num_items) return;
  // prefill: item = (sequence s, KV head g, column span ct); shared-prefix
  // pass: (KV head g, column group ct), the groups of a head adjacent so
  // that they read its keys through one L2
  const int ct = item % pp.tiles;
  const int g = SH ? item / pp.tiles : (item / pp.tiles) % p.Hkv;
  const int s = SH ? 0 : item / (pp.tiles * p.Hkv);
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int row = lane & 15;
  const int j = lane >> 4;
  // query rows, kept inside [0, T) whatever query_start holds
  const int q0 = SH ? 0 : (pp.qstart ? min(max(pp.qstart[s], 0), pp.T) : s);
  const int n = SH ? pp.T : (pp.qstart ? min(max(pp.qstart[s + 1], q0), pp.T) - q0 : 1);
  const int ncol = (SH ? n : min(n, pp.maxq)) * p.G;   // positions still follow the whole chunk
  constexpr int cpw = 16 * NT;                   // columns per wave
  // this wave's first column (the shared-prefix pass: the workgroup's, the
  // same for its four waves, so that they leave together or not at all)
  const int c0 = SH ? ct * cpw : (ct * kNW + w) * cpw;
  if (c0 >= ncol) return;                        // prefill: no barrier follows, waves are independent
  const int cols = min(cpw, ncol - c0);

  const int ctx = SH ? pp.prefix_len : clamp_ctx(p.ctx[s], p.W * B);
  const int first = ctx - n;                     // position of the chunk's token 0
  // shared-prefix pass: this wave's keys [k0, k1) of the prefix
  const int k0 = SH ? w * pp.chunk_len : 0;
  const int k1 = SH ? min(k0 + pp.chunk_len, pp.prefix_len) : 0;
  // a column's keys end at its limit; t_end is the wave's largest limit and
  // every valid column sees the keys below lim_lo (its smallest): steps
  // wholly below it need no mask.  Prefill: causal limits, column c0's the
  // smallest; shared-prefix pass: min(ctx_s, k1) of the column's sequence
  int t_end, lim_lo;
  if constexpr (SH) {
    int hi = 0, lo = k1;
    for (int c = lane; c < cols; c += kWave) {
      const int l = min(max(p.ctx[(c0 + c) / p.G], 0), k1);
      hi = max(hi, l);
      lo = min(lo, l);
    }
    t_end = wave_max_i(hi);
    lim_lo = wave_min_i(lo);
  } else {
    t_end = max(0, first + (c0 + cols - 1) / p.G + 1);
    lim_lo = max(0, first + c0 / p.G + 1);
  }
  const int nsteps = (t_end + kStep - 1) / kStep;
  // one query per sequence (a decode step) may attend to a sliding window:
  // positions [t_lo, ctx); the steps start at the one holding t_lo and the
  // keys before it are masked (their blocks may hold anything).  The
  // shared-prefix pass starts at its chunk (a multiple of kStep).
  const int t_lo = SH ? k0 : (pp.qstart ? 0 : window_lo(ctx, p.win));
  const int s0 = t_lo / kStep;
  const int32_t* bt_row = p.bt + (int64_t)s * p.W;

  // per tile: this lane's column limit (keys [0, lim)) and the query as the
  // B operand (columns past the chunk read column c0's query, limit 0); with
  // the K channel scales folded in (int8 per channel, INT4), set 0 is the
  // bf16 hi part of the folded query and set 1 its lo part (the next D
  // elements of the row), both multiplying the same K operand
  constexpr int NQ = (KVT == PKV_KV_INT8_CHANNEL || I4) ? 2 : 1;
  bf16x8 qop[NT][NQ][T::KK];
  float qsum[NT];   // INT4: the column's sum of q over all dims
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int cl = 16 * nt + row;
    const bool valid = cl < cols;
    const int c = c0 + (valid ? cl : 0);
    lim[nt] = !valid ? 0 : (SH ? min(max(p.ctx[c / p.G], 0), k1) : max(0, first + c / p.G + 1));
    const uint16_t* qh = p.q + ((int64_t)(q0 + c / p.G) * p.Hq + g * p.G + c % p.G) * p.q_stride;
#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk)
        // a prefill reads each query once and writes each output row once:
        // both move with the non-temporal hint, so that they leave the L2s
        // to the K/V tiles, which the chunk's column tiles read again (the
        // shared-prefix pass re-reads its rows to merge, and keeps them cached)
        qop[nt][n][kk] = __builtin_bit_cast(
            bf16x8, SH ? *reinterpret_cast<const u32x4*>(qh + n * D + q_dim0<QL>(kk, j))
                       : __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qh + n * D + q_dim0<QL>(kk, j))));
    qsum[nt] = 0.f;
    if constexpr (I4) {
      float a = 0.f;
#pragma unroll
      for (int n = 0; n < NQ; ++n)
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk)
#pragma unroll
          for (int e = 0; e < 8; ++e) a += (float)qop[nt][n][kk][e];
      qsum[nt] = sum_x32(sum_x16(a));   // lanes of one column hold its 4 dim slots
    } else if constexpr (I8K) {
      // the fp16 operand, and the sum of exactly the values it holds
      float a = 0.f;
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        const u32x4 wq = __builtin_bit_cast(u32x4, qop[nt][0][kk]);
        u32x4 hq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hq[e] = pack_f16x2(bf16_lo(wq[e]) * kInt8QShift, bf16_hi(wq[e]) * kInt8QShift);
          a += f16_lo(hq[e]) + f16_hi(hq[e]);
        }
        qop[nt][0][kk] = __builtin_bit_cast(bf16x8, hq);
      }
      qsum[nt] = sum_x32(sum_x16(a));
    }
  }

  f32x4 acc[NT][T::NC];
  float m_run[NT], l_run[NT];   // reference max of scaled logits (log2 domain) and partial sum, column `row`
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int cc = 0; cc < T::NC; ++cc) acc[nt][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](StepRegs<D, KVT>& r, int tok0) __attribute__((always_inline)) {
    // K operands, widened once for every tile
    bf16x8 ka[2][T::KK];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        if constexpr (I4) {
          const uint32_t wk = r.k[h][0][kk];        // word kk: dims 32 kk + 8 j .. + 7
          ka[h][kk] = __builtin_bit_cast(
              bf16x8, u32x4{int4_pair(wk, 0), int4_pair(wk, 1), int4_pair(wk, 2), int4_pair(wk, 3)});
        } else if constexpr (I8K) {
          const u32x4 wv = r.k[h][kk >> 1];
          ka[h][kk] = (kk & 1) ? int8x8_to_f16x8(wv[2], wv[3]) : int8x8_to_f16x8(wv[0], wv[1]);
        } else if constexpr (E == 2) {
          ka[h][kk] = __builtin_bit_cast(bf16x8, r.k[h][kk]);
        } else {
          const u32x4 wv = r.k[h][kk >> 1];
          ka[h][kk] = (kk & 1) ? widen8<KVT>(wv[2], wv[3]) : widen8<KVT>(wv[0], wv[1]);
        }
      }
    }
    f32x4 z[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < T::KK; ++kk) {
          if constexpr (I8K) {
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ka[h][kk]),
                                                       __builtin_bit_cast(f16x8, qop[nt][0][kk]), c, 0, 0, 0);
          } else {
#pragma unroll
            for (int n = 0; n < NQ; ++n)
              c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[h][kk], qop[nt][n][kk], c, 0, 0, 0);
          }
        }
        if constexpr (I4) c -= kInt4Bias * qsum[nt];    // the K operand held 136 + code
        if constexpr (I8K) c -= kInt8Bias * qsum[nt];   // the K operand held 1152 + code
        z[nt][h] = c;
      }
    }
    float alpha[NT], m_use[NT];
    bool any_rescale = false;
    // raw logits (int8: times the token's K scale); the softmax scale s > 0
    // is applied to the max and inside the exponent's fma, max(z) s = max(z s)
    const bool unmasked = tok0 + kStep <= lim_lo && tok0 >= t_lo;   // uniform
    float mlocs[NT];
    if (unmasked) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mloc = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (KVT == PKV_KV_INT8) z[nt][h][i] *= r.ksc[h][i];
            mloc = fmaxf(mloc, z[nt][h][i]);
          }
        mlocs[nt] = mloc;
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mloc = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tok0 + 16 * h + 4 * j + i;
            float zz = z[nt][h][i];
            if constexpr (KVT == PKV_KV_INT8) zz *= r.ksc[h][i];
            zz = (t < lim[nt] && t >= t_lo) ? zz : -INFINITY;   // causal: this column's keys only
            z[nt][h][i] = zz;
            mloc = fmaxf(mloc, zz);
          }
        mlocs[nt] = mloc;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mloc = max_x32(max_x16(mlocs[nt])) * qks;   // the column's scaled max over the step
      const bool bump = mloc > m_run[nt] + kPrefillSlack;   // false while the column has no key
      const float m_ref = bump ? mloc : m_run[nt];
      alpha[nt] = bump ? __builtin_amdgcn_exp2f(m_run[nt] - m_ref) : 1.0f;
      any_rescale |= bump && m_run[nt] > -INFINITY;   // the accumulator is zero until the first raise
      m_run[nt] = m_ref;
      // a column with no key yet keeps reference -inf; its exponents use 0 so
      // that p is 0, not NaN
      m_use[nt] = m_ref == -INFINITY ? 0.f : m_ref;
    }
    if (__builtin_amdgcn_ballot_w64(any_rescale)) {   // uniform branch, rarely taken
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int cc = 0; cc < T::NC; ++cc) acc[nt][cc] = acc[nt][cc] * alpha[nt];
    }
    // keys at or past the wave's largest limit may be unwritten slots (any
    // bits): their V is zeroed, in the step's own registers (the next load
    // overwrites them anyway); keys below it are written data, masked by p = 0
    // (INT4 codes, and INT8 codes read as fp16, are finite whatever the bytes: p = 0 masks them)
    if (E == 2 && !I4 && (tok0 + kStep > t_end || tok0 < t_lo)) {
      // bf16 operand quads: chunk 0 tokens tb0 .. tb0 + 3, chunk 1 tokens tb1 .. tb1 + 3
      const int tb0 = tok0 + 4 * j, tb1 = tok0 + 16 + 4 * j;
      const u32x4 m = u32x4{tok_mask16(tb0, t_lo, t_end), tok_mask16(tb0 + 2, t_lo, t_end),
                            tok_mask16(tb1, t_lo, t_end), tok_mask16(tb1 + 2, t_lo, t_end)};
#pragma unroll
      for (int cc = 0; cc < T::NC; ++cc) r.v[cc / T::VLOADS][cc % T::VLOADS] &= m;
    } else if (E != 2 && !I4 && !I8V && (tok0 + kStep > t_end || tok0 < t_lo)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tb = tok0 + 16 * h + 4 * j;      // lane j's 4 tokens of the chunk
#pragma unroll
        for (int u = 0; u < T::VLOADS; ++u) {
#pragma unroll
          for (int e = 0; e < 4; ++e) r.v[h][u][e] &= tok_mask8(tb, t_lo, t_end);   // 8-bit: tokens tb .. tb + 3
        }
      }
    }
    bf16x8 pop[NT], pop_lo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float psum = 0.f;
      uint32_t ph[2][2], pl[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[nt][h][i], qks, -m_use[nt]));
          psum += pv[i];
          if constexpr (KVT == PKV_KV_INT8) {
            const int t = tok0 + 16 * h + 4 * j + i;
            pv[i] = (unmasked || (t < lim[nt] && t >= t_lo)) ? pv[i] * r.vsc[h][i] : 0.f;   // fold the V scale into p
          }
        }
        if constexpr (I8V) {   // fp16 parts for the fp16 V operand
          ph[h][0] = pack_f16x2(pv[0], pv[1]);
          ph[h][1] = pack_f16x2(pv[2], pv[3]);
          if constexpr (!P1) {
            pl[h][0] = pack_f16x2(pv[0] - f16_lo(ph[h][0]), pv[1] - f16_hi(ph[h][0]));
            pl[h][1] = pack_f16x2(pv[2] - f16_lo(ph[h][1]), pv[3] - f16_hi(ph[h][1]));
          }
        } else {
          ph[h][0] = pack_bf16x2(pv[0], pv[1]);
          ph[h][1] = pack_bf16x2(pv[2], pv[3]);
          if constexpr (!P1) {
            pl[h][0] = pack_bf16x2(pv[0] - bf16_lo(ph[h][0]), pv[1] - bf16_hi(ph[h][0]));
            pl[h][1] = pack_bf16x2(pv[2] - bf16_lo(ph[h][1]), pv[3] - bf16_hi(ph[h][1]));
          }
        }
      }
      if constexpr (I8V) {
        // the sum the 1152 offset of V is taken back with: that of the p the
        // products use, which is also the softmax denominator
        psum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            psum += f16_lo(ph[h][e]) + f16_hi(ph[h][e]);
            if constexpr (!P1) psum += f16_lo(pl[h][e]) + f16_hi(pl[h][e]);
          }
      }
      if constexpr (I4 || (P1 && !I8V && KVT != PKV_KV_INT8)) {
        // INT4: the sum the 136 offset of V is taken back with; with one
        // part, the sum of the rounded p: that of the p the products use,
        // which is also the softmax denominator
        psum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            psum += bf16_lo(ph[h][e]) + bf16_hi(ph[h][e]);
            if constexpr (!P1) psum += bf16_lo(pl[h][e]) + bf16_hi(pl[h][e]);
          }
      }
      l_run[nt] = l_run[nt] * alpha[nt] + psum;
      pop[nt] = __builtin_bit_cast(bf16x8, u32x4{ph[0][0], ph[0][1], ph[1][0], ph[1][1]});
      if constexpr (!P1) pop_lo[nt] = __builtin_bit_cast(bf16x8, u32x4{pl[0][0], pl[0][1], pl[1][0], pl[1][1]});
    }
#pragma unroll
    for (int cc = 0; cc < T::NC; ++cc) {
      uint32_t a0, a1, a2, a3;
      if constexpr (I4) {
        // word cc / 2 of the V piece: pairs (cc % 2) and 2 + (cc % 2) are
        // tokens 0, 1 and 2, 3 of the group, dim 16 cc + row
        const uint32_t w0 = r.v[0][0][cc >> 1], w1 = r.v[1][0][cc >> 1];
        a0 = int4_pair(w0, cc & 1);
        a1 = int4_pair(w0, 2 + (cc & 1));
        a2 = int4_pair(w1, cc & 1);
        a3 = int4_pair(w1, 2 + (cc & 1));
      } else if constexpr (I8V) {
        const int u = cc >> 2, e = cc & 3;
        a0 = int8x2_to_f16x2<false>(r.v[0][u][e]);
        a1 = int8x2_to_f16x2<true>(r.v[0][u][e]);
        a2 = int8x2_to_f16x2<false>(r.v[1][u][e]);
        a3 = int8x2_to_f16x2<true>(r.v[1][u][e]);
      } else if constexpr (E == 2) {
        const u32x4 q4 = r.v[cc / T::VLOADS][cc % T::VLOADS];   // the operand quad (issue_step_bf16)
        a0 = q4[0];
        a1 = q4[1];
        a2 = q4[2];
        a3 = q4[3];
      } else {
        const int u = cc >> 2, e = cc & 3;
        widen4<KVT>(r.v[0][u][e], a0, a1);
        widen4<KVT>(r.v[1][u][e], a2, a3);
      }
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{a0, a1, a2, a3});
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (I8V) {
          acc[nt][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va),
                                                               __builtin_bit_cast(f16x8, pop[nt]), acc[nt][cc], 0, 0, 0);
          if constexpr (!P1)
            acc[nt][cc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va),
                                                                 __builtin_bit_cast(f16x8, pop_lo[nt]), acc[nt][cc], 0, 0, 0);
        } else {
          acc[nt][cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop[nt], acc[nt][cc], 0, 0, 0);
          if constexpr (!P1) acc[nt][cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop_lo[nt], acc[nt][cc], 0, 0, 0);
        }
      }
    }
  };

  // NB - 1 steps in flight ahead of the one computed.  Every iteration issues
  // the same loads (a step past the end reads a tile the table clamps into
  // the pool, unused) so that each wait covers exactly one step's loads.
  StepRegs<D, KVT> r[NB];
  auto issue = [&](StepRegs<D, KVT>& rr, int tok0) __attribute__((always_inline)) {
    if constexpr (I4)
      issue_step_int4<D, B>(rr, p, bt_row, g, tok0, lane);
    else if constexpr (E == 2)
      issue_step_bf16<D, B>(rr, p, bt_row, g, tok0, lane);
    else
      issue_step<D, KVT, B>(rr, p, bt_row, g, tok0, 0, lane);
  };
  static_for<NB - 1>([&](auto b) __attribute__((always_inline)) { issue(r[b], (s0 + (int)b) * kStep); });
  int i = s0;
  while (i < nsteps) {
    static_for<NB>([&](auto b) __attribute__((always_inline)) {   // buffer indices are constants
      if (i < nsteps) {
        issue(r[(b + NB - 1) % NB], (i + NB - 1) * kStep);
        compute(r[b], i * kStep);
        ++i;
      }
    });
  }

  // outputs: column `row` of tile nt; this lane holds dims acc_dim(cc, j, .).
  // The shared-prefix pass writes them, and the column's (m, l), as this
  // wave's partial into LDS.
  constexpr int kPartFloats = SH ? kNW * NT * 16 * D : 1;
  __shared__ __attribute__((aligned(16))) float lds_o[kPartFloats];
  __shared__ f32x2 lds_ml[SH ? kNW * NT * 16 : 1];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int cl = 16 * nt + row;
    const float L = sum_x32(sum_x16(l_run[nt]));
    if (cl >= cols) continue;
    const int cq = c0 + cl;
    float* orow = p.out + ((int64_t)(q0 + cq / p.G) * p.Hq + g * p.G + cq % p.G) * D;
    float* prow = lds_o + ((w * NT + nt) * 16 + row) * D;
    auto put = [&](int d, f32x4 v) __attribute__((always_inline)) {   // dims d .. d + 3
      if constexpr (SH)
        *reinterpret_cast<f32x4*>(prow + d) = v;
      else
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(orow + d));
    };
    const float inv = L > 0.f ? 1.f / L : 0.f;   // no key at all (position < 0): zero row
    float o[T::NC][4];
#pragma unroll
    for (int cc = 0; cc < T::NC; ++cc)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const int d = acc_dim<AL>(cc, j, i2);
        // INT4: the V operand held 136 + code
        const float a = I4 ? acc[nt][cc][i2] - kInt4Bias * L
                           : (I8V ? acc[nt][cc][i2] - kInt8Bias * L : acc[nt][cc][i2]);
        o[cc][i2] = a * inv * (p.vs_ch ? p.vs_ch[g * D + d] : p.out_scale);
      }
    if constexpr (I4) {
      // tile cc holds dims 16 cc + 4j + {0 .. 3}
#pragma unroll
      for (int cc = 0; cc < T::NC; ++cc) put(16 * cc + 4 * j, f32x4{o[cc][0], o[cc][1], o[cc][2], o[cc][3]});
    } else if constexpr (E == 2) {
      // tiles 2u, 2u + 1 hold dims 32u + 8j + 2 i2 + {0, 1}: 8 consecutive floats
#pragma unroll
      for (int u = 0; u < T::NC / 2; ++u) {
        put(32 * u + 8 * j, f32x4{o[2 * u][0], o[2 * u + 1][0], o[2 * u][1], o[2 * u + 1][1]});
        put(32 * u + 8 * j + 4, f32x4{o[2 * u][2], o[2 * u + 1][2], o[2 * u][3], o[2 * u + 1][3]});
      }
    } else {
      // tiles 4u .. 4u + 3 hold dims 64u + 16j + 4 i2 + {0 .. 3}
#pragma unroll
      for (int u = 0; u < T::NC / 4; ++u)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
          put(64 * u + 16 * j + 4 * i2, f32x4{o[4 * u][i2], o[4 * u + 1][i2], o[4 * u + 2][i2], o[4 * u + 3][i2]});
    }
    if constexpr (SH) {
      if (j == 0) lds_ml[(w * NT + nt) * 16 + row] = f32x2{m_run[nt], L};
    }
  }
  if constexpr (SH) {
    // Wave nt (< NT) merges tile nt's columns: the four waves' partials and
    // the result of the other positions in out.  With (m, l) per part
    // (reference max of the scaled logits in log2 units, sum relative to
    // it; l = 0 for a part that attended nothing), weight w = l 2^(m - M)
    // over M the largest m of a non-empty part; out = sum w o / sum w, zero
    // when every part is empty.  Lane (j, row): column row, dims j D / 4 ..
    __syncthreads();
    if (w >= NT) return;
    constexpr int DL = D / 4;
    const int cl = 16 * w + row;
    if (cl >= cols) return;
    const int cq = c0 + cl;
    const int64_t oi = (int64_t)(cq / p.G) * p.Hq + g * p.G + cq % p.G;
    float* orow = p.out + oi * D + j * DL;
    const f32x2 mls = *reinterpret_cast<const f32x2*>(pp.merge_ml + oi * 2);
    f32x4 a[DL / 4];
#pragma unroll
    for (int u = 0; u < DL / 4; ++u) a[u] = *reinterpret_cast<const f32x4*>(orow + 4 * u);
    f32x2 ml[kNW];
    float M = mls[1] > 0.f ? mls[0] : -INFINITY;
#pragma unroll
    for (int k = 0; k < kNW; ++k) {
      ml[k] = lds_ml[(k * NT + w) * 16 + row];
      if (ml[k][1] > 0.f) M = fmaxf(M, ml[k][0]);
    }
    const float ws = mls[1] > 0.f ? mls[1] * __builtin_amdgcn_exp2f(mls[0] - M) : 0.f;
    float W = ws;
#pragma unroll
    for (int u = 0; u < DL / 4; ++u) a[u] = a[u] * ws;
#pragma unroll
    for (int k = 0; k < kNW; ++k) {
      const float wk = ml[k][1] > 0.f ? ml[k][1] * __builtin_amdgcn_exp2f(ml[k][0] - M) : 0.f;
      W += wk;
      const float* src = lds_o + ((k * NT + w) * 16 + row) * D + j * DL;
#pragma unroll
      for (int u = 0; u < DL / 4; ++u) a[u] += wk * *reinterpret_cast<const f32x4*>(src + 4 * u);
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int u = 0; u < DL / 4; ++u) *reinterpret_cast<f32x4*>(orow + 4 * u) = a[u] * inv;
  }
}

template <int D, int KVT, int B, bool P1>
__global__ __launch_bounds__(kWave * kNW) __attribute__((amdgpu_waves_per_eu(kPrefillWavesPerSimd, kPrefillWavesPerSimd)))
void pa_prefill_kernel(const PrefillParams pp) {
  prefill_body<D, KVT, B, prefill_nt<D, KVT, B>(), kPrefillBuf, false, P1>(pp);
}

// The shared-prefix pass of a decode: one wave per SIMD holding kPrefixBuf
// steps of K/V (a wave streams one key chunk, a few steps, so their loads
// are kept in flight rather than covered by a second wave on the SIMD).
template <int D, int KVT, int B>
__global__ __launch_bounds__(kWave * kNW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void pa_prefix_kernel(const PrefillParams pp) {
  prefill_body<D, KVT, B, prefill_nt<D, KVT, B>(), kPrefixBuf, true, false>(pp);
}

// prefill_nt() of the variant the call runs
int prefill_tiles_per_wave(int D, int kvt, int B) {
  return with_variant<true>(D, kvt, B, [](auto dc, auto kc, auto bc) {
    return prefill_nt<decltype(dc)::value, decltype(kc)::value, decltype(bc)::value>();
  });
}

hipError_t launch_prefill(const PrefillParams& p, int D, int kvt, int B, int grid, bool one_part,
                          hipStream_t stream) {
  return with_variant<true>(D, kvt, B, [&](auto dc, auto kc, auto bc) {
    constexpr int D_ = decltype(dc)::value, K_ = decltype(kc)::value, B_ = decltype(bc)::value;
    if (one_part)
      hipLaunchKernelGGL((pa_prefill_kernel<D_, K_, B_, true>), dim3(grid), dim3(kWave * kNW), 0, stream, p);
    else
      hipLaunchKernelGGL((pa_prefill_kernel<D_, K_, B_, false>), dim3(grid), dim3(kWave * kNW), 0, stream, p);
    return hipGetLastError();
  });
}

hipError_t launch_prefix(const PrefillParams& p, int D, int kvt, int B, int grid, hipStream_t stream) {
  return with_variant<true>(D, kvt, B, [&](auto dc, auto kc, auto bc) {
    hipLaunchKernelGGL((pa_prefix_kernel<decltype(dc)::value, decltype(kc)::value, decltype(bc)::value>),
                       dim3(grid), dim3(kWave * kNW), 0, stream, p);
    return hipGetLastError();
  });
}

}  // namespace

// A decode step as a prefill of one token per sequence: the single-pass
// decode of storage types the single-pass decode kernel does not read (INT4).
hipError_t launch_prefill_as_decode(const PrefillDecodeArgs& a, hipStream_t stream) {
  const pkv_pool_config& c = a.pool->cfg;
  const int32_t G = a.num_q_heads / c.num_kv_heads;
  const int64_t span = 16 * prefill_tiles_per_wave(c.head_dim, c.kv_dtype, c.block_size) * kNW;
  const int64_t tiles = (G + span - 1) / span;
  const int64_t items = (int64_t)a.num_seqs * c.num_kv_heads * tiles;
  if (items > INT32_MAX / 2) return hipErrorInvalidValue;
  PrefillParams pp{};
  DecodeParams& p = pp.d;
  p.q = a.q;
  p.q_stride = a.q_stride;
  p.vs_ch = a.vs_ch;
  p.out = a.out;
  p.k = static_cast<char*>(a.pool->k) + (uint64_t)a.layer * a.pool->layer_bytes;
  p.v = static_cast<char*>(a.pool->v) + (uint64_t)a.layer * a.pool->layer_bytes;
  p.ks = a.ks;
  p.vs = a.vs;
  p.bt = a.block_tables;
  p.ctx = a.context_lens;
  p.W = a.table_width;
  p.S = a.num_seqs;
  p.Hq = a.num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = G;
  p.QT = 1;
  p.num_blocks = c.num_blocks;
  p.num_items = (int32_t)items;
  p.win = a.sliding_window;
  p.qk_scale = a.qk_scale;
  p.out_scale = a.out_scale;
  pp.qstart = nullptr;
  pp.tiles = (int32_t)tiles;
  pp.T = a.num_seqs;
  pp.maxq = 1;
  return launch_prefill(pp, c.head_dim, c.kv_dtype, c.block_size, (int)((items + 7) / 8 * 8), false, stream);
}

// Geometry of the shared-prefix pass: workgroups of 16 prefill_nt()
// columns of one KV head, whose four waves split the prefix's steps evenly.
bool prefix_pass_geometry(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t kv_dtype, int32_t block_size, int32_t prefix_len, PrefixPassGeometry* g) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || prefix_len <= 0) return false;
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t ncol = (int64_t)num_seqs * G;
  const int64_t cols = 16 * (int64_t)prefill_tiles_per_wave(head_dim, kv_dtype, block_size);
  const int64_t tiles = (ncol + cols - 1) / cols;
  const int64_t steps = ((int64_t)prefix_len + kStep - 1) / kStep;
  const int64_t items = (int64_t)num_kv_heads * tiles;
  if (items > INT32_MAX / 2) return false;
  g->tiles = (int32_t)tiles;
  g->chunk_len = (int32_t)((steps + kNW - 1) / kNW * kStep);
  return true;
}

hipError_t launch_prefix_pass(const PrefixPassArgs& a, hipStream_t stream) {
  const pkv_pool_config& c = a.d.pool->cfg;
  const int64_t items = (int64_t)c.num_kv_heads * a.geo.tiles;
  PrefillParams pp{};
  DecodeParams& p = pp.d;
  p.q = a.d.q;
  p.q_stride = a.d.q_stride;
  p.vs_ch = a.d.vs_ch;
  p.out = a.d.out;
  p.k = static_cast<char*>(a.d.pool->k) + (uint64_t)a.d.layer * a.d.pool->layer_bytes;
  p.v = static_cast<char*>(a.d.pool->v) + (uint64_t)a.d.layer * a.d.pool->layer_bytes;
  p.ks = a.d.ks;
  p.vs = a.d.vs;
  p.bt = a.d.block_tables;
  p.ctx = a.d.context_lens;
  p.W = a.d.table_width;
  p.S = a.d.num_seqs;
  p.Hq = a.d.num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = a.d.num_q_heads / c.num_kv_heads;
  p.QT = 1;
  p.num_blocks = c.num_blocks;
  p.num_items = (int32_t)items;
  p.win = 0;
  p.qk_scale = a.d.qk_scale;
  p.out_scale = a.d.out_scale;
  pp.qstart = nullptr;
  pp.tiles = a.geo.tiles;
  pp.T = a.d.num_seqs;
  pp.maxq = 1;
  pp.merge_ml = a.merge_ml;
  pp.prefix_len = a.prefix_len;
  pp.chunk_len = a.geo.chunk_len;
  return launch_prefix(pp, c.head_dim, c.kv_dtype, c.block_size, (int)((items + 7) / 8 * 8), stream);
}

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status paged_attn_prefill_ex(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                            const int32_t* block_tables, int32_t table_width,
                                            const int32_t* context_lens, const int32_t* query_start,
                                            int32_t num_seqs, int32_t num_queries, int32_t max_query_len,
                                            int32_t num_q_heads, float scale, int32_t kv_dtype,
                                            const pkv_kv_scales* kv_scales, uint32_t flags, hipStream_t stream) {
  if (flags & ~PKV_PREFILL_P_ONE_PART) {
    set_error("unknown prefill flags 0x%x", flags);
    return PKV_ERR_INVALID;
  }
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  const pkv_pool_config& c = pool->cfg;
  if (kv_dtype != c.kv_dtype) {
    set_error("kv_dtype %d does not match the pool's %d", kv_dtype, c.kv_dtype);
    return PKV_ERR_INVALID;
  }
  if (layer < 0 || layer >= c.num_layers) {
    set_error("layer %d outside [0, %d)", layer, c.num_layers);
    return PKV_ERR_INVALID;
  }
  if (num_seqs < 0 || num_queries < 0 || max_query_len < 0)
    return fail(PKV_ERR_INVALID, "num_seqs, num_queries and max_query_len must not be negative");
  if (num_seqs == 0 || num_queries == 0 || max_query_len == 0) { clear_error(); return PKV_OK; }
  if (!out || !q || !block_tables || !context_lens || !query_start) return fail(PKV_ERR_INVALID, "NULL device pointer");
  if (num_q_heads <= 0 || num_q_heads % c.num_kv_heads != 0) {
    set_error("num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads, c.num_kv_heads);
    return PKV_ERR_INVALID;
  }
  if (table_width <= 0) return fail(PKV_ERR_INVALID, "table_width must be positive");
  if ((int64_t)table_width * c.block_size > INT32_MAX / 2) return fail(PKV_ERR_INVALID, "table_width too large");
  if (!(scale > 0.f) || !(scale < INFINITY)) return fail(PKV_ERR_INVALID, "scale must be positive and finite");
  if (c.head_dim != 64 && c.head_dim != 128) {
    set_error("head_dim %d not built (64, 128)", c.head_dim);
    return PKV_ERR_UNSUPPORTED;
  }
  if (c.block_size != 8 && c.block_size != 16 && c.block_size != 32) {
    set_error("block_size %d not built (8, 16, 32)", c.block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (((uintptr_t)q) % 16 || ((uintptr_t)out) % 16) return fail(PKV_ERR_INVALID, "q and out must be 16-byte aligned");
  float ksc = 1.f, vsc = 1.f;
  if (tensor_scales(c.kv_dtype, kv_scales, &ksc, &vsc) != PKV_OK) return PKV_ERR_INVALID;
  // K channel scales (folded into the query); the pool's V channel scales,
  // where it has them, multiply the output
  const bool channel = has_k_channel_scales(c.kv_dtype);
  if (channel && (const void*)out == q)
    return fail(PKV_ERR_INVALID, "out must not alias q for storage with per-channel scales");
  const int32_t G = num_q_heads / c.num_kv_heads;
  const int64_t span = 16 * prefill_tiles_per_wave(c.head_dim, c.kv_dtype, c.block_size) * kNW;   // columns per workgroup
  const int64_t tiles = ((int64_t)max_query_len * G + span - 1) / span;
  const int64_t items = (int64_t)num_seqs * c.num_kv_heads * tiles;
  if (items > INT32_MAX / 2) return fail(PKV_ERR_INVALID, "too many query tiles in one call");
  const uint64_t scale_layer = channel ? (uint64_t)c.num_kv_heads * c.head_dim
                                      : (uint64_t)c.num_blocks * c.num_kv_heads * c.block_size;
  float* ksl = pool->k_scale ? pool->k_scale + layer * scale_layer : nullptr;
  float* vsl = pool->v_scale ? pool->v_scale + layer * scale_layer : nullptr;
  const uint16_t* qk = static_cast<const uint16_t*>(q);
  int32_t q_stride = c.head_dim;
  if (channel) {   // the K channel scales folded into the query, written into the output rows first
    const int64_t n = (int64_t)num_queries * num_q_heads * c.head_dim;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > INT32_MAX) return fail(PKV_ERR_INVALID, "too many queries in one call");
    hipLaunchKernelGGL(fold_q_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, qk,
                       reinterpret_cast<uint16_t*>(out), ksl, n, num_q_heads, G, c.head_dim);
    qk = reinterpret_cast<const uint16_t*>(out);
    q_stride = 2 * c.head_dim;
  }
  PrefillParams pp{};
  DecodeParams& p = pp.d;
  p.q = qk;
  p.q_stride = q_stride;
  p.vs_ch = channel ? vsl : nullptr;
  p.out = out;
  p.k = static_cast<char*>(pool->k) + (uint64_t)layer * pool->layer_bytes;
  p.v = static_cast<char*>(pool->v) + (uint64_t)layer * pool->layer_bytes;
  p.ks = ksl;
  p.vs = vsl;
  p.bt = block_tables;
  p.ctx = context_lens;
  p.W = table_width;
  p.S = num_seqs;
  p.Hq = num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = G;
  p.QT = 1;
  p.num_blocks = c.num_blocks;
  p.num_items = (int32_t)items;
  p.win = 0;
  p.qk_scale = scale * kLog2e * ksc;
  p.out_scale = vsc;
  pp.qstart = query_start;
  pp.tiles = (int32_t)tiles;
  pp.T = num_queries;
  pp.maxq = max_query_len;
  const hipError_t e = launch_prefill(pp, c.head_dim, c.kv_dtype, c.block_size, (int)((items + 7) / 8 * 8),
                                      (flags & PKV_PREFILL_P_ONE_PART) != 0, stream);
  if (e != hipSuccess) {
    set_error("paged_attn_prefill launch failed: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  clear_error();
  return PKV_OK;
}

extern "C" pkv_status paged_attn_prefill(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                         const int32_t* block_tables, int32_t table_width,
                                         const int32_t* context_lens, const int32_t* query_start,
                                         int32_t num_seqs, int32_t num_queries, int32_t max_query_len,
                                         int32_t num_q_heads, float scale, int32_t kv_dtype,
                                         const pkv_kv_scales* kv_scales, hipStream_t stream) {
  return paged_attn_prefill_ex(out, q, pool, layer, block_tables, table_width, context_lens, query_start, num_seqs,
                               num_queries, max_query_len, num_q_heads, scale, kv_dtype, kv_scales, 0u, stream);
}
