// Paged decode attention for gfx950 (CDNA4).
//
// For each sequence s and query head h the kernel computes
//     out[s][h] = softmax(scale * q[s][h] . K^T) V
// over the ctx_s cached tokens of KV head h / G (bjdmk.com.cn article, §2.1),
// fetching each token's K/V through the sequence's block table ("KV Cache
// 原理与 PagedAttention", §三 工作方式 step 4).  Query heads sharing a KV head
// (same page, §一 GQA / MQA) are served by one workgroup so their K/V is read
// from HBM once.  8-bit K/V is widened exactly to bf16 and its scale applied in
// fp32 before it meets q or p (same page, §四: dequantise before compute).
//
// Work decomposition
//   workgroup  = (sequence, KV head, tile of <= 16 query heads, partition)
//   wavefront  = every NW-th "step" of 32 consecutive tokens of the partition
//   step       = two 16-token chunks; each chunk is one 16x16 matrix-core tile
// Per step a wavefront
//   1. loads the chunks' K tiles (1 KB contiguous per load instruction) and V
//      tiles straight into matrix-core operand registers, one step ahead;
//   2. computes logits[16 tokens][16 heads] per chunk with
//      v_mfma_f32_16x16x32_bf16 (A = K rows, B = the query group);
//   3. updates a running max / sum per head (online softmax, exp2 domain);
//   4. accumulates acc^T[d][head] += V^T[d][32 tokens] . P[32 tokens][head]
//      with 16x16x32 MFMAs per 16 dims (P split into bf16 hi and lo parts):
//      the logits' register layout is exactly the B-operand layout of this
//      product, so P needs no shuffle.
// Waves then merge their (max, sum, acc) through LDS.  With one partition the
// workgroup writes the normalised output; otherwise it writes the partition's
// (max, sum, acc) and pa_reduce_kernel merges the partitions:
//     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWave = 64;
constexpr int kNW = 4;            // wavefronts per workgroup
constexpr int kStep = 32;         // tokens per step
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DecodeParams {
  const uint16_t* q;          // [S][Hq][D] bf16
  float* out;                 // [S][Hq][D]          (single pass)
  float* part_acc;            // [S][Hq][NP][D]      (split)
  float* part_ml;             // [S][Hq][NP][2]      (split: max, sum)
  const char* k;              // this layer's K region
  const char* v;              // this layer's V region
  const float* ks;            // this layer's K scales (int8) or null
  const float* vs;            // this layer's V scales (int8) or null
  const int32_t* bt;          // [S][W]
  const int32_t* ctx;         // [S]
  int32_t W, S, Hq, Hkv, G, QT, NP, P, num_blocks;
  int32_t num_items;          // S * Hkv * QT * NP
  float qk_scale;             // softmax scale * log2(e) (* fp8 k scale)
  float out_scale;            // fp8 v scale, else 1
};

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

// Four bytes of w (byte i = token i) -> 4 bf16 in 2 dwords.
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
                                           int g, int tok0, int ctx_lim, int lane) {
  using T = Tile<D, KVT>;
  constexpr int E = T::E;
  const int row = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = tok0 + 16 * h;                   // first token of the chunk (multiple of 16)
    int lb = t / B;
    lb = lb < p.W ? lb : p.W - 1;                  // never index past the table row
    int phys = bt_row[lb];
    phys = phys < 0 ? 0 : (phys >= p.num_blocks ? p.num_blocks - 1 : phys);  // stay inside the pool
    const int toff = t % B;                        // chunk offset inside the block (0 or 16)
    const int64_t tile = ((int64_t)phys * p.Hkv + g) * (int64_t)(B * D * E);
    const char* kt = p.k + tile;
    const char* vt = p.v + tile;
    // K: piece c holds dims [X*c, X*c+X) of all B tokens, 16 bytes per token
#pragma unroll
    for (int u = 0; u < T::KLOADS; ++u) r.k[h][u] = ld16(kt + ((int64_t)((4 * u + j) * B + toff + row)) * 16);
    // V: token group (toff/4 + j), 4 tokens x dims as 4E-byte words
    const int grp = (toff >> 2) + j;
#pragma unroll
    for (int u = 0; u < T::VLOADS; ++u) {
      const int d = (E == 2) ? (32 * u + 2 * row) : (64 * u + 4 * row);
      r.v[h][u] = ld16(vt + ((int64_t)(grp * D + d)) * 4 * E);
    }
    if constexpr (KVT == PKV_KV_INT8) {
      const int64_t so = ((int64_t)phys * p.Hkv + g) * B + toff + 4 * j;
      r.ksc[h] = *reinterpret_cast<const f32x4*>(p.ks + so);
      r.vsc[h] = *reinterpret_cast<const f32x4*>(p.vs + so);
    }
  }
  (void)ctx_lim;
}

template <int D, int KVT, int B>
__global__ __launch_bounds__(kWave * kNW) void pa_decode_kernel(const DecodeParams p) {
  using T = Tile<D, KVT>;
  constexpr int E = T::E;
  __shared__ float sm_ml[kNW][2][16];
  __shared__ float sm_acc[kNW][16][D + 4];

  // ---- which item: XCD-aware order so that consecutive items (partitions of
  // one sequence and KV head) run on the same XCD
  const int nwg = (int)gridDim.x;
  const int xcd = (int)blockIdx.x % 8;
  const int per_xcd = (nwg + 7) / 8;
  const int item = xcd * per_xcd + (int)blockIdx.x / 8;
  if (item >= p.num_items) return;
  const int part = item % p.NP;
  const int qt = (item / p.NP) % p.QT;
  const int g = (item / (p.NP * p.QT)) % p.Hkv;
  const int s = item / (p.NP * p.QT * p.Hkv);

  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int row = lane & 15;
  const int j = lane >> 4;
  const int gt = min(16, p.G - qt * 16);           // query heads in this tile
  const int h0 = g * p.G + qt * 16;                // first query head of the tile

  int ctx = p.ctx[s];
  ctx = ctx < 0 ? 0 : (ctx > p.W * B ? p.W * B : ctx);
  const int t_begin = p.P > 0 ? part * p.P : 0;
  const int t_end = p.P > 0 ? min(t_begin + p.P, ctx) : ctx;
  if (t_begin >= t_end) {
    if (p.P == 0) {  // empty context: zero output rows
      for (int i = threadIdx.x; i < gt * D; i += blockDim.x)
        p.out[((int64_t)s * p.Hq + h0 + i / D) * D + i % D] = 0.f;
    }
    return;  // split: the reduce kernel ignores partitions past ctx
  }
  const int nsteps = (t_end - t_begin + kStep - 1) / kStep;
  const int32_t* bt_row = p.bt + (int64_t)s * p.W;

  // ---- query tile as the B operand of q.K: lane (j, row) holds head row,
  // dims d0(kk, j) .. +7 (the same dims the K operand of that lane slot holds)
  bf16x8 qop[T::KK];
  {
    const bool valid = row < gt;
    const uint16_t* qh = p.q + ((int64_t)s * p.Hq + h0 + (valid ? row : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
      const int d0 = (E == 2) ? (32 * kk + 8 * j) : (64 * (kk >> 1) + 16 * j + 8 * (kk & 1));
      u32x4 raw = *reinterpret_cast<const u32x4*>(qh + d0);
      if (!valid) raw = u32x4{0, 0, 0, 0};
      qop[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x4 acc[T::NC];
#pragma unroll
  for (int c = 0; c < T::NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of scaled logits (log2 domain), head `row`
  float l_run = 0.f;         // running sum of p over this lane's tokens

  auto compute = [&](const StepRegs<D, KVT>& r, int tok0) {
    // logits: C[token 4j+i][head row] per chunk
    f32x4 z[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        bf16x8 a;
        if constexpr (E == 2) {
          a = __builtin_bit_cast(bf16x8, r.k[h][kk]);
        } else {
          const u32x4 wv = r.k[h][kk >> 1];
          a = (kk & 1) ? widen8<KVT>(wv[2], wv[3]) : widen8<KVT>(wv[0], wv[1]);
        }
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[kk], c, 0, 0, 0);
      }
      z[h] = c;
    }
    // scale, mask, max
    float mloc = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tok0 + 16 * h + 4 * j + i;
        float zz = z[h][i] * p.qk_scale;
        if constexpr (KVT == PKV_KV_INT8) zz *= r.ksc[h][i];
        zz = t < t_end ? zz : -INFINITY;
        z[h][i] = zz;
        mloc = fmaxf(mloc, zz);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    // p enters the P.V product as bf16 hi + lo parts (two MFMAs), so the
    // product carries ~16 significant bits of p instead of 8
    uint32_t ph[2][2], pl[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(z[h][i] - m_new);
        psum += pv[i];
        if constexpr (KVT == PKV_KV_INT8) {
          const int t = tok0 + 16 * h + 4 * j + i;
          pv[i] = t < t_end ? pv[i] * r.vsc[h][i] : 0.f;   // fold the V scale into p
        }
      }
      ph[h][0] = pack_bf16x2(pv[0], pv[1]);
      ph[h][1] = pack_bf16x2(pv[2], pv[3]);
      pl[h][0] = pack_bf16x2(pv[0] - bf16_lo(ph[h][0]), pv[1] - bf16_hi(ph[h][0]));
      pl[h][1] = pack_bf16x2(pv[2] - bf16_lo(ph[h][1]), pv[3] - bf16_hi(ph[h][1]));
    }
    l_run = l_run * alpha + psum;
    const bf16x8 pop = __builtin_bit_cast(bf16x8, u32x4{ph[0][0], ph[0][1], ph[1][0], ph[1][1]});
    const bf16x8 pop_lo = __builtin_bit_cast(bf16x8, u32x4{pl[0][0], pl[0][1], pl[1][0], pl[1][1]});
    // zero V of masked tokens so that garbage (NaN/inf bit patterns in unwritten
    // slots) cannot reach the accumulator through 0 * NaN
    const bool tail = tok0 + kStep > t_end;
    // P.V: A = V^T[d][tokens], slots 0..3 = chunk 0 tokens 4j..4j+3, 4..7 = chunk 1
#pragma unroll
    for (int c = 0; c < T::NC; ++c) {
      uint32_t a0, a1, a2, a3;
      if constexpr (E == 2) {
        const int u = c >> 1, e = c & 1;   // load u holds dims (32u + 2row, +1) x 4 tokens
        a0 = r.v[0][u][2 * e];
        a1 = r.v[0][u][2 * e + 1];
        a2 = r.v[1][u][2 * e];
        a3 = r.v[1][u][2 * e + 1];
      } else {
        const int u = c >> 2, e = c & 3;   // load u holds dims (64u + 4row .. +3) x 4 tokens
        widen4<KVT>(r.v[0][u][e], a0, a1);
        widen4<KVT>(r.v[1][u][e], a2, a3);
      }
      if (tail) {
        const int tb0 = tok0 + 4 * j, tb1 = tok0 + 16 + 4 * j;
        a0 = tb0 + 0 < t_end ? (tb0 + 1 < t_end ? a0 : (a0 & 0xffffu)) : 0u;
        a1 = tb0 + 2 < t_end ? (tb0 + 3 < t_end ? a1 : (a1 & 0xffffu)) : 0u;
        a2 = tb1 + 0 < t_end ? (tb1 + 1 < t_end ? a2 : (a2 & 0xffffu)) : 0u;
        a3 = tb1 + 2 < t_end ? (tb1 + 3 < t_end ? a3 : (a3 & 0xffffu)) : 0u;
      }
      const bf16x8 aop = __builtin_bit_cast(bf16x8, u32x4{a0, a1, a2, a3});
      acc[c] = acc[c] * alpha;
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, pop, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, pop_lo, acc[c], 0, 0, 0);
    }
  };

  // ---- main loop: wave w takes steps w, w+NW, ...; loads run one step ahead
  StepRegs<D, KVT> r0, r1;
  int i = w;
  if (i < nsteps) issue_step<D, KVT, B>(r0, p, bt_row, g, t_begin + i * kStep, t_end, lane);
  while (i < nsteps) {
    int nx = i + kNW;
    if (nx < nsteps) issue_step<D, KVT, B>(r1, p, bt_row, g, t_begin + nx * kStep, t_end, lane);
    compute(r0, t_begin + i * kStep);
    i = nx;
    if (i >= nsteps) break;
    nx = i + kNW;
    if (nx < nsteps) issue_step<D, KVT, B>(r0, p, bt_row, g, t_begin + nx * kStep, t_end, lane);
    compute(r1, t_begin + i * kStep);
    i = nx;
  }

  // ---- merge the waves: per head max, sum and accumulator through LDS
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (j == 0) {
    sm_ml[w][0][row] = m_run;
    sm_ml[w][1][row] = l_run;
  }
  // acc^T rows: lane (j, row) holds head `row`, dims
  //   bf16: 32u + 8j + 2i + e  (c = 2u + e)    8-bit: 64u + 16j + 4i + e (c = 4u + e)
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      int d;
      if constexpr (E == 2) d = 32 * (c >> 1) + 8 * j + 2 * i2 + (c & 1);
      else d = 64 * (c >> 2) + 16 * j + 4 * i2 + (c & 3);
      sm_acc[w][row][d] = acc[c][i2];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < gt * D; idx += blockDim.x) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, sm_ml[ww][0][hh]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      const float mw = sm_ml[ww][0][hh];
      const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f * sm_ml[ww][1][hh];
      A += f * sm_acc[ww][hh][d];
    }
    const int64_t sh = (int64_t)s * p.Hq + h0 + hh;
    if (p.P == 0) {
      p.out[sh * D + d] = A / L * p.out_scale;
    } else {
      p.part_acc[(sh * p.NP + part) * D + d] = A;
      if (d == 0) {
        p.part_ml[(sh * p.NP + part) * 2 + 0] = M;
        p.part_ml[(sh * p.NP + part) * 2 + 1] = L;
      }
    }
  }
}

// One workgroup of D threads per (sequence, query head): merge the partitions.
template <int D>
__global__ __launch_bounds__(D) void pa_reduce_kernel(float* __restrict__ out, const float* __restrict__ part_acc,
                                                      const float* __restrict__ part_ml,
                                                      const int32_t* __restrict__ ctx_lens, int32_t Hq,
                                                      int32_t NP, int32_t P, int32_t max_ctx, float out_scale) {
  const int sh = blockIdx.x;
  const int s = sh / Hq;
  const int d = threadIdx.x;
  int ctx = ctx_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
  const int np = (ctx + P - 1) / P;
  if (np == 0) {
    out[(int64_t)sh * D + d] = 0.f;
    return;
  }
  const float* ml = part_ml + (int64_t)sh * NP * 2;
  float M = -INFINITY;
  for (int k = 0; k < np; ++k) M = fmaxf(M, ml[2 * k]);
  float L = 0.f, A = 0.f;
  const float* pa = part_acc + (int64_t)sh * NP * D + d;
  for (int k = 0; k < np; ++k) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * k] - M);
    L += f * ml[2 * k + 1];
    A += f * pa[(int64_t)k * D];
  }
  out[(int64_t)sh * D + d] = A / L * out_scale;
}

template <int D, int KVT, int B>
hipError_t launch(const DecodeParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((pa_decode_kernel<D, KVT, B>), dim3(grid), dim3(kWave * kNW), 0, stream, p);
  return hipGetLastError();
}

template <int D, int KVT>
hipError_t launch_b(const DecodeParams& p, int B, int grid, hipStream_t stream) {
  return B == 16 ? launch<D, KVT, 16>(p, grid, stream) : launch<D, KVT, 32>(p, grid, stream);
}

template <int D>
hipError_t launch_kv(const DecodeParams& p, int kvt, int B, int grid, hipStream_t stream) {
  switch (kvt) {
    case PKV_KV_BF16: return launch_b<D, PKV_KV_BF16>(p, B, grid, stream);
    case PKV_KV_FP8_E5M2: return launch_b<D, PKV_KV_FP8_E5M2>(p, B, grid, stream);
    default: return launch_b<D, PKV_KV_INT8>(p, B, grid, stream);
  }
}

uint64_t part_acc_bytes(int32_t S, int32_t Hq, int32_t D, int32_t NP) {
  return align_up((uint64_t)S * Hq * NP * D * sizeof(float));
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" uint64_t paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                               int32_t table_width, int32_t block_size,
                                               int32_t partition_size) {
  if (partition_size <= 0 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || table_width <= 0 ||
      block_size <= 0)
    return 0;
  const int64_t np = ((int64_t)table_width * block_size + partition_size - 1) / partition_size;
  return part_acc_bytes(num_seqs, num_q_heads, head_dim, (int32_t)np) +
         align_up((uint64_t)num_seqs * num_q_heads * np * 2 * sizeof(float));
}

extern "C" pkv_status paged_attn_decode(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                        const int32_t* block_tables, int32_t table_width,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        float scale, int32_t kv_dtype, const pkv_kv_scales* kv_scales,
                                        int32_t partition_size, void* workspace, uint64_t workspace_bytes,
                                        hipStream_t stream) {
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
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs is negative");
  if (num_seqs == 0) { clear_error(); return PKV_OK; }
  if (!out || !q || !block_tables || !context_lens) return fail(PKV_ERR_INVALID, "NULL device pointer");
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
  if (c.block_size != 16 && c.block_size != 32) {
    set_error("block_size %d not built (16, 32)", c.block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (pool->layer_bytes > (uint64_t)INT64_MAX) return fail(PKV_ERR_INVALID, "pool too large");
  if (((uintptr_t)q) % 16 || ((uintptr_t)out) % 16) return fail(PKV_ERR_INVALID, "q and out must be 16-byte aligned");
  float ksc = 1.f, vsc = 1.f;
  if (kv_scales && c.kv_dtype == PKV_KV_FP8_E5M2) {
    ksc = kv_scales->k_scale;
    vsc = kv_scales->v_scale;
    if (!(ksc > 0.f) || !(vsc > 0.f) || !(ksc < INFINITY) || !(vsc < INFINITY))
      return fail(PKV_ERR_INVALID, "fp8 scales must be positive and finite");
  }
  const int32_t G = num_q_heads / c.num_kv_heads;
  const int32_t QT = (G + 15) / 16;
  int32_t NP = 1;
  if (partition_size != 0) {
    if (partition_size < 0 || partition_size % kStep != 0) {
      set_error("partition_size %d must be 0 or a positive multiple of %d", partition_size, kStep);
      return PKV_ERR_INVALID;
    }
    NP = (int32_t)(((int64_t)table_width * c.block_size + partition_size - 1) / partition_size);
    const uint64_t need = paged_attn_workspace_bytes(num_seqs, num_q_heads, c.head_dim, table_width, c.block_size,
                                                     partition_size);
    if (!workspace || workspace_bytes < need) {
      set_error("workspace of %llu bytes needed, got %llu", (unsigned long long)need,
                (unsigned long long)workspace_bytes);
      return PKV_ERR_INVALID;
    }
    if (((uintptr_t)workspace) % 256) return fail(PKV_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  const int64_t items = (int64_t)num_seqs * c.num_kv_heads * QT * NP;
  const int64_t grid = (items + 7) / 8 * 8;
  if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "too many work items");

  DecodeParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.out = out;
  if (partition_size != 0) {
    p.part_acc = static_cast<float*>(workspace);
    p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         part_acc_bytes(num_seqs, num_q_heads, c.head_dim, NP));
  }
  p.k = static_cast<const char*>(pool->k) + (uint64_t)layer * pool->layer_bytes;
  p.v = static_cast<const char*>(pool->v) + (uint64_t)layer * pool->layer_bytes;
  const uint64_t scale_layer = (uint64_t)c.num_blocks * c.num_kv_heads * c.block_size;
  p.ks = pool->k_scale ? pool->k_scale + layer * scale_layer : nullptr;
  p.vs = pool->v_scale ? pool->v_scale + layer * scale_layer : nullptr;
  p.bt = block_tables;
  p.ctx = context_lens;
  p.W = table_width;
  p.S = num_seqs;
  p.Hq = num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.G = G;
  p.QT = QT;
  p.NP = NP;
  p.P = partition_size;
  p.num_blocks = c.num_blocks;
  p.num_items = (int32_t)items;
  p.qk_scale = scale * kLog2e * ksc;
  p.out_scale = vsc;

  hipError_t e = c.head_dim == 64 ? launch_kv<64>(p, c.kv_dtype, c.block_size, (int)grid, stream)
                                  : launch_kv<128>(p, c.kv_dtype, c.block_size, (int)grid, stream);
  if (e == hipSuccess && partition_size != 0) {
    const int64_t rg = (int64_t)num_seqs * num_q_heads;
    const int32_t max_ctx = table_width * c.block_size;
    if (c.head_dim == 64)
      hipLaunchKernelGGL(pa_reduce_kernel<64>, dim3((uint32_t)rg), dim3(64), 0, stream, out, p.part_acc, p.part_ml,
                         context_lens, num_q_heads, NP, partition_size, max_ctx, vsc);
    else
      hipLaunchKernelGGL(pa_reduce_kernel<128>, dim3((uint32_t)rg), dim3(128), 0, stream, out, p.part_acc,
                         p.part_ml, context_lens, num_q_heads, NP, partition_size, max_ctx, vsc);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    set_error("paged_attn_decode launch failed: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  clear_error();
  return PKV_OK;
}
