// Paged decode attention for gfx950 (CDNA4).
//
// For each sequence s and query head h the kernels compute
//     out[s][h] = softmax(scale * q[s][h] . K^T) V
// over the ctx_s cached tokens of KV head h / G (bjdmk.com.cn article, §2.1),
// fetching each token's K/V through the sequence's block table ("KV Cache
// 原理与 PagedAttention", §三 工作方式 step 4).  Query heads sharing a KV head
// (same page, §一 GQA / MQA) are served together so their K/V is read from
// HBM once.  8-bit K/V is widened exactly to bf16 and its scale applied in
// fp32 before it meets q or p (same page, §四: dequantise before compute).
//
// Matrix-core formulation, per 16-token chunk of one KV head:
//   logits^T[16 tokens][16 heads] = K[16 tokens][D] . Q^T[D][16 heads]
//       v_mfma_f32_16x16x32_bf16, A = K rows, B = the query group;
//   acc^T[D][16 heads] += V^T[D][16 tokens] . P[16 tokens][16 heads]
//       v_mfma_f32_16x16x16_bf16 (one chunk) or 16x16x32 (two chunks), with P
//       split into bf16 hi and lo parts so the product carries ~16 bits of p.
// The logits' accumulator layout is exactly the B-operand layout of the P.V
// product, so P never moves between lanes.  The softmax is the streaming form
// (running max and sum per head, exp2 domain).
//
// Two launch forms:
//   partition_size == 0  pa_decode_kernel: one workgroup per (sequence, KV
//       head, tile of <= 16 query heads); its four waves split the context and
//       merge through LDS; it writes the output directly.
//   partition_size  > 0  split-context: pa_split_kernel is a persistent grid
//       sized to the GPU.  The work of all (sequence, KV head, head tile)
//       rows is laid end to end as a list of fixed-size token steps and every
//       wavefront takes one equal contiguous range of it, so all waves finish
//       together whatever the context lengths.  A wave keeps NBUF-1 steps of
//       K/V loads in flight, across row boundaries too.  It emits one partial
//       (running max m, sum l, unnormalised acc) per segment: the part of its
//       range inside one row.  The wave that completes a row combines the
//       row's partials:
//           out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,  M = max m_k.
#include <atomic>
#include <chrono>
#include <mutex>

#include "decode_common.h"

namespace pkv {
namespace {

// =====================================================================
// Single-pass kernel (partition_size == 0); its parameter block and step
// loads are in decode_common.h
// =====================================================================
template <int D, int KVT, int B>
__global__ __launch_bounds__(kWave * kNW) void pa_decode_kernel(const DecodeParams p) {
  using T = Tile<D, KVT>;
  constexpr int E = T::E;
  __shared__ float sm_ml[kNW][2][16];
  __shared__ float sm_acc[kNW][16][D + 4];

  // XCD-aware order: consecutive items run on the same XCD
  const int nwg = (int)gridDim.x;
  const int xcd = (int)blockIdx.x % 8;
  const int per_xcd = (nwg + 7) / 8;
  const int item = xcd * per_xcd + (int)blockIdx.x / 8;
  if (item >= p.num_items) return;
  const int qt = item % p.QT;
  const int g = (item / p.QT) % p.Hkv;
  const int s = item / (p.QT * p.Hkv);

  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int row = lane & 15;
  const int j = lane >> 4;
  const int gt = min(16, p.G - qt * 16);           // query heads in this tile
  const int h0 = g * p.G + qt * 16;                // first query head of the tile

  const int t_end = clamp_ctx(p.ctx[s], p.W * B);
  if (t_end == 0) {  // empty context: zero output rows
    for (int i = threadIdx.x; i < gt * D; i += blockDim.x)
      p.out[((int64_t)s * p.Hq + h0 + i / D) * D + i % D] = 0.f;
    return;
  }
  const int nsteps = (t_end + kStep - 1) / kStep;
  const int t_lo = window_lo(t_end, p.win);
  const int32_t* bt_row = p.bt + (int64_t)s * p.W;

  // query tile as the B operand of q.K: lane (j, row) holds head row; with
  // the K channel scales folded in, set 0 is the bf16 hi part of the folded
  // query and set 1 its lo part (the next D elements of the row)
  constexpr int NQ = KVT == PKV_KV_INT8_CHANNEL ? 2 : 1;
  bf16x8 qop[NQ][T::KK];
  {
    const bool valid = row < gt;
    const uint16_t* qh = p.q + ((int64_t)s * p.Hq + h0 + (valid ? row : 0)) * p.q_stride;
#pragma unroll
    for (int n = 0; n < NQ; ++n)
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(qh + n * D + q_dim0<E>(kk, j));
        if (!valid) raw = u32x4{0, 0, 0, 0};
        qop[n][kk] = __builtin_bit_cast(bf16x8, raw);
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
#pragma unroll
        for (int n = 0; n < NQ; ++n) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[n][kk], c, 0, 0, 0);
      }
      z[h] = c;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tok0 + 16 * h + 4 * j + i;
        float zz = z[h][i] * p.qk_scale;
        if constexpr (KVT == PKV_KV_INT8) zz *= r.ksc[h][i];
        zz = (t < t_end && t >= t_lo) ? zz : -INFINITY;
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
          pv[i] = tok_in(t, t_lo, t_end) ? pv[i] * r.vsc[h][i] : 0.f;   // fold the V scale into p
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
    // slots, blocks before a window) cannot reach the accumulator through 0 * NaN
    const bool edge = tok0 + kStep > t_end || tok0 < t_lo;
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
      if (edge) {
        const int tb0 = tok0 + 4 * j, tb1 = tok0 + 16 + 4 * j;
        a0 &= tok_mask16(tb0, t_lo, t_end);
        a1 &= tok_mask16(tb0 + 2, t_lo, t_end);
        a2 &= tok_mask16(tb1, t_lo, t_end);
        a3 &= tok_mask16(tb1 + 2, t_lo, t_end);
      }
      const bf16x8 aop = __builtin_bit_cast(bf16x8, u32x4{a0, a1, a2, a3});
      acc[c] = acc[c] * alpha;
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, pop, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, pop_lo, acc[c], 0, 0, 0);
    }
  };

  // wave w takes steps i0 + w, i0 + w + NW, ... (i0: the step holding the
  // window's first position); loads run one step ahead
  StepRegs<D, KVT> r0, r1;
  int i = t_lo / kStep + w;
  if (i < nsteps) issue_step<D, KVT, B>(r0, p, bt_row, g, i * kStep, t_lo, lane);
  while (i < nsteps) {
    int nx = i + kNW;
    if (nx < nsteps) issue_step<D, KVT, B>(r1, p, bt_row, g, nx * kStep, t_lo, lane);
    compute(r0, i * kStep);
    i = nx;
    if (i >= nsteps) break;
    nx = i + kNW;
    if (nx < nsteps) issue_step<D, KVT, B>(r0, p, bt_row, g, nx * kStep, t_lo, lane);
    compute(r1, i * kStep);
    i = nx;
  }

  // merge the waves: per head max, sum and accumulator through LDS
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (j == 0) {
    sm_ml[w][0][row] = m_run;
    sm_ml[w][1][row] = l_run;
  }
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) sm_acc[w][row][acc_dim<E>(c, j, i2)] = acc[c][i2];
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
    p.out[((int64_t)s * p.Hq + h0 + hh) * D + d] = A / L * (p.vs_ch ? p.vs_ch[g * D + d] : p.out_scale);
  }
}

// =====================================================================
// Split-context persistent kernel (partition_size > 0)
// =====================================================================
// A "row" x = (sequence s, KV head g, head tile qt), numbered head-major:
// x = xi * S + s with xi = g * QT + qt (HQ = Hkv * QT values).  Row x has
// n_s = ceil(ctx_s / TS) steps of TS tokens.  The flat step list is row 0's
// steps, then row 1's, ...: all sequences of xi = 0, then of xi = 1, ...;
// row x starts at xi * T + cum_s where cum_s = sum over s' < s of n_s' and
// T = cum_S.  Each wave of the NWV takes one contiguous range of the list.
// Head-major order gives each XCD (one eighth of the list) the rows of a few
// KV heads: when sequences share prefix blocks, the prefix tiles of those
// heads fit the XCD's L2 and are fetched from memory about once, where a
// sequence-major order would stream every head's prefix through every L2.
// The grid is one workgroup of four waves per CU.  Workgroups are dispatched
// to the eight XCDs in turn (workgroup b runs on XCD b % 8), and waves are
// numbered so that XCD x holds waves [x * WX, (x + 1) * WX), WX = NWV / 8.
// Measured on MI355X, waves on odd-numbered XCDs stream 10-16% slower than
// those on even ones (it varies from board to board), so XCD x takes a share
// of the flat list proportional to kXcdWeight[x], split equally among its
// waves, and the waves finish at about the same time.  The split depends
// only on N and the grid, never on timing.
// The partials the merge combines are the segments of a row that the waves
// cover: the part of row x inside wave w's range is stored in partial slot
// x + w.  Walking the (row, wave) pairs of the flat list in order raises x or
// w (or both) at every step, so the sum is unique, and slots number at most
// rows + NWV - 1.  A wave carries its running (m, l, o) across everything it
// computes of one row: that running state after any prefix of the row's
// tokens is the merge of the partials of that prefix, so a fixed partition
// length (a partial every P tokens, merged afterwards) would give the same
// result up to rounding while adding partials for the final merge to read.
// The partition size therefore only selects this form.
// When a wave has computed its whole range it makes its partials visible
// (device-scope release) and adds, for every row it touched, the number of
// that row's steps it computed to the row's counter.  The wave whose addition
// completes the row (the sum reaches n_s) merges all of the row's partials
// into the output.  A counter is 64 bits: the call's epoch (a number the host
// draws anew for every call) above the step count, updated by compare-and-
// swap; a counter carrying any other epoch counts as zero, so the workspace
// needs no clearing between calls, whatever sizes earlier calls had.
// Row counters sit 128 bytes apart: every wave covering a row updates its
// counter at about the same time, from all eight XCDs, and counters sharing a
// cache line would serialise the updates of all their rows.
constexpr int kCounterStride = 16;   // uint64 words

struct SplitParams {
  const uint16_t* q;          // [S][Hq][D] bf16
  float* out;                 // [S][Hq][D]
  char* k;                    // this layer's K region (written only when appending)
  char* v;
  float* ks;
  float* vs;
  const uint16_t* new_k;      // appending decode: [S][Hkv][D] bf16 new tokens, else null
  const uint16_t* new_v;
  float enc_k, enc_v;         // fp8 per-tensor scales for encoding the new token
  const int32_t* bt;
  const int32_t* ctx;
  uint64_t* row_done;         // workspace: [rows][kCounterStride] (epoch << 32) | steps reported, in word 0
  float* part_ml;             // workspace: [slots][16][2]  (m, l)
  float* part_acc;            // workspace: [slots][NC][64 lanes][4]
  uint32_t acc_bytes;         // size of part_acc in bytes (< 4 GiB)
  uint32_t ml_bytes;          // size of part_ml in bytes
  int32_t W, S, Hq, Hkv, G, QT, HQ, num_blocks;
  int32_t NWV;                // waves in the grid
  int32_t win;                // sliding window (positions), 0 = whole context
  uint32_t epoch;             // this call's tag for row_done
  float qk_scale;
  float out_scale;
  const float* ks_ch;         // int8 per channel, INT4: this layer's K / V scales [Hkv][D], else null
  const float* vs_ch;         // (the K scales are folded into the query as it is loaded)
  int32_t prefix_len;         // shared-prefix decode: positions below it are left to the prefix pass, else 0
  float* ml_out;              // shared-prefix decode: [S][Hq] (m, l) of every output row, else null
};

// First attended position of a row: the sliding window's start, or, in a
// shared-prefix decode, the end of the shared prefix (the prefix pass
// attends the positions before it), and the row's first step and step count
// from there (no step when nothing is left to attend).
__device__ __forceinline__ int split_lo(int ctx, const SplitParams& p) {
  return p.prefix_len > 0 ? min(ctx, p.prefix_len) : window_lo(ctx, p.win);
}
template <int TS>
__device__ __forceinline__ int split_base(int ctx, const SplitParams& p) { return split_lo(ctx, p) / TS * TS; }
template <int TS>
__device__ __forceinline__ int split_steps(int ctx, const SplitParams& p) {
  const int lo = split_lo(ctx, p);
  return lo >= ctx ? 0 : (ctx - lo / TS * TS + TS - 1) / TS;
}

template <int D, int KVT>
struct SplitGeo {
  static constexpr bool I4 = KVT == PKV_KV_INT4;
  static constexpr bool BF = KVT == PKV_KV_BF16;
  static constexpr bool FP8 = KVT == PKV_KV_FP8_E5M2;
  static constexpr bool TOK = KVT == PKV_KV_INT8;                  // per-(token, head) scales
  static constexpr bool CHAN = KVT == PKV_KV_INT8_CHANNEL || I4;   // K channel scales folded into q
  static constexpr int E = BF ? 2 : 1;            // bytes per stored element (INT4: half a byte)
  static constexpr int CH = BF ? 1 : (I4 ? 4 : 2);   // 16-token chunks per step (8 KiB of K + V, 4 KiB for INT4)
  static constexpr int TS = 16 * CH;              // tokens per step
  static constexpr int LPC = I4 ? 1 : D * E / 64; // loads per chunk per lane, for K and for V
                                                  // (INT4: one load of D / 8 bytes)
  static constexpr int KK = D / 32;               // q.K matrix-core steps per chunk
  static constexpr int NC = D / 16;               // accumulator tiles of 16 dims
  static constexpr int QL = I4 ? 2 : E;           // query dim layout (q_dim0)
  static constexpr int AL = I4 ? 0 : E;           // accumulator dim layout (acc_dim)
  static constexpr int NQ = CHAN ? 2 : 1;         // query operand sets: the folded query as bf16 hi + lo
  static constexpr int P4 = D / 8;                // INT4: bytes per piece
  // bytes of one token's K (V) inside a tile, as an offset from the tile start
  // for a token at offset t of its block: K pieces are runs of tokens, V
  // groups of 4 tokens are stored dim by dim (see the pool layout)
  static constexpr int KTOK = I4 ? P4 : 16;
  static constexpr int VTOK = I4 ? 4 * P4 : D * E;
  static constexpr int LPS = CH * 2 * LPC + (TOK ? 2 * CH : 0);   // vector loads of one step
};

// Registers of one step: K and V loads of each chunk, and the per-token int8
// scales of the lane's four tokens per chunk.
template <int D, int KVT>
struct SplitBuf {
  using G_ = SplitGeo<D, KVT>;
  u32x4 k[G_::CH][G_::LPC];
  u32x4 v[G_::CH][G_::LPC];
  f32x4 ksc[G_::TOK ? G_::CH : 1];
  f32x4 vsc[G_::TOK ? G_::CH : 1];
};

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// The query group of one row as the B operand of q.K: lane (j, row) holds
// head row of the tile; with folded channel scales, set 0 is the bf16 hi part
// and set 1 the lo part of the folded query (q' = hi + lo to ~16 bits).
template <int KK, int NQ>
struct QRegs {
  bf16x8 q[NQ][KK];
};

template <int D, int KVT>
__device__ __forceinline__ QRegs<SplitGeo<D, KVT>::KK, SplitGeo<D, KVT>::NQ> load_q(const SplitParams& p, int s,
                                                                                    int h0, int gt, int lane) {
  using GE = SplitGeo<D, KVT>;
  const int row = lane & 15;
  const int j = lane >> 4;
  // rows past the tile's heads read a valid head; their columns are never stored
  const int h = h0 + (row < gt ? row : 0);
  const uint16_t* qh = p.q + ((int64_t)s * p.Hq + h) * D;
  QRegs<GE::KK, GE::NQ> r;
  if constexpr (GE::CHAN) {
    // the K channel scales folded into the query as it is loaded:
    // q' = fp32(q) * s_k[g][d], hi = bf16(q'), lo = bf16(q' - hi), both
    // rounded to nearest even (the query fold kernel's arithmetic)
    const float* ksc = p.ks_ch + (h / p.G) * D;
#pragma unroll
    for (int kk = 0; kk < GE::KK; ++kk) {
      const int d0 = q_dim0<GE::QL>(kk, j);
      const bf16x8 raw = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + d0));
      const f32x4 sa = *reinterpret_cast<const f32x4*>(ksc + d0);
      const f32x4 sb = *reinterpret_cast<const f32x4*>(ksc + d0 + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)raw[e] * (e < 4 ? sa[e] : sb[e - 4]);
        const __bf16 hi = (__bf16)x;
        r.q[0][kk][e] = hi;
        r.q[1][kk][e] = (__bf16)(x - (float)hi);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < GE::KK; ++kk)
      r.q[0][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + q_dim0<GE::QL>(kk, j)));
  }
  return r;
}

// INT4: the sum over all dims of the row's head's (folded) query, which the
// 136 offset of the K operand is taken back with.
template <int D, int KVT>
__device__ __forceinline__ float query_sum(const QRegs<SplitGeo<D, KVT>::KK, SplitGeo<D, KVT>::NQ>& q) {
  using GE = SplitGeo<D, KVT>;
  float a = 0.f;
#pragma unroll
  for (int n = 0; n < GE::NQ; ++n)
#pragma unroll
    for (int kk = 0; kk < GE::KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) a += (float)q.q[n][kk][e];
  return sum_x32(sum_x16(a));      // lanes of one head row hold its 4 dim slots
}

// Lane-constant byte offsets of a lane's loads inside a tile (or, for the
// int8 scales, inside a block's scale row).  K: lane (j, row) reads token
// row of the chunk, piece j (+ 4 u); V and scales: lane j reads tokens
// 4 j .. 4 j + 3, V dims by row.  With 8-token blocks a chunk covers two
// blocks: the token (group) index inside its block wraps at 8 (2 groups).
template <int D, int KVT, int B>
struct LaneOff {
  uint32_t k, v, s;
  __device__ __forceinline__ LaneOff(int lane) {
    using GE = SplitGeo<D, KVT>;
    constexpr int TM = (B < 16 ? B : 16) - 1;
    constexpr int JM = B < 16 ? 1 : 3;
    const int row = lane & 15;
    const int j = lane >> 4;
    if constexpr (GE::I4) {
      k = (uint32_t)((j * B + (row & TM)) * GE::P4);
      v = (uint32_t)(((j & JM) * 16 + row) * GE::P4);
    } else {
      k = (uint32_t)((j * B + (row & TM)) * 16);
      v = (uint32_t)(((j & JM) * D + (GE::E == 2 ? 2 * row : 4 * row)) * 4 * GE::E);
    }
    s = (uint32_t)(16 * (j & JM));
  }
};

// K/V tiles (and per-token scales).  When every block belongs to one
// sequence (NT), a decode reads each (block, head) tile once, and the tiles
// are loaded with the non-temporal hint, so that the streamed bytes do not
// displace the lines that are reused (queries, tables, partials) from the
// L2 and the MALL: measured on one box, 70B step 289 -> 275 us per launch,
// 8B-shaped layer 120 -> 110 us, 32K fp8 116 -> 103 us.  When tables share
// blocks (forked sequences, a cached prompt), the other readers of a block
// find it in the L2 or the MALL only if it was loaded with the default
// policy (!NT): the copy-on-write run's decode took 0.235 s streamed
// against 0.160 s cached.
template <bool NT, class V>
__device__ __forceinline__ V ld_kv(const char* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  return *reinterpret_cast<const V*>(p);
}

// Load the K/V (and int8 scales) of one step of tokens [t0, t0 + TS) of KV
// head g.  ph holds the step's table entries (one per 16-token chunk when
// blocks are smaller than a step, two per chunk with 8-token blocks), read
// for logical blocks clamped to the row's attended range: a chunk outside
// [t_lo, t_end) re-reads a block of the row and is masked.  The tile base is
// wave-uniform (scalar registers); the lane offsets are constant, so a step
// costs no per-lane address arithmetic except with 8-token blocks, where
// the two halves of a chunk come from two tiles.
template <int D, int KVT, int B, int NE, bool NT>
__device__ __forceinline__ void issue_step(SplitBuf<D, KVT>& r, const SplitParams& p, const int (&ph)[NE], int g,
                                           int t0, const LaneOff<D, KVT, B>& lo, int lane) {
  using GE = SplitGeo<D, KVT>;
  constexpr uint32_t TB = GE::I4 ? (uint32_t)(B * D / 2) : (uint32_t)(B * D * GE::E);
  const int row = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int h = 0; h < GE::CH; ++h) {
    const char* kb;
    const char* vb;
    const float* kscb = nullptr;
    const float* vscb = nullptr;
    if constexpr (B >= 16) {
      // the chunk lies in one block: the step's only entry at token offset
      // t0 % B + 16 h, or (steps longer than a block, which start at a block
      // boundary) entry 16 h / B at offset 16 h % B
      constexpr bool one = B >= GE::TS;
      const uint32_t tok = one ? ((uint32_t)t0 % B) + 16u * h : (16u * h) % B;
      const uint32_t tile = (uint32_t)ph[one ? 0 : (16 * h) / B] * (uint32_t)p.Hkv + (uint32_t)g;
      const uint64_t off = (uint64_t)tile * TB;
      kb = p.k + off + tok * GE::KTOK;
      vb = p.v + off + tok * GE::VTOK;
      if constexpr (GE::TOK) {
        kscb = p.ks + ((uint64_t)tile * B + tok);
        vscb = p.vs + ((uint64_t)tile * B + tok);
      }
    } else {
      // 8-token blocks: tokens 0-7 of the chunk in entry 2h, 8-15 in 2h + 1
      const uint64_t oa = (uint64_t)((uint32_t)ph[2 * h] * (uint32_t)p.Hkv + (uint32_t)g);
      const uint64_t ob = (uint64_t)((uint32_t)ph[2 * h + 1] * (uint32_t)p.Hkv + (uint32_t)g);
      kb = p.k + (row < 8 ? oa : ob) * TB;
      vb = p.v + (j < 2 ? oa : ob) * TB;
      if constexpr (GE::TOK) {
        kscb = p.ks + (j < 2 ? oa : ob) * B;
        vscb = p.vs + (j < 2 ? oa : ob) * B;
      }
    }
    if constexpr (GE::I4) {
      if constexpr (GE::P4 == 16) {
        r.k[h][0] = ld_kv<NT, u32x4>(kb + lo.k);
        r.v[h][0] = ld_kv<NT, u32x4>(vb + lo.v);
      } else {
        const u32x2 k2 = ld_kv<NT, u32x2>(kb + lo.k);
        const u32x2 v2 = ld_kv<NT, u32x2>(vb + lo.v);
        r.k[h][0] = u32x4{k2[0], k2[1], 0u, 0u};
        r.v[h][0] = u32x4{v2[0], v2[1], 0u, 0u};
      }
    } else {
#pragma unroll
      for (int u = 0; u < GE::LPC; ++u) r.k[h][u] = ld_kv<NT, u32x4>(kb + lo.k + u * 64 * B);
#pragma unroll
      for (int u = 0; u < GE::LPC; ++u) r.v[h][u] = ld_kv<NT, u32x4>(vb + lo.v + u * 256);
    }
    if constexpr (GE::TOK) {
      r.ksc[h] = ld_kv<NT, f32x4>(reinterpret_cast<const char*>(kscb) + lo.s);
      r.vsc[h] = ld_kv<NT, f32x4>(reinterpret_cast<const char*>(vscb) + lo.s);
    }
  }
}

// ---- appending decode.  Before streaming its range, a wave stores the new
// token (position ctx - 1) of every row whose last step lies in that range,
// encoded exactly as reshape_and_cache stores it, and waits until those
// stores have completed (s_waitcnt vmcnt(0)) before it issues its first K/V
// load.  The wave reads that tile again at the row's last step.  A completed
// store has reached the L2 of the wave's XCD and has updated or invalidated
// the line in its CU's vector L1, which every wave of that CU shares (the
// vector L1 is write-through; this is why, in the AMDGPU memory model for
// gfx942 and gfx950 outside threadgroup-split mode, a workgroup-scope
// release needs only that wait and an acquire no cache invalidation), so the
// later load returns the token even when the line is shared with other KV
// heads' tiles or int8 scale rows that other waves read (the step loads'
// non-temporal hint changes how lines are allocated and replaced, not what a
// load observes).  No other wave
// reads the token's own bytes: its block is not shared (copy-on-write runs
// before the append), the rest of its tile belongs to other steps, and when
// a KV head has several 16-head rows, each of their last-step waves stores
// the same bytes itself before reading them.  Stores cover the token's bytes
// only.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ uint32_t half_of(uint32_t w, int i) { return i ? (w >> 16) : (w & 0xffffu); }
__device__ __forceinline__ float abs_bf16(uint32_t b) { return fabsf(bf16_bits_to_float(b & 0xffffu)); }

template <int D, int KVT, int B>
__device__ __forceinline__ void append_token_bytes(const SplitParams& p, int s, int g, int ctx, int lane) {
  constexpr int E = KVT == PKV_KV_BF16 ? 2 : 1;
  constexpr int X = 16 / E;    // dims per 16-byte K piece
  constexpr int NPC = D / X;   // K pieces per token (<= 16): lane pc < NPC stores piece pc
  constexpr int VD = D / 64;   // V dims per lane: lane l stores dims VD*l ..
  const int pos = ctx - 1;     // ctx <= W * B, so the table index is inside the row
  int phys = uniform_load(p.bt + (int64_t)s * p.W + pos / B);
  phys = phys < 0 ? 0 : (phys >= p.num_blocks ? p.num_blocks - 1 : phys);  // stay inside the pool
  const int t = pos % B;
  const int64_t tile = (int64_t)phys * p.Hkv + g;
  char* kt = p.k + tile * (int64_t)(B * D * E);
  char* vt = p.v + tile * (int64_t)(B * D * E);
  const uint16_t* kx = p.new_k + ((int64_t)s * p.Hkv + g) * D;
  const uint16_t* vx = p.new_v + ((int64_t)s * p.Hkv + g) * D;
  const bool kl = lane < NPC;
  u32x4 kin[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};   // bf16 values of the lane's K piece
  if (kl) {
    kin[0] = *reinterpret_cast<const u32x4*>(kx + X * lane);
    if constexpr (E == 1) kin[1] = *reinterpret_cast<const u32x4*>(kx + X * lane + 8);
  }
  uint32_t vin;                                                 // bf16 values of the lane's V dims
  if constexpr (VD == 2) vin = *reinterpret_cast<const uint32_t*>(vx + 2 * lane);
  else vin = vx[lane];
  float sk = 0.f, sv = 0.f;
  if constexpr (KVT == PKV_KV_INT8) {
    float mk = 0.f, mv = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) mk = fmaxf(mk, fmaxf(abs_bf16(kin[h][e]), abs_bf16(kin[h][e] >> 16)));
#pragma unroll
    for (int i = 0; i < VD; ++i) mv = fmaxf(mv, abs_bf16(vin >> (16 * i)));
    sk = int8_scale(wave_max(mk));
    sv = int8_scale(wave_max(mv));
  }
  if (kl) {
    u32x4 kout;
    if constexpr (E == 2) {
      kout = kin[0];
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {   // output word q4 = dims 4q4 .. 4q4+3 of the piece
        const uint32_t x0 = kin[q4 >> 1][(q4 & 1) * 2], x1 = kin[q4 >> 1][(q4 & 1) * 2 + 1];
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x = half_of(i < 2 ? x0 : x1, i & 1);
          if constexpr (KVT == PKV_KV_FP8_E5M2) {
            b[i] = fp8_store(x, p.enc_k);
          } else if constexpr (KVT == PKV_KV_INT8) {
            b[i] = int8_store(x, sk);
          } else {   // calibrated: per tensor, or per channel (dim X * lane + 4 * q4 + i)
            b[i] = int8_store(x, p.ks_ch ? p.ks_ch[g * D + X * lane + 4 * q4 + i] : p.enc_k);
          }
        }
        kout[q4] = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      }
    }
    *reinterpret_cast<u32x4*>(kt + (lane * B + t) * 16) = kout;
  }
#pragma unroll
  for (int i = 0; i < VD; ++i) {
    const int d = VD * lane + i;
    const uint32_t x = half_of(vin, i);
    const int64_t el = ((int64_t)(t >> 2) * D + d) * 4 + (t & 3);
    if constexpr (E == 2) {
      reinterpret_cast<uint16_t*>(vt)[el] = (uint16_t)x;
    } else {
      uint32_t code;
      if constexpr (KVT == PKV_KV_FP8_E5M2) code = fp8_store(x, p.enc_v);
      else if constexpr (KVT == PKV_KV_INT8) code = int8_store(x, sv);
      else code = int8_store(x, p.vs_ch ? p.vs_ch[g * D + d] : p.enc_v);
      reinterpret_cast<uint8_t*>(vt)[el] = (uint8_t)code;
    }
  }
  if constexpr (KVT == PKV_KV_INT8) {
    if (lane == 0) {
      p.ks[tile * B + t] = sk;
      p.vs[tile * B + t] = sv;
    }
  }
}

template <int D, int KVT, int B>
__device__ __forceinline__ void append_token(const SplitParams& p, int s, int g, int ctx, int lane) {
  if constexpr (KVT == PKV_KV_INT4) {
    // as the INT4 cache write: lane b < D / 2 stores K byte b and V byte b of
    // the token, each byte holding two of its codes (+ 8)
    const int pos = ctx - 1;
    int phys = uniform_load(p.bt + (int64_t)s * p.W + pos / B);
    phys = phys < 0 ? 0 : (phys >= p.num_blocks ? p.num_blocks - 1 : phys);
    const int t = pos % B;
    const int64_t tile = (int64_t)phys * p.Hkv + g;
    uint8_t* kt = reinterpret_cast<uint8_t*>(p.k) + tile * (int64_t)(B * D / 2);
    uint8_t* vt = reinterpret_cast<uint8_t*>(p.v) + tile * (int64_t)(B * D / 2);
    const uint16_t* kx = p.new_k + ((int64_t)s * p.Hkv + g) * D;
    const uint16_t* vx = p.new_v + ((int64_t)s * p.Hkv + g) * D;
    const float* ksc = p.ks_ch + g * D;
    const float* vsc = p.vs_ch + g * D;
    constexpr int P = D / 8;
    if (lane < D / 2) {
      const int j = lane / P, o = lane % P, kk = o >> 2, bw = o & 3;
      const int d0 = 32 * kk + 8 * j + int4_k_lo_elem(bw);
      kt[(j * B + t) * P + o] = (uint8_t)(int4_store(kx[d0], ksc[d0]) | (int4_store(kx[d0 + 2], ksc[d0 + 2]) << 4));
      const int m = lane % 16, w = lane / 16, r = t & 3;
      const int e0 = 32 * w + m, e1 = e0 + 16;
      vt[((t >> 2) * 16 + m) * P + 4 * w + 2 * (r & 1) + (r >> 1)] =
          (uint8_t)(int4_store(vx[e0], vsc[e0]) | (int4_store(vx[e1], vsc[e1]) << 4));
    }
    return;
  } else {
    append_token_bytes<D, KVT, B>(p, s, g, ctx, lane);
  }
}

// Rescale threshold of the streaming softmax, in log2 units: the reference
// max m_run is only raised when a logit exceeds it by more than this, so p
// stays below 2^8 and the accumulator is rescaled a handful of times per
// segment instead of every step.  Any reference gives the same softmax.
constexpr float kRescaleSlack = 8.0f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}
// Packed fp16 pair plus c (both halves), rounded to nearest even.
__device__ __forceinline__ uint32_t add_f16x2(uint32_t w, _Float16 c) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, w) + f16x2{c, c});
}

// V words (4 tokens of one dim, one byte each) -> fp16 pairs of tokens
// (0, 1) and (2, 3), exactly.  e5m2 is the upper byte of an fp16 with the
// same exponent bias, so the byte moves into place; an int8 code c is stored
// as the fp16 1024 + (c + 128) (the byte c ^ 0x80 under the exponent bits of
// 1024) and 1152 is taken back, exactly, in fp16.
template <int KVT>
__device__ __forceinline__ void v_to_f16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (KVT == PKV_KV_FP8_E5M2) {
    lo = __builtin_amdgcn_perm(0u, w, 0x010c000cu);
    hi = __builtin_amdgcn_perm(0u, w, 0x030c020cu);
  } else {
    const uint32_t u = w ^ 0x80808080u;
    lo = add_f16x2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u), (_Float16)-1152.0f);
    hi = add_f16x2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u), (_Float16)-1152.0f);
  }
}
// INT4 V: pair k of a word (nibbles at bits 4k and 16 + 4k, u = code + 8)
// as fp16 subnormals, exactly: pairs 0 and 2 (the latter from the word
// shifted by 8) are u * 2^-24, pairs 1 and 3, masked in place, u * 2^-20.
// One AND per pair and one shift per word; a tile's operand holds pairs of
// one scale, and when a segment ends its accumulator is scaled back and
// 8 * (sum of the p that entered the products) taken off (kInt4VScale).
__device__ __forceinline__ uint32_t int4_pair_sub(uint32_t w, int k) {
  const uint32_t x = k & 2 ? w >> 8 : w;
  return x & (k & 1 ? 0x00F000F0u : 0x000F000Fu);
}
// The factor that turns an INT4 accumulator tile c back into sum p * u.
__device__ __forceinline__ constexpr float kInt4VScale(int c) { return c & 1 ? 0x1p20f : 0x1p24f; }

// K operand of q.K step kk of chunk h, as bf16 (exact: 8-bit codes and e5m2
// widen without rounding; INT4 nibbles become 136 + code).
template <int D, int KVT>
__device__ __forceinline__ bf16x8 k_operand(const SplitBuf<D, KVT>& r, int h, int kk) {
  using GE = SplitGeo<D, KVT>;
  if constexpr (GE::I4) {
    const uint32_t wk = r.k[h][0][kk];          // word kk: dims 32 kk + 8 j .. + 7
    return __builtin_bit_cast(bf16x8, u32x4{int4_pair(wk, 0), int4_pair(wk, 1), int4_pair(wk, 2), int4_pair(wk, 3)});
  } else if constexpr (GE::E == 2) {
    return __builtin_bit_cast(bf16x8, r.k[h][kk]);
  } else {
    const u32x4 wv = r.k[h][kk >> 1];
    return (kk & 1) ? widen8<KVT == PKV_KV_FP8_E5M2 ? PKV_KV_FP8_E5M2 : PKV_KV_INT8>(wv[2], wv[3])
                    : widen8<KVT == PKV_KV_FP8_E5M2 ? PKV_KV_FP8_E5M2 : PKV_KV_INT8>(wv[0], wv[1]);
  }
}

// Online-softmax update of (m_run, l_run, acc) with one step of tokens
// [t0, t0 + TS).  Only an edge step (one reaching past t_end or starting
// before t_lo) masks: its logits outside [t_lo, t_end) become -inf, and the
// V elements (or p, when per-token scales multiply it) of those tokens are
// zeroed so that unwritten slots and blocks before a window (any bit
// pattern) cannot reach the accumulator through 0 * NaN.
// P.V: bf16 storage meets p as bf16 hi + lo parts (~16 bits of p); 8-bit and
// 4-bit storage converts V exactly to fp16 and meets p rounded to fp16
// (11 bits), one matrix-core step per tile.
template <int D, int KVT>
__device__ __forceinline__ void compute_step(const SplitBuf<D, KVT>& r,
                                             const QRegs<SplitGeo<D, KVT>::KK, SplitGeo<D, KVT>::NQ>& qop,
                                             float qs, float qk_scale, int t0, int t_lo, int t_end, bool edge,
                                             int lane, float& m_run, float& l_run,
                                             f32x4 (&acc)[SplitGeo<D, KVT>::NC], f32x4& psum16) {
  using GE = SplitGeo<D, KVT>;
  constexpr int CH = GE::CH;
  const int j = lane >> 4;
  f32x4 z[CH];
#pragma unroll
  for (int h = 0; h < CH; ++h) {
    f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < GE::KK; ++kk) {
      const bf16x8 a = k_operand<D, KVT>(r, h, kk);
#pragma unroll
      for (int n = 0; n < GE::NQ; ++n) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop.q[n][kk], c, 0, 0, 0);
    }
    if constexpr (GE::I4) c -= kInt4Bias * qs;   // the K operand held 136 + code
    if constexpr (GE::TOK) c *= r.ksc[h];
    z[h] = c;
  }
  if (edge) {
#pragma unroll
    for (int h = 0; h < CH; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[h][i] = tok_in(t0 + 16 * h + 4 * j + i, t_lo, t_end) ? z[h][i] : -INFINITY;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int h = 0; h < CH; ++h) mloc = fmaxf(fmaxf(mloc, fmaxf(z[h][0], z[h][1])), fmaxf(z[h][2], z[h][3]));
  // finite: every step holds a token of [t_lo, t_end); qk_scale > 0
  const float ms = max_x32(max_x16(mloc)) * qk_scale;
  const bool bump = ms > m_run + kRescaleSlack;   // always true on a segment's first step
  const float m_ref = bump ? ms : m_run;
  const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_ref) : 1.0f;
  // the accumulator is zero until the first step has run, so only a raise of a
  // finite reference needs the rescale (wave-uniform branch)
  if (__builtin_amdgcn_ballot_w64(bump && m_run > -INFINITY)) {
#pragma unroll
    for (int c = 0; c < GE::NC; ++c) acc[c] = acc[c] * alpha;
    if constexpr (GE::I4) psum16 = psum16 * alpha;
  }
  m_run = m_ref;
  float pv[CH][4];
  float psum = 0.f;
#pragma unroll
  for (int h = 0; h < CH; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[h][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[h][i], qk_scale, -m_ref));
      psum += pv[h][i];
    }
  l_run = l_run * alpha + psum;
  if constexpr (GE::TOK) {
    // fold the V scale into p (masked tokens: p = 0 whatever their scale)
#pragma unroll
    for (int h = 0; h < CH; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[h][i] *= r.vsc[h][i];
      if (edge) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[h][i] = tok_in(t0 + 16 * h + 4 * j + i, t_lo, t_end) ? pv[h][i] : 0.f;
      }
    }
  }
  if constexpr (GE::BF) {
    uint32_t ph[2], pl[2];
    ph[0] = pack_bf16x2(pv[0][0], pv[0][1]);
    ph[1] = pack_bf16x2(pv[0][2], pv[0][3]);
    pl[0] = pack_bf16x2(pv[0][0] - bf16_lo(ph[0]), pv[0][1] - bf16_hi(ph[0]));
    pl[1] = pack_bf16x2(pv[0][2] - bf16_lo(ph[1]), pv[0][3] - bf16_hi(ph[1]));
    const s16x4 pop = __builtin_bit_cast(s16x4, u32x2{ph[0], ph[1]});
    const s16x4 pop_lo = __builtin_bit_cast(s16x4, u32x2{pl[0], pl[1]});
    u32x4 v[GE::LPC];
#pragma unroll
    for (int u = 0; u < GE::LPC; ++u) v[u] = r.v[0][u];
    if (edge) {
      const int tb = t0 + 4 * j;
      const u32x4 m = u32x4{tok_mask16(tb, t_lo, t_end), tok_mask16(tb + 2, t_lo, t_end),
                            tok_mask16(tb, t_lo, t_end), tok_mask16(tb + 2, t_lo, t_end)};
#pragma unroll
      for (int u = 0; u < GE::LPC; ++u) v[u] &= m;
    }
#pragma unroll
    for (int c = 0; c < GE::NC; ++c) {
      const int u = c >> 1, e = c & 1;      // load u holds dims (32u + 2row, +1) x 4 tokens
      const s16x4 aop = __builtin_bit_cast(s16x4, u32x2{v[u][2 * e], v[u][2 * e + 1]});
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, pop, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, pop_lo, acc[c], 0, 0, 0);
    }
  } else {
    // one 16x16x32 product per tile and pair of chunks
    f16x8 pop[CH / 2];
#pragma unroll
    for (int hp = 0; hp < CH / 2; ++hp)
      pop[hp] = __builtin_bit_cast(f16x8, u32x4{pack_f16x2(pv[2 * hp][0], pv[2 * hp][1]),
                                                pack_f16x2(pv[2 * hp][2], pv[2 * hp][3]),
                                                pack_f16x2(pv[2 * hp + 1][0], pv[2 * hp + 1][1]),
                                                pack_f16x2(pv[2 * hp + 1][2], pv[2 * hp + 1][3])});
    // fp8 codes of masked tokens may be inf / NaN patterns: zero them on an
    // edge step (two copies of the loop, so that other steps carry no mask);
    // other codes decode to finite values, which p = 0 cancels
    auto pv_tiles = [&](auto maskc) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(maskc)::value;
      uint32_t mk[CH] = {};
      if constexpr (MASK) {
#pragma unroll
        for (int h = 0; h < CH; ++h) mk[h] = tok_mask8(t0 + 16 * h + 4 * j, t_lo, t_end);
      }
#pragma unroll
      for (int hp = 0; hp < CH / 2; ++hp)
#pragma unroll
        for (int c = 0; c < GE::NC; ++c) {
          uint32_t a0, a1, a2, a3;
          if constexpr (GE::I4) {
            // word c / 2 of the V piece: pairs (c % 2) and 2 + (c % 2) are
            // tokens 0, 1 and 2, 3 of the group, dim 16 c + row
            const uint32_t w0 = r.v[2 * hp][0][c >> 1], w1 = r.v[2 * hp + 1][0][c >> 1];
            a0 = int4_pair_sub(w0, c & 1);
            a1 = int4_pair_sub(w0, 2 + (c & 1));
            a2 = int4_pair_sub(w1, c & 1);
            a3 = int4_pair_sub(w1, 2 + (c & 1));
          } else {
            const int u = c >> 2, e = c & 3;    // load u holds dims (64u + 4row .. +3) x 4 tokens
            uint32_t w0 = r.v[2 * hp][u][e], w1 = r.v[2 * hp + 1][u][e];
            if constexpr (MASK) {
              w0 &= mk[2 * hp];
              w1 &= mk[2 * hp + 1];
            }
            v_to_f16<KVT>(w0, a0, a1);
            v_to_f16<KVT>(w1, a2, a3);
          }
          const f16x8 aop = __builtin_bit_cast(f16x8, u32x4{a0, a1, a2, a3});
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, pop[hp], acc[c], 0, 0, 0);
        }
      if constexpr (GE::I4) {
        // the sum of the fp16 p that entered the products, per head (every
        // row of the product: a matrix of ones times P)
        const _Float16 one = (_Float16)1.0f;
#pragma unroll
        for (int hp = 0; hp < CH / 2; ++hp)
          psum16 = __builtin_amdgcn_mfma_f32_16x16x32_f16(f16x8{one, one, one, one, one, one, one, one}, pop[hp],
                                                          psum16, 0, 0, 0);
      }
    };
    if (GE::FP8 && edge) pv_tiles(std::true_type{});
    else pv_tiles(std::false_type{});
  }
}

// Where a walk over the flat step list stands, with the constants of its
// row (recomputed only when the row changes).
struct Cursor {
  int s, xi, j;     // sequence, row within the sequence, step within the row
  int n;            // steps of sequence s's rows (from the window's first step)
  int ctx;          // context length of sequence s
  int tb;           // first token of the rows' first step (window start, rounded down)
  int lo;           // first attended position (window start, or 0)
  int g;            // KV head of the row
  int h0, gt;       // first query head of the row's tile, and its number of heads
};

// Row constants of the cursor's row.
__device__ __forceinline__ void cursor_row(Cursor& c, const SplitParams& p) {
  c.g = p.QT == 1 ? c.xi : c.xi / p.QT;
  const int qt = c.xi - c.g * p.QT;
  c.h0 = c.g * p.G + qt * 16;
  c.gt = min(16, p.G - qt * 16);
}

// Move to the first step of the next row that has any (the caller knows
// there is one: the wave's range reaches it): the next sequence with steps,
// past the last one the first of the next head tile.
template <int TS, bool kRowConsts = true>
__device__ __forceinline__ void cursor_next_row(Cursor& c, const SplitParams& p, int max_ctx) {
  c.j = 0;
  bool next_head = false;
  do {
    if (++c.s == p.S) {
      c.s = 0;
      next_head = true;
    }
    c.ctx = clamp_ctx(uniform_load(p.ctx + c.s), max_ctx);
    c.n = split_steps<TS>(c.ctx, p);
  } while (c.n == 0);
  if (next_head) ++c.xi;
  c.tb = split_base<TS>(c.ctx, p);
  c.lo = split_lo(c.ctx, p);
  if constexpr (kRowConsts) cursor_row(c, p);
}

// (m, l) of one (slot, head) in the partial (m, l) region.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ml_rsrc(const SplitParams& p) {
  return __builtin_amdgcn_make_buffer_rsrc(p.part_ml, (short)0, p.ml_bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t ml_offset(int slot, int head) { return ((uint32_t)slot * 16u + (uint32_t)head) * 8u; }

// The accumulator block of one partial slot (NC * 1 KiB) as a buffer
// resource; every access through it stays inside the slot.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(float* acc, int slot, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(acc + (int64_t)slot * (bytes / 4), (short)0, bytes, 0x00020000);
}

constexpr int kXcdWeight[8] = {256, 224, 256, 224, 256, 224, 256, 224};

// First flat step of XCD x's share of N steps.
__device__ __forceinline__ int xcd_begin(int N, int x) {
  int64_t acc = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc += i < x ? kXcdWeight[i] : 0;
    tot += kXcdWeight[i];
  }
  return (int)((int64_t)N * acc / tot);
}

// Flat steps [a, e) of wave w; WX waves per XCD.
__device__ __forceinline__ void wave_range(int N, int w, int WX, int& a, int& e) {
  const int x = w / WX, li = w - x * WX;
  const int b0 = xcd_begin(N, x), b1 = xcd_begin(N, x + 1);
  const int per = (b1 - b0 + WX - 1) / WX;
  a = min(b0 + li * per, b1);
  e = min(a + per, b1);
}

// Merge the partials of row x into the output rows of its query heads.
// Wave-cooperative, in the accumulator lane layout: lane (j, row) holds query
// head row of the tile.  With gt <= 8 heads, the 16 / gp lane groups of the
// tile (gp = gt rounded up to a power of two) each take a share of the slots,
// lane (j, row) merging head row % gp, and the groups combine at the end, so
// that all lanes load.  The slots are those of the waves covering flat steps
// [sx, sx + ns), which are consecutive waves minus those with empty ranges:
// lane i tests wave first + i, a ballot gives the set, and the slot of rank n
// is the n-th wave of the set.  merge_slots() slots per lane group are loaded
// at a time so that their latencies overlap.
template <int D>
constexpr int merge_slots() { return D == 64 ? 16 : 12; }

// Position of the n-th (from 0) set bit of mask, n < popcount(mask).
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int n) {
  if ((mask & (mask + 1)) == 0) return n;      // one run from bit 0: the usual case
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __builtin_popcountll((mask >> pos) & ((1ull << w) - 1));
    if (n >= c) {
      n -= c;
      pos += w;
    }
  }
  return pos;
}

// (M, L, A) <- the merge of (M, L, A) and (m, l, a); an empty side has
// M = -inf, L = 0, A = 0 and contributes nothing.
template <int NC>
__device__ __forceinline__ void merge_into(float& M, float& L, f32x4 (&A)[NC], float m, float l,
                                           const f32x4 (&a)[NC]) {
  const float Mn = fmaxf(M, m);
  const float fa = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
  const float fk = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - Mn);
  L = L * fa + l * fk;
#pragma unroll
  for (int c = 0; c < NC; ++c) A[c] = A[c] * fa + a[c] * fk;
  M = Mn;
}

// Normalised output rows of one (sequence, KV head, head tile) row from its
// merged state: lane (j, row) holds head row of the tile in the accumulator
// layout AL; L is the softmax denominator of that head.
// A shared-prefix decode also keeps each output row's softmax state (m, l)
// (reference max of the scaled logits in log2 units, and the sum relative to
// it), which the prefix pass merges its own with.
__device__ __forceinline__ void store_ml(const SplitParams& p, int s, int h, float m, float l) {
  *reinterpret_cast<f32x2*>(p.ml_out + ((int64_t)s * p.Hq + h) * 2) = f32x2{m, l};
}

template <int D, int AL>
__device__ __forceinline__ void store_out(const SplitParams& p, int s, int g, int h0, int gt, const f32x4 (&A)[D / 16],
                                          float M, float L, int lane) {
  constexpr int NC = D / 16;
  const int row = lane & 15;
  const int j = lane >> 4;
  if (row < gt) {
    if (p.ml_out && j == 0) store_ml(p, s, h0 + row, M, L);
    float* orow = p.out + ((int64_t)s * p.Hq + h0 + row) * D;
    const float inv = p.out_scale / L;
    const float* vch = p.vs_ch ? p.vs_ch + g * D : nullptr;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = acc_dim<AL>(c, j, i);
        orow[dd] = vch ? A[c][i] / L * vch[dd] : A[c][i] * inv;
      }
  }
}

// Output rows of a whole-row segment straight from the accumulator (storage
// without per-channel V scales): 16-byte stores of 4 consecutive dims,
// through a buffer resource spanning the tile's gt output rows, which drops
// the stores of lanes whose head lies past them.
template <int D, int AL>
__device__ __forceinline__ void store_out_direct(const SplitParams& p, int s, int h0, int gt, const f32x4 (&A)[D / 16],
                                                 float M, float L, int lane) {
  static_assert(AL == 1 || AL == 2, "direct output covers the bf16 and 8-bit accumulator layouts");
  const int row = lane & 15;
  const int j = lane >> 4;
  if (p.ml_out && j == 0 && row < gt) store_ml(p, s, h0 + row, M, L);
  const float inv = p.out_scale / L;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(p.out + ((int64_t)s * p.Hq + h0) * D, (short)0,
                                                                     gt * D * 4, 0x00020000);
  const int lo = (row * D + (AL == 2 ? 8 : 16) * j) * 4;
  if constexpr (AL == 2) {
    // tiles 2u, 2u + 1 hold dims 32u + 8j + 2i and 32u + 8j + 2i + 1
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const f32x4 a = A[2 * u] * inv, b = A[2 * u + 1] * inv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{a[0], b[0], a[1], b[1]}), r,
                                             lo + 128 * u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{a[2], b[2], a[3], b[3]}), r,
                                             lo + 128 * u + 16, 0, 0);
    }
  } else {
    // tiles 4u + e hold dims 64u + 16j + 4i + e
#pragma unroll
    for (int u = 0; u < D / 64; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{A[4 * u][i], A[4 * u + 1][i], A[4 * u + 2][i], A[4 * u + 3][i]} * inv),
            r, lo + 256 * u + 16 * i, 0, 0);
  }
}

template <int D, int AL>
__device__ __forceinline__ void merge_row(const SplitParams& p, int x, int s, int xi, int ns, int sx, int N,
                                          int xbv, int lane) {
  constexpr int NC = D / 16;
  constexpr int KS = merge_slots<D>();
  const int g = xi / p.QT;
  const int qt = xi - g * p.QT;
  const int row = lane & 15;
  const int j = lane >> 4;
  const int gt = min(16, p.G - qt * 16);
  const int h0 = g * p.G + qt * 16;
  const int gp = gt > 8 ? 16 : gt > 4 ? 8 : gt > 2 ? 4 : gt > 1 ? 2 : 1;
  const int hs = 16 / gp;                      // lane groups per head
  const int hr = row & (gp - 1);               // head merged by this lane
  const int grp = row / gp;                    // its lane group
  const int src = (j * 16 + hr) * 16;          // byte offset of that head's values in a slot's tile
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(p.part_acc, (short)0, p.acc_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t mr = ml_rsrc(p);
  float M = -INFINITY, L = 0.f;
  f32x4 A[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) A[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int WX = p.NWV / 8;
  const int end = sx + ns;
  // the loads below follow the counter update that found the row complete
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // the wave holding step sx (lane i < 9 of xbv holds the first step of XCD
  // i's share of the list)
  const int xc = __builtin_popcountll(__ballot(lane >= 1 && lane <= 7 && sx >= xbv));
  const int b0 = __builtin_amdgcn_readlane(xbv, xc), b1 = __builtin_amdgcn_readlane(xbv, xc + 1);
  int first = xc * WX + (sx - b0) / ((b1 - b0 + WX - 1) / WX);
  while (true) {
    // lane i: does wave first + i hold a partial of this row?
    const int wl = first + lane;
    const int xl = min(wl / WX, 8);
    const int l0 = __shfl(xbv, xl, kWave), l1 = __shfl(xbv, min(xl + 1, 8), kWave);
    const int al = min(l0 + (wl - xl * WX) * ((l1 - l0 + WX - 1) / WX), l1);   // its first step
    const uint64_t set = __ballot(xl < 8 && al < l1 && al < end);
    const int cnt = __builtin_popcountll(set);
    for (int nb = 0; nb < cnt; nb += KS * hs) {
      int slot[KS];
      bool live[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int n = nb + k * hs + grp;
        live[k] = n < cnt;
        slot[k] = x + first + nth_set_bit(set, live[k] ? n : 0);
      }
      f32x2 ml[KS];
      f32x4 av[KS][NC];
      if (hr < gt) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          if (nb + k * hs >= cnt) break;         // no lane group has a slot k this round
          ml[k] = ld_agent2(mr, ml_offset(slot[k], hr));
          const uint32_t base = (uint32_t)slot[k] * (NC * 1024u) + src;
#pragma unroll
          for (int c = 0; c < NC; ++c) av[k][c] = ld_agent4(pr, base + c * 1024);
        }
#pragma unroll
        for (int k = 0; k < KS; ++k)
          if (nb + k * hs < cnt && live[k]) merge_into<NC>(M, L, A, ml[k][0], ml[k][1], av[k]);
      }
    }
    // the next 64 waves, if the last one tested starts inside the row
    if (__builtin_amdgcn_readlane(xl < 8 && al < end ? 1 : 0, kWave - 1) == 0) break;
    first += kWave;
  }
  // combine the lane groups of each head (partner lanes stay inside the
  // 16-lane run of one j)
  for (int off = gp; off < 16; off <<= 1) {
    const float m2 = __shfl_xor(M, off, kWave);
    const float l2 = __shfl_xor(L, off, kWave);
    f32x4 a2[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) a2[c][i] = __shfl_xor(A[c][i], off, kWave);
    merge_into<NC>(M, L, A, m2, l2, a2);
  }
  store_out<D, AL>(p, s, g, h0, gt, A, M, L, lane);
}

// Launched with one workgroup (one wave per SIMD) per CU, so the compiler may
// use the whole register file for a wave's in-flight loads.
template <int D, int KVT, int B, int NBUF, bool NT>
__global__ __launch_bounds__(kWave * kNW) __attribute__((amdgpu_waves_per_eu(1, 1))) void pa_split_kernel(
    const SplitParams p) {
  using GE = SplitGeo<D, KVT>;
  constexpr int TS = GE::TS;
  const int lane = threadIdx.x % kWave;
  const int row = lane & 15;
  const int j = lane >> 4;
  // XCD-aware numbering: workgroup b runs on XCD b % 8; each XCD gets a
  // contiguous run of wave ranges
  const int nwg = (int)gridDim.x;                  // a multiple of 8
  const int b = (int)blockIdx.x;
  const int wg = (b % 8) * (nwg / 8) + b / 8;
  // wave-uniform, and said so: everything derived from it stays in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(wg * kNW + (int)threadIdx.x / kWave);
  const int max_ctx = p.W * B;

  // ---- total steps N (wave 0 also zeroes the output of empty sequences),
  // this wave's range, and the sequence holding its first step.  Context
  // lengths are read kSeqRegs * 64 at a time with independent loads; up to
  // that many sequences they are read once and kept in registers.
  constexpr int kSeqRegs = 4;
  int cv[kSeqRegs];          // clamped context length of sequence base + 64k + lane
  auto load_ctx = [&](int base) __attribute__((always_inline)) {
    // unconditional loads (a lane past the last sequence re-reads it), so
    // that all of them are in flight before the first is waited for
    int raw[kSeqRegs];
#pragma unroll
    for (int k = 0; k < kSeqRegs; ++k) raw[k] = p.ctx[min(base + k * kWave + lane, p.S - 1)];
#pragma unroll
    for (int k = 0; k < kSeqRegs; ++k) cv[k] = base + k * kWave + lane < p.S ? clamp_ctx(raw[k], max_ctx) : 0;
  };
  int total = 0;
  for (int base = 0; base < p.S; base += kSeqRegs * kWave) {
    load_ctx(base);
#pragma unroll
    for (int k = 0; k < kSeqRegs; ++k) {
      const int n = split_steps<TS>(cv[k], p);
      total += wave_sum(n);
      if (w == 0) {
        const int b0 = base + k * kWave;
        uint64_t empty = __ballot(b0 + lane < p.S && n == 0);
        while (empty) {
          const int se = b0 + __builtin_ctzll(empty);
          empty &= empty - 1;
          float* o = p.out + (int64_t)se * p.Hq * D;
          for (int i = lane * 4; i < p.Hq * D; i += kWave * 4)
            *reinterpret_cast<f32x4*>(o + i) = f32x4{0.f, 0.f, 0.f, 0.f};
          if (p.ml_out)   // nothing attended: the prefix pass takes its own state alone
            for (int h = lane; h < p.Hq; h += kWave) store_ml(p, se, h, -INFINITY, 0.f);
        }
      }
    }
  }
  const int T = __builtin_amdgcn_readfirstlane(total);   // steps of one head tile's rows
  const int N = T * p.HQ;
  if (N == 0) return;
  int start, stop;
  wave_range(N, w, p.NWV / 8, start, stop);
  if (start >= stop) return;
  const int nsteps = stop - start;

  // locate the first step: head tile xi = start / T, then the sequence s
  // with cum_s <= start - xi T < cum_{s+1}
  Cursor cur{};
  int cum0 = 0;
  const int xi0 = start / T;
  const int rem0 = start - xi0 * T;
  {
    int acc0 = 0;
    bool found = false;
    for (int base = 0; base < p.S && !found; base += kSeqRegs * kWave) {
      if (p.S > kSeqRegs * kWave) load_ctx(base);   // else still held from the count
#pragma unroll
      for (int k = 0; k < kSeqRegs; ++k) {
        if (found) break;
        const int c = cv[k];
        const int n = split_steps<TS>(c, p);
        const int incl = wave_incl_scan(n, lane);
        const bool hit = acc0 + incl - n <= rem0 && rem0 < acc0 + incl;
        const uint64_t m = __ballot(hit);
        if (m) {
          const int l = __builtin_ctzll(m);
          cur.s = base + k * kWave + l;
          cur.n = __shfl(n, l, kWave);
          cur.ctx = __shfl(c, l, kWave);
          cum0 = acc0 + __shfl(incl - n, l, kWave);
          cur.xi = xi0;
          cur.j = rem0 - cum0;
          found = true;
        }
        acc0 += __shfl(incl, kWave - 1, kWave);
      }
    }
  }
  cur.s = __builtin_amdgcn_readfirstlane(cur.s);
  cur.n = __builtin_amdgcn_readfirstlane(cur.n);
  cur.ctx = __builtin_amdgcn_readfirstlane(cur.ctx);
  cur.tb = split_base<TS>(cur.ctx, p);
  cur.lo = split_lo(cur.ctx, p);
  cur.xi = __builtin_amdgcn_readfirstlane(cur.xi);
  cur.j = __builtin_amdgcn_readfirstlane(cur.j);
  cum0 = __builtin_amdgcn_readfirstlane(cum0);
  const Cursor first = cur;

  // ---- appending decode: store the new token of every row that ends in this
  // range, then wait until the stores have completed, before the load of any
  // step holding such a token is issued.  When the range's first row ends
  // past the pipeline's first NBUF - 1 steps (every later row ends later),
  // those steps' loads are issued first, so the append's own loads, encoding
  // and stores overlap their memory latency; otherwise the append runs first.
  auto append_rows = [&]() __attribute__((always_inline)) {
    int as = cur.s, axi = cur.xi, aj = cur.j, an = cur.n, actx = cur.ctx, left = nsteps;
    while (left > 0) {
      const int mine = min(left, an - aj);
      if (aj + mine == an) {
        append_token<D, KVT, B>(p, as, p.QT == 1 ? axi : axi / p.QT, actx, lane);
      }
      left -= mine;
      aj = 0;
      if (left > 0) {
        do {
          if (++as == p.S) {
            as = 0;
            ++axi;
          }
          actx = clamp_ctx(uniform_load(p.ctx + as), max_ctx);
          an = split_steps<TS>(actx, p);
        } while (an == 0);
      }
    }
    wait_vm_all();
  };
  const bool append_first = p.new_k && cur.n - cur.j - 1 < NBUF - 1;
  if (append_first) append_rows();

  cursor_row(cur, p);

  constexpr int NE = B >= TS ? 1 : TS / B;          // table entries per step
  const LaneOff<D, KVT, B> lo(lane);
  // issue side: the cursor of the next step to load, its row's table, and
  // that step's table entries (fetched one step ahead, as they are read: the
  // scalar loads' results are first used, to clamp them into the pool, when
  // that step is issued, so their latency hides behind a step's compute)
  Cursor ic = cur;
  const int32_t* bt_row = p.bt + (int64_t)ic.s * p.W;
  int ph_raw[NE];
  auto fetch = [&]() __attribute__((always_inline)) {
    // logical blocks clamped to those holding attended positions, so a chunk
    // outside [lo, ctx) never reads a table entry past the context or before
    // the window (those may name any block)
    const uint32_t lb0 = (uint32_t)(ic.tb + ic.j * TS) / B;
    const uint32_t lmin = (uint32_t)ic.lo / B, lmax = (uint32_t)(ic.ctx - 1) / B;
#pragma unroll
    for (int e = 0; e < NE; ++e) ph_raw[e] = uniform_load(bt_row + min(max(lb0 + e, lmin), lmax));
  };
  fetch();
  // compute side: the cursor of the next step to compute
  Cursor cc = cur;

  using QR = QRegs<GE::KK, GE::NQ>;
  SplitBuf<D, KVT> buf[NBUF];
  QR qbuf[NBUF];   // q of a row that starts at the step in the same-index buffer
  QR qop;          // q of the row being computed
  float qs = 0.f;  // INT4: the sum of qop over the head's dims
  int issued = 0, consumed = 0;

  // Issue the step at the issue cursor into buffer r (and, when it starts a
  // row in this wave, the row's q into qr), then advance the cursor and
  // fetch the next step's table entries.  Past the end of the range the
  // cursor stays and the loads repeat the last step's (never consumed): every
  // step issues the same loads, so the compiler's wait before each compute
  // covers exactly that step's loads and the later ones stay in flight.  A
  // row's q goes with its first step into the register set of that step's
  // buffer, so every load is consumed a fixed number of issues after it was
  // made.
  auto issue = [&](SplitBuf<D, KVT>& r, QR& qr) __attribute__((always_inline)) {
    if (issued < nsteps && (ic.j == 0 || issued == 0)) qr = load_q<D, KVT>(p, ic.s, ic.h0, ic.gt, lane);
    int ph[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)   // stay inside the pool
      ph[e] = ph_raw[e] < 0 ? 0 : (ph_raw[e] >= p.num_blocks ? p.num_blocks - 1 : ph_raw[e]);
    issue_step<D, KVT, B, NE, NT>(r, p, ph, ic.g, ic.tb + ic.j * TS, lo, lane);
    ++issued;
    if (issued < nsteps) {
      if (++ic.j == ic.n) {
        const int s0 = ic.s;
        cursor_next_row<TS>(ic, p, max_ctx);
        if (ic.s != s0) bt_row = p.bt + (int64_t)ic.s * p.W;
      }
      fetch();
    }
  };

  f32x4 acc[GE::NC];
#pragma unroll
  for (int c = 0; c < GE::NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 psum16 = f32x4{0.f, 0.f, 0.f, 0.f};   // INT4: sum of the fp16 p per head (all four entries)
  float m_run = -INFINITY;
  float l_run = 0.f;

  // Compute the step at the compute cursor from buffer r.  At the end of a
  // segment (the row's last step, or the range's): a segment that is the
  // whole row (storage without per-channel V scales) writes the row's output
  // directly; any other writes its partial.  Only the range's first row can
  // end inside the range without being whole; when its end leaves NBUF steps
  // of the range, its partial is reported to the row's counter NBUF steps
  // later (by then its stores have completed, below), so that the wave is
  // rarely the one completing that row and the rows it merges when its
  // range ends are at most its last.
  constexpr bool kDirect = !GE::CHAN;
  const int len0 = first.n - first.j;              // steps of the first row in this range (if it ends here)
  const int whole_from = first.j > 0 ? len0 + 1 : 1;   // consumed count from which a row end closes a whole row
  const int pend_at = (first.j > 0 && len0 + NBUF <= nsteps) ? len0 + NBUF : -1;
  unsigned long long pend_old = 0;  // lane 0: the first row's counter before this wave's addition
  auto consume = [&](const SplitBuf<D, KVT>& r, const QR& qr) __attribute__((always_inline)) {
    if (cc.j == 0 || consumed == 0) {
      qop = qr;
      if constexpr (GE::I4) qs = query_sum<D, KVT>(qop);
    }
    const int t0 = cc.tb + cc.j * TS;
    const bool edge = t0 < cc.lo || t0 + TS > cc.ctx;
    compute_step<D, KVT>(r, qop, qs, p.qk_scale, t0, cc.lo, cc.ctx, edge, lane, m_run, l_run, acc, psum16);
    ++consumed;
    if (cc.j + 1 == cc.n || consumed == nsteps) {
      const float l = sum_x32(sum_x16(l_run));
      if constexpr (GE::I4) {
#pragma unroll
        for (int c = 0; c < GE::NC; ++c) acc[c] = acc[c] * kInt4VScale(c) - 8.0f * psum16[0];
        psum16 = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const int g = p.QT == 1 ? cc.xi : cc.xi / p.QT;
      const int qt = cc.xi - g * p.QT;
      const int gt = min(16, p.G - qt * 16);
      if (kDirect && cc.j + 1 == cc.n && consumed >= whole_from) {
        if constexpr (kDirect) store_out_direct<D, GE::AL>(p, cc.s, g * p.G + qt * 16, gt, acc, m_run, l, lane);
      } else {
        if (row < gt) {
          const int slot = cc.xi * p.S + cc.s + w;
          const __amdgpu_buffer_rsrc_t pr = slot_rsrc(p.part_acc, slot, GE::NC * 1024);
#pragma unroll
          for (int c = 0; c < GE::NC; ++c) st_agent4(pr, c * 1024 + lane * 16, acc[c]);
          if (j == 0) st_agent2(ml_rsrc(p), ml_offset(slot, row), m_run, l);
        }
      }
#pragma unroll
      for (int c = 0; c < GE::NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    if (consumed == pend_at) {
      // the NBUF steps issued since the partial's stores are all younger than
      // them, and vector memory operations of a wave complete in issue order:
      // with at most that many outstanding, the stores have completed
      vm_wait_at_most<(NBUF * GE::LPS < 63 ? NBUF * GE::LPS : 63)>();
      __builtin_amdgcn_sched_barrier(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0)
        pend_old = report_steps(p.row_done + (int64_t)(first.xi * p.S + first.s) * kCounterStride, p.epoch, len0);
    }
    if (consumed < nsteps && ++cc.j == cc.n) cursor_next_row<TS, false>(cc, p, max_ctx);
  };

  // ---- pipeline: NBUF - 1 steps of loads in flight ahead of the one computed
  // (the buffer indices must be compile-time constants, or the buffers move
  // to scratch memory: the steps are expanded from an index sequence rather
  // than left to loop unrolling)
  static_for<NBUF - 1>([&](auto bbc) {
    constexpr int bb = decltype(bbc)::value;
    issue(buf[bb], qbuf[bb]);
  });
  if (p.new_k && !append_first) append_rows();
  for (int base = 0; base < nsteps; base += NBUF) {
    static_for<NBUF>([&](auto bbc) {
      constexpr int bb = decltype(bbc)::value;
      constexpr int nb = (bb + NBUF - 1) % NBUF;
      issue(buf[nb], qbuf[nb]);
      if (base + bb < nsteps) consume(buf[bb], qbuf[bb]);
    });
  }

  // ---- report the rows this range wrote partials of; the wave completing a
  // row merges it.
  // this wave's partial stores have completed (and, being agent-scope, are
  // visible to every XCD) before any counter below is raised
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  wait_vm_all();
  // rows go 64 at a time, one per lane: their counters are raised by
  // concurrent atomics (the first row's by lane 0, possibly inside the loop),
  // then the rows this wave completed are merged
  int rs = first.s, rxi = first.xi, rn = first.n, rj = first.j, rcum = cum0;
  const int xbv = lane <= 8 ? xcd_begin(N, lane) : 0;     // XCD boundaries of the flat list, for merges
  int left = nsteps;
  bool first_row = true;
  while (left > 0) {
    int lx = -1, lmine = 0, ln = 0, ls = 0, lxi = 0, lsx = 0;
    bool lpend = false;
    for (int k = 0; k < kWave && left > 0; ++k) {
      const int mine = min(left, rn - rj);
      // a whole row written directly has no partial and no counter
      if (!(kDirect && mine == rn)) {
        if (lane == k) {
          lx = rxi * p.S + rs;
          lmine = mine;
          ln = rn;
          ls = rs;
          lxi = rxi;
          lsx = rxi * T + rcum;
          lpend = first_row && pend_at > 0;
        }
      } else {
        --k;     // the lane stays free for the next row
      }
      first_row = false;
      left -= mine;
      rj = 0;
      if (left > 0) {
        do {
          rcum += rn;
          if (++rs == p.S) {
            rs = 0;
            rcum = 0;
            ++rxi;
          }
          rn = split_steps<TS>(clamp_ctx(uniform_load(p.ctx + rs), max_ctx), p);
        } while (rn == 0);
      }
    }
    int done_now = 0;
    if (lx >= 0) {
      uint64_t* ctr = p.row_done + (int64_t)lx * kCounterStride;
      done_now = report_total(ctr, p.epoch, lmine, lpend ? pend_old : report_steps(ctr, p.epoch, lmine));
    }
    uint64_t complete = __ballot(lx >= 0 && done_now == ln);   // every partial of the row is in place
    while (complete) {
      const int l = __builtin_ctzll(complete);
      complete &= complete - 1;
      merge_row<D, GE::AL>(p, __builtin_amdgcn_readlane(lx, l), __builtin_amdgcn_readlane(ls, l),
                          __builtin_amdgcn_readlane(lxi, l), __builtin_amdgcn_readlane(ln, l),
                          __builtin_amdgcn_readlane(lsx, l), N, xbv, lane);
    }
  }
}

// ---------------------------------------------------------------- launches
hipError_t launch_single(const DecodeParams& p, int D, int kvt, int B, int grid, hipStream_t stream) {
  return with_variant<false>(D, kvt, B, [&](auto dc, auto kc, auto bc) {
    hipLaunchKernelGGL((pa_decode_kernel<decltype(dc)::value, decltype(kc)::value, decltype(bc)::value>), dim3(grid),
                       dim3(kWave * kNW), 0, stream, p);
    return hipGetLastError();
  });
}

// Steps of K/V registers per wave: one computed, the rest in flight (about
// 40 KB per wave, 160 KB per CU with one wave per SIMD).
template <int D, int KVT>
constexpr int split_nbuf() { return D == 64 ? 8 : (KVT == PKV_KV_INT4 ? 4 : 5); }

// f(IC<D>, IC<KVT>, IC<B>) for the split kernel's variants: every storage
// type has its own (per-channel INT8 folds its K scales into the query as hi
// + lo parts, which the per-tensor codes kernel does not read).
template <class F>
auto with_split_variant(int D, int kvt, int B, F&& f) {
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
      case PKV_KV_INT4: return by_b(dc, IC<PKV_KV_INT4>{});
      default: return by_b(dc, IC<PKV_KV_INT8>{});
    }
  };
  return D == 64 ? by_kv(IC<64>{}) : by_kv(IC<128>{});
}
constexpr int kMaxBlocksPerCU = 1;       // persistent grid: one workgroup (a wave per SIMD) per CU

const void* split_kernel_fn(int D, int kvt, int B) {
  return with_split_variant(D, kvt, B, [](auto dc, auto kc, auto bc) {
    constexpr int Dv = decltype(dc)::value, Kv = decltype(kc)::value, Bv = decltype(bc)::value;
    return reinterpret_cast<const void*>(&pa_split_kernel<Dv, Kv, Bv, split_nbuf<Dv, Kv>(), true>);
  });
}

// Compute units of the current device (cached per device).
int device_cus(int* cus) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    cache[dev] = n;
  }
  *cus = cache[dev];
  return 0;
}

// Resident workgroups per CU of one split-kernel variant (cached).
int split_blocks_per_cu(int D, int kvt, int B) {
  static std::mutex mu;
  static int cache[64][2][6][3] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  const int di = D == 64 ? 0 : 1, bi = B == 8 ? 0 : (B == 16 ? 1 : 2);
  std::lock_guard<std::mutex> lk(mu);
  int& c = cache[dev][di][kvt][bi];
  if (c == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, split_kernel_fn(D, kvt, B), kWave * kNW, 0) != hipSuccess)
      n = 1;
    c = n < 1 ? 1 : (n > kMaxBlocksPerCU ? kMaxBlocksPerCU : n);
  }
  return c;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A fresh tag per split-context call.  The sequence starts at a value drawn
// from the clock and the address space, so stale counters left in reused
// memory by another process are not mistaken for this call's.
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{(uint32_t)(std::chrono::steady_clock::now().time_since_epoch().count() ^
                                                  (uintptr_t)&counter ^ 0x9e3779b9u)};
  return counter.fetch_add(1, std::memory_order_relaxed);
}

// Workgroups of the split kernel: one resident wave per SIMD slot the
// variant can use, but never more waves than there are steps.
int64_t split_grid(int64_t steps_ub, int cus, int blocks_per_cu) {
  int64_t nwg = (int64_t)cus * blocks_per_cu;
  nwg = std::min<int64_t>(nwg, ceil_div(steps_ub, kNW));
  return std::max<int64_t>(8, ceil_div(nwg, 8) * 8);
}

struct SplitSizes {
  int64_t rows, slots_cap, cnt_bytes, ml_bytes, acc_bytes;
};

// Scratch of paged_attn_decode_noalloc: the split form's row counters and
// partials, in a static device array that every GPU the library runs on
// holds until the process ends.  Its contents need no clearing: the row
// counters are tagged with each call's epoch, and partials are written
// before they are read.
constexpr uint64_t kScratchBytes = 32ull << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// The device address of this device's scratch array, looked up once per
// device with that device current (in host code `scratch` names a host-side
// stand-in, never a device address).
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return -1;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return 0;
}

// Workspace regions for the largest grid any variant may launch.  rows_or_0:
// the call's (sequence, KV head, head tile) rows when known, else 0 for the
// bound S * Hq (one head per row when G == 1), which sizes a workspace
// without the pool's head count.
bool split_sizes(int32_t S, int32_t Hq, int32_t rows_or_0, int32_t D, int32_t W, int32_t B, int32_t P,
                 SplitSizes* z) {
  int cus = 0;
  if (device_cus(&cus) != 0) return false;
  z->rows = rows_or_0 > 0 ? (int64_t)rows_or_0 : (int64_t)S * Hq;
  (void)P;                       // partials are per (row, wave) segment, whatever the partition size
  const int64_t steps_ub = z->rows * ceil_div((int64_t)W * B, 16);
  const int64_t waves_cap = split_grid(steps_ub, cus, kMaxBlocksPerCU) * kNW;
  z->slots_cap = z->rows + waves_cap;
  z->cnt_bytes = align_up((uint64_t)z->rows * kCounterStride * sizeof(uint64_t));
  z->ml_bytes = align_up((uint64_t)z->slots_cap * 16 * 2 * sizeof(float));
  z->acc_bytes = align_up((uint64_t)z->slots_cap * (D / 16) * 256 * sizeof(float));
  return true;
}

// keep_cached: load K/V with the default cache policy (tables that share
// blocks) instead of streaming them
void launch_split(const SplitParams& p, int D, int kvt, int B, int grid, bool keep_cached, hipStream_t stream) {
  with_split_variant(D, kvt, B, [&](auto dc, auto kc, auto bc) {
    constexpr int Dv = decltype(dc)::value, Kv = decltype(kc)::value, Bv = decltype(bc)::value;
    if (keep_cached)
      hipLaunchKernelGGL((pa_split_kernel<Dv, Kv, Bv, split_nbuf<Dv, Kv>(), false>), dim3(grid), dim3(kWave * kNW), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((pa_split_kernel<Dv, Kv, Bv, split_nbuf<Dv, Kv>(), true>), dim3(grid), dim3(kWave * kNW), 0,
                         stream, p);
    return 0;
  });
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
  SplitSizes z;
  if (!split_sizes(num_seqs, num_q_heads, 0, head_dim, table_width, block_size, partition_size, &z)) return 0;
  return (uint64_t)(z.cnt_bytes + z.ml_bytes + z.acc_bytes);
}

namespace {

// The shared-prefix form's arguments and workspace regions past the split
// form's own (which comes first, as for paged_attn_decode).
struct SharedPrefixCall {
  const int32_t* prefix_table;
  int32_t prefix_len;
  float* ml;               // [S][Hq] (m, l) of the rows the split pass writes
  uint16_t* qfold;         // [S][Hq][2 D] the query with K channel scales folded in (those storage types)
  PrefixPassGeometry geo;
};

// A decode call.  With use_scratch the split form's workspace is this
// device's copy of the static scratch array (sized exactly for the call and
// refused beyond kScratchBytes) and the workspace arguments are ignored.
pkv_status decode_impl(float* out, const void* q, const pkv_pool* pool, int32_t layer, const void* key,
                       const void* value, const int32_t* block_tables, int32_t table_width,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                       int32_t kv_dtype, const pkv_kv_scales* kv_scales, int32_t partition_size,
                       int32_t sliding_window, void* workspace, uint64_t workspace_bytes, hipStream_t stream,
                       bool use_scratch = false, const SharedPrefixCall* sp = nullptr, uint32_t flags = 0) {
  const bool append = key != nullptr || value != nullptr;
  if (flags & ~PKV_DECODE_KEEP_KV_CACHED) {
    set_error("unknown decode flags 0x%x", flags);
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
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs is negative");
  if (num_seqs == 0) { clear_error(); return PKV_OK; }
  if (!out || !q || !block_tables || !context_lens) return fail(PKV_ERR_INVALID, "NULL device pointer");
  if (append && (!key || !value)) return fail(PKV_ERR_INVALID, "key and value must both be given");
  if (sliding_window < 0) return fail(PKV_ERR_INVALID, "sliding_window is negative");
  if (append && partition_size == 0)
    return fail(PKV_ERR_UNSUPPORTED, "the appending decode runs in the split-context form (partition_size > 0)");
  if (append && ((uintptr_t)key % 16 || (uintptr_t)value % 16))
    return fail(PKV_ERR_INVALID, "key and value must be 16-byte aligned");
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
  const int32_t QT = (G + 15) / 16;
  const int64_t rows = (int64_t)num_seqs * c.num_kv_heads * QT;
  const uint64_t scale_layer = channel ? (uint64_t)c.num_kv_heads * c.head_dim
                                      : (uint64_t)c.num_blocks * c.num_kv_heads * c.block_size;
  char* kl = static_cast<char*>(pool->k) + (uint64_t)layer * pool->layer_bytes;
  char* vl = static_cast<char*>(pool->v) + (uint64_t)layer * pool->layer_bytes;
  float* ksl = pool->k_scale ? pool->k_scale + layer * scale_layer : nullptr;
  float* vsl = pool->v_scale ? pool->v_scale + layer * scale_layer : nullptr;
  // the split form's sizes and workspace, checked before anything is launched
  SplitSizes z{};
  int64_t split_grid_wg = 0;
  void* ws_base = workspace;
  if (partition_size != 0) {
    if (partition_size < 0 || partition_size % 32 != 0) {
      set_error("partition_size %d must be 0 or a positive multiple of 32", partition_size);
      return PKV_ERR_INVALID;
    }
    const int TS = c.kv_dtype == PKV_KV_BF16 ? 16 : (c.kv_dtype == PKV_KV_INT4 ? 64 : 32);
    const int64_t steps_ub = rows * ceil_div((int64_t)table_width * c.block_size, TS);
    if (steps_ub > INT32_MAX / 2) return fail(PKV_ERR_INVALID, "problem too large for one call");
    if (!split_sizes(num_seqs, num_q_heads, use_scratch ? (int32_t)rows : 0, c.head_dim, table_width,
                     c.block_size, partition_size, &z))
      return fail(PKV_ERR_HIP, "could not query the current device");
    const uint64_t need = (uint64_t)(z.cnt_bytes + z.ml_bytes + z.acc_bytes);
    if (z.acc_bytes > (int64_t)UINT32_MAX)
      return fail(PKV_ERR_INVALID, "too many (sequence, KV head) rows for one split-context call: split the batch");
    if (use_scratch) {
      if (need > kScratchBytes) {
        set_error("this call needs %llu bytes of scratch, the static scratch holds %llu: split the batch",
                  (unsigned long long)need, (unsigned long long)kScratchBytes);
        return PKV_ERR_INVALID;
      }
      if (scratch_address(&ws_base) != 0) return fail(PKV_ERR_HIP, "could not find the scratch array on this device");
    } else {
      if (!workspace || workspace_bytes < need) {
        set_error("workspace of %llu bytes needed, got %llu", (unsigned long long)need,
                  (unsigned long long)workspace_bytes);
        return PKV_ERR_INVALID;
      }
      if (((uintptr_t)workspace) % 256) return fail(PKV_ERR_INVALID, "workspace must be 256-byte aligned");
    }
    int cus = 0;
    device_cus(&cus);
    const int bpc = split_blocks_per_cu(c.head_dim, c.kv_dtype, c.block_size);
    split_grid_wg = split_grid(steps_ub, cus, bpc);
    if (split_grid_wg * kNW + z.rows > z.slots_cap) return fail(PKV_ERR_INVALID, "internal: workspace sizing");
  }
  // the query the kernels read: q itself, or (K channel scales, single-pass
  // forms) q with the scales folded in, written into the output rows first;
  // the split form folds them as it loads each query
  const uint16_t* qk = static_cast<const uint16_t*>(q);
  int32_t q_stride = c.head_dim;
  if (channel && partition_size == 0) {
    const int64_t n = (int64_t)num_seqs * num_q_heads * c.head_dim;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > INT32_MAX) return fail(PKV_ERR_INVALID, "too many queries in one call");
    hipLaunchKernelGGL(fold_q_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, qk,
                       reinterpret_cast<uint16_t*>(out), ksl, n, num_q_heads, num_q_heads / c.num_kv_heads,
                       c.head_dim);
    qk = reinterpret_cast<const uint16_t*>(out);
    q_stride = 2 * c.head_dim;
  }

  hipError_t e = hipSuccess;
  if (partition_size == 0 && c.kv_dtype == PKV_KV_INT4) {
    // one query per sequence through the prefill kernel, which reads INT4
    PrefillDecodeArgs a{};
    a.out = out;
    a.q = qk;
    a.q_stride = q_stride;
    a.pool = pool;
    a.layer = layer;
    a.block_tables = block_tables;
    a.table_width = table_width;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.sliding_window = sliding_window;
    a.qk_scale = scale * kLog2e * ksc;
    a.out_scale = vsc;
    a.ks = ksl;
    a.vs = vsl;
    a.vs_ch = vsl;
    e = launch_prefill_as_decode(a, stream);
  } else if (partition_size == 0) {
    const int64_t grid = (rows + 7) / 8 * 8;
    if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "too many work items");
    DecodeParams p{};
    p.q = qk;
    p.q_stride = q_stride;
    p.vs_ch = channel ? vsl : nullptr;
    p.out = out;
    p.k = kl;
    p.v = vl;
    p.ks = ksl;
    p.vs = vsl;
    p.bt = block_tables;
    p.ctx = context_lens;
    p.W = table_width;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = c.num_kv_heads;
    p.G = G;
    p.QT = QT;
    p.num_blocks = c.num_blocks;
    p.num_items = (int32_t)rows;
    p.win = sliding_window;
    p.qk_scale = scale * kLog2e * ksc;
    p.out_scale = vsc;
    e = launch_single(p, c.head_dim, c.kv_dtype, c.block_size, (int)grid, stream);
  } else {
    const int64_t grid = split_grid_wg;
    SplitParams p{};
    p.q = qk;
    p.ks_ch = channel ? ksl : nullptr;
    p.vs_ch = channel ? vsl : nullptr;
    p.out = out;
    p.k = kl;
    p.v = vl;
    p.ks = ksl;
    p.vs = vsl;
    p.bt = block_tables;
    p.ctx = context_lens;
    p.new_k = static_cast<const uint16_t*>(key);
    p.new_v = static_cast<const uint16_t*>(value);
    p.enc_k = ksc;
    p.enc_v = vsc;
    char* ws = static_cast<char*>(ws_base);
    p.row_done = reinterpret_cast<uint64_t*>(ws);
    p.part_ml = reinterpret_cast<float*>(ws + z.cnt_bytes);
    p.part_acc = reinterpret_cast<float*>(ws + z.cnt_bytes + z.ml_bytes);
    p.acc_bytes = (uint32_t)z.acc_bytes;
    p.ml_bytes = (uint32_t)z.ml_bytes;
    p.W = table_width;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.Hkv = c.num_kv_heads;
    p.G = G;
    p.QT = QT;
    p.HQ = c.num_kv_heads * QT;
    p.num_blocks = c.num_blocks;
    p.NWV = (int32_t)(grid * kNW);
    p.win = sliding_window;
    p.epoch = next_epoch();
    p.qk_scale = scale * kLog2e * ksc;
    p.out_scale = vsc;
    p.prefix_len = sp ? sp->prefix_len : 0;
    p.ml_out = sp ? sp->ml : nullptr;
    launch_split(p, c.head_dim, c.kv_dtype, c.block_size, (int)grid, (flags & PKV_DECODE_KEEP_KV_CACHED) != 0, stream);
    e = hipGetLastError();
    if (e == hipSuccess && sp) {
      // the shared prefix, attended once per KV head for all sequences and
      // merged into the rows the split pass wrote
      PrefixPassArgs a{};
      a.d.q = qk;
      a.d.q_stride = q_stride;
      if (channel) {   // the prefill kernel's products read the folded query
        const int64_t n = (int64_t)num_seqs * num_q_heads * c.head_dim;
        hipLaunchKernelGGL(fold_q_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, qk, sp->qfold,
                           ksl, n, num_q_heads, G, c.head_dim);
        a.d.q = sp->qfold;
        a.d.q_stride = 2 * c.head_dim;
      }
      a.d.out = out;
      a.d.pool = pool;
      a.d.layer = layer;
      a.d.block_tables = sp->prefix_table;
      a.d.table_width = sp->prefix_len / c.block_size;
      a.d.context_lens = context_lens;
      a.d.num_seqs = num_seqs;
      a.d.num_q_heads = num_q_heads;
      a.d.sliding_window = 0;
      a.d.qk_scale = p.qk_scale;
      a.d.out_scale = vsc;
      a.d.ks = ksl;
      a.d.vs = vsl;
      a.d.vs_ch = channel ? vsl : nullptr;
      a.prefix_len = sp->prefix_len;
      a.merge_ml = sp->ml;
      a.geo = sp->geo;
      e = launch_prefix_pass(a, stream);
    }
  }
  if (e != hipSuccess) {
    set_error("paged_attn_decode launch failed: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  clear_error();
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status paged_attn_decode(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                        const int32_t* block_tables, int32_t table_width,
                                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                        float scale, int32_t kv_dtype, const pkv_kv_scales* kv_scales,
                                        int32_t partition_size, void* workspace, uint64_t workspace_bytes,
                                        hipStream_t stream) {
  return decode_impl(out, q, pool, layer, nullptr, nullptr, block_tables, table_width, context_lens, num_seqs,
                     num_q_heads, scale, kv_dtype, kv_scales, partition_size, 0, workspace, workspace_bytes,
                     stream);
}

extern "C" pkv_status paged_attn_decode_append(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                               const void* key, const void* value, const int32_t* block_tables,
                                               int32_t table_width, const int32_t* context_lens,
                                               int32_t num_seqs, int32_t num_q_heads, float scale,
                                               int32_t kv_dtype, const pkv_kv_scales* kv_scales,
                                               int32_t partition_size, void* workspace,
                                               uint64_t workspace_bytes, hipStream_t stream) {
  if (!key || !value) return fail(PKV_ERR_INVALID, "key and value must be non-NULL");
  return decode_impl(out, q, pool, layer, key, value, block_tables, table_width, context_lens, num_seqs,
                     num_q_heads, scale, kv_dtype, kv_scales, partition_size, 0, workspace, workspace_bytes,
                     stream);
}

extern "C" pkv_status paged_attn_decode_ex(const pkv_decode_args* a, hipStream_t stream) {
  if (!a) return fail(PKV_ERR_INVALID, "NULL argument block");
  if ((a->key == nullptr) != (a->value == nullptr)) return fail(PKV_ERR_INVALID, "key and value must both be given");
  return decode_impl(a->out, a->q, a->pool, a->layer, a->key, a->value, a->block_tables, a->table_width,
                     a->context_lens, a->num_seqs, a->num_q_heads, a->scale, a->kv_dtype, a->kv_scales,
                     a->partition_size, a->sliding_window, a->workspace, a->workspace_bytes, stream, false, nullptr,
                     a->flags);
}

extern "C" pkv_status paged_attn_decode_noalloc(const pkv_decode_args* a, hipStream_t stream) {
  if (!a) return fail(PKV_ERR_INVALID, "NULL argument block");
  if ((a->key == nullptr) != (a->value == nullptr)) return fail(PKV_ERR_INVALID, "key and value must both be given");
  return decode_impl(a->out, a->q, a->pool, a->layer, a->key, a->value, a->block_tables, a->table_width,
                     a->context_lens, a->num_seqs, a->num_q_heads, a->scale, a->kv_dtype, a->kv_scales,
                     a->partition_size, a->sliding_window, nullptr, 0, stream, true, nullptr, a->flags);
}

namespace {

// Workspace layout of a shared-prefix decode: the split form's regions, the
// rows' (m, l), then the folded query (storage with K channel scales).
struct SharedPrefixSizes {
  uint64_t split, ml, qfold, total;
  PrefixPassGeometry geo;
};
bool shared_prefix_sizes(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t W, int32_t B, int32_t kvt,
                         int32_t prefix_len, SharedPrefixSizes* z) {
  SplitSizes sz;
  if (!split_sizes(S, Hq, 0, D, W, B, 1, &sz)) return false;
  if (!prefix_pass_geometry(S, Hq, Hkv, D, kvt, B, prefix_len, &z->geo)) return false;
  z->split = (uint64_t)(sz.cnt_bytes + sz.ml_bytes + sz.acc_bytes);
  z->ml = align_up((uint64_t)S * Hq * 2 * sizeof(float));
  z->qfold = has_k_channel_scales(kvt) ? align_up((uint64_t)S * Hq * 2 * D * sizeof(uint16_t)) : 0;
  z->total = z->split + z->ml + z->qfold;
  return true;
}

}  // namespace

extern "C" uint64_t paged_attn_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                             int32_t num_kv_heads, int32_t head_dim,
                                                             int32_t table_width, int32_t block_size,
                                                             int32_t kv_dtype, int32_t prefix_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 ||
      table_width <= 0 || block_size <= 0 || prefix_len < 0)
    return 0;
  if (prefix_len == 0) return paged_attn_workspace_bytes(num_seqs, num_q_heads, head_dim, table_width, block_size, 32);
  SharedPrefixSizes z;
  if (!shared_prefix_sizes(num_seqs, num_q_heads, num_kv_heads, head_dim, table_width, block_size, kv_dtype,
                           prefix_len, &z))
    return 0;
  return z.total;   // every region grows with num_seqs: it also serves smaller batches
}

extern "C" pkv_status paged_attn_decode_shared_prefix(const pkv_decode_args* a, const int32_t* prefix_table,
                                                      int32_t prefix_len, hipStream_t stream) {
  if (!a) return fail(PKV_ERR_INVALID, "NULL argument block");
  if ((a->key == nullptr) != (a->value == nullptr)) return fail(PKV_ERR_INVALID, "key and value must both be given");
  if (prefix_len < 0) return fail(PKV_ERR_INVALID, "prefix_len is negative");
  if (prefix_len == 0)
    return decode_impl(a->out, a->q, a->pool, a->layer, a->key, a->value, a->block_tables, a->table_width,
                       a->context_lens, a->num_seqs, a->num_q_heads, a->scale, a->kv_dtype, a->kv_scales,
                       a->partition_size, a->sliding_window, a->workspace, a->workspace_bytes, stream, false, nullptr,
                       a->flags);
  pkv_status st = check_pool(a->pool);
  if (st != PKV_OK) return st;
  const pkv_pool_config& c = a->pool->cfg;
  if (prefix_len % c.block_size != 0) {
    set_error("prefix_len %d is not a multiple of the block size %d", prefix_len, c.block_size);
    return PKV_ERR_INVALID;
  }
  if (prefix_len > INT32_MAX / 2) return fail(PKV_ERR_INVALID, "prefix_len too large");
  if (!prefix_table) return fail(PKV_ERR_INVALID, "NULL prefix_table");
  if (a->partition_size == 0)
    return fail(PKV_ERR_UNSUPPORTED, "the shared-prefix decode runs in the split-context form (partition_size > 0)");
  if (a->sliding_window != 0) return fail(PKV_ERR_UNSUPPORTED, "the shared-prefix decode takes no sliding window");
  if (a->num_seqs <= 0) return decode_impl(a->out, a->q, a->pool, a->layer, a->key, a->value, a->block_tables,
                                           a->table_width, a->context_lens, a->num_seqs, a->num_q_heads, a->scale,
                                           a->kv_dtype, a->kv_scales, a->partition_size, 0, a->workspace,
                                           a->workspace_bytes, stream, false, nullptr, a->flags);
  if (a->num_q_heads <= 0 || a->num_q_heads % c.num_kv_heads != 0 || a->table_width <= 0)
    return decode_impl(a->out, a->q, a->pool, a->layer, a->key, a->value, a->block_tables, a->table_width,
                       a->context_lens, a->num_seqs, a->num_q_heads, a->scale, a->kv_dtype, a->kv_scales,
                       a->partition_size, 0, a->workspace, a->workspace_bytes, stream, false, nullptr,
                       a->flags);   // reports the error
  SharedPrefixSizes z;
  if (!shared_prefix_sizes(a->num_seqs, a->num_q_heads, c.num_kv_heads, c.head_dim, a->table_width, c.block_size,
                           c.kv_dtype, prefix_len, &z))
    return fail(PKV_ERR_INVALID, "shared-prefix decode too large for one call");
  if (!a->workspace || a->workspace_bytes < z.total) {
    set_error("workspace of %llu bytes needed, got %llu", (unsigned long long)z.total,
              (unsigned long long)a->workspace_bytes);
    return PKV_ERR_INVALID;
  }
  if (((uintptr_t)a->workspace) % 256) return fail(PKV_ERR_INVALID, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(a->workspace);
  SharedPrefixCall sp{};
  sp.prefix_table = prefix_table;
  sp.prefix_len = prefix_len;
  sp.ml = reinterpret_cast<float*>(ws + z.split);
  sp.qfold = z.qfold ? reinterpret_cast<uint16_t*>(ws + z.split + z.ml) : nullptr;
  sp.geo = z.geo;
  return decode_impl(a->out, a->q, a->pool, a->layer, a->key, a->value, a->block_tables, a->table_width,
                     a->context_lens, a->num_seqs, a->num_q_heads, a->scale, a->kv_dtype, a->kv_scales,
                     a->partition_size, 0, a->workspace, z.split, stream, false, &sp, a->flags);
}
