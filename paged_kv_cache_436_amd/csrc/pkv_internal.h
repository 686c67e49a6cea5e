// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline pkv_status fail(pkv_status st, const char* msg) {
  set_error("%s", msg);
  return st;
}

// Bits per stored K/V element; 0 for an unknown dtype.
inline int elem_bits(int32_t kv_dtype) {
  switch (kv_dtype) {
    case PKV_KV_BF16: return 16;
    case PKV_KV_FP8_E5M2: return 8;
    case PKV_KV_INT8: return 8;
    case PKV_KV_INT8_TENSOR: return 8;
    case PKV_KV_INT8_CHANNEL: return 8;
    case PKV_KV_INT4: return 4;
    case PKV_KV_INT8_KCHANNEL_VTENSOR: return 8;
    default: return 0;
  }
}

// Bytes of one (block, head) tile of K (or V).
inline uint64_t tile_bytes_of(const pkv_pool_config& c) {
  return (uint64_t)c.block_size * c.head_dim * elem_bits(c.kv_dtype) / 8;
}

// Calibrated per-(layer, head, dim) scales kept in the pool, for K and for V.
inline bool has_channel_scales(int32_t kv_dtype) {
  return kv_dtype == PKV_KV_INT8_CHANNEL || kv_dtype == PKV_KV_INT4;
}

// Calibrated per-(layer, head, dim) K scales kept in the pool (the decode
// kernels fold them into the query); V may have its own granularity.
inline bool has_k_channel_scales(int32_t kv_dtype) {
  return has_channel_scales(kv_dtype) || kv_dtype == PKV_KV_INT8_KCHANNEL_VTENSOR;
}

// The call's per-tensor scales: K and V (fp8, INT8 per tensor), or V only.
inline bool has_tensor_k_scale(int32_t kv_dtype) {
  return kv_dtype == PKV_KV_FP8_E5M2 || kv_dtype == PKV_KV_INT8_TENSOR;
}
inline bool has_tensor_v_scale(int32_t kv_dtype) {
  return has_tensor_k_scale(kv_dtype) || kv_dtype == PKV_KV_INT8_KCHANNEL_VTENSOR;
}

// The call's per-tensor scales of this storage type, checked: *ks / *vs keep
// 1.0 where the type has no such scale or scales is NULL.
inline pkv_status tensor_scales(int32_t kv_dtype, const pkv_kv_scales* scales, float* ks, float* vs) {
  *ks = 1.f;
  *vs = 1.f;
  if (!scales) return PKV_OK;
  if (has_tensor_k_scale(kv_dtype)) {
    *ks = scales->k_scale;
    if (!(*ks > 0.f) || !(*ks < INFINITY)) return fail(PKV_ERR_INVALID, "per-tensor scales must be positive and finite");
  }
  if (has_tensor_v_scale(kv_dtype)) {
    *vs = scales->v_scale;
    if (!(*vs > 0.f) || !(*vs < INFINITY)) return fail(PKV_ERR_INVALID, "per-tensor scales must be positive and finite");
  }
  return PKV_OK;
}

constexpr uint64_t kRegionAlign = 256;
inline uint64_t align_up(uint64_t n) { return (n + kRegionAlign - 1) / kRegionAlign * kRegionAlign; }

// Region byte offsets of a pool; false if the configuration is invalid
// (message set).
struct Regions {
  uint64_t k, v, ks, vs, total, kv_bytes, scale_bytes;
};
bool pool_regions(const pkv_pool_config* cfg, Regions* r);

pkv_status check_pool(const pkv_pool* pool);

// The single-pass decode of one query per sequence run by the prefill kernel
// (prefill_kernels.hip), for storage the single-pass decode kernel does not
// read.  Arguments are checked by the caller; q is the query the kernels read
// (folded for per-channel scales, q_stride elements between rows).
struct PrefillDecodeArgs {
  float* out;
  const uint16_t* q;
  int32_t q_stride;
  const pkv_pool* pool;
  int32_t layer;
  const int32_t* block_tables;
  int32_t table_width;
  const int32_t* context_lens;
  int32_t num_seqs, num_q_heads;
  int32_t sliding_window;   // 0: whole context; w > 0: the last w positions
  float qk_scale;           // softmax scale * log2(e) (* fp8 k scale)
  float out_scale;          // per-tensor v scale, else 1
  const float* ks;          // this layer's K / V scale regions, or null
  const float* vs;
  const float* vs_ch;       // per-channel V scales of the layer, or null
};
hipError_t launch_prefill_as_decode(const PrefillDecodeArgs& a, hipStream_t stream);

// The shared-prefix pass of a decode (prefill_kernels.hip): for every KV
// head, the (sequence, head) pairs of all sequences attend the shared prefix
// (positions [0, min(ctx_s, prefix_len)), read through d.block_tables = the
// prefix table of d.table_width entries), and their results are merged with
// the result already in d.out, whose (m, l) per row are in merge_ml.
// d.sliding_window must be 0.
struct PrefixPassGeometry {
  int32_t tiles;       // column groups per KV head (one workgroup each)
  int32_t chunk_len;   // prefix positions per wave (multiple of 32)
};
bool prefix_pass_geometry(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t kv_dtype, int32_t block_size, int32_t prefix_len, PrefixPassGeometry* g);
struct PrefixPassArgs {
  PrefillDecodeArgs d;
  int32_t prefix_len;
  const float* merge_ml;   // [S][Hq] (m, l) of d.out's rows
  PrefixPassGeometry geo;
};
hipError_t launch_prefix_pass(const PrefixPassArgs& a, hipStream_t stream);

}  // namespace pkv
