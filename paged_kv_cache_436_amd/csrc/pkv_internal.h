// Internal helpers shared by the library's translation units (not installed).
#pragma once

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
    default: return 0;
  }
}

// Bytes of one (block, head) tile of K (or V).
inline uint64_t tile_bytes_of(const pkv_pool_config& c) {
  return (uint64_t)c.block_size * c.head_dim * elem_bits(c.kv_dtype) / 8;
}

// Calibrated per-(layer, head, dim) scales kept in the pool.
inline bool has_channel_scales(int32_t kv_dtype) {
  return kv_dtype == PKV_KV_INT8_CHANNEL || kv_dtype == PKV_KV_INT4;
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

}  // namespace pkv
