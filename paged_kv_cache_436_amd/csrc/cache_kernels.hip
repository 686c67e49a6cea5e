// Cache write (reshape_and_cache) and copy-on-write block copy (copy_blocks)
// for gfx950.
//
// reshape_and_cache puts the newest token's K and V into the slot its block
// table names ("KV Cache 原理与 PagedAttention", §一 decode step: only K_t and
// V_t are computed and appended; §三 工作方式 steps 2-3), quantising on the way
// in for 8-bit storage (same page, §四; bjdmk.com.cn article, §5.2 per-token-
// head scales).  copy_blocks copies a shared block before its writer is
// repointed (bjdmk.com.cn article, §3.2 Copy-on-Write).  swap_blocks moves
// blocks between the device pool and a pool in pinned host memory, for
// requests that are preempted and later resumed (same article, §6.1).
#include <hip/hip_runtime.h>

#include "pkv_codecs.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ------------------------------------------------------------------ kernels
// One wavefront per (token, kv head).  Lane i handles dims i, i+64, ...
// Tile offsets follow the documented layout: K (t, d) at
// ((d / X) * B + t) * X + d % X, V (t, d) at ((t / 4) * D + d) * 4 + t % 4.
template <int KVT>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    const int64_t* __restrict__ slots, int32_t num_tokens, int32_t H, int32_t D, int32_t B,
    int64_t num_slots, void* __restrict__ kdst, void* __restrict__ vdst,
    float* __restrict__ kscale, float* __restrict__ vscale, float k_scale, float v_scale) {
  const int wave = (int)(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (wave >= num_tokens * H) return;
  const int n = wave / H;
  const int h = wave % H;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / B;
  const int t = (int)(slot % B);
  const int64_t tile = (blk * H + h) * (int64_t)B * D;  // in elements
  const uint16_t* kx = key + ((int64_t)n * H + h) * D;
  const uint16_t* vx = value + ((int64_t)n * H + h) * D;

  if constexpr (KVT == PKV_KV_BF16) {
    uint16_t* kd = static_cast<uint16_t*>(kdst) + tile;
    uint16_t* vd = static_cast<uint16_t*>(vdst) + tile;
    for (int d = lane; d < D; d += kWave) {
      kd[((d >> 3) * B + t) * 8 + (d & 7)] = kx[d];
      vd[((t >> 2) * D + d) * 4 + (t & 3)] = vx[d];
    }
  } else if constexpr (KVT == PKV_KV_FP8_E5M2) {
    uint8_t* kd = static_cast<uint8_t*>(kdst) + tile;
    uint8_t* vd = static_cast<uint8_t*>(vdst) + tile;
    for (int d = lane; d < D; d += kWave) {
      kd[((d >> 4) * B + t) * 16 + (d & 15)] = (uint8_t)fp8_store(kx[d], k_scale);
      vd[((t >> 2) * D + d) * 4 + (t & 3)] = (uint8_t)fp8_store(vx[d], v_scale);
    }
  } else if constexpr (KVT == PKV_KV_INT8_TENSOR || KVT == PKV_KV_INT8_CHANNEL) {
    // calibrated scales: one per tensor (the call's) or per (head, dim) (this
    // layer's channel scales, [H][D])
    int8_t* kd = static_cast<int8_t*>(kdst) + tile;
    int8_t* vd = static_cast<int8_t*>(vdst) + tile;
    for (int d = lane; d < D; d += kWave) {
      // (per channel with no V channel scales: V per tensor, the call's)
      const float ks = KVT == PKV_KV_INT8_TENSOR ? k_scale : kscale[h * D + d];
      const float vs = KVT == PKV_KV_INT8_TENSOR ? v_scale : (vscale ? vscale[h * D + d] : v_scale);
      kd[((d >> 4) * B + t) * 16 + (d & 15)] = (int8_t)int8_store(kx[d], ks);
      vd[((t >> 2) * D + d) * 4 + (t & 3)] = (int8_t)int8_store(vx[d], vs);
    }
  } else if constexpr (KVT == PKV_KV_INT4) {
    // two codes per byte, each byte belonging to one token; lane b < D / 2
    // writes K byte b and V byte b of the token (nibble placement as the
    // pool layout documents)
    uint8_t* kd = static_cast<uint8_t*>(kdst) + tile / 2;
    uint8_t* vd = static_cast<uint8_t*>(vdst) + tile / 2;
    const int P = D / 8;                            // bytes per piece
    const float* ksc = kscale + h * D;
    const float* vsc = vscale + h * D;
    if (lane < D / 2) {
      // K: piece (j, t), byte o = 4 kk + bw; the byte's low / high nibbles are
      // elements i and i + 2 of dims 32 kk + 8 j + i
      const int j = lane / P, o = lane % P, kk = o >> 2, bw = o & 3;
      const int d0 = 32 * kk + 8 * j + int4_k_lo_elem(bw);
      kd[(j * B + t) * P + o] = (uint8_t)(int4_store(kx[d0], ksc[d0]) | (int4_store(kx[d0 + 2], ksc[d0 + 2]) << 4));
      // V: piece (t / 4, m), word w, byte 2 (r % 2) + r / 2 (r = t % 4) holds
      // dims 16 (2w) + m (low) and 16 (2w + 1) + m (high)
      const int m = lane % 16, w = lane / 16, r = t & 3;
      const int e0 = 32 * w + m, e1 = e0 + 16;
      vd[((t >> 2) * 16 + m) * P + 4 * w + 2 * (r & 1) + (r >> 1)] =
          (uint8_t)(int4_store(vx[e0], vsc[e0]) | (int4_store(vx[e1], vsc[e1]) << 4));
    }
  } else {  // INT8, symmetric per (token, head)
    int8_t* kd = static_cast<int8_t*>(kdst) + tile;
    int8_t* vd = static_cast<int8_t*>(vdst) + tile;
    float kmax = 0.f, vmax = 0.f;
    for (int d = lane; d < D; d += kWave) {
      kmax = fmaxf(kmax, fabsf(bf16_bits_to_float(kx[d])));
      vmax = fmaxf(vmax, fabsf(bf16_bits_to_float(vx[d])));
    }
    kmax = wave_max(kmax);
    vmax = wave_max(vmax);
    const float ks = int8_scale(kmax);
    const float vs = int8_scale(vmax);
    for (int d = lane; d < D; d += kWave) {
      kd[((d >> 4) * B + t) * 16 + (d & 15)] = (int8_t)int8_store(kx[d], ks);
      vd[((t >> 2) * D + d) * 4 + (t & 3)] = (int8_t)int8_store(vx[d], vs);
    }
    if (lane == 0) {
      const int64_t so = (blk * H + h) * (int64_t)B + t;
      kscale[so] = ks;
      vscale[so] = vs;
    }
  }
}

// One workgroup per (pair, layer, region).  A block of one layer is a single
// contiguous run of H tiles in the K and in the V region (H * B floats in each
// scale region), so the copy is a straight 16-byte-vector memcpy.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    const int64_t* __restrict__ pairs, int32_t num_pairs, int32_t num_layers, int32_t num_blocks,
    char* __restrict__ k, char* __restrict__ v, char* __restrict__ ks, char* __restrict__ vs,
    uint64_t block_bytes, uint64_t scale_block_bytes) {
  const int pi = blockIdx.x / num_layers;
  const int layer = blockIdx.x % num_layers;
  const int region = blockIdx.y;  // 0 K, 1 V, 2 K scales, 3 V scales
  if (pi >= num_pairs) return;
  const int64_t src = pairs[2 * pi], dst = pairs[2 * pi + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* base = region == 0 ? k : region == 1 ? v : region == 2 ? ks : vs;
  const uint64_t bytes = region < 2 ? block_bytes : scale_block_bytes;
  const uint64_t layer_off = (uint64_t)layer * num_blocks * bytes;
  const uint4* s = reinterpret_cast<const uint4*>(base + layer_off + (uint64_t)src * bytes);
  uint4* d = reinterpret_cast<uint4*>(base + layer_off + (uint64_t)dst * bytes);
  const uint64_t n16 = bytes / 16;
  for (uint64_t i = threadIdx.x; i < n16; i += blockDim.x) d[i] = s[i];
}

// One workgroup per (pair, layer, region), copying between two pools of the
// same shape; either may be pinned host memory that the device reads and
// writes directly over the host link.  Four 16-byte loads per thread are in
// flight before their stores, to cover that link's latency.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const int64_t* __restrict__ pairs, int32_t num_pairs, int32_t num_layers, int32_t src_blocks,
    int32_t dst_blocks, const char* __restrict__ sk, const char* __restrict__ sv, const char* __restrict__ sks,
    const char* __restrict__ svs, char* __restrict__ dk, char* __restrict__ dv, char* __restrict__ dks,
    char* __restrict__ dvs, uint64_t block_bytes, uint64_t scale_block_bytes) {
  const int pi = blockIdx.x / num_layers;
  const int layer = blockIdx.x % num_layers;
  const int region = blockIdx.y;  // 0 K, 1 V, 2 K scales, 3 V scales
  if (pi >= num_pairs) return;
  const int64_t src = pairs[2 * pi], dst = pairs[2 * pi + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const char* sbase = region == 0 ? sk : region == 1 ? sv : region == 2 ? sks : svs;
  char* dbase = region == 0 ? dk : region == 1 ? dv : region == 2 ? dks : dvs;
  const uint64_t bytes = region < 2 ? block_bytes : scale_block_bytes;
  const uint4* s = reinterpret_cast<const uint4*>(sbase + ((uint64_t)layer * src_blocks + (uint64_t)src) * bytes);
  uint4* d = reinterpret_cast<uint4*>(dbase + ((uint64_t)layer * dst_blocks + (uint64_t)dst) * bytes);
  const uint64_t n16 = bytes / 16;
  constexpr int U = 4;
  uint64_t i = threadIdx.x;
  for (; i + (U - 1) * blockDim.x < n16; i += U * blockDim.x) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = s[i + u * blockDim.x];
#pragma unroll
    for (int u = 0; u < U; ++u) d[i + u * blockDim.x] = x[u];
  }
  for (; i < n16; i += blockDim.x) d[i] = s[i];
}

// Device address of memory a pool description points into: device memory as
// it is, pinned host memory through its device mapping; anything else (for
// instance pageable host memory) is refused.
bool device_view(const void* p, const char* what, char** out) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // do not leave the error for the next launch check
    set_error("%s: not device or pinned host memory (%s)", what, hipGetErrorString(e));
    return false;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
    *out = static_cast<char*>(const_cast<void*>(p));
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer) {
    // pinned host memory: its device mapping must also be known to
    // hipHostGetDevicePointer, which refuses anything not allocated or
    // registered as pinned
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      set_error("%s: host memory is not pinned for the device", what);
      return false;
    }
    const char* host = static_cast<const char*>(a.hostPointer);
    char* mapped = static_cast<char*>(a.devicePointer) + (static_cast<const char*>(p) - host);
    if (mapped != static_cast<char*>(d)) {
      set_error("%s: inconsistent device mapping of pinned host memory", what);
      return false;
    }
    *out = mapped;
    return true;
  }
  set_error("%s: memory is not mapped for the device", what);
  return false;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status reshape_and_cache(const pkv_pool* pool, int32_t layer, const void* key,
                                        const void* value, const int64_t* slot_mapping,
                                        int32_t num_tokens, const pkv_kv_scales* scales,
                                        hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  const pkv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers) {
    set_error("layer %d outside [0, %d)", layer, c.num_layers);
    return PKV_ERR_INVALID;
  }
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens is negative");
  if (num_tokens == 0) { clear_error(); return PKV_OK; }
  if (!key || !value || !slot_mapping) return fail(PKV_ERR_INVALID, "key, value and slot_mapping must be non-NULL");
  float ksc = 1.f, vsc = 1.f;
  st = tensor_scales(c.kv_dtype, scales, &ksc, &vsc);
  if (st != PKV_OK) return st;
  const int64_t waves = (int64_t)num_tokens * c.num_kv_heads;
  const int64_t grid = (waves + 3) / 4;
  if (grid > INT32_MAX) return fail(PKV_ERR_INVALID, "too many tokens in one call");
  char* kl = static_cast<char*>(pool->k) + (uint64_t)layer * pool->layer_bytes;
  char* vl = static_cast<char*>(pool->v) + (uint64_t)layer * pool->layer_bytes;
  const uint64_t scale_layer = has_k_channel_scales(c.kv_dtype)
                                  ? (uint64_t)c.num_kv_heads * c.head_dim
                                  : (uint64_t)c.num_blocks * c.num_kv_heads * c.block_size;
  float* ksl = pool->k_scale ? pool->k_scale + layer * scale_layer : nullptr;
  float* vsl = pool->v_scale ? pool->v_scale + layer * scale_layer : nullptr;
  const int64_t num_slots = (int64_t)c.num_blocks * c.block_size;
  const auto* kx = static_cast<const uint16_t*>(key);
  const auto* vx = static_cast<const uint16_t*>(value);
  switch (c.kv_dtype) {
    case PKV_KV_BF16:
      hipLaunchKernelGGL(reshape_and_cache_kernel<PKV_KV_BF16>, dim3((uint32_t)grid), dim3(256), 0, stream,
                         kx, vx, slot_mapping, num_tokens, c.num_kv_heads, c.head_dim, c.block_size,
                         num_slots, kl, vl, ksl, vsl, ksc, vsc);
      break;
    case PKV_KV_FP8_E5M2:
      hipLaunchKernelGGL(reshape_and_cache_kernel<PKV_KV_FP8_E5M2>, dim3((uint32_t)grid), dim3(256), 0,
                         stream, kx, vx, slot_mapping, num_tokens, c.num_kv_heads, c.head_dim,
                         c.block_size, num_slots, kl, vl, ksl, vsl, ksc, vsc);
      break;
    case PKV_KV_INT8_TENSOR:
      hipLaunchKernelGGL(reshape_and_cache_kernel<PKV_KV_INT8_TENSOR>, dim3((uint32_t)grid), dim3(256), 0,
                         stream, kx, vx, slot_mapping, num_tokens, c.num_kv_heads, c.head_dim, c.block_size,
                         num_slots, kl, vl, ksl, vsl, ksc, vsc);
      break;
    case PKV_KV_INT8_CHANNEL:
    case PKV_KV_INT8_KCHANNEL_VTENSOR:   // no V channel scales: vsl is NULL, V takes vsc
      hipLaunchKernelGGL(reshape_and_cache_kernel<PKV_KV_INT8_CHANNEL>, dim3((uint32_t)grid), dim3(256), 0,
                         stream, kx, vx, slot_mapping, num_tokens, c.num_kv_heads, c.head_dim, c.block_size,
                         num_slots, kl, vl, ksl, vsl, ksc, vsc);
      break;
    case PKV_KV_INT4:
      hipLaunchKernelGGL(reshape_and_cache_kernel<PKV_KV_INT4>, dim3((uint32_t)grid), dim3(256), 0, stream,
                         kx, vx, slot_mapping, num_tokens, c.num_kv_heads, c.head_dim, c.block_size,
                         num_slots, kl, vl, ksl, vsl, ksc, vsc);
      break;
    default:
      hipLaunchKernelGGL(reshape_and_cache_kernel<PKV_KV_INT8>, dim3((uint32_t)grid), dim3(256), 0, stream,
                         kx, vx, slot_mapping, num_tokens, c.num_kv_heads, c.head_dim, c.block_size,
                         num_slots, kl, vl, ksl, vsl, ksc, vsc);
      break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("reshape_and_cache launch failed: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  clear_error();
  return PKV_OK;
}

extern "C" pkv_status copy_blocks(const pkv_pool* pool, const int64_t* pairs, int32_t num_pairs,
                                  hipStream_t stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return fail(PKV_ERR_INVALID, "num_pairs is negative");
  if (num_pairs == 0) { clear_error(); return PKV_OK; }
  if (!pairs) return fail(PKV_ERR_INVALID, "pairs is NULL");
  const pkv_pool_config& c = pool->cfg;
  const uint64_t block_bytes = (uint64_t)c.num_kv_heads * pool->tile_bytes;
  const uint64_t scale_block_bytes = (uint64_t)c.num_kv_heads * c.block_size * sizeof(float);
  if (block_bytes % 16 || scale_block_bytes % 16) return fail(PKV_ERR_UNSUPPORTED, "block bytes not a multiple of 16");
  const int64_t gx = (int64_t)num_pairs * c.num_layers;
  if (gx > INT32_MAX) return fail(PKV_ERR_INVALID, "too many pairs in one call");
  const int regions = c.kv_dtype == PKV_KV_INT8 ? 4 : 2;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)gx, regions), dim3(256), 0, stream, pairs,
                     num_pairs, c.num_layers, c.num_blocks, static_cast<char*>(pool->k),
                     static_cast<char*>(pool->v), reinterpret_cast<char*>(pool->k_scale),
                     reinterpret_cast<char*>(pool->v_scale), block_bytes, scale_block_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("copy_blocks launch failed: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  clear_error();
  return PKV_OK;
}

extern "C" pkv_status swap_blocks(const pkv_pool* from, const pkv_pool* to, const int64_t* pairs,
                                  int32_t num_pairs, hipStream_t stream) {
  pkv_status st = check_pool(from);
  if (st != PKV_OK) return st;
  st = check_pool(to);
  if (st != PKV_OK) return st;
  const pkv_pool_config& a = from->cfg;
  const pkv_pool_config& b = to->cfg;
  if (a.num_layers != b.num_layers || a.block_size != b.block_size || a.num_kv_heads != b.num_kv_heads ||
      a.head_dim != b.head_dim || a.kv_dtype != b.kv_dtype)
    return fail(PKV_ERR_INVALID, "the two pools differ in more than num_blocks");
  if (num_pairs < 0) return fail(PKV_ERR_INVALID, "num_pairs is negative");
  if (num_pairs == 0) { clear_error(); return PKV_OK; }
  if (!pairs) return fail(PKV_ERR_INVALID, "pairs is NULL");
  char* ptr[8];
  const void* src[8] = {from->k, from->v, from->k_scale, from->v_scale, to->k, to->v, to->k_scale, to->v_scale};
  const char* names[8] = {"from K", "from V", "from K scales", "from V scales",
                          "to K", "to V", "to K scales", "to V scales"};
  const int regions = a.kv_dtype == PKV_KV_INT8 ? 4 : 2;
  for (int i = 0; i < 8; ++i) {
    ptr[i] = nullptr;
    if (i % 4 >= regions) continue;
    if (!device_view(src[i], names[i], &ptr[i])) return PKV_ERR_INVALID;
  }
  const uint64_t block_bytes = (uint64_t)a.num_kv_heads * from->tile_bytes;
  const uint64_t scale_block_bytes = (uint64_t)a.num_kv_heads * a.block_size * sizeof(float);
  if (block_bytes % 16 || scale_block_bytes % 16) return fail(PKV_ERR_UNSUPPORTED, "block bytes not a multiple of 16");
  const int64_t gx = (int64_t)num_pairs * a.num_layers;
  if (gx > INT32_MAX) return fail(PKV_ERR_INVALID, "too many pairs in one call");
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((uint32_t)gx, regions), dim3(256), 0, stream, pairs, num_pairs,
                     a.num_layers, a.num_blocks, b.num_blocks, ptr[0], ptr[1], ptr[2], ptr[3], ptr[4], ptr[5],
                     ptr[6], ptr[7], block_bytes, scale_block_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("swap_blocks launch failed: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  clear_error();
  return PKV_OK;
}
