// Pool sizing and description, error reporting and host-side validators.
//
// The pool holds K and V for num_blocks fixed-size blocks per layer, the
// preallocated memory pool of "KV Cache 原理与 PagedAttention" §三 and of the
// aiworkagent.org Q17 notes (PagedAttention 的关键数据结构); its K/V payload is
// the per-layer KV-size formula of the first page's §一 (2 x heads x tokens x
// head_dim x bytes) applied to num_blocks * block_size token slots.
#include <cstring>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
}

void clear_error() { g_error.clear(); }

bool pool_regions(const pkv_pool_config* cfg, Regions* r) {
  if (!cfg) { set_error("pool config is NULL"); return false; }
  const int bits = elem_bits(cfg->kv_dtype);
  if (bits == 0) { set_error("kv_dtype %d is not a pkv_kv_dtype", cfg->kv_dtype); return false; }
  if (cfg->num_layers <= 0 || cfg->num_blocks <= 0 || cfg->block_size <= 0 ||
      cfg->num_kv_heads <= 0 || cfg->head_dim <= 0) {
    set_error("pool dimensions must be positive (layers %d blocks %d block_size %d heads %d dim %d)",
              cfg->num_layers, cfg->num_blocks, cfg->block_size, cfg->num_kv_heads, cfg->head_dim);
    return false;
  }
  if (cfg->block_size % 4 != 0) { set_error("block_size %d is not a multiple of 4", cfg->block_size); return false; }
  const int dmul = bits == 4 ? 32 : 128 / bits;     // dims per 16-byte piece (INT4: per 32-bit word group)
  if (cfg->head_dim % dmul != 0) {
    set_error("head_dim %d is not a multiple of %d", cfg->head_dim, dmul);
    return false;
  }
  const uint64_t tile = tile_bytes_of(*cfg);
  const uint64_t kv = (uint64_t)cfg->num_layers * cfg->num_blocks * cfg->num_kv_heads * tile;
  r->kv_bytes = kv;
  r->k = 0;
  r->v = align_up(kv);
  r->total = align_up(r->v + kv);
  r->ks = r->vs = 0;
  r->scale_bytes = 0;
  if (cfg->kv_dtype == PKV_KV_INT8 || has_k_channel_scales(cfg->kv_dtype)) {
    const uint64_t sb = cfg->kv_dtype == PKV_KV_INT8
                            ? (uint64_t)cfg->num_layers * cfg->num_blocks * cfg->num_kv_heads * cfg->block_size *
                                  sizeof(float)
                            : (uint64_t)cfg->num_layers * cfg->num_kv_heads * cfg->head_dim * sizeof(float);
    r->scale_bytes = sb;
    r->ks = r->total;
    r->total = align_up(r->ks + sb);
    if (cfg->kv_dtype == PKV_KV_INT8 || has_channel_scales(cfg->kv_dtype)) {   // V scales too
      r->vs = r->total;
      r->total = align_up(r->vs + sb);
    }
  }
  return true;
}

pkv_status check_pool(const pkv_pool* pool) {
  if (!pool) return fail(PKV_ERR_INVALID, "pool is NULL");
  Regions r;
  if (!pool_regions(&pool->cfg, &r)) return PKV_ERR_INVALID;
  if (!pool->k || !pool->v) return fail(PKV_ERR_INVALID, "pool has no K/V pointers (use kv_pool_create)");
  const int32_t t = pool->cfg.kv_dtype;
  if (((t == PKV_KV_INT8 || has_k_channel_scales(t)) && !pool->k_scale) ||
      ((t == PKV_KV_INT8 || has_channel_scales(t)) && !pool->v_scale))
    return fail(PKV_ERR_INVALID, "pool has no scale pointers");
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

uint64_t kv_pool_bytes(const pkv_pool_config* cfg) {
  Regions r;
  if (!pool_regions(cfg, &r)) return 0;
  return r.total;
}

int64_t kv_pool_num_blocks_for_budget(const pkv_pool_config* cfg, uint64_t budget_bytes) {
  if (!cfg) { set_error("pool config is NULL"); return -1; }
  pkv_pool_config c = *cfg;
  c.num_blocks = 1;
  Regions r;
  if (!pool_regions(&c, &r)) return -1;
  // bytes grow linearly in num_blocks apart from alignment padding: start
  // from the payload estimate and step down until the padded size fits
  uint64_t per_block = 2ull * c.num_layers * c.num_kv_heads * tile_bytes_of(c);
  if (c.kv_dtype == PKV_KV_INT8) per_block += 2ull * c.num_layers * c.num_kv_heads * c.block_size * 4;
  // (per-channel scales do not grow with the block count: the exact check below covers them)
  int64_t nb = (int64_t)(budget_bytes / per_block);
  if (nb > INT32_MAX) nb = INT32_MAX;
  while (nb > 0) {
    c.num_blocks = (int32_t)nb;
    if (pool_regions(&c, &r) && r.total <= budget_bytes) break;
    --nb;
  }
  clear_error();
  return nb;
}

pkv_status kv_pool_create(const pkv_pool_config* cfg, void* dev_mem, uint64_t bytes, pkv_pool* out) {
  if (!out) return fail(PKV_ERR_INVALID, "out is NULL");
  Regions r;
  if (!pool_regions(cfg, &r)) return PKV_ERR_INVALID;
  if (!dev_mem) return fail(PKV_ERR_INVALID, "dev_mem is NULL");
  if (((uintptr_t)dev_mem) % kRegionAlign != 0) return fail(PKV_ERR_INVALID, "dev_mem is not 256-byte aligned");
  if (bytes < r.total) {
    set_error("pool needs %llu bytes, got %llu", (unsigned long long)r.total, (unsigned long long)bytes);
    return PKV_ERR_INVALID;
  }
  std::memset(out, 0, sizeof *out);
  out->cfg = *cfg;
  out->base = dev_mem;
  out->bytes = bytes;
  char* b = static_cast<char*>(dev_mem);
  out->k = b + r.k;
  out->v = b + r.v;
  if (r.scale_bytes) out->k_scale = reinterpret_cast<float*>(b + r.ks);
  if (r.vs) out->v_scale = reinterpret_cast<float*>(b + r.vs);
  out->tile_bytes = tile_bytes_of(*cfg);
  out->layer_bytes = (uint64_t)cfg->num_blocks * cfg->num_kv_heads * out->tile_bytes;
  clear_error();
  return PKV_OK;
}

pkv_status pkv_check_slots(const int64_t* slots, int32_t n, int64_t num_slots) {
  if (n < 0 || (n > 0 && !slots)) return fail(PKV_ERR_INVALID, "bad slot array");
  std::vector<uint8_t> seen((size_t)(num_slots > 0 ? num_slots : 0), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = slots[i];
    if (s < 0) continue;
    if (s >= num_slots) {
      set_error("slot[%d] = %lld is outside the pool (%lld slots)", i, (long long)s, (long long)num_slots);
      return PKV_ERR_INVALID;
    }
    if (seen[(size_t)s]) {
      set_error("slot[%d] = %lld repeats an earlier slot", i, (long long)s);
      return PKV_ERR_INVALID;
    }
    seen[(size_t)s] = 1;
  }
  clear_error();
  return PKV_OK;
}

pkv_status pkv_check_pairs(const int64_t* pairs, int32_t n, int32_t num_blocks) {
  if (n < 0 || (n > 0 && !pairs) || num_blocks <= 0) return fail(PKV_ERR_INVALID, "bad pair array");
  std::vector<uint8_t> role((size_t)num_blocks, 0);  // bit0 src, bit1 dst
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) {
      set_error("pair %d (%lld, %lld) is outside [0, %d)", i, (long long)s, (long long)d, num_blocks);
      return PKV_ERR_INVALID;
    }
    role[(size_t)s] |= 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t d = pairs[2 * i + 1];
    if (role[(size_t)d] & 1) {
      set_error("pair %d: destination %lld is also a source", i, (long long)d);
      return PKV_ERR_INVALID;
    }
    if (role[(size_t)d] & 2) {
      set_error("pair %d: destination %lld repeats", i, (long long)d);
      return PKV_ERR_INVALID;
    }
    role[(size_t)d] |= 2;
  }
  clear_error();
  return PKV_OK;
}

pkv_status pkv_check_tables(const int32_t* tables, const int32_t* context_lens, int32_t num_seqs,
                            int32_t table_width, int32_t block_size, int32_t num_blocks) {
  if (num_seqs < 0 || table_width <= 0 || block_size <= 0 || num_blocks <= 0 ||
      (num_seqs > 0 && (!tables || !context_lens)))
    return fail(PKV_ERR_INVALID, "bad table arguments");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t c = context_lens[s];
    if (c < 0 || c > (int64_t)table_width * block_size) {
      set_error("context_lens[%d] = %lld does not fit %d blocks of %d", s, (long long)c, table_width,
                block_size);
      return PKV_ERR_INVALID;
    }
    const int64_t nb = (c + block_size - 1) / block_size;
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t b = tables[(int64_t)s * table_width + i];
      if (b < 0 || b >= num_blocks) {
        set_error("block_tables[%d][%lld] = %d is outside [0, %d)", s, (long long)i, b, num_blocks);
        return PKV_ERR_INVALID;
      }
    }
  }
  clear_error();
  return PKV_OK;
}

}  // extern "C"
