// Host block manager: the bookkeeping side of paging.
//
// Physical blocks of a preallocated pool are handed to sequences on demand and
// reused when sequences end ("KV Cache 原理与 PagedAttention", §三 工作方式
// steps 1-3; aiworkagent.org Q17, KV Memory Pool).  Each sequence has a block
// table mapping logical block i to a physical block.  Forked sequences share
// their parent's blocks; the first write into a shared block copies it and
// repoints the writer's table (bjdmk.com.cn article, §3.1 and §3.2
// Copy-on-Write).  Prompt blocks can be found again by content: a full block's
// key hashes its tokens and the key of the block before it, and a request
// whose prompt starts with a cached run of blocks reuses them (same article,
// §4.1 prefix caching; §4.3: only an exact, position-aligned prefix is
// reused).  Alternatively the cached prompt blocks form a radix tree over
// their token ids (same article, §4.2): a request takes the longest matching
// prefix, also one ending inside a block (that block is copied), and the
// least recently used leaves are evicted first.  The tie-break rules that
// make tables, slots and copy pairs unique are stated with the declarations
// in pkv.h.
#include <algorithm>
#include <deque>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv_internal.h"
#include "sha256.h"

namespace {
struct DigestHash {
  size_t operator()(const pkv::Digest& d) const {
    size_t h;
    std::memcpy(&h, d.data(), sizeof h);
    return h;
  }
};
}  // namespace

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // FIFO of free blocks: pop front, push back.  An entry is live while its
  // generation is the block's current one and the block is unreferenced; a
  // cached free block that a prefix hit takes back leaves a dead entry
  // behind, skipped when it reaches the front.
  std::deque<std::pair<int32_t, uint32_t>> free_list;
  std::vector<uint32_t> gen;
  int64_t num_free = 0;
  std::vector<int32_t> ref;                 // per physical block
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
  };
  std::unordered_map<int32_t, Seq> seqs;
  int64_t failed_allocs = 0;
  // prefix cache: key -> block; a block's own key while it holds one
  std::unordered_map<pkv::Digest, int32_t, DigestHash> cache;
  std::vector<pkv::Digest> block_key;
  std::vector<uint8_t> keyed;
  int64_t lookups = 0, hits = 0;

  // which prefix cache is in use: none yet, the hash chain, or the radix tree
  enum Mode { kNone, kHash, kRadix } mode = kNone;
  // radix tree: a node is a cached full prompt block.  parent: the node of
  // the block before it (kRoot for block 0), kNoNode for blocks outside the
  // tree; children in insertion order; the B token ids of node b at
  // tokens[b * B ..).  In radix mode num_free also counts the cached blocks
  // nobody references (idle), which eviction hands out leaves first, least
  // recently used first.
  static constexpr int32_t kRoot = -1, kNoNode = -2;
  std::vector<int32_t> parent;
  std::vector<std::vector<int32_t>> children;
  std::vector<int32_t> root_children;
  std::vector<int32_t> tokens;
  std::vector<int64_t> last_use;
  std::vector<int32_t> depth;
  std::set<std::tuple<int64_t, int32_t, int32_t>> evictable;   // (last use, -depth, block) of idle leaves
  int64_t idle = 0;
  int64_t clock = 0;
  int64_t radix_lookups = 0, radix_hits = 0;

  bool in_tree(int32_t b) const { return !parent.empty() && parent[(size_t)b] != kNoNode; }
  std::vector<int32_t>& kids(int32_t b) { return b == kRoot ? root_children : children[(size_t)b]; }
  std::tuple<int64_t, int32_t, int32_t> ev_key(int32_t b) const {
    return {last_use[(size_t)b], -depth[(size_t)b], b};
  }
  void radix_arrays() {
    if (parent.empty()) {
      parent.assign((size_t)num_blocks, kNoNode);
      children.resize((size_t)num_blocks);
      tokens.resize((size_t)num_blocks * (size_t)block_size);
      last_use.assign((size_t)num_blocks, 0);
      depth.assign((size_t)num_blocks, 0);
    }
  }
  // a tree node that nobody references becomes idle (and evictable once it
  // is a leaf)
  void make_idle(int32_t b) {
    last_use[(size_t)b] = clock;
    ++idle;
    ++num_free;
    if (children[(size_t)b].empty()) evictable.insert(ev_key(b));
  }
  // an idle node gains a reference
  void wake(int32_t b) {
    if (children[(size_t)b].empty()) evictable.erase(ev_key(b));
    --idle;
    --num_free;
  }
  // remove the least recently used idle leaf from the tree; its parent may
  // become an idle leaf in turn
  int32_t evict() {
    const int32_t b = std::get<2>(*evictable.begin());
    evictable.erase(evictable.begin());
    const int32_t pa = parent[(size_t)b];
    std::vector<int32_t>& sib = kids(pa);
    sib.erase(std::find(sib.begin(), sib.end(), b));
    if (pa != kRoot && sib.empty() && ref[(size_t)pa] == 0) evictable.insert(ev_key(pa));
    parent[(size_t)b] = kNoNode;
    --idle;
    --num_free;
    return b;
  }

  void push_free(int32_t b) {
    free_list.emplace_back(b, ++gen[(size_t)b]);
    ++num_free;
  }
  void release(int32_t b) {
    if (--ref[(size_t)b] == 0) {
      if (in_tree(b)) make_idle(b);
      else push_free(b);
    }
  }
  void unkey(int32_t b) {
    if (keyed[(size_t)b]) {
      cache.erase(block_key[(size_t)b]);
      keyed[(size_t)b] = 0;
    }
  }
  // The front live free block (radix mode: an evicted idle leaf once the
  // free list holds none), now referenced once; it leaves the cache (its
  // content is about to be overwritten).
  int32_t take() {
    if (mode == kRadix && num_free == idle) {
      const int32_t b = evict();
      ref[(size_t)b] = 1;
      return b;
    }
    while (true) {
      const auto e = free_list.front();
      free_list.pop_front();
      if (e.second != gen[(size_t)e.first] || ref[(size_t)e.first] != 0) continue;   // dead entry
      ref[(size_t)e.first] = 1;
      --num_free;
      unkey(e.first);
      return e.first;
    }
  }
};

using namespace pkv;

extern "C" {

pkv_status kv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order,
                        pkv_bm** out) {
  if (!out) return fail(PKV_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return fail(PKV_ERR_INVALID, "num_blocks and block_size must be positive");
  pkv_bm* bm = new (std::nothrow) pkv_bm;
  if (!bm) return fail(PKV_ERR_INVALID, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign((size_t)num_blocks, 0);
  bm->gen.assign((size_t)num_blocks, 0);
  bm->block_key.resize((size_t)num_blocks);
  bm->keyed.assign((size_t)num_blocks, 0);
  if (initial_order) {
    std::vector<uint8_t> seen((size_t)num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_order[i];
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        delete bm;
        set_error("initial_order is not a permutation of 0..%d (entry %d = %d)", num_blocks - 1, i, b);
        return PKV_ERR_INVALID;
      }
      seen[(size_t)b] = 1;
      bm->push_free(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->push_free(b);
  }
  *out = bm;
  clear_error();
  return PKV_OK;
}

void kv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status kv_bm_add_seq(pkv_bm* bm, int32_t seq, int32_t ctx_len) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (ctx_len < 0) return fail(PKV_ERR_INVALID, "ctx_len is negative");
  if (bm->seqs.count(seq)) {
    set_error("sequence %d already exists", seq);
    return PKV_ERR_INVALID;
  }
  const int64_t need = ((int64_t)ctx_len + bm->block_size - 1) / bm->block_size;
  if (need > bm->num_free) {
    bm->failed_allocs++;
    set_error("sequence %d needs %lld blocks, %lld free", seq, (long long)need, (long long)bm->num_free);
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  pkv_bm::Seq s;
  s.table.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->take());
  s.len = ctx_len;
  bm->seqs.emplace(seq, std::move(s));
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_fork(pkv_bm* bm, int32_t parent, int32_t child) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) {
    set_error("parent %d does not exist", parent);
    return PKV_ERR_INVALID;
  }
  if (bm->seqs.count(child)) {
    set_error("child %d already exists", child);
    return PKV_ERR_INVALID;
  }
  pkv_bm::Seq c = it->second;
  for (int32_t b : c.table) bm->ref[(size_t)b]++;
  bm->seqs.emplace(child, std::move(c));
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_append(pkv_bm* bm, const int32_t* seqs, int32_t n, int64_t* slots, int64_t* cow_pairs,
                        int32_t* num_pairs) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_pairs)
    return fail(PKV_ERR_INVALID, "bad append arguments");
  *num_pairs = 0;
  const int32_t B = bm->block_size;
  std::vector<pkv_bm::Seq*> ptr((size_t)n);
  {
    std::unordered_map<int32_t, int32_t> dup;
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seqs[i]);
      if (it == bm->seqs.end()) {
        set_error("sequence %d does not exist", seqs[i]);
        return PKV_ERR_INVALID;
      }
      if (dup.count(seqs[i])) {
        set_error("sequence %d appears twice in one append", seqs[i]);
        return PKV_ERR_INVALID;
      }
      dup[seqs[i]] = i;
      ptr[(size_t)i] = &it->second;
    }
  }
  // dry run: fresh blocks the whole batch needs
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> ref_delta;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq& s = *ptr[(size_t)i];
    if (s.len % B == 0) {
      ++need;
    } else {
      const int32_t last = s.table[(size_t)(s.len / B)];
      auto d = ref_delta.find(last);
      const int32_t delta = d == ref_delta.end() ? 0 : d->second;
      if (bm->ref[(size_t)last] + delta > 1) {
        ++need;
        ref_delta[last] = delta - 1;
      }
    }
  }
  if (need > bm->num_free) {
    bm->failed_allocs++;
    set_error("append needs %lld blocks, %lld free", (long long)need, (long long)bm->num_free);
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    pkv_bm::Seq& s = *ptr[(size_t)i];
    const int32_t pos = s.len;
    const size_t lb = (size_t)(pos / B);
    if (pos % B == 0) {
      s.table.push_back(bm->take());
    } else {
      const int32_t last = s.table[lb];
      if (bm->ref[(size_t)last] > 1) {
        const int32_t dst = bm->take();
        bm->ref[(size_t)last]--;
        s.table[lb] = dst;
        cow_pairs[2 * np] = last;
        cow_pairs[2 * np + 1] = dst;
        ++np;
      }
    }
    slots[i] = (int64_t)s.table[lb] * B + pos % B;
    s.len = pos + 1;
  }
  *num_pairs = np;
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_free_seq(pkv_bm* bm, int32_t seq) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) {
    set_error("sequence %d does not exist", seq);
    return PKV_ERR_INVALID;
  }
  ++bm->clock;
  for (int32_t b : it->second.table) bm->release(b);
  bm->seqs.erase(it);
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_block_tables(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t* tables,
                              int32_t width, int32_t* context_lens) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (n < 0 || width <= 0 || (n > 0 && (!seqs || !tables))) return fail(PKV_ERR_INVALID, "bad table arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) {
      set_error("sequence %d does not exist", seqs[i]);
      return PKV_ERR_INVALID;
    }
    if ((int64_t)it->second.table.size() > width) {
      set_error("sequence %d holds %zu blocks, wider than %d", seqs[i], it->second.table.size(), width);
      return PKV_ERR_INVALID;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + (int64_t)i * width;
    size_t j = 0;
    for (; j < s.table.size(); ++j) row[j] = s.table[j];
    for (; j < (size_t)width; ++j) row[j] = 0;
    if (context_lens) context_lens[i] = s.len;
  }
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_stats(const pkv_bm* bm, int32_t* used, int32_t* total, int64_t* failed_allocs) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (used) *used = bm->num_blocks - (int32_t)bm->num_free;
  if (total) *total = bm->num_blocks;
  if (failed_allocs) *failed_allocs = bm->failed_allocs;
  return PKV_OK;
}

int32_t kv_bm_ref_count(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[(size_t)block];
}

pkv_status kv_bm_block_key(const uint8_t* parent, const int32_t* tokens, int32_t n, uint8_t* out) {
  if (!out || n < 0 || (n > 0 && !tokens)) return fail(PKV_ERR_INVALID, "bad key arguments");
  pkv::Sha256 h;
  uint8_t zero[32] = {0};
  h.update(parent ? parent : zero, 32);
  // token ids as little-endian 32-bit words, in one buffer
  std::vector<uint8_t> buf((size_t)n * 4);
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t t = (uint32_t)tokens[i];
    buf[(size_t)4 * i] = (uint8_t)t;
    buf[(size_t)4 * i + 1] = (uint8_t)(t >> 8);
    buf[(size_t)4 * i + 2] = (uint8_t)(t >> 16);
    buf[(size_t)4 * i + 3] = (uint8_t)(t >> 24);
  }
  h.update(buf.data(), buf.size());
  const pkv::Digest d = h.finish();
  std::memcpy(out, d.data(), 32);
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_add_seq_tokens(pkv_bm* bm, int32_t seq, const int32_t* tokens, int32_t n,
                                int32_t* cached_tokens) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (n < 0 || (n > 0 && !tokens)) return fail(PKV_ERR_INVALID, "bad token arguments");
  if (bm->seqs.count(seq)) {
    set_error("sequence %d already exists", seq);
    return PKV_ERR_INVALID;
  }
  if (bm->mode == pkv_bm::kRadix)
    return fail(PKV_ERR_UNSUPPORTED, "this block manager's prefix cache is the radix tree (kv_bm_add_seq_radix)");
  const int32_t B = bm->block_size;
  const int64_t full = n / B;
  const int64_t total = ((int64_t)n + B - 1) / B;
  // blocks that may be reused: those wholly before the prompt's last token,
  // which is always left to compute (its forward pass yields the first
  // generated token, and its K/V would otherwise be rewritten into a block
  // other sequences share)
  const int64_t eligible = n > 0 ? ((int64_t)n - 1) / B : 0;
  std::vector<pkv::Digest> keys((size_t)full);
  for (int64_t i = 0; i < full; ++i)
    kv_bm_block_key(i ? keys[(size_t)(i - 1)].data() : nullptr, tokens + i * B, B, keys[(size_t)i].data());
  // the longest run of leading eligible blocks already cached
  int64_t matched = 0, matched_free = 0;
  while (matched < eligible) {
    auto it = bm->cache.find(keys[(size_t)matched]);
    if (it == bm->cache.end()) break;
    if (bm->ref[(size_t)it->second] == 0) ++matched_free;
    ++matched;
  }
  if (total - matched > bm->num_free - matched_free) {
    bm->failed_allocs++;
    set_error("sequence %d needs %lld fresh blocks, %lld free", seq, (long long)(total - matched),
              (long long)(bm->num_free - matched_free));
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  bm->mode = pkv_bm::kHash;
  bm->lookups += eligible;
  bm->hits += matched;
  pkv_bm::Seq s;
  s.table.reserve((size_t)total);
  for (int64_t i = 0; i < matched; ++i) {
    const int32_t b = bm->cache.find(keys[(size_t)i])->second;
    if (bm->ref[(size_t)b] == 0) --bm->num_free;   // its free-list entry dies
    bm->ref[(size_t)b]++;
    s.table.push_back(b);
  }
  for (int64_t i = matched; i < total; ++i) {
    const int32_t b = bm->take();
    s.table.push_back(b);
    if (i < full) {   // a full prompt block: findable by its key from now on
      auto it = bm->cache.find(keys[(size_t)i]);
      if (it != bm->cache.end()) bm->keyed[(size_t)it->second] = 0;   // an older holder of the key loses it
      bm->cache[keys[(size_t)i]] = b;
      bm->block_key[(size_t)b] = keys[(size_t)i];
      bm->keyed[(size_t)b] = 1;
    }
  }
  s.len = n;
  bm->seqs.emplace(seq, std::move(s));
  if (cached_tokens) *cached_tokens = (int32_t)(matched * B);
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_prefix_stats(const pkv_bm* bm, int64_t* lookups, int64_t* hits, int32_t* cached_blocks) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (lookups) *lookups = bm->lookups;
  if (hits) *hits = bm->hits;
  if (cached_blocks) *cached_blocks = (int32_t)bm->cache.size();
  return PKV_OK;
}

pkv_status kv_bm_add_seq_radix(pkv_bm* bm, int32_t seq, const int32_t* tokens, int32_t n,
                               int32_t* cached_tokens, int64_t* copy_pair) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  if (n < 0 || (n > 0 && !tokens) || !copy_pair) return fail(PKV_ERR_INVALID, "bad token arguments");
  if (bm->seqs.count(seq)) {
    set_error("sequence %d already exists", seq);
    return PKV_ERR_INVALID;
  }
  if (bm->mode == pkv_bm::kHash)
    return fail(PKV_ERR_UNSUPPORTED, "this block manager's prefix cache is the hash chain (kv_bm_add_seq_tokens)");
  bm->radix_arrays();
  const int32_t B = bm->block_size;
  const int64_t full = n / B;
  const int64_t total = ((int64_t)n + B - 1) / B;
  const int64_t last = n > 0 ? n - 1 : 0;   // tokens that may be reused (the last one is always computed)
  auto same = [&](int32_t b, int64_t blk) {
    return std::equal(tokens + blk * B, tokens + (blk + 1) * B, bm->tokens.begin() + (int64_t)b * B);
  };
  // whole blocks along the tree
  int32_t node = pkv_bm::kRoot;
  std::vector<int32_t> path;
  while ((int64_t)(path.size() + 1) * B <= last) {
    const int64_t blk = (int64_t)path.size();
    int32_t nxt = -1;
    for (int32_t c : bm->kids(node))
      if (same(c, blk)) {
        nxt = c;
        break;
      }
    if (nxt < 0) break;
    path.push_back(nxt);
    node = nxt;
  }
  const int64_t i = (int64_t)path.size();
  // the child sharing the most leading tokens of the next block
  const int64_t lim = std::min<int64_t>(B, last - i * B);
  int32_t src = -1;
  int64_t l = 0;
  if (lim > 0) {
    for (int32_t c : bm->kids(node)) {
      const int32_t* t = bm->tokens.data() + (int64_t)c * B;
      int64_t k = 0;
      while (k < lim && t[k] == tokens[i * B + k]) ++k;
      if (k > l) {
        src = c;
        l = k;
      }
    }
  }
  int64_t pinned = src >= 0 && bm->ref[(size_t)src] == 0 ? 1 : 0;
  for (int32_t b : path) pinned += bm->ref[(size_t)b] == 0 ? 1 : 0;
  if (total - i > bm->num_free - pinned) {
    bm->failed_allocs++;
    set_error("sequence %d needs %lld fresh blocks, %lld obtainable", seq, (long long)(total - i),
              (long long)(bm->num_free - pinned));
    return PKV_ERR_OUT_OF_BLOCKS;
  }
  bm->mode = pkv_bm::kRadix;
  ++bm->clock;
  std::vector<int32_t> used = path;
  if (src >= 0) used.push_back(src);
  for (int32_t b : used) {
    if (bm->ref[(size_t)b] == 0) bm->wake(b);
    bm->ref[(size_t)b]++;
    bm->last_use[(size_t)b] = bm->clock;
  }
  pkv_bm::Seq s;
  s.table = path;
  s.table.reserve((size_t)total);
  int32_t par = node;
  bool insert = true;
  for (int64_t k = i; k < total; ++k) {
    const int32_t b = bm->take();
    s.table.push_back(b);
    if (!insert || k >= full) continue;
    bool dup = false;
    for (int32_t c : bm->kids(par)) dup = dup || same(c, k);
    if (dup) {   // a sibling holds these tokens: the chain stops here
      insert = false;
      continue;
    }
    bm->parent[(size_t)b] = par;
    bm->kids(par).push_back(b);
    std::copy(tokens + k * B, tokens + (k + 1) * B, bm->tokens.begin() + (int64_t)b * B);
    bm->depth[(size_t)b] = (int32_t)k;
    bm->last_use[(size_t)b] = bm->clock;
    par = b;
  }
  if (src >= 0 && --bm->ref[(size_t)src] == 0) bm->make_idle(src);   // held only while blocks were taken
  copy_pair[0] = src >= 0 ? src : -1;
  copy_pair[1] = src >= 0 ? s.table[(size_t)i] : -1;
  s.len = n;
  bm->seqs.emplace(seq, std::move(s));
  bm->radix_lookups += last;
  bm->radix_hits += i * B + l;
  if (cached_tokens) *cached_tokens = (int32_t)(i * B + l);
  clear_error();
  return PKV_OK;
}

pkv_status kv_bm_radix_stats(const pkv_bm* bm, int64_t* lookup_tokens, int64_t* hit_tokens, int32_t* cached_blocks,
                             int32_t* idle_blocks) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm is NULL");
  int32_t nodes = 0;
  for (size_t b = 0; b < bm->parent.size(); ++b) nodes += bm->parent[b] != pkv_bm::kNoNode ? 1 : 0;
  if (lookup_tokens) *lookup_tokens = bm->radix_lookups;
  if (hit_tokens) *hit_tokens = bm->radix_hits;
  if (cached_blocks) *cached_blocks = nodes;
  if (idle_blocks) *idle_blocks = (int32_t)bm->idle;
  return PKV_OK;
}

}  // extern "C"
