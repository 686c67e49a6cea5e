// Drives the host side of the C ABI - pool sizing and description, the host
// validators, the block manager with forks, copy-on-write appends and prefix
// caching - through fixed cases and a long seeded random walk, checking after
// every operation what pkv.h promises: reference counts equal the number of
// tables naming a block, tables hold ceil(len / B) blocks, an append's slot
// is table[pos / B] * B + pos % B, a copy-on-write pair copies a block that
// was shared into one that was free, a refused call changes nothing; and the
// radix-tree prefix cache with a simulated pool memory (below).
// tests/test_host_sanitize.py builds it with AddressSanitizer and
// UndefinedBehaviorSanitizer together with pool.cpp and block_manager.cpp.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <map>
#include <set>
#include <vector>

#include "pkv.h"

#define CHECK(c)                                                                                     \
  do {                                                                                               \
    if (!(c)) {                                                                                      \
      std::fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, #c,        \
                   pkv_last_error());                                                                \
      std::exit(1);                                                                                  \
    }                                                                                                \
  } while (0)

namespace {

struct Lcg {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
  }
  int below(int n) { return (int)(next() % (uint32_t)n); }
};

void pool_sizing() {
  for (int dt = 0; dt <= 6; ++dt)
    for (int D : {64, 128})
      for (int B : {8, 16, 32}) {
        pkv_pool_config c{3, 37, B, 2, D, dt};
        const uint64_t bytes = kv_pool_bytes(&c);
        CHECK(bytes > 0 && bytes % 256 == 0);
        const int64_t nb = kv_pool_num_blocks_for_budget(&c, bytes);
        CHECK(nb >= 37);
        pkv_pool_config c2 = c;
        c2.num_blocks = (int32_t)nb + 1;
        CHECK(kv_pool_bytes(&c2) > bytes);
        CHECK(kv_pool_num_blocks_for_budget(&c, 0) == 0);
        // a host buffer stands in for device memory: kv_pool_create only records pointers
        void* mem = std::aligned_alloc(256, (size_t)bytes);
        CHECK(mem);
        pkv_pool p;
        CHECK(kv_pool_create(&c, mem, bytes, &p) == PKV_OK);
        char* b = static_cast<char*>(mem);
        const uint64_t payload = (uint64_t)c.num_layers * p.layer_bytes;
        CHECK((char*)p.k >= b && (char*)p.k + payload <= (char*)p.v);
        CHECK((char*)p.v + payload <= b + bytes);
        const bool vscales = dt == PKV_KV_INT8 || dt == PKV_KV_INT8_CHANNEL || dt == PKV_KV_INT4;
        const bool kscales = vscales || dt == PKV_KV_INT8_KCHANNEL_VTENSOR;
        CHECK((p.k_scale != nullptr) == kscales && (p.v_scale != nullptr) == vscales);
        if (kscales) CHECK((char*)p.k_scale >= (char*)p.v + payload && (char*)p.k_scale < b + bytes);
        if (vscales) CHECK((char*)p.v_scale > (char*)p.k_scale && (char*)p.v_scale < b + bytes);
        CHECK(kv_pool_create(&c, mem, bytes - 1, &p) == PKV_ERR_INVALID);
        CHECK(kv_pool_create(&c, b + 16, bytes, &p) == PKV_ERR_INVALID);
        CHECK(kv_pool_create(&c, nullptr, bytes, &p) == PKV_ERR_INVALID);
        CHECK(kv_pool_create(&c, mem, bytes, nullptr) == PKV_ERR_INVALID);
        std::free(mem);
      }
  pkv_pool_config bad{1, 4, 16, 1, 128, 9};
  CHECK(kv_pool_bytes(&bad) == 0 && std::strlen(pkv_last_error()) > 0);
  bad.kv_dtype = 0;
  bad.block_size = 6;
  CHECK(kv_pool_bytes(&bad) == 0);
  bad.block_size = 16;
  bad.num_layers = 0;
  CHECK(kv_pool_bytes(&bad) == 0);
  CHECK(kv_pool_bytes(nullptr) == 0);
  CHECK(kv_pool_num_blocks_for_budget(nullptr, 1 << 20) == -1);
}

void validators() {
  const int64_t slots_ok[] = {0, 5, -1, 63, -7};
  CHECK(pkv_check_slots(slots_ok, 5, 64) == PKV_OK);
  const int64_t slots_dup[] = {3, 4, 3};
  CHECK(pkv_check_slots(slots_dup, 3, 64) == PKV_ERR_INVALID);
  const int64_t slots_big[] = {64};
  CHECK(pkv_check_slots(slots_big, 1, 64) == PKV_ERR_INVALID);
  CHECK(pkv_check_slots(nullptr, 0, 64) == PKV_OK);
  CHECK(pkv_check_slots(nullptr, 2, 64) == PKV_ERR_INVALID);
  const int64_t pairs_ok[] = {0, 1, 0, 2, 5, 6};
  CHECK(pkv_check_pairs(pairs_ok, 3, 8) == PKV_OK);
  const int64_t pairs_chain[] = {0, 1, 1, 2};
  CHECK(pkv_check_pairs(pairs_chain, 2, 8) == PKV_ERR_INVALID);
  const int64_t pairs_dup[] = {0, 3, 1, 3};
  CHECK(pkv_check_pairs(pairs_dup, 2, 8) == PKV_ERR_INVALID);
  const int64_t pairs_out[] = {0, 8};
  CHECK(pkv_check_pairs(pairs_out, 1, 8) == PKV_ERR_INVALID);
  const int32_t tables[] = {1, 2, 99, 3, 0, 0};
  const int32_t ctx_ok[] = {17, 1};
  CHECK(pkv_check_tables(tables, ctx_ok, 2, 3, 8, 4) == PKV_ERR_INVALID);   // entry 99 is read (ctx 17 = 3 blocks)
  const int32_t ctx_short[] = {16, 1};
  CHECK(pkv_check_tables(tables, ctx_short, 2, 3, 8, 4) == PKV_OK);         // ... but not for ctx 16
  const int32_t ctx_long[] = {25, 1};
  CHECK(pkv_check_tables(tables, ctx_long, 2, 3, 8, 100) == PKV_ERR_INVALID);
  const int32_t ctx_neg[] = {-1, 1};
  CHECK(pkv_check_tables(tables, ctx_neg, 2, 3, 8, 100) == PKV_ERR_INVALID);
}

// Host model of what the manager must hold, rebuilt from its own tables.
struct View {
  std::map<int32_t, std::vector<int32_t>> tab;
  std::map<int32_t, int32_t> len;
};

View snapshot(const pkv_bm* bm, const std::set<int32_t>& live, int width) {
  View v;
  std::vector<int32_t> seqs(live.begin(), live.end());
  std::vector<int32_t> t(seqs.size() * (size_t)width + 1), c(seqs.size() + 1);
  CHECK(kv_bm_block_tables(bm, seqs.data(), (int32_t)seqs.size(), t.data(), width, c.data()) == PKV_OK);
  for (size_t i = 0; i < seqs.size(); ++i) {
    v.tab[seqs[i]].assign(t.begin() + (long)(i * width), t.begin() + (long)(i * width + width));
    v.len[seqs[i]] = c[i];
  }
  return v;
}

void invariants(const pkv_bm* bm, const View& v, int NB, int B, int width) {
  std::vector<int32_t> refs((size_t)NB, 0);
  for (const auto& [s, row] : v.tab) {
    const int32_t n = (v.len.at(s) + B - 1) / B;
    CHECK(n <= width);
    for (int i = 0; i < n; ++i) {
      CHECK(row[(size_t)i] >= 0 && row[(size_t)i] < NB);
      refs[(size_t)row[(size_t)i]]++;
    }
    for (int i = n; i < width; ++i) CHECK(row[(size_t)i] == 0);
  }
  int used = 0;
  for (int b = 0; b < NB; ++b) {
    CHECK(kv_bm_ref_count(bm, b) == refs[(size_t)b]);
    used += refs[(size_t)b] > 0;
  }
  int32_t u = -1, total = -1;
  int64_t failed = -1;
  CHECK(kv_bm_stats(bm, &u, &total, &failed) == PKV_OK);
  CHECK(u == used && total == NB && failed >= 0);
  CHECK(kv_bm_ref_count(bm, -1) == -1 && kv_bm_ref_count(bm, NB) == -1);
}

void block_manager_walk(uint64_t seed) {
  const int NB = 96, B = 4, width = 40;
  Lcg r{seed};
  std::vector<int32_t> order(NB);
  for (int i = 0; i < NB; ++i) order[(size_t)i] = i;
  for (int i = NB - 1; i > 0; --i) std::swap(order[(size_t)i], order[(size_t)r.below(i + 1)]);
  pkv_bm* bm = nullptr;
  CHECK(kv_bm_create(NB, B, order.data(), &bm) == PKV_OK && bm);
  std::set<int32_t> live;
  int32_t next_id = 0;
  int64_t last_lookups = 0, last_hits = 0;
  int64_t n_cow = 0, n_refused = 0, n_appended = 0;
  // prompts: a shared system prompt of 3 blocks + own tokens, from a small vocabulary
  std::vector<int32_t> system(3 * B + 1);
  for (auto& t : system) t = r.below(50);
  for (int it = 0; it < 6000; ++it) {
    const View before = snapshot(bm, live, width);
    const int op = r.below(10);
    if (op == 0 || live.empty()) {                    // new sequence
      const int32_t n = r.below(4 * B);
      const pkv_status st = kv_bm_add_seq(bm, next_id, n);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
      if (st == PKV_OK) live.insert(next_id);
      ++next_id;
    } else if (op == 1) {                             // prompt with the shared prefix
      std::vector<int32_t> toks(system.begin(), system.begin() + r.below((int)system.size()) + 1);
      const int extra = r.below(2 * B);
      for (int i = 0; i < extra; ++i) toks.push_back(50 + r.below(5));
      int32_t cached = -1;
      const pkv_status st = kv_bm_add_seq_tokens(bm, next_id, toks.data(), (int32_t)toks.size(), &cached);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
      if (st == PKV_OK) {
        live.insert(next_id);
        CHECK(cached >= 0 && cached % B == 0 && cached < (int32_t)toks.size());
      }
      ++next_id;
      int64_t lookups = -1, hits = -1;
      int32_t nkeys = -1;
      CHECK(kv_bm_prefix_stats(bm, &lookups, &hits, &nkeys) == PKV_OK);
      CHECK(lookups >= last_lookups && hits >= last_hits && hits <= lookups && nkeys >= 0 && nkeys <= NB);
      last_lookups = lookups;
      last_hits = hits;
    } else if (op == 2) {                             // fork
      auto p = live.begin();
      std::advance(p, r.below((int)live.size()));
      CHECK(kv_bm_fork(bm, *p, next_id) == PKV_OK);
      live.insert(next_id++);
    } else if (op <= 7) {                             // batch append
      std::vector<int32_t> seqs;
      for (int32_t s : live)
        if (r.below(3) == 0 && before.len.at(s) < (width - 1) * B) seqs.push_back(s);
      for (size_t i = seqs.size(); i > 1; --i) std::swap(seqs[i - 1], seqs[(size_t)r.below((int)i)]);
      std::vector<int64_t> slots(seqs.size() + 1), pairs(2 * seqs.size() + 2);
      int32_t np = -1;
      const pkv_status st =
          kv_bm_append(bm, seqs.data(), (int32_t)seqs.size(), slots.data(), pairs.data(), &np);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
      const View after = snapshot(bm, live, width);
      if (st != PKV_OK) {
        CHECK(after.tab == before.tab && after.len == before.len);   // all or nothing
        ++n_refused;
      } else {
        n_cow += np;
        n_appended += (int64_t)seqs.size();
        std::vector<int32_t> ref_before((size_t)NB, 0);
        for (const auto& [s, row] : before.tab)
          for (int i = 0; i < (before.len.at(s) + B - 1) / B; ++i) ref_before[(size_t)row[(size_t)i]]++;
        CHECK(np >= 0 && np <= (int32_t)seqs.size());
        for (int32_t k = 0; k < np; ++k) {
          const int64_t src = pairs[(size_t)(2 * k)], dst = pairs[(size_t)(2 * k + 1)];
          CHECK(src >= 0 && src < NB && dst >= 0 && dst < NB && src != dst);
          CHECK(ref_before[(size_t)src] > 1 && ref_before[(size_t)dst] == 0);
        }
        for (size_t i = 0; i < seqs.size(); ++i) {
          const int32_t s = seqs[i], pos = before.len.at(s);
          CHECK(after.len.at(s) == pos + 1);
          CHECK(slots[i] == (int64_t)after.tab.at(s)[(size_t)(pos / B)] * B + pos % B);
          CHECK(kv_bm_ref_count(bm, after.tab.at(s)[(size_t)(pos / B)]) == 1);   // the written block is unshared
        }
      }
    } else {                                          // free
      auto p = live.begin();
      std::advance(p, r.below((int)live.size()));
      CHECK(kv_bm_free_seq(bm, *p) == PKV_OK);
      live.erase(p);
    }
    invariants(bm, snapshot(bm, live, width), NB, B, width);
  }
  // argument errors leave the state alone
  const View v = snapshot(bm, live, width);
  CHECK(kv_bm_add_seq(bm, *live.begin(), 3) == PKV_ERR_INVALID || live.empty());
  CHECK(kv_bm_add_seq(bm, next_id, -1) == PKV_ERR_INVALID);
  CHECK(kv_bm_fork(bm, -12345, next_id) == PKV_ERR_INVALID);
  CHECK(kv_bm_free_seq(bm, -12345) == PKV_ERR_INVALID);
  if (!live.empty()) {
    const int32_t twice[] = {*live.begin(), *live.begin()};
    int64_t sl[2], pr[4];
    int32_t np = 0;
    CHECK(kv_bm_append(bm, twice, 2, sl, pr, &np) == PKV_ERR_INVALID);
    int32_t row[1];
    const int32_t one[] = {*live.rbegin()};
    if ((v.len.at(one[0]) + B - 1) / B > 1) CHECK(kv_bm_block_tables(bm, one, 1, row, 1, nullptr) == PKV_ERR_INVALID);
  }
  CHECK(kv_bm_append(nullptr, nullptr, 0, nullptr, nullptr, nullptr) == PKV_ERR_INVALID);
  const View w = snapshot(bm, live, width);
  CHECK(w.tab == v.tab && w.len == v.len);
  for (int32_t s : live) CHECK(kv_bm_free_seq(bm, s) == PKV_OK);
  for (int b = 0; b < NB; ++b) CHECK(kv_bm_ref_count(bm, b) == 0);
  kv_bm_destroy(bm);
  // the walk must have reached the interesting paths
  CHECK(n_cow > 0 && n_refused > 0 && n_appended > 0 && last_hits > 0);
  std::printf("walk %llu: %lld appends, %lld copy-on-write pairs, %lld refused appends, %lld prefix hits of %lld\n",
              (unsigned long long)seed, (long long)n_appended, (long long)n_cow, (long long)n_refused,
              (long long)last_hits, (long long)last_lookups);
}

void create_errors_and_keys() {
  pkv_bm* bm = nullptr;
  CHECK(kv_bm_create(0, 16, nullptr, &bm) == PKV_ERR_INVALID && bm == nullptr);
  const int32_t not_perm[] = {0, 0, 1};
  CHECK(kv_bm_create(3, 16, not_perm, &bm) == PKV_ERR_INVALID && bm == nullptr);
  CHECK(kv_bm_create(3, 16, nullptr, nullptr) == PKV_ERR_INVALID);
  uint8_t k1[32], k2[32], k3[32];
  const int32_t toks[] = {1, 2, 3, 4};
  CHECK(kv_bm_block_key(nullptr, toks, 4, k1) == PKV_OK);
  CHECK(kv_bm_block_key(nullptr, toks, 4, k2) == PKV_OK && std::memcmp(k1, k2, 32) == 0);
  CHECK(kv_bm_block_key(k1, toks, 4, k3) == PKV_OK && std::memcmp(k1, k3, 32) != 0);
  CHECK(kv_bm_block_key(nullptr, nullptr, 4, k3) == PKV_ERR_INVALID);
  CHECK(kv_bm_block_key(nullptr, toks, 4, nullptr) == PKV_ERR_INVALID);
  kv_bm_destroy(nullptr);
}

// The radix-tree prefix cache on a small pool (eviction runs often), with a
// simulated pool memory: each slot holds the token id whose K/V it stores.
// A request writes its tokens from the cached count on after copying its
// pair, an append writes one token after its copy-on-write pairs, and every
// live sequence must read back its own tokens after every call.
void radix_walk(uint64_t seed) {
  const int NB = 40, width = 64;
  Lcg r{seed * 7 + 1};
  const int sizes[] = {1, 2, 3, 4, 8, 16};
  const int B = sizes[seed % 6];
  pkv_bm* bm = nullptr;
  CHECK(kv_bm_create(NB, B, nullptr, &bm) == PKV_OK);
  std::vector<std::vector<int32_t>> mem((size_t)NB, std::vector<int32_t>((size_t)B, -1));
  std::map<int32_t, std::vector<int32_t>> hist;
  std::set<int32_t> live;
  std::vector<std::vector<int32_t>> stems(4);
  for (auto& st : stems) {
    st.resize((size_t)r.below(5 * B + 2));
    for (auto& t : st) t = r.below(3);
  }
  int32_t next_id = 0;
  int64_t n_partial = 0, n_hit_tokens = 0;
  auto slot_of = [&](const View& v, int32_t s, int32_t pos) -> int32_t& {
    return mem[(size_t)v.tab.at(s)[(size_t)(pos / B)]][(size_t)(pos % B)];
  };
  for (int it = 0; it < 3000; ++it) {
    const int op = r.below(10);
    if (op < 4) {
      const auto& st = stems[(size_t)r.below(4)];
      std::vector<int32_t> toks(st.begin(), st.begin() + r.below((int)st.size() + 1));
      for (int k = r.below(2 * B + 2); k > 0; --k) toks.push_back(r.below(3));
      int32_t cached = -1;
      int64_t pair[2] = {-7, -7};
      const pkv_status s = kv_bm_add_seq_radix(bm, next_id, toks.data(), (int32_t)toks.size(), &cached, pair);
      CHECK(s == PKV_OK || s == PKV_ERR_OUT_OF_BLOCKS);
      if (s == PKV_OK) {
        live.insert(next_id);
        const View v = snapshot(bm, live, width);
        CHECK(cached >= 0 && (toks.empty() ? cached == 0 : cached < (int32_t)toks.size()));
        CHECK((pair[0] >= 0) == (cached % B != 0));
        if (pair[0] >= 0) {
          CHECK(pair[0] < NB && pair[1] == v.tab.at(next_id)[(size_t)(cached / B)]);
          mem[(size_t)pair[1]] = mem[(size_t)pair[0]];
          ++n_partial;
        }
        for (int32_t p = 0; p < (int32_t)toks.size(); ++p) {
          int32_t& m = slot_of(v, next_id, p);
          if (p < cached) CHECK(m == toks[(size_t)p]);
          else m = toks[(size_t)p];
        }
        hist[next_id] = toks;
        n_hit_tokens += cached;
      }
      ++next_id;
    } else if (op < 6 && !live.empty()) {
      std::vector<int32_t> seqs;
      for (int32_t s : live)
        if (r.below(2)) seqs.push_back(s);
      if (seqs.empty()) continue;
      std::vector<int64_t> slots(seqs.size()), pairs(2 * seqs.size());
      int32_t np = -1;
      const pkv_status st =
          kv_bm_append(bm, seqs.data(), (int32_t)seqs.size(), slots.data(), pairs.data(), &np);
      CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_BLOCKS);
      if (st != PKV_OK) continue;
      for (int32_t k = 0; k < np; ++k) mem[(size_t)pairs[(size_t)(2 * k + 1)]] = mem[(size_t)pairs[(size_t)(2 * k)]];
      for (size_t k = 0; k < seqs.size(); ++k) {
        const int32_t t = r.below(3);
        mem[(size_t)(slots[k] / B)][(size_t)(slots[k] % B)] = t;
        hist[seqs[k]].push_back(t);
      }
    } else if (op < 7 && !live.empty()) {
      auto p = live.begin();
      std::advance(p, r.below((int)live.size()));
      CHECK(kv_bm_fork(bm, *p, next_id) == PKV_OK);
      hist[next_id] = hist[*p];
      live.insert(next_id++);
    } else if (!live.empty()) {
      auto p = live.begin();
      std::advance(p, r.below((int)live.size()));
      CHECK(kv_bm_free_seq(bm, *p) == PKV_OK);
      hist.erase(*p);
      live.erase(p);
    }
    const View v = snapshot(bm, live, width);
    invariants(bm, v, NB, B, width);
    for (const auto& [s, toks] : hist)
      for (int32_t p = 0; p < (int32_t)toks.size(); ++p) CHECK(slot_of(v, s, p) == toks[(size_t)p]);
    int64_t lookups = -1, hits = -1;
    int32_t nodes = -1, idle = -1;
    CHECK(kv_bm_radix_stats(bm, &lookups, &hits, &nodes, &idle) == PKV_OK);
    CHECK(hits == n_hit_tokens && hits <= lookups && idle >= 0 && idle <= nodes && nodes <= NB);
  }
  // one prefix cache per manager; bad arguments
  int32_t cached = 0;
  int64_t pair[2];
  const int32_t t3[] = {0, 1, 2};
  CHECK(kv_bm_add_seq_tokens(bm, next_id, t3, 3, &cached) == PKV_ERR_UNSUPPORTED);
  CHECK(kv_bm_add_seq_radix(bm, next_id, t3, 3, &cached, nullptr) == PKV_ERR_INVALID);
  CHECK(kv_bm_add_seq_radix(bm, next_id, nullptr, 3, &cached, pair) == PKV_ERR_INVALID);
  CHECK(kv_bm_add_seq_radix(nullptr, next_id, t3, 3, &cached, pair) == PKV_ERR_INVALID);
  CHECK(kv_bm_radix_stats(nullptr, nullptr, nullptr, nullptr, nullptr) == PKV_ERR_INVALID);
  CHECK(n_partial > 0 || B == 1);   // with one-token blocks every match is whole
  std::printf("radix walk %llu: B %d, %lld partial matches, %lld cached tokens\n", (unsigned long long)seed, B,
              (long long)n_partial, (long long)n_hit_tokens);
  for (int32_t s : live) CHECK(kv_bm_free_seq(bm, s) == PKV_OK);
  kv_bm_destroy(bm);
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 436;
  pool_sizing();
  validators();
  create_errors_and_keys();
  for (uint64_t k = 0; k < 4; ++k) block_manager_walk(seed + k);
  for (uint64_t k = 0; k < 6; ++k) radix_walk(seed + k);
  std::printf("host api check passed\n");
  return 0;
}
