// Host block allocator of libpkv: free list, refcounts, per-sequence block
// tables, fork and copy-on-write.
//
// The pages fix the mechanism: fixed 16-token blocks, a per-request table from
// logical to physical block, blocks taken on demand and returned the moment a
// request ends ([p1] chanyi.net.cn/article/49 §三; [p2] lqnn.cn/news/235768
// §3.2), shared prefixes pointing at the same physical blocks with a copy made
// only when one sharer forks off ([p1] §三), and a capped pool that makes a
// request wait instead of overflowing ([p2] §5.2). They leave the policy open;
// this file fixes it so results are reproducible bit for bit:
//   - the free list is a LIFO stack seeded so the first block handed out is
//     free_order[0]; freeing a sequence pushes its blocks in reverse logical
//     order;
//   - one reservation takes blocks token by token, in logical order;
//   - a write at a non-zero offset of a block with refcount > 1 moves the
//     writer to a fresh block and reports the (old, new) pair to copy;
//   - a reservation either succeeds whole or changes nothing.
//
// Prefix cache ([p2] §4.3: K/V kept block by block with the order of the
// blocks recorded; a request whose prefix matches reuses those blocks and
// computes only the rest; eviction left to tuning):
//   - only full blocks are cached, each identified by its 16 token ids and
//     its predecessor (the cached block before it, or none); matching
//     compares the ids themselves, the 64-bit key only narrows the search;
//   - a lookup takes the longest matching chain of a prompt's leading full
//     blocks, at most floor((n - 1) / 16), so the last token is computed;
//   - the cache holds one reference per cached block; a block only the cache
//     holds, with no cached block after it, is evictable;
//   - least recently used first: a hit or an insert marks its chain's blocks
//     used, last block first, so a block is always newer than its followers;
//   - a reservation short of free blocks evicts just enough first, or, if
//     free plus cache-only blocks are too few, changes nothing.
#include <algorithm>
#include <array>
#include <cstring>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // logical block -> physical block
  int32_t len = 0;             // tokens held
};

}  // namespace

namespace {

struct CacheEntry {
  int32_t pred = -1;  // cached block before this one, -1 for a first block
  std::array<int32_t, PKV_BLOCK_TOKENS> ids{};
  uint64_t tick = 0;  // last use
};

uint64_t content_key(int32_t pred, const int32_t* ids) {
  uint64_t h = 0x9E3779B97F4A7C15ull ^ uint64_t(uint32_t(pred));
  for (int i = 0; i < PKV_BLOCK_TOKENS; ++i) {
    h ^= uint64_t(uint32_t(ids[i])) + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    h *= 0xBF58476D1CE4E5B9ull;
    h ^= h >> 31;
  }
  return h;
}

}  // namespace

struct pkv_pool {
  pkv_config cfg;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;         // per physical block
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 1;
  // prefix cache
  std::vector<char> cached;                                      // per block
  std::vector<CacheEntry> entry;                                 // per block, valid if cached
  std::vector<int32_t> children;                                 // cached blocks following each block
  std::unordered_multimap<uint64_t, int32_t> by_key;             // content key -> cached block
  std::set<std::pair<uint64_t, int32_t>> lru;                    // (tick, block) of cached blocks
  uint64_t tick = 0;
};

namespace {

Seq* find(pkv_pool* p, int64_t id) {
  auto it = p->seqs.find(id);
  return it == p->seqs.end() ? nullptr : &it->second;
}
const Seq* find(const pkv_pool* p, int64_t id) {
  auto it = p->seqs.find(id);
  return it == p->seqs.end() ? nullptr : &it->second;
}

int64_t ceil_blocks(int64_t tokens) { return (tokens + PKV_BLOCK_TOKENS - 1) / PKV_BLOCK_TOKENS; }

// The cached block with these ids after `pred`, or -1.
int32_t cache_find(const pkv_pool* p, int32_t pred, const int32_t* ids) {
  auto range = p->by_key.equal_range(content_key(pred, ids));
  for (auto it = range.first; it != range.second; ++it) {
    const CacheEntry& e = p->entry[it->second];
    if (e.pred == pred && std::equal(e.ids.begin(), e.ids.end(), ids)) return it->second;
  }
  return -1;
}

// Mark a chain used, last block first (a block stays newer than its followers).
void cache_touch(pkv_pool* p, const std::vector<int32_t>& chain) {
  for (auto it = chain.rbegin(); it != chain.rend(); ++it) {
    CacheEntry& e = p->entry[*it];
    p->lru.erase({e.tick, *it});
    e.tick = ++p->tick;
    p->lru.insert({e.tick, *it});
  }
}

int32_t cache_reclaimable(const pkv_pool* p) {
  int32_t n = 0;
  for (const auto& tb : p->lru) n += p->ref[tb.second] == 1;
  return n;
}

// Evict the least recently used block only the cache holds and no cached
// block follows; returns it, or -1.
int32_t cache_evict_one(pkv_pool* p) {
  for (auto it = p->lru.begin(); it != p->lru.end(); ++it) {
    const int32_t b = it->second;
    if (p->ref[b] != 1 || p->children[b] != 0) continue;
    CacheEntry& e = p->entry[b];
    auto range = p->by_key.equal_range(content_key(e.pred, e.ids.data()));
    for (auto k = range.first; k != range.second; ++k)
      if (k->second == b) {
        p->by_key.erase(k);
        break;
      }
    if (e.pred >= 0) --p->children[e.pred];
    p->lru.erase(it);
    p->cached[b] = 0;
    e = CacheEntry{};
    if (--p->ref[b] == 0) p->free_stack.push_back(b);
    return b;
  }
  return -1;
}

}  // namespace

namespace pkv {
int32_t pool_num_blocks(const pkv_pool* pool) { return pool->cfg.num_blocks; }
}  // namespace pkv

extern "C" {

int pkv_pool_create(const pkv_config* cfg, const int32_t* free_order, int32_t n, pkv_pool** out) {
  int st = pkv::validate_config(cfg);
  if (st != PKV_OK) return st;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const int32_t N = cfg->num_blocks;
  std::vector<int32_t> order(N);
  if (free_order) {
    if (n != N) return pkv::fail(PKV_ERR_INVALID_ARG, "free_order has %d entries, pool has %d", n, N);
    std::vector<char> seen(N, 0);
    for (int32_t i = 0; i < N; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= N || seen[b])
        return pkv::fail(PKV_ERR_INVALID_ARG, "free_order is not a permutation of 0..%d", N - 1);
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < N; ++i) order[i] = i;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "out of host memory");
  p->cfg = *cfg;
  p->free_stack.assign(order.rbegin(), order.rend());
  p->ref.assign(N, 0);
  p->cached.assign(N, 0);
  p->entry.assign(N, CacheEntry{});
  p->children.assign(N, 0);
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_seq_create(pkv_pool* pool, int64_t* seq) {
  if (!pool || !seq) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  int64_t id = pool->next_id++;
  pool->seqs.emplace(id, Seq{});
  *seq = id;
  return PKV_OK;
}

int pkv_seq_free(pkv_pool* pool, int64_t seq) {
  if (!pool) return pkv::fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  Seq* s = find(pool, seq);
  if (!s) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq);
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it) {
    int32_t b = *it;
    if (pool->ref[b] <= 0) return pkv::fail(PKV_ERR_REFCOUNT, "block %d refcount underflow", b);
  }
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it) {
    int32_t b = *it;
    if (--pool->ref[b] == 0) pool->free_stack.push_back(b);
  }
  pool->seqs.erase(seq);
  return PKV_OK;
}

int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t* child) {
  if (!pool || !child) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  const Seq* ps = find(pool, parent);
  if (!ps) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)parent);
  Seq c = *ps;  // copy before inserting: the map may rehash
  for (int32_t b : c.table) ++pool->ref[b];
  int64_t id = pool->next_id++;
  pool->seqs.emplace(id, std::move(c));
  *child = id;
  return PKV_OK;
}

int pkv_seq_reserve(pkv_pool* pool, int64_t seq, int32_t n, int32_t* slots_out, int32_t* cow_pairs_out,
                    int32_t cow_cap, int32_t* n_cow) {
  if (!pool) return pkv::fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (n > 0 && !slots_out) return pkv::fail(PKV_ERR_INVALID_ARG, "slots_out is NULL");
  Seq* s = find(pool, seq);
  if (!s) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq);
  const int64_t len = s->len;
  if (len + n > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence length overflows int32");
  // Plan: blocks opened by tokens at offset 0, plus one copy-on-write if the
  // first token lands at a non-zero offset of a shared tail block.
  int64_t need = ceil_blocks(len + n) - ceil_blocks(len);
  bool cow = n > 0 && (len % PKV_BLOCK_TOKENS) != 0 && pool->ref[s->table.back()] > 1;
  if (cow) {
    ++need;
    if (!cow_pairs_out || cow_cap < 1)
      return pkv::fail(PKV_ERR_INVALID_ARG, "copy-on-write needed but cow_cap < 1");
  }
  if (need > int64_t(pool->free_stack.size())) {
    const int64_t have = int64_t(pool->free_stack.size()) + cache_reclaimable(pool);
    if (need > have)
      return pkv::fail(PKV_ERR_NO_BLOCKS, "need %lld blocks, %zu free, %lld with the cache-only ones",
                       (long long)need, pool->free_stack.size(), (long long)have);
    while (need > int64_t(pool->free_stack.size()))
      if (cache_evict_one(pool) < 0) return pkv::fail(PKV_ERR_REFCOUNT, "prefix cache bookkeeping is inconsistent");
  }
  // Apply.
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t pos = len + i;
    const int32_t lblk = int32_t(pos / PKV_BLOCK_TOKENS), off = int32_t(pos % PKV_BLOCK_TOKENS);
    int32_t blk;
    if (off == 0) {
      blk = pool->free_stack.back();
      pool->free_stack.pop_back();
      pool->ref[blk] = 1;
      s->table.push_back(blk);
    } else {
      blk = s->table[lblk];
      if (pool->ref[blk] > 1) {
        int32_t fresh = pool->free_stack.back();
        pool->free_stack.pop_back();
        pool->ref[fresh] = 1;
        --pool->ref[blk];
        s->table[lblk] = fresh;
        cow_pairs_out[2 * ncow] = blk;
        cow_pairs_out[2 * ncow + 1] = fresh;
        ++ncow;
        blk = fresh;
      }
    }
    slots_out[i] = blk * PKV_BLOCK_TOKENS + off;
  }
  s->len = int32_t(len + n);
  if (n_cow) *n_cow = ncow;
  return PKV_OK;
}

int pkv_seq_len(const pkv_pool* pool, int64_t seq, int32_t* len) {
  if (!pool || !len) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  const Seq* s = find(pool, seq);
  if (!s) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq);
  *len = s->len;
  return PKV_OK;
}

int pkv_seq_block_table(const pkv_pool* pool, int64_t seq, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  const Seq* s = find(pool, seq);
  if (!s) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq);
  *n = int32_t(s->table.size());
  if (cap < *n || (*n > 0 && !out))
    return pkv::fail(PKV_ERR_INVALID_ARG, "table has %d blocks, cap is %d", *n, cap);
  if (*n) std::memcpy(out, s->table.data(), sizeof(int32_t) * size_t(*n));
  return PKV_OK;
}

int pkv_block_refcount(const pkv_pool* pool, int32_t block, int32_t* ref) {
  if (!pool || !ref) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (block < 0 || block >= pool->cfg.num_blocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "block %d out of range", block);
  *ref = pool->ref[block];
  return PKV_OK;
}

int pkv_num_free(const pkv_pool* pool, int32_t* n) {
  if (!pool || !n) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *n = int32_t(pool->free_stack.size());
  return PKV_OK;
}

int pkv_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *n = int32_t(pool->free_stack.size());
  if (cap < *n || (*n > 0 && !out))
    return pkv::fail(PKV_ERR_INVALID_ARG, "%d free blocks, cap is %d", *n, cap);
  for (int32_t i = 0; i < *n; ++i) out[i] = pool->free_stack[size_t(*n - 1 - i)];
  return PKV_OK;
}

int pkv_build_block_tables(const pkv_pool* pool, const int64_t* seqs, int32_t B, int32_t max_blocks,
                           int32_t* tables_host, int32_t* ctx_lens_host) {
  if (!pool || !seqs || !tables_host || !ctx_lens_host)
    return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (B < 0 || max_blocks < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "negative size");
  for (int32_t b = 0; b < B; ++b) {
    const Seq* s = find(pool, seqs[b]);
    if (!s) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seqs[b]);
    if (int64_t(s->table.size()) > max_blocks)
      return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld has %zu blocks > max_blocks %d",
                       (long long)seqs[b], s->table.size(), max_blocks);
  }
  for (int32_t b = 0; b < B; ++b) {
    const Seq* s = find(pool, seqs[b]);
    int32_t* row = tables_host + int64_t(b) * max_blocks;
    size_t nb = s->table.size();
    for (size_t j = 0; j < nb; ++j) row[j] = s->table[j];
    for (int32_t j = int32_t(nb); j < max_blocks; ++j) row[j] = -1;
    ctx_lens_host[b] = s->len;
  }
  return PKV_OK;
}

int pkv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int32_t n, int64_t* seq, int32_t* n_cached) {
  if (!pool || !seq || !n_cached || (n > 0 && !tokens)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  Seq s;
  int32_t pred = -1;
  const int32_t blocks = n > 0 ? (n - 1) / PKV_BLOCK_TOKENS : 0;
  for (int32_t j = 0; j < blocks; ++j) {
    const int32_t b = cache_find(pool, pred, tokens + int64_t(j) * PKV_BLOCK_TOKENS);
    if (b < 0) break;
    s.table.push_back(b);
    pred = b;
  }
  for (int32_t b : s.table) ++pool->ref[b];
  s.len = int32_t(s.table.size()) * PKV_BLOCK_TOKENS;
  cache_touch(pool, s.table);
  const int64_t id = pool->next_id++;
  *n_cached = s.len;
  pool->seqs.emplace(id, std::move(s));
  *seq = id;
  return PKV_OK;
}

int pkv_prefix_cache_insert(pkv_pool* pool, int64_t seq, const int32_t* tokens, int32_t n, int32_t* n_added) {
  if (!pool || (n > 0 && !tokens)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  Seq* s = find(pool, seq);
  if (!s) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seq);
  const int32_t nfull = std::min(n, s->len) / PKV_BLOCK_TOKENS;
  std::vector<int32_t> chain;
  int32_t pred = -1, added = 0;
  for (int32_t j = 0; j < nfull; ++j) {
    const int32_t b = s->table[j];
    const int32_t* ids = tokens + int64_t(j) * PKV_BLOCK_TOKENS;
    const int32_t have = cache_find(pool, pred, ids);
    if (have < 0) {
      if (pool->cached[b]) break;  // cached under other content: the ids do not describe this table
      CacheEntry& e = pool->entry[b];
      e.pred = pred;
      std::copy(ids, ids + PKV_BLOCK_TOKENS, e.ids.begin());
      e.tick = 0;
      pool->cached[b] = 1;
      pool->by_key.emplace(content_key(pred, ids), b);
      pool->lru.insert({0, b});
      ++pool->ref[b];
      if (pred >= 0) ++pool->children[pred];
      ++added;
    } else if (have != b) {
      break;  // this content is already cached as another block
    }
    chain.push_back(b);
    pred = b;
  }
  cache_touch(pool, chain);
  if (n_added) *n_added = added;
  return PKV_OK;
}

int pkv_prefix_cache_evict(pkv_pool* pool, int32_t max_blocks, int32_t* evicted_out, int32_t* n_evicted) {
  if (!pool || !n_evicted || (max_blocks > 0 && !evicted_out)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (max_blocks < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "max_blocks must be >= 0");
  int32_t k = 0;
  while (k < max_blocks) {
    const int32_t b = cache_evict_one(pool);
    if (b < 0) break;
    evicted_out[k++] = b;
  }
  *n_evicted = k;
  return PKV_OK;
}

int pkv_prefix_cache_stats(const pkv_pool* pool, int32_t* n_cached, int32_t* n_reclaimable) {
  if (!pool || !n_cached || !n_reclaimable) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *n_cached = int32_t(pool->lru.size());
  *n_reclaimable = cache_reclaimable(pool);
  return PKV_OK;
}

int pkv_prefix_cache_entry(const pkv_pool* pool, int32_t block, int32_t* is_cached, int32_t* pred, int32_t* ids,
                           int64_t* last_use) {
  if (!pool || !is_cached || !pred || !ids || !last_use) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (block < 0 || block >= pool->cfg.num_blocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "block %d out of range", block);
  const CacheEntry& e = pool->entry[block];
  *is_cached = pool->cached[block];
  *pred = pool->cached[block] ? e.pred : -1;
  for (int i = 0; i < PKV_BLOCK_TOKENS; ++i) ids[i] = pool->cached[block] ? e.ids[i] : 0;
  *last_use = pool->cached[block] ? int64_t(e.tick) : 0;
  return PKV_OK;
}

int32_t pkv_plan_ints(int32_t B) { return B < 0 ? 0 : 2 * B + (B / 2) * PKV_PREFIX_GROUP_INTS; }

int pkv_plan_shared_prefix(const pkv_pool* pool, const int64_t* seqs, int32_t B, int32_t min_blocks,
                           int32_t max_members, int32_t* plan_host, int32_t plan_cap, int32_t* n_groups) {
  if (!pool || !seqs || !plan_host || !n_groups) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (B < 0 || min_blocks < 1 || max_members < 1 || max_members > PKV_MAX_SHARERS)
    return pkv::fail(PKV_ERR_INVALID_ARG, "need B >= 0, min_blocks >= 1, max_members in [1, %d]", PKV_MAX_SHARERS);
  if (plan_cap < pkv_plan_ints(B))
    return pkv::fail(PKV_ERR_INVALID_ARG, "plan_cap %d < %d", plan_cap, pkv_plan_ints(B));
  std::vector<const Seq*> sq(B);
  for (int32_t b = 0; b < B; ++b) {
    sq[b] = find(pool, seqs[b]);
    if (!sq[b]) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld is not live", (long long)seqs[b]);
  }
  // blocks that may be shared: full, and before the block of the last token
  auto shareable = [&](int32_t b) { return sq[b]->len >= 1 ? (sq[b]->len - 1) / PKV_BLOCK_TOKENS : 0; };
  // sequences keyed by their first block, keys in order of first appearance
  std::vector<int32_t> keys;
  std::unordered_map<int32_t, std::vector<int32_t>> by_first;
  for (int32_t b = 0; b < B; ++b) {
    if (shareable(b) < min_blocks) continue;
    const int32_t first = sq[b]->table[0];
    auto it = by_first.find(first);
    if (it == by_first.end()) {
      keys.push_back(first);
      by_first[first] = {b};
    } else {
      it->second.push_back(b);
    }
  }
  for (int32_t b = 0; b < B; ++b) {
    plan_host[2 * b] = 0;
    plan_host[2 * b + 1] = -1;
  }
  int32_t ng = 0;
  for (int32_t key : keys) {
    const std::vector<int32_t>& all = by_first[key];
    for (size_t c0 = 0; c0 < all.size(); c0 += size_t(max_members)) {
      const size_t c1 = std::min(all.size(), c0 + size_t(max_members));
      if (c1 - c0 < 2) continue;
      int32_t np = shareable(all[c0]);
      for (size_t i = c0 + 1; i < c1; ++i) np = std::min(np, shareable(all[i]));
      const std::vector<int32_t>& t0 = sq[all[c0]]->table;
      int32_t lcp = 0;
      while (lcp < np) {
        bool same = true;
        for (size_t i = c0 + 1; i < c1 && same; ++i) same = sq[all[i]]->table[lcp] == t0[lcp];
        if (!same) break;
        ++lcp;
      }
      if (lcp < min_blocks) continue;
      int32_t* gd = plan_host + 2 * int64_t(B) + int64_t(ng) * PKV_PREFIX_GROUP_INTS;
      gd[0] = lcp;
      gd[1] = int32_t(c1 - c0);
      for (int32_t m = 0; m < PKV_MAX_SHARERS; ++m) gd[2 + m] = m < int32_t(c1 - c0) ? all[c0 + m] : -1;
      for (size_t i = c0; i < c1; ++i) {
        plan_host[2 * all[i]] = lcp;
        plan_host[2 * all[i] + 1] = ng * 64 + int32_t(i - c0);
      }
      ++ng;
    }
  }
  *n_groups = ng;
  return PKV_OK;
}

}  // extern "C"
