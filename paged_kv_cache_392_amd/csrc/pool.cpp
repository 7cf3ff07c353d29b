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
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // logical block -> physical block
  int32_t len = 0;             // tokens held
};

}  // namespace

struct pkv_pool {
  pkv_config cfg;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;         // per physical block
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 1;
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

}  // namespace

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
  if (need > int64_t(pool->free_stack.size()))
    return pkv::fail(PKV_ERR_NO_BLOCKS, "need %lld blocks, %zu free", (long long)need,
                     pool->free_stack.size());
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
