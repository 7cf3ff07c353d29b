// Continuous-batching step planner of libpkv, over the block allocator and
// its prefix cache.
//
// The pages fix the behaviour: after every decode step finished requests
// leave the batch at once and free their blocks, and waiting requests are
// brought in ([p2] §3.3); blocks are taken on demand in block-sized pieces
// ([p2] §3.2, §3.3); a capped pool makes requests wait instead of running
// the device out of memory ([p2] §5.2); a request reuses the cached blocks
// of a matching prefix and computes only the rest ([p2] §4.3). The policy
// (fixed here so results are reproducible):
//   - a request is its token list (prompt, then each generated token) and
//     `computed`, the tokens whose K/V are in the cache;
//   - a step plans, in order: (1) decode: every running request with no
//     chunk left and a pending newest token gets one slot, in admission
//     order; a refusal preempts the newest running request (its sequence is
//     freed, it goes back to the front of the queue and is recomputed
//     later), repeated until the slot is granted or the request itself
//     yielded; (2) admission: while fewer than max_running run, the first
//     waiting request starts from the prefix cache and reserves the rest of
//     its tokens, or stays first and admission stops; (3) prefill: running
//     requests with tokens left get chunks in admission order, at most
//     prefill_budget tokens in all;
//   - commit: each item that computed its request's newest token hands the
//     request its next token; a request with max_new generated tokens
//     inserts its computed tokens into the prefix cache and frees its
//     sequence; a request whose prompt is first computed inserts it.
#include <algorithm>
#include <deque>
#include <memory>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Request {
  int64_t id = 0;
  int32_t prompt_len = 0;
  int32_t max_new = 0;
  std::vector<int32_t> tokens;
  int32_t generated = 0;
  int64_t seq = 0;  // 0: none
  int32_t computed = 0;
  bool pending = false;           // a reservation still being computed in chunks
  std::vector<int32_t> pend_slots;  // slots of tokens pend_base .. tokens.size() - 1
  int32_t pend_base = 0;
  bool prompt_cached = false;
  int32_t state = PKV_REQ_WAITING;
};

}  // namespace

struct pkv_sched {
  pkv_pool* pool = nullptr;
  int32_t max_running = 0, prefill_budget = 0;
  std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
  std::deque<Request*> waiting;
  std::vector<Request*> running;
  int32_t n_finished = 0;
  // the last plan's items, for commit
  std::vector<pkv_step_item> last_items;
};

namespace {

int reserve(pkv_pool* pool, int64_t seq, int32_t n, std::vector<int32_t>& slots, std::vector<int32_t>& cow) {
  slots.assign(size_t(std::max(n, 1)), 0);
  int32_t pair[2];
  int32_t ncow = 0;
  int st = pkv_seq_reserve(pool, seq, n, slots.data(), pair, 1, &ncow);
  slots.resize(size_t(n));
  if (st == PKV_OK && ncow) cow.insert(cow.end(), pair, pair + 2);
  return st;
}

Request* preempt_newest(pkv_sched* s) {
  Request* v = s->running.back();
  s->running.pop_back();
  pkv_seq_free(s->pool, v->seq);
  v->seq = 0;
  v->computed = 0;
  v->pending = false;
  v->pend_slots.clear();
  v->state = PKV_REQ_WAITING;
  s->waiting.push_front(v);
  return v;
}

void advance(pkv_sched* s, Request* r, int32_t token, std::vector<int64_t>& done) {
  r->tokens.push_back(token);
  ++r->generated;
  if (r->generated >= r->max_new) {
    pkv_prefix_cache_insert(s->pool, r->seq, r->tokens.data(), r->computed, nullptr);
    pkv_seq_free(s->pool, r->seq);
    r->seq = 0;
    s->running.erase(std::find(s->running.begin(), s->running.end(), r));
    r->state = PKV_REQ_FINISHED;
    ++s->n_finished;
    done.push_back(r->id);
  }
}

}  // namespace

extern "C" {

int pkv_sched_create(pkv_pool* pool, int32_t max_running, int32_t prefill_budget, pkv_sched** out) {
  if (!pool || !out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (max_running < 1 || prefill_budget < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_running and prefill_budget must be >= 1");
  pkv_sched* s = new (std::nothrow) pkv_sched;
  if (!s) return pkv::fail(PKV_ERR_INVALID_ARG, "out of host memory");
  s->pool = pool;
  s->max_running = max_running;
  s->prefill_budget = prefill_budget;
  *out = s;
  return PKV_OK;
}

void pkv_sched_destroy(pkv_sched* s) { delete s; }

int pkv_sched_limits(int32_t max_running, int32_t prefill_budget, int32_t* max_items, int32_t* max_slots) {
  if (!max_items || !max_slots) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (max_running < 1 || prefill_budget < 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "max_running and prefill_budget must be >= 1");
  *max_items = max_running;                    // a running request has at most one item a step
  *max_slots = max_running + prefill_budget;  // one decode slot each, plus the chunks
  return PKV_OK;
}

int pkv_sched_submit(pkv_sched* s, int64_t req, const int32_t* prompt, int32_t n, int32_t max_new) {
  if (!s || !prompt) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (n < 1 || max_new < 1) return pkv::fail(PKV_ERR_INVALID_ARG, "need a prompt and max_new >= 1");
  if (s->reqs.count(req)) return pkv::fail(PKV_ERR_INVALID_ARG, "request %lld already submitted", (long long)req);
  // a request that cannot fit the whole pool would wait at the head of the queue forever
  const int64_t blocks = (int64_t(n) + max_new + PKV_BLOCK_TOKENS - 1) / PKV_BLOCK_TOKENS;
  if (blocks > pkv::pool_num_blocks(s->pool))
    return pkv::fail(PKV_ERR_INVALID_ARG, "request %lld needs %lld blocks, the pool has %d", (long long)req,
                     (long long)blocks, pkv::pool_num_blocks(s->pool));
  auto r = std::make_unique<Request>();
  r->id = req;
  r->prompt_len = n;
  r->max_new = max_new;
  r->tokens.assign(prompt, prompt + n);
  s->waiting.push_back(r.get());
  s->reqs.emplace(req, std::move(r));
  return PKV_OK;
}

int pkv_sched_step(pkv_sched* s, pkv_step_plan* p) {
  if (!s || !p) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  int32_t mi = 0, ms = 0;
  pkv_sched_limits(s->max_running, s->prefill_budget, &mi, &ms);
  if (!p->items || p->item_cap < mi || !p->slots || p->slot_cap < ms || !p->cow_pairs || p->cow_cap < mi ||
      !p->preempted || p->preempted_cap < mi || !p->admitted || !p->admitted_cached || p->admitted_cap < mi)
    return pkv::fail(PKV_ERR_INVALID_ARG, "plan arrays below the limits (%d items, %d slots)", mi, ms);
  std::vector<pkv_step_item> items;
  std::vector<int32_t> slots, cow, tmp;
  std::vector<int64_t> pre, adm;
  std::vector<int32_t> adm_hit;
  // 1. decode
  for (size_t i = 0; i < s->running.size();) {
    Request* r = s->running[i];
    if (r->pending || r->computed != int32_t(r->tokens.size()) - 1) {
      ++i;
      continue;
    }
    bool granted = false;
    for (;;) {
      const int st = reserve(s->pool, r->seq, 1, tmp, cow);
      if (st == PKV_OK) {
        granted = true;
        break;
      }
      if (st != PKV_ERR_NO_BLOCKS) return st;
      Request* v = preempt_newest(s);
      pre.push_back(v->id);
      if (v == r) break;
    }
    if (granted) {
      items.push_back({r->id, r->seq, PKV_STEP_DECODE, r->computed, 1, int32_t(slots.size()), 1});
      slots.push_back(tmp[0]);
      ++i;
    }
  }
  // 2. admission
  while (int32_t(s->running.size()) < s->max_running && !s->waiting.empty()) {
    Request* r = s->waiting.front();
    int64_t seq = 0;
    int32_t hit = 0;
    int st = pkv_seq_create_cached(s->pool, r->tokens.data(), int32_t(r->tokens.size()), &seq, &hit);
    if (st != PKV_OK) return st;
    std::vector<int32_t> rs;
    st = reserve(s->pool, seq, int32_t(r->tokens.size()) - hit, rs, cow);
    if (st == PKV_ERR_NO_BLOCKS) {
      pkv_seq_free(s->pool, seq);
      break;
    }
    if (st != PKV_OK) return st;
    s->waiting.pop_front();
    r->seq = seq;
    r->computed = hit;
    r->pending = true;
    r->pend_base = hit;
    r->pend_slots = std::move(rs);
    r->state = PKV_REQ_RUNNING;
    s->running.push_back(r);
    adm.push_back(r->id);
    adm_hit.push_back(hit);
  }
  // 3. prefill chunks
  int32_t budget = s->prefill_budget;
  for (Request* r : s->running) {
    if (budget == 0) break;
    if (!r->pending) continue;
    const int32_t n = int32_t(r->tokens.size());
    const int32_t c = std::min(n - r->computed, budget);
    const int32_t lo = r->computed - r->pend_base;
    items.push_back({r->id, r->seq, PKV_STEP_PREFILL, r->computed, c, int32_t(slots.size()),
                     r->computed + c == n ? 1 : 0});
    slots.insert(slots.end(), r->pend_slots.begin() + lo, r->pend_slots.begin() + lo + c);
    r->computed += c;
    budget -= c;
    if (r->computed == n) {
      r->pending = false;
      r->pend_slots.clear();
    }
  }
  if (int32_t(items.size()) > p->item_cap || int32_t(slots.size()) > p->slot_cap ||
      int32_t(cow.size()) > 2 * p->cow_cap || int32_t(pre.size()) > p->preempted_cap ||
      int32_t(adm.size()) > p->admitted_cap)
    return pkv::fail(PKV_ERR_REFCOUNT, "step plan exceeded its limits");
  std::copy(items.begin(), items.end(), p->items);
  std::copy(slots.begin(), slots.end(), p->slots);
  std::copy(cow.begin(), cow.end(), p->cow_pairs);
  std::copy(pre.begin(), pre.end(), p->preempted);
  std::copy(adm.begin(), adm.end(), p->admitted);
  std::copy(adm_hit.begin(), adm_hit.end(), p->admitted_cached);
  p->n_items = int32_t(items.size());
  p->n_slots = int32_t(slots.size());
  p->n_cow = int32_t(cow.size() / 2);
  p->n_preempted = int32_t(pre.size());
  p->n_admitted = int32_t(adm.size());
  s->last_items = std::move(items);
  return PKV_OK;
}

int pkv_sched_commit(pkv_sched* s, const int32_t* next_tokens, int32_t n, int64_t* finished, int32_t fin_cap,
                     int32_t* n_finished) {
  if (!s || !n_finished || (n > 0 && !next_tokens)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  int32_t want = 0;
  for (const auto& it : s->last_items) want += it.completes;
  if (n != want) return pkv::fail(PKV_ERR_INVALID_ARG, "%d next tokens for %d completing items", n, want);
  if (want > 0 && (!finished || fin_cap < want))
    return pkv::fail(PKV_ERR_INVALID_ARG, "finished array below %d entries", want);
  std::vector<int64_t> done;
  int32_t k = 0;
  for (const auto& it : s->last_items) {
    Request* r = s->reqs.at(it.req).get();
    if (it.kind == PKV_STEP_DECODE) {
      ++r->computed;
      advance(s, r, next_tokens[k++], done);
    } else if (it.completes) {
      if (!r->prompt_cached) {
        pkv_prefix_cache_insert(s->pool, r->seq, r->tokens.data(), r->prompt_len, nullptr);
        r->prompt_cached = true;
      }
      advance(s, r, next_tokens[k++], done);
    }
  }
  s->last_items.clear();
  std::copy(done.begin(), done.end(), finished);
  *n_finished = int32_t(done.size());
  return PKV_OK;
}

int pkv_sched_request(const pkv_sched* s, int64_t req, int32_t* tokens, int32_t cap, int32_t* n_tokens,
                      int32_t* computed, int64_t* seq, int32_t* state) {
  if (!s || !n_tokens || !computed || !seq || !state) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  auto it = s->reqs.find(req);
  if (it == s->reqs.end()) return pkv::fail(PKV_ERR_INVALID_ARG, "unknown request %lld", (long long)req);
  const Request& r = *it->second;
  *n_tokens = int32_t(r.tokens.size());
  *computed = r.computed;
  *seq = r.seq;
  *state = r.state;
  if (tokens) {
    if (cap < *n_tokens) return pkv::fail(PKV_ERR_INVALID_ARG, "request has %d tokens, cap is %d", *n_tokens, cap);
    std::copy(r.tokens.begin(), r.tokens.end(), tokens);
  }
  return PKV_OK;
}

int pkv_sched_counts(const pkv_sched* s, int32_t* n_waiting, int32_t* n_running, int32_t* n_finished) {
  if (!s || !n_waiting || !n_running || !n_finished) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *n_waiting = int32_t(s->waiting.size());
  *n_running = int32_t(s->running.size());
  *n_finished = s->n_finished;
  return PKV_OK;
}

}  // extern "C"
