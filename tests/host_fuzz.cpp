// Random operation sequences against the host side of libpkv (allocator,
// copy-on-write, block tables, prefix cache, shared-prefix planner and the
// batching planner), for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer. Test infrastructure: every call's status is
// checked against the documented contract and the pool's block accounting
// (free blocks + distinct referenced blocks = pool size) after every step.
// Exit status 0 = all checks held and the sanitizers reported nothing.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

namespace {

int fails = 0;
// how often the interesting paths ran (reported; the test requires each)
long n_cache_hits = 0, n_cow = 0, n_no_blocks = 0, n_evicted = 0, n_groups = 0, n_finished = 0, n_preempted = 0;
#define CHECK(c)                                                                  \
  do {                                                                            \
    if (!(c)) {                                                                   \
      std::fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c,   \
                   pkv_last_error());                                            \
      ++fails;                                                                    \
    }                                                                             \
  } while (0)

struct Live {
  int64_t id;
  std::vector<int32_t> tokens;  // token ids it holds, for the prefix cache
};

// free blocks + blocks referenced by any live sequence or the cache == N
void check_accounting(pkv_pool* pool, const std::vector<Live>& live, int N) {
  int32_t nfree = -1;
  CHECK(pkv_num_free(pool, &nfree) == PKV_OK);
  std::vector<int32_t> fl(N);
  int32_t nf2 = -1;
  CHECK(pkv_free_list(pool, fl.data(), N, &nf2) == PKV_OK);
  CHECK(nf2 == nfree);
  std::set<int32_t> freeset(fl.begin(), fl.begin() + std::max(0, nf2));
  CHECK(int(freeset.size()) == nf2);  // no block listed twice
  int used = 0;
  for (int b = 0; b < N; ++b) {
    int32_t ref = -1;
    CHECK(pkv_block_refcount(pool, b, &ref) == PKV_OK);
    CHECK(ref >= 0);
    if (ref > 0) {
      ++used;
      CHECK(!freeset.count(b));
    }
  }
  CHECK(used + nfree == N);
  for (const Live& s : live) {
    int32_t len = -1, n = -1;
    CHECK(pkv_seq_len(pool, s.id, &len) == PKV_OK);
    CHECK(len == int32_t(s.tokens.size()));
    std::vector<int32_t> tab(N);
    CHECK(pkv_seq_block_table(pool, s.id, tab.data(), N, &n) == PKV_OK);
    CHECK(n == (len + 15) / 16);
    for (int j = 0; j < n; ++j) {
      int32_t ref = 0;
      CHECK(tab[j] >= 0 && tab[j] < N);
      CHECK(pkv_block_refcount(pool, tab[j], &ref) == PKV_OK && ref >= 1);
    }
  }
}

// a prompt: one of four shared bases (so cached blocks match) + a random tail
std::vector<int32_t> make_prompt(std::mt19937& rng, int max_tail) {
  static const int base_len[4] = {0, 20, 48, 80};
  const int which = int(rng() % 4);
  std::vector<int32_t> p;
  for (int i = 0; i < base_len[which]; ++i) p.push_back(int32_t((i * 7 + which) % 5));
  const int tail = 1 + int(rng() % unsigned(max_tail));
  for (int i = 0; i < tail; ++i) p.push_back(int32_t(rng() % 5));
  return p;
}

void allocator_round(std::mt19937& rng, int N) {
  pkv_config cfg = {1, N, 16, 2, 64, PKV_F16};
  std::vector<int32_t> order(N);
  for (int i = 0; i < N; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_pool* pool = nullptr;
  CHECK(pkv_pool_create(&cfg, order.data(), N, &pool) == PKV_OK);
  std::vector<Live> live;
  std::vector<int32_t> slots(4096), cow(2 * 64);
  for (int op = 0; op < 600; ++op) {
    const int kind = int(rng() % 10);
    if (kind <= 1 || live.empty()) {  // new sequence, maybe from the prefix cache
      const std::vector<int32_t> prompt = make_prompt(rng, 30);
      Live s;
      int32_t cached = -1;
      const int st = pkv_seq_create_cached(pool, prompt.data(), int32_t(prompt.size()), &s.id, &cached);
      CHECK(st == PKV_OK);
      if (st != PKV_OK) continue;
      CHECK(cached >= 0 && cached % 16 == 0 && cached <= int32_t(prompt.size()) - 1);
      n_cache_hits += cached > 0;
      s.tokens.assign(prompt.begin(), prompt.begin() + cached);
      const int rest = int(prompt.size()) - cached;
      int32_t ncow = 0;
      const int rs = pkv_seq_reserve(pool, s.id, rest, slots.data(), cow.data(), 64, &ncow);
      CHECK(rs == PKV_OK || rs == PKV_ERR_NO_BLOCKS);
      n_no_blocks += rs == PKV_ERR_NO_BLOCKS;
      if (rs == PKV_OK) s.tokens.assign(prompt.begin(), prompt.end());
      live.push_back(s);
    } else if (kind <= 4) {  // grow a sequence
      Live& s = live[rng() % live.size()];
      const int n = 1 + int(rng() % 40);
      int32_t ncow = -1;
      const int rs = pkv_seq_reserve(pool, s.id, n, slots.data(), cow.data(), 64, &ncow);
      CHECK(rs == PKV_OK || rs == PKV_ERR_NO_BLOCKS);
      n_no_blocks += rs == PKV_ERR_NO_BLOCKS;
      if (rs == PKV_OK) {
        CHECK(ncow >= 0 && ncow <= 1);
        n_cow += ncow;
        for (int i = 0; i < n; ++i) {
          CHECK(slots[i] >= 0 && slots[i] < N * 16);
          s.tokens.push_back(int32_t(rng() % 3));
        }
      }
    } else if (kind == 5) {  // fork
      Live& p = live[rng() % live.size()];
      Live c;
      CHECK(pkv_seq_fork(pool, p.id, &c.id) == PKV_OK);
      c.tokens = p.tokens;
      live.push_back(c);
    } else if (kind == 6) {  // register a sequence's blocks in the prefix cache
      Live& s = live[rng() % live.size()];
      int32_t added = -1;
      CHECK(pkv_prefix_cache_insert(pool, s.id, s.tokens.data(), int32_t(s.tokens.size()), &added) == PKV_OK);
      CHECK(added >= 0);
    } else if (kind == 7) {  // evict
      std::vector<int32_t> ev(8);
      int32_t nev = -1;
      CHECK(pkv_prefix_cache_evict(pool, 8, ev.data(), &nev) == PKV_OK);
      CHECK(nev >= 0 && nev <= 8);
      n_evicted += nev;
    } else if (kind == 8) {  // tables and a shared-prefix plan over a random batch
      std::vector<size_t> pick(live.size());
      for (size_t i = 0; i < pick.size(); ++i) pick[i] = i;
      std::shuffle(pick.begin(), pick.end(), rng);  // distinct sequences in a random order
      const int B = 1 + int(rng() % std::min<size_t>(live.size(), 40));
      std::vector<int64_t> ids(B);
      int max_blocks = 1;
      for (int b = 0; b < B; ++b) {
        ids[b] = live[pick[b]].id;
        int32_t len = 0;
        pkv_seq_len(pool, ids[b], &len);
        max_blocks = std::max(max_blocks, (len + 15) / 16);
      }
      std::vector<int32_t> tab(size_t(B) * max_blocks), lens(B);
      CHECK(pkv_build_block_tables(pool, ids.data(), B, max_blocks, tab.data(), lens.data()) == PKV_OK);
      const int32_t cap = pkv_plan_ints(B);
      std::vector<int32_t> plan(cap);
      int32_t ng = -1;
      CHECK(pkv_plan_shared_prefix(pool, ids.data(), B, 1, PKV_MAX_SHARERS, plan.data(), cap, &ng) == PKV_OK);
      CHECK(ng >= 0 && ng <= B / 2);
      n_groups += ng;
    } else {  // free
      const size_t i = rng() % live.size();
      CHECK(pkv_seq_free(pool, live[i].id) == PKV_OK);
      live.erase(live.begin() + long(i));
    }
    check_accounting(pool, live, N);
  }
  // error paths leave the pool as it was
  CHECK(pkv_seq_free(pool, 1 << 30) == PKV_ERR_UNKNOWN_SEQ);
  int32_t ref = 0;
  CHECK(pkv_block_refcount(pool, N, &ref) == PKV_ERR_INVALID_ARG);
  check_accounting(pool, live, N);
  for (const Live& s : live) CHECK(pkv_seq_free(pool, s.id) == PKV_OK);
  live.clear();
  check_accounting(pool, live, N);
  pkv_pool_destroy(pool);
}

void sched_round(std::mt19937& rng, int N) {
  pkv_config cfg = {1, N, 16, 2, 64, PKV_F16};
  pkv_pool* pool = nullptr;
  CHECK(pkv_pool_create(&cfg, nullptr, 0, &pool) == PKV_OK);
  const int max_running = 1 + int(rng() % 12), budget = 16 + int(rng() % 200);
  pkv_sched* sched = nullptr;
  CHECK(pkv_sched_create(pool, max_running, budget, &sched) == PKV_OK);
  int32_t max_items = 0, max_slots = 0;
  CHECK(pkv_sched_limits(max_running, budget, &max_items, &max_slots) == PKV_OK);
  std::vector<pkv_step_item> items(max_items);
  std::vector<int32_t> slots(max_slots), cowp(2 * size_t(max_items));
  std::vector<int64_t> pre(max_items), adm(max_items), fin(max_items);
  std::vector<int32_t> admc(max_items), next(max_items);
  pkv_step_plan plan;
  std::memset(&plan, 0, sizeof(plan));
  plan.items = items.data();
  plan.item_cap = max_items;
  plan.slots = slots.data();
  plan.slot_cap = max_slots;
  plan.cow_pairs = cowp.data();
  plan.cow_cap = max_items;
  plan.preempted = pre.data();
  plan.preempted_cap = max_items;
  plan.admitted = adm.data();
  plan.admitted_cached = admc.data();
  plan.admitted_cap = max_items;
  const int nreq = 4 + int(rng() % 30);
  for (int r = 0; r < nreq; ++r) {
    const std::vector<int32_t> prompt = make_prompt(rng, 60);
    const int st = pkv_sched_submit(sched, r, prompt.data(), int32_t(prompt.size()), 1 + int(rng() % 40));
    CHECK(st == PKV_OK || st == PKV_ERR_INVALID_ARG);
  }
  int32_t waiting = 0, running = 0, finished = 0;
  for (int step = 0; step < 5000; ++step) {
    CHECK(pkv_sched_counts(sched, &waiting, &running, &finished) == PKV_OK);
    if (waiting + running == 0) break;
    CHECK(pkv_sched_step(sched, &plan) == PKV_OK);
    int completing = 0;
    for (int i = 0; i < plan.n_items; ++i) {
      CHECK(plan.items[i].slot_index >= 0 && plan.items[i].slot_index + plan.items[i].count <= plan.n_slots);
      completing += plan.items[i].completes ? 1 : 0;
    }
    for (int i = 0; i < completing; ++i) next[i] = int32_t(rng() % 4);
    int32_t nfin = -1;
    CHECK(pkv_sched_commit(sched, next.data(), completing, fin.data(), max_items, &nfin) == PKV_OK);
    CHECK(nfin >= 0 && nfin <= completing);
    n_finished += nfin;
    n_preempted += plan.n_preempted;
  }
  CHECK(pkv_sched_counts(sched, &waiting, &running, &finished) == PKV_OK);
  CHECK(waiting + running == 0);
  pkv_sched_destroy(sched);
  pkv_pool_destroy(pool);
}

}  // namespace

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? unsigned(std::atoi(argv[1])) : 1u;
  std::mt19937 rng(seed);
  for (int round = 0; round < 6; ++round) {
    allocator_round(rng, 48 + int(rng() % 200));
    sched_round(rng, 12 + int(rng() % 60));
  }
  std::printf("host fuzz seed %u: %d failed checks; cache hits %ld, copy-on-write %ld, refused %ld, "
              "evicted %ld, plan groups %ld, finished %ld, preempted %ld\n",
              seed, fails, n_cache_hits, n_cow, n_no_blocks, n_evicted, n_groups, n_finished, n_preempted);
  return fails == 0 ? 0 : 1;
}
