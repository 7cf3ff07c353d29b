"""Reference continuous-batching step loop over the reference prefix cache.
Test infrastructure only (see the package header).

What the pages fix: after every decode step the requests that finished
leave the batch at once and free their blocks, and waiting requests are
brought in ([p2] §3.3); blocks are taken on demand, a new request needs
only block-sized pieces ([p2] §3.2, §3.3); a capped pool makes requests
wait instead of running the device out of memory ([p2] §5.2); a request
reuses the cached blocks of a matching prefix and computes only the rest
([p2] §4.3).

Readings taken here (the plainest ones; each is pinned by a test):

* A request is its token list: the prompt, then each generated token. Its
  K/V are computed in order; ``computed`` counts the tokens whose K/V are in
  the cache.
* One step, in this order:
  1. decode: every running request with no chunk left to compute and whose
     newest token still needs its K/V gets one slot, in admission order. If
     the pool refuses, the newest running request is preempted: its
     sequence is freed and it goes back to the front of the queue, to be
     recomputed later (its cached prefix blocks may spare most of that);
     this repeats until the slot is granted or the request itself was the
     one preempted;
  2. admission: while fewer than ``max_running`` requests run, the first
     waiting request starts a sequence from the prefix cache and reserves
     slots for the rest of its tokens; if the pool refuses, it stays first in
     the queue and admission stops for this step;
  3. prefill: running requests with tokens left to compute get chunks in
     admission order, at most ``prefill_budget`` tokens per step in all.
* Commit, after the device work: each decoded request and each request
  whose last chunk completed its tokens receives its next token; a request
  with ``max_new`` generated tokens finishes, its computed tokens are
  inserted into the prefix cache and its sequence is freed. A request whose
  prompt is first computed inserts it into the prefix cache.
"""

from collections import deque

from .allocator import NoBlocks


class Request:
    def __init__(self, rid, prompt, max_new):
        self.rid = rid
        self.prompt = [int(t) for t in prompt]
        self.tokens = list(self.prompt)
        self.max_new = int(max_new)
        self.generated = 0
        self.seq = None
        self.computed = 0
        self.pending = None  # (first token, slots, cow pairs) of a reservation still being computed
        self.prompt_cached = False


class RefScheduler:
    def __init__(self, cache, max_running, prefill_budget):
        if max_running < 1 or prefill_budget < 1:
            raise ValueError("max_running and prefill_budget must be >= 1")
        self.cache = cache
        self.max_running = max_running
        self.prefill_budget = prefill_budget
        self.waiting = deque()
        self.running = []
        self.requests = {}
        self.finished = []

    def submit(self, rid, prompt, max_new):
        if rid in self.requests or not prompt or max_new < 1:
            raise ValueError("bad request")
        r = Request(rid, prompt, max_new)
        self.requests[rid] = r
        self.waiting.append(r)

    def _preempt_newest(self):
        v = self.running.pop()
        self.cache.seq_free(v.seq)
        v.seq, v.computed, v.pending = None, 0, None
        self.waiting.appendleft(v)
        return v

    def step(self):
        """Plan one step. Returns a dict of
        ``decode``: [(rid, seq, slot, cow_pairs)],
        ``prefill``: [(rid, seq, start, count, slots, cow_pairs)],
        ``preempted``: [rid], ``admitted``: [(rid, cached_tokens)]."""
        plan = {"decode": [], "prefill": [], "preempted": [], "admitted": []}
        # 1. decode
        i = 0
        while i < len(self.running):
            r = self.running[i]
            if r.pending is not None or r.computed != len(r.tokens) - 1:
                i += 1
                continue
            while True:
                try:
                    slots, cow = self.cache.seq_reserve(r.seq, 1)
                    plan["decode"].append((r.rid, r.seq, slots[0], cow))
                    break
                except NoBlocks:
                    v = self._preempt_newest()
                    plan["preempted"].append(v.rid)
                    if v is r:
                        break
            if r.seq is not None:
                i += 1
        # 2. admission
        while len(self.running) < self.max_running and self.waiting:
            r = self.waiting[0]
            seq, hit = self.cache.seq_create_cached(r.tokens)
            try:
                slots, cow = self.cache.seq_reserve(seq, len(r.tokens) - hit)
            except NoBlocks:
                self.cache.seq_free(seq)
                break
            self.waiting.popleft()
            r.seq, r.computed = seq, hit
            r.pending = (hit, slots, cow)
            self.running.append(r)
            plan["admitted"].append((r.rid, hit))
        # 3. prefill chunks
        budget = self.prefill_budget
        for r in self.running:
            if budget == 0:
                break
            if r.pending is None:
                continue
            base, slots, cow = r.pending
            c = min(len(r.tokens) - r.computed, budget)
            lo = r.computed - base
            plan["prefill"].append((r.rid, r.seq, r.computed, c, slots[lo:lo + c], cow if lo == 0 else []))
            r.computed += c
            budget -= c
            if r.computed == len(r.tokens):
                r.pending = None
        return plan

    def commit(self, plan, next_tokens):
        """``next_tokens[rid]`` for every request decoded this step and every
        request whose last chunk completed its tokens. Returns finished rids."""
        done = []
        for rid, seq, _slot, _cow in plan["decode"]:
            r = self.requests[rid]
            r.computed += 1
            self._advance(r, next_tokens[rid], done)
        for rid, seq, start, count, _slots, _cow in plan["prefill"]:
            r = self.requests[rid]
            if r.seq != seq or start + count != len(r.tokens):
                continue
            if not r.prompt_cached:
                self.cache.insert(r.seq, r.prompt)
                r.prompt_cached = True
            self._advance(r, next_tokens[rid], done)
        return done

    def _advance(self, r, token, done):
        r.tokens.append(int(token))
        r.generated += 1
        if r.generated >= r.max_new:
            self.cache.insert(r.seq, r.tokens[:r.computed])
            self.cache.seq_free(r.seq)
            self.running.remove(r)
            r.seq = None
            self.finished.append(r.rid)
            done.append(r.rid)
