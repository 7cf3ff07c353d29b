"""Planted mistakes: each test puts one plausible bug into the oracle (on the
CPU, through monkeypatch) and checks that at least one pin catches it. This
shows the pins constrain every part of the oracle, not only its happy path."""

import math

import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.allocator as alc
import oracle.quant as qnt
import oracle.sizes as sz
import workloads
from test_oracle_allocator import hand_trace, random_ops, check_invariants
from test_oracle_decode import (check_against_brute, check_against_sdpa,
                                check_gather_matches_contiguous,
                                test_shared_prefix_equals_private_copy)
from test_oracle_quant import check_error_bound
from test_oracle_sizes import check_printed_sizes


def _decode_with(mapping=None, scale_override=None, sign=1.0, swap_kv=False):
    def decode(cache, q, block_tables, context_lens, layer=0, scale=None):
        q = np.asarray(q)
        B, Hq, D = q.shape
        Hkv = cache.kv_heads
        G = Hq // Hkv
        sc = 1.0 / math.sqrt(D) if scale is None else scale
        if scale_override is not None:
            sc = scale_override
        out = np.empty((B, Hq, D))
        for b in range(B):
            n = int(context_lens[b])
            for h in range(Hq):
                g = mapping(h, G, Hkv) if mapping else h // G
                Kc = att.gather(cache.K, layer, block_tables[b], n, g, cache.scales, 0)
                Vc = att.gather(cache.V, layer, block_tables[b], n, g, cache.scales, 1)
                if swap_kv:
                    Kc, Vc = Vc, Kc
                s = sign * (Kc @ q[b, h].astype(np.float64)) * sc
                e = np.exp(s - s.max())
                out[b, h] = (e / e.sum()) @ Vc
        return out
    return decode


def test_interleaved_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "decode", _decode_with(mapping=lambda h, G, Hkv: h % Hkv))
    with pytest.raises(AssertionError):
        check_against_sdpa(workloads.c1_tiny())


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "decode", _decode_with(scale_override=1.0))
    with pytest.raises(AssertionError):
        check_against_brute(workloads.c1_tiny())


def test_sign_flip_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "decode", _decode_with(sign=-1.0))
    with pytest.raises(AssertionError):
        check_against_brute(workloads.c1_tiny())


def test_swapped_k_and_v_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "decode", _decode_with(swap_kv=True))
    with pytest.raises(AssertionError):
        check_against_brute(workloads.c1_tiny())


def test_gather_off_by_one_is_caught(monkeypatch):
    real = att.gather

    def shifted(store, layer, table, n, g, scales=None, which=0):
        rows = real(store, layer, table, n + 1 if n % 16 else n, g, scales, which)
        return rows[1:n + 1] if len(rows) > n else np.roll(rows, 1, axis=0)

    monkeypatch.setattr(oracle, "gather", shifted)
    with pytest.raises(AssertionError):
        check_gather_matches_contiguous(0)


def test_fifo_free_list_is_caught(monkeypatch):
    def seq_free(self, sid):
        self._check(sid)
        for blk in reversed(self.tables[sid]):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.insert(0, blk)
        del self.tables[sid]
        del self.lens[sid]

    monkeypatch.setattr(alc.RefAllocator, "seq_free", seq_free)
    with pytest.raises(AssertionError):
        hand_trace()


def test_missing_copy_on_write_is_caught(monkeypatch):
    def seq_reserve(self, sid, n):
        self._check(sid)
        table, length = self.tables[sid], self.lens[sid]
        need = sum(1 for pos in range(length, length + n) if pos % 16 == 0)
        if need > len(self.free):
            raise oracle.NoBlocks(sid)
        slots = []
        for pos in range(length, length + n):
            lblk, off = divmod(pos, 16)
            if off == 0:
                blk = self.free.pop()
                self.ref[blk] = 1
                table.append(blk)
            slots.append(table[lblk] * 16 + off)
        self.lens[sid] = length + n
        return slots, []

    monkeypatch.setattr(alc.RefAllocator, "seq_reserve", seq_reserve)
    with pytest.raises(AssertionError):
        test_shared_prefix_equals_private_copy()
    with pytest.raises(AssertionError):
        hand_trace()


def test_leaked_block_on_free_is_caught(monkeypatch):
    def seq_free(self, sid):
        self._check(sid)
        for blk in reversed(self.tables[sid][1:]):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
        del self.tables[sid]
        del self.lens[sid]

    monkeypatch.setattr(alc.RefAllocator, "seq_free", seq_free)
    with pytest.raises(AssertionError):
        random_ops(oracle.RefAllocator(12, np.arange(12)), np.random.default_rng(1), 100)


def test_floor_quantiser_is_caught(monkeypatch):
    monkeypatch.setattr(qnt.np, "rint", np.floor)
    with pytest.raises(AssertionError):
        check_error_bound(1)


def test_size_formula_without_factor_two_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "kv_cache_bytes",
                        lambda L, H, D, E, n, B=1: L * H * D * E * n * B)
    with pytest.raises(AssertionError):
        check_printed_sizes(__import__("os").path.join(__import__("os").path.dirname(__file__), "golden"))


def test_append_without_requantising_is_caught(monkeypatch):
    """A quantise-on-write that raises the scale but keeps the old codes
    breaks the bound on earlier rows."""
    from test_oracle_quant import test_append_beyond_range_requantises_the_block

    real = qnt.append_row_int8

    def lazy(codes, scale, off, x):
        new_codes, new_scale = real(codes, scale, off, x)
        new_codes[:off] = np.asarray(codes)[:off]
        return new_codes, new_scale

    monkeypatch.setattr(oracle, "append_row_int8", lazy)
    with pytest.raises(AssertionError):
        test_append_beyond_range_requantises_the_block()


def test_causal_off_by_one_is_caught(monkeypatch):
    """A prefill whose token does not see itself (positions < p instead of
    <= p) fails the SDPA pin."""
    from test_oracle_prefill import check_prefill_against_sdpa

    def prefill(cache, q, q_lens, block_tables, context_lens, layer=0, scale=None):
        q = np.asarray(q)
        T, Hq, D = q.shape
        G = Hq // cache.kv_heads
        sc = 1.0 / math.sqrt(D) if scale is None else scale
        out = np.zeros((T, Hq, D))
        row0 = 0
        for b, ql in enumerate(q_lens):
            n = int(context_lens[b])
            for g in range(cache.kv_heads):
                Kc = att.gather(cache.K, layer, block_tables[b], n, g)
                Vc = att.gather(cache.V, layer, block_tables[b], n, g)
                for i in range(ql):
                    p = n - ql + i
                    for h in range(g * G, (g + 1) * G):
                        s = (Kc[:max(p, 1)] @ q[row0 + i, h].astype(np.float64)) * sc
                        e = np.exp(s - s.max())
                        out[row0 + i, h] = (e / e.sum()) @ Vc[:max(p, 1)]
            row0 += ql
        return out

    monkeypatch.setattr(oracle, "prefill", prefill)
    with pytest.raises(AssertionError):
        check_prefill_against_sdpa(workloads.prefill_chunks(11, [5, 0], [12, 30], 8, 2, 64))


def test_prefill_grouping_mixup_is_caught(monkeypatch):
    """Interleaved head grouping in the prefill fails the SDPA pin."""
    from test_oracle_prefill import check_prefill_against_sdpa
    real = att.prefill

    def prefill(cache, q, q_lens, block_tables, context_lens, layer=0, scale=None):
        q = np.asarray(q)
        G = q.shape[1] // cache.kv_heads
        perm = [(h % cache.kv_heads) * G + h // cache.kv_heads for h in range(q.shape[1])]
        out = real(cache, q[:, perm], q_lens, block_tables, context_lens, layer, scale)
        inv = np.argsort(perm)
        return out[:, inv]

    monkeypatch.setattr(oracle, "prefill", prefill)
    with pytest.raises(AssertionError):
        check_prefill_against_sdpa(workloads.prefill_chunks(11, [5, 0], [12, 30], 8, 2, 64))


# ---------------------------------------------------------------------------
# prefix cache

def test_prefix_match_without_predecessor_is_caught(monkeypatch):
    """Matching a block by its ids alone would hand a request a block cached
    after a different predecessor; the brute-force lookup pin fails."""
    import oracle.prefix_cache as pcm
    from test_oracle_prefix_cache import brute_lookup, toks

    def create(self, tokens):
        tokens = [int(t) for t in tokens]
        sid = self.seq_create()
        chain = []
        for j in range(max(len(tokens) - 1, 0) // 16):
            ids = tuple(tokens[j * 16:(j + 1) * 16])
            hit = [b for b, (p, i) in self.entries.items() if i == ids]
            if not hit:
                break
            chain.append(hit[0])
        for b in chain:
            self.ref[b] += 1
        self.tables[sid] = chain
        self.lens[sid] = 16 * len(chain)
        return sid, self.lens[sid]

    monkeypatch.setattr(pcm.RefPrefixCache, "seq_create_cached", create)
    c = pcm.RefPrefixCache(8)
    a, _ = c.seq_create_cached(toks((0, 33)))
    c.seq_reserve(a, 33)
    c.insert(a, toks((0, 33)))
    prompt = toks((16, 16), (0, 5))  # the second block's ids, now in first position
    expect = brute_lookup(c, prompt)
    with pytest.raises(AssertionError):
        sid, hit = c.seq_create_cached(prompt)
        assert c.tables[sid] == expect


def test_prefix_lookup_taking_the_last_token_is_caught(monkeypatch):
    """Taking floor(n / 16) blocks leaves no token to compute for a prompt of
    whole blocks; the hand-traced scenario fails."""
    import oracle.prefix_cache as pcm
    from test_oracle_prefix_cache import test_hand_traced_scenario
    real = pcm.RefPrefixCache.seq_create_cached

    def create(self, tokens):
        return real(self, list(tokens) + [0])

    monkeypatch.setattr(pcm.RefPrefixCache, "seq_create_cached", create)
    with pytest.raises(AssertionError):
        test_hand_traced_scenario()


def test_eviction_of_a_block_with_followers_is_caught(monkeypatch):
    """Evicting the least recently used block even when cached blocks follow
    it leaves orphans; the invariants fail on a random program."""
    import oracle.prefix_cache as pcm
    from test_oracle_prefix_cache import random_program

    def evictable(self):
        return [b for b in self.entries if self.ref[b] == 1]

    def touch(self, chain):  # root first: predecessors become the older ones
        for blk in chain:
            self.tick += 1
            self.used[blk] = self.tick

    monkeypatch.setattr(pcm.RefPrefixCache, "_evictable", evictable)
    monkeypatch.setattr(pcm.RefPrefixCache, "_touch", touch)
    with pytest.raises((AssertionError, KeyError)):
        for seed in (1, 2, 3):
            random_program(seed)


# ---------------------------------------------------------------------------
# continuous batching

def test_static_batching_is_caught(monkeypatch):
    """Admitting only into an empty batch (wait for the whole batch to
    finish) fails the hand trace: request 3 must start as soon as 1 and 2
    have left."""
    import oracle.batching as bm
    from test_oracle_batching import test_hand_trace
    real = bm.RefScheduler.step

    # a batch that never takes new requests while any request runs
    def step_static(self):
        if self.running:
            saved = self.waiting
            self.waiting = bm.deque()
            try:
                return real(self)
            finally:
                self.waiting = saved
        return real(self)

    monkeypatch.setattr(bm.RefScheduler, "step", step_static)
    with pytest.raises(AssertionError):
        test_hand_trace()


def test_preempting_the_oldest_is_caught(monkeypatch):
    import oracle.batching as bm
    from test_oracle_batching import test_preemption_recomputes_and_keeps_the_tokens

    def preempt_oldest(self):
        v = self.running.pop(0)
        self.cache.seq_free(v.seq)
        v.seq, v.computed, v.pending = None, 0, None
        self.waiting.appendleft(v)
        return v

    monkeypatch.setattr(bm.RefScheduler, "_preempt_newest", preempt_oldest)
    with pytest.raises((AssertionError, KeyError, ValueError)):
        test_preemption_recomputes_and_keeps_the_tokens()


def test_finishing_without_freeing_is_caught(monkeypatch):
    import oracle.batching as bm
    from test_oracle_batching import test_random_workloads_finish_and_keep_invariants

    def advance(self, r, token, done):
        r.tokens.append(int(token))
        r.generated += 1
        if r.generated >= r.max_new:
            self.running.remove(r)  # leaves without releasing its sequence
            self.finished.append(r.rid)
            done.append(r.rid)

    monkeypatch.setattr(bm.RefScheduler, "_advance", advance)
    with pytest.raises(AssertionError):
        test_random_workloads_finish_and_keep_invariants(1)
