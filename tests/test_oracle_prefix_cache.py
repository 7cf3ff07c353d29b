"""Pins of the oracle's prefix cache: a hand-traced scenario, invariants
after every operation of random programs, brute-force lookup and eviction
choices computed independently of the cache's own indexes, and the
all-or-nothing reservation under pressure."""

import copy
import random

import numpy as np
import pytest

import oracle
from oracle import RefPrefixCache, NoBlocks

BT = 16


def toks(*runs):
    """Token ids from (start, count) runs."""
    out = []
    for start, count in runs:
        out += list(range(start, start + count))
    return out


def check_invariants(c):
    held = {}
    for sid, table in c.tables.items():
        assert len(table) == -(-c.lens[sid] // BT)
        for j, b in enumerate(table):
            held[b] = held.get(b, 0) + 1
            # a sequence holding a cached block holds its predecessor just before it
            if b in c.entries:
                pred = c.entries[b][0]
                assert pred == (table[j - 1] if j else -1) or c.entries.get(table[j - 1] if j else -1) is None
    for b in range(c.num_blocks):
        assert c.ref[b] == held.get(b, 0) + (1 if b in c.entries else 0), b
    assert sorted(c.free) == sorted(b for b in range(c.num_blocks) if c.ref[b] == 0)
    kids = {}
    for b, (pred, ids) in c.entries.items():
        assert len(ids) == BT
        assert pred == -1 or pred in c.entries
        if pred >= 0:
            kids[pred] = kids.get(pred, 0) + 1
        assert c.by_content[(pred, ids)] == b
    assert len(c.by_content) == len(c.entries)
    for b in c.entries:
        assert c.children.get(b, 0) == kids.get(b, 0)
        # marked after every block that follows it
        for f, (pred, _) in c.entries.items():
            if pred == b:
                assert c.used[b] > c.used[f]


def brute_lookup(c, tokens):
    """Longest chain of cached blocks matching the prompt, from the entries
    alone (a scan, no content index)."""
    chain, pred = [], -1
    for j in range((len(tokens) - 1) // BT if tokens else 0):
        ids = tuple(tokens[j * BT:(j + 1) * BT])
        nxt = [b for b, (p, i) in c.entries.items() if p == pred and i == ids]
        if not nxt:
            break
        assert len(nxt) == 1
        chain.append(nxt[0])
        pred = nxt[0]
    return chain


def test_hand_traced_scenario():
    c = RefPrefixCache(8)
    a, hit = c.seq_create_cached(toks((0, 40)))
    assert hit == 0
    slots, _ = c.seq_reserve(a, 40)
    assert c.tables[a] == [0, 1, 2]
    assert c.insert(a, toks((0, 40))) == 2  # blocks 0 and 1 are full; 2 holds 8 tokens
    assert c.entries[0] == (-1, tuple(range(16))) and c.entries[1] == (0, tuple(range(16, 32)))
    assert c.ref[:3] == [2, 2, 1]
    c.seq_free(a)
    assert c.ref[:3] == [1, 1, 0] and c.free_list()[0] == 2
    # same first 32 tokens, then different: both cached blocks are reused
    b, hit = c.seq_create_cached(toks((0, 32), (900, 13)))
    assert hit == 32 and c.tables[b] == [0, 1] and c.ref[:2] == [2, 2]
    c.seq_reserve(b, 13)
    assert c.tables[b] == [0, 1, 2]
    # a prompt of exactly 32 tokens takes only one block: its last token is computed
    d, hit = c.seq_create_cached(toks((0, 32)))
    assert hit == 16 and c.tables[d] == [0]
    # same second block content after a different first block: no match
    e, hit = c.seq_create_cached(toks((500, 16), (16, 16), (0, 5)))
    assert hit == 0
    check_invariants(c)
    # pressure: 8 blocks; 0, 1 held by b and d; block 2 by b; free 3..7
    c.seq_free(b)
    c.seq_free(d)
    assert c.reclaimable() == 2 and c.num_free() == 6
    f, _ = c.seq_create_cached([7] * 129)  # needs 9 blocks: 6 free + 2 reclaimable are too few
    before = copy.deepcopy(c.__dict__)
    with pytest.raises(NoBlocks):
        c.seq_reserve(f, 129)
    assert c.__dict__ == before
    c.seq_reserve(f, 113)  # 8 blocks: both cached blocks are evicted, follower first
    assert not c.entries and c.num_free() == 0
    # block 1 went back to the free stack first, then 0: the stack hands out 0, 1, then 2..7
    assert c.tables[f] == [0, 1, 2, 3, 4, 5, 6, 7]
    check_invariants(c)


def random_program(seed, steps=300, N=24):
    rng = random.Random(seed)
    c = RefPrefixCache(N, list(np.random.default_rng(seed).permutation(N)))
    prompts = [toks((1000 * k, 16 * rng.randint(1, 4))) for k in range(4)]
    live = {}
    log = []
    for _ in range(steps):
        op = rng.random()
        if op < 0.35:
            base = rng.choice(prompts)
            tail = [rng.randint(0, 3) for _ in range(rng.randint(0, 40))]
            cut = rng.randint(0, len(base))
            tokens = base[:cut] + tail
            if not tokens:
                tokens = [1]
            expect = brute_lookup(c, tokens)
            sid, hit = c.seq_create_cached(tokens)
            assert c.tables[sid] == expect and hit == BT * len(expect)
            try:
                c.seq_reserve(sid, len(tokens) - hit)
                live[sid] = tokens
                log.append(("admit", sid, hit))
            except NoBlocks:
                c.seq_free(sid)
                log.append(("refused",))
        elif op < 0.6 and live:
            sid = rng.choice(sorted(live))
            c.insert(sid, live[sid])
        elif op < 0.75 and live:
            sid = rng.choice(sorted(live))
            try:
                c.seq_reserve(sid, rng.randint(1, 20))
                live[sid] = live[sid] + [rng.randint(0, 3) for _ in range(c.lens[sid] - len(live[sid]))]
            except NoBlocks:
                pass
        elif op < 0.9 and live:
            sid = rng.choice(sorted(live))
            c.seq_free(sid)
            del live[sid]
        else:
            want = rng.randint(1, 4)
            cands = sorted((c.used[b], b) for b in c.entries if c.ref[b] == 1 and c.children.get(b, 0) == 0)
            got = c.evict(want)
            if got:
                assert got[0] == cands[0][1]  # least recently used evictable block first
        check_invariants(c)
    return c, log


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_random_programs_keep_invariants(seed):
    c, log = random_program(seed)
    assert any(e[0] == "admit" and e[2] > 0 for e in log)  # the cache was hit


def test_reserve_evicts_just_enough_least_recent_first():
    c = RefPrefixCache(6)
    for k in range(3):
        s, _ = c.seq_create_cached(toks((100 * k, 17)))
        c.seq_reserve(s, 17)
        c.insert(s, toks((100 * k, 17)))
        c.seq_free(s)
    # each prompt's partial block went back to the free stack and was taken
    # again first: cached blocks 0, 1, 2 (used in that order), three free
    assert sorted(c.entries) == [0, 1, 2] and c.num_free() == 3
    s, _ = c.seq_create_cached([9] * 70)
    c.seq_reserve(s, 70)  # 5 blocks: 3 free + the two least recently used
    assert sorted(c.entries) == [2]
    check_invariants(c)


def test_lookup_hit_marks_the_chain_used():
    c = RefPrefixCache(6)
    for k in range(2):
        s, _ = c.seq_create_cached(toks((100 * k, 17)))
        c.seq_reserve(s, 17)
        c.insert(s, toks((100 * k, 17)))
        c.seq_free(s)
    s, hit = c.seq_create_cached(toks((0, 20)))  # hit the older one (block 0)
    assert hit == 16
    c.seq_free(s)
    assert c.evict(1) == [1]  # the other one is now the least recently used
