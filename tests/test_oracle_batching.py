"""Pins of the oracle's continuous-batching step loop: a hand trace,
invariants and liveness on random workloads, admission as soon as a
request finishes, recompute preemption that leaves every request's tokens
unchanged, and prefix reuse on admission."""

import random

import pytest

import oracle
from oracle import RefPrefixCache, RefScheduler
from test_oracle_prefix_cache import check_invariants


def next_token(rid, tokens):
    """A stand-in for sampling: depends only on the request and its tokens."""
    return (7 * rid + 3 * len(tokens) + tokens[-1]) % 50


def run(sched, max_steps=500, check=None):
    plans = []
    for _ in range(max_steps):
        if not sched.running and not sched.waiting:
            break
        plan = sched.step()
        toks = {}
        for rid, *_ in plan["decode"]:
            toks[rid] = next_token(rid, sched.requests[rid].tokens)
        for rid, seq, start, count, slots, cow in plan["prefill"]:
            r = sched.requests[rid]
            if start + count == len(r.tokens):
                toks[rid] = next_token(rid, r.tokens)
        plan["finished"] = sched.commit(plan, toks)
        plans.append(plan)
        if check:
            check(sched, plan)
    return plans


def test_hand_trace():
    c = RefPrefixCache(8)
    s = RefScheduler(c, max_running=2, prefill_budget=20)
    s.submit(1, list(range(20)), 3)  # 2 blocks for the prompt
    s.submit(2, list(range(100, 120)), 4)
    s.submit(3, list(range(200, 210)), 1)
    p = s.step()
    assert p["admitted"] == [(1, 0), (2, 0)] and p["decode"] == []
    assert [(rid, start, count) for rid, _, start, count, _, _ in p["prefill"]] == [(1, 0, 20)]  # budget 20
    assert s.commit(p, {1: 5}) == []
    p = s.step()
    assert [rid for rid, *_ in p["decode"]] == [1] and p["admitted"] == []
    assert [(rid, start, count) for rid, _, start, count, _, _ in p["prefill"]] == [(2, 0, 20)]
    assert s.commit(p, {1: 6, 2: 7}) == []
    p = s.step()
    assert [rid for rid, *_ in p["decode"]] == [1, 2]
    assert s.commit(p, {1: 8, 2: 9}) == [1]  # 1 has its 3 tokens and leaves at once
    assert s.requests[1].tokens == list(range(20)) + [5, 6, 8]
    # 3 takes the free place while 2 is still decoding
    p = s.step()
    assert [rid for rid, *_ in p["decode"]] == [2] and p["admitted"] == [(3, 0)]
    assert [(rid, start, count) for rid, _, start, count, _, _ in p["prefill"]] == [(3, 0, 10)]
    assert s.commit(p, {2: 10, 3: 1}) == [3]
    p = s.step()
    assert s.commit(p, {2: 11}) == [2]
    assert s.requests[2].tokens == list(range(100, 120)) + [7, 9, 10, 11]
    assert not s.running and not s.waiting


def invariant_check(max_running, budget):
    def check(sched, plan):
        assert len(sched.running) <= max_running
        assert sum(count for _, _, _, count, _, _ in plan["prefill"]) <= budget
        check_invariants(sched.cache)
        for r in sched.running:
            # after commit: a request still computing chunks holds slots for all its
            # tokens; any other holds exactly its computed tokens, the newest one pending
            if r.pending is not None:
                assert sched.cache.lens[r.seq] == len(r.tokens)
            else:
                assert sched.cache.lens[r.seq] == r.computed == len(r.tokens) - 1
        # every live sequence belongs to a running request
        assert sorted(sched.cache.tables) == sorted(r.seq for r in sched.running)
    return check


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_workloads_finish_and_keep_invariants(seed):
    rng = random.Random(seed)
    c = RefPrefixCache(40)
    s = RefScheduler(c, max_running=4, prefill_budget=48)
    systems = [[1000 * k + i for i in range(rng.choice([16, 32, 40]))] for k in range(3)]
    for rid in range(1, 25):
        prompt = rng.choice(systems) + [rng.randint(0, 9) for _ in range(rng.randint(1, 40))]
        s.submit(rid, prompt, rng.randint(1, 30))
    plans = run(s, check=invariant_check(4, 48))
    assert sorted(s.finished) == list(range(1, 25))
    for rid, r in s.requests.items():
        assert r.generated == r.max_new and len(r.tokens) == len(r.prompt) + r.max_new
    assert any(hit > 0 for p in plans for _, hit in p["admitted"])  # system prompts were reused
    assert c.num_free() + c.reclaimable() == 40  # everything is back or only cached


def test_preemption_recomputes_and_keeps_the_tokens():
    def workload(N):
        c = RefPrefixCache(N)
        s = RefScheduler(c, max_running=3, prefill_budget=64)
        for rid in range(1, 4):
            s.submit(rid, [rid * 100 + i for i in range(30)], 60)
        return s

    free = workload(100)
    run(free)
    tight = workload(12)  # three requests of 90 tokens (6 blocks each) cannot all grow at once
    plans = run(tight)
    first = next(p["preempted"] for p in plans if p["preempted"])
    assert first[0] == 3  # the newest running request yields
    assert sorted(tight.finished) == [1, 2, 3]
    for rid in (1, 2, 3):
        assert tight.requests[rid].tokens == free.requests[rid].tokens


def test_prefix_reuse_on_admission():
    c = RefPrefixCache(20)
    s = RefScheduler(c, max_running=1, prefill_budget=100)
    system = list(range(48))
    s.submit(1, system + [1, 2, 3], 2)
    s.submit(2, system + [4, 5], 1)
    plans = run(s)
    admitted = [a for p in plans for a in p["admitted"]]
    assert admitted == [(1, 0), (2, 48)]
    # request 2 computed only its own two tokens
    assert [(rid, start, count) for p in plans for rid, _, start, count, _, _ in p["prefill"] if rid == 2] == [(2, 48, 2)]


def test_bad_arguments():
    c = RefPrefixCache(4)
    with pytest.raises(ValueError):
        RefScheduler(c, 0, 10)
    s = RefScheduler(c, 1, 10)
    s.submit(1, [1], 1)
    with pytest.raises(ValueError):
        s.submit(1, [2], 1)
    with pytest.raises(ValueError):
        s.submit(2, [], 1)
