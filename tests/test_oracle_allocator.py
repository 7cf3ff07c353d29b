"""Pins of the oracle allocator: a hand-traced example, invariants after every
operation, brute-force enumeration of short operation sequences, and the
exact-fit and all-or-nothing behaviour."""

import copy
import itertools

import numpy as np
import pytest

import oracle
from oracle.sizes import BLOCK_TOKENS


def snapshot(a):
    return (list(a.free), list(a.ref), copy.deepcopy(a.tables), dict(a.lens), a.next_id)


def check_invariants(a):
    """Properties the paging rules fix, whatever the free-list policy."""
    N = a.num_blocks
    used = set()
    count = [0] * N
    for sid, table in a.tables.items():
        # each sequence holds exactly as many blocks as its tokens need
        assert len(table) == -(-a.lens[sid] // BLOCK_TOKENS), sid
        assert len(set(table)) == len(table)
        for blk in table:
            count[blk] += 1
            used.add(blk)
    # the refcount of a block is the number of tables that point at it
    assert count == a.ref
    # free blocks carry no reference and appear once
    assert len(set(a.free)) == len(a.free)
    for blk in a.free:
        assert a.ref[blk] == 0
    # every block is either referenced or free
    assert len(used) + len(a.free) == N
    assert used.isdisjoint(a.free)


def hand_trace():
    """Worked by hand from the rules in the allocator's docstring."""
    a = oracle.RefAllocator(6, [3, 1, 4, 0, 5, 2])
    A = a.seq_create()
    assert A == 1
    slots, cow = a.seq_reserve(A, 20)
    assert slots == list(range(48, 64)) + [16, 17, 18, 19] and cow == []
    assert a.tables[A] == [3, 1]
    B = a.seq_create()
    slots, cow = a.seq_reserve(B, 5)
    assert slots == [64, 65, 66, 67, 68] and cow == []
    C = a.seq_fork(A)
    assert C == 3 and a.tables[C] == [3, 1] and a.lens[C] == 20
    assert a.ref[3] == 2 and a.ref[1] == 2
    # the child writes at offset 4 of the shared tail: copy-on-write
    slots, cow = a.seq_reserve(C, 1)
    assert cow == [(1, 0)] and slots == [4] and a.tables[C] == [3, 0]
    assert a.ref[1] == 1 and a.ref[0] == 1
    # the parent now owns its tail alone and writes in place
    slots, cow = a.seq_reserve(A, 1)
    assert cow == [] and slots == [20]
    a.seq_free(A)
    assert a.free_list() == [1, 5, 2]
    slots, cow = a.seq_reserve(B, 12)
    assert slots == list(range(69, 80)) + [16] and a.tables[B] == [4, 1]
    before = snapshot(a)
    with pytest.raises(oracle.NoBlocks):
        a.seq_reserve(B, 100)
    assert snapshot(a) == before
    a.seq_free(C)
    assert a.free_list() == [3, 0, 5, 2]
    a.seq_free(B)
    assert a.num_free() == 6
    return a


def test_hand_trace():
    hand_trace()


def random_ops(a, rng, steps):
    live = []
    for _ in range(steps):
        op = rng.integers(0, 5)
        if op == 0 or not live:
            live.append(a.seq_create())
        elif op == 1:
            sid = live[rng.integers(len(live))]
            n = int(rng.integers(0, 40))
            before = snapshot(a)
            try:
                slots, cow = a.seq_reserve(sid, n)
                assert len(slots) == n and len(cow) <= 1
            except oracle.NoBlocks:
                assert snapshot(a) == before
        elif op == 2:
            live.append(a.seq_fork(live[rng.integers(len(live))]))
        else:
            a.seq_free(live.pop(rng.integers(len(live))))
        check_invariants(a)
    for sid in live:
        a.seq_free(sid)
    check_invariants(a)
    # everything returns to the pool the moment its requests end
    assert a.num_free() == a.num_blocks


@pytest.mark.parametrize("seed", range(20))
def test_random_ops_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 24))
    random_ops(oracle.RefAllocator(N, rng.permutation(N)), rng, 200)


OPS = ["create", "r1", "r7", "r16", "fork", "free"]


def apply(a, live, op):
    if op == "create" or not live:
        live.append(a.seq_create())
        return
    if op == "fork":
        live.append(a.seq_fork(live[-1]))
    elif op == "free":
        a.seq_free(live.pop(0))
    else:
        n = int(op[1:])
        before = snapshot(a)
        try:
            a.seq_reserve(live[-1], n)
        except oracle.NoBlocks:
            assert snapshot(a) == before


@pytest.mark.parametrize("N", [1, 2, 3])
def test_brute_force_short_sequences(N):
    for length in range(1, 6):
        for ops in itertools.product(OPS, repeat=length):
            a = oracle.RefAllocator(N)
            live = []
            for op in ops:
                apply(a, live, op)
                check_invariants(a)


def test_slots_are_distinct_and_addressed_through_table():
    rng = np.random.default_rng(7)
    a = oracle.RefAllocator(40, rng.permutation(40))
    seen = set()
    sids = [a.seq_create() for _ in range(3)]
    for _ in range(30):
        sid = sids[rng.integers(3)]
        start = a.lens[sid]
        slots, cow = a.seq_reserve(sid, int(rng.integers(1, 9)))
        assert cow == []
        for i, slot in enumerate(slots):
            pos = start + i
            assert slot == a.tables[sid][pos // 16] * 16 + pos % 16
            assert slot not in seen
            seen.add(slot)


def test_exact_fit_pool_is_empty_after_append():
    # 8 sequences of 1024 tokens plus one appended token need 8 * 65 blocks
    a = oracle.RefAllocator(520, np.random.default_rng(2).permutation(520))
    sids = [a.seq_create() for _ in range(8)]
    for s in sids:
        a.seq_reserve(s, 1024)
    assert a.num_free() == 8
    for s in sids:
        a.seq_reserve(s, 1)
    assert a.num_free() == 0
    before = snapshot(a)
    with pytest.raises(oracle.NoBlocks):
        a.seq_reserve(sids[0], 16)
    # 15 more tokens still fit in the partly filled tail block
    a.seq_reserve(sids[0], 15)
    with pytest.raises(oracle.NoBlocks):
        a.seq_reserve(sids[0], 1)
    assert snapshot(a)[2][sids[1]] == before[2][sids[1]]


def test_unknown_sequence():
    a = oracle.RefAllocator(4)
    with pytest.raises(oracle.UnknownSeq):
        a.seq_reserve(5, 1)
    s = a.seq_create()
    a.seq_free(s)
    with pytest.raises(oracle.UnknownSeq):
        a.seq_free(s)
    with pytest.raises(oracle.UnknownSeq):
        a.seq_fork(s)


def test_full_shared_block_needs_no_copy():
    a = oracle.RefAllocator(8)
    p = a.seq_create()
    a.seq_reserve(p, 32)
    c = a.seq_fork(p)
    slots, cow = a.seq_reserve(c, 1)
    assert cow == [] and a.tables[c][:2] == a.tables[p]
    assert a.ref[a.tables[p][0]] == 2 and a.ref[a.tables[p][1]] == 2
