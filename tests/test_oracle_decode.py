"""Pins of the oracle's gather and decode: brute force, a library routine
(torch scaled_dot_product_attention in fp64 on the CPU), closed forms and the
paging invariants (any physical order, shared prefix == private copy)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle_driver import OracleRun


# ---------------------------------------------------------------------------
# helpers

def fill_sequences(N, Hkv, D, seqs, free_order, shared_prefix=None):
    """Write token K/V arrays ``seqs[i] = (k, v)`` through the allocator and
    cache; returns (alloc, cache, sids)."""
    a = oracle.RefAllocator(N, free_order)
    c = oracle.RefCache(1, N, Hkv, D)
    sids = []
    for k, v in seqs:
        s = a.seq_create()
        slots, cow = a.seq_reserve(s, len(k))
        c.copy_blocks(cow)
        c.append(0, k, v, slots)
        sids.append(s)
    return a, c, sids


def contiguous_twin(k):
    """The pseudocode's per-layer cache ``kv_cache[:len]``: rows in token
    order, built without any block table ([p2] §2.2)."""
    return np.asarray(k, np.float64)


def sdpa(q, Kc, Vc, scale):
    """torch.nn.functional.scaled_dot_product_attention in fp64 on the CPU,
    one query row against ``Kc, Vc [n, D]``."""
    qt = torch.tensor(np.asarray(q, np.float64)).reshape(1, 1, 1, -1)
    kt = torch.tensor(Kc).reshape(1, 1, *Kc.shape)
    vt = torch.tensor(Vc).reshape(1, 1, *Vc.shape)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out.reshape(-1).numpy()


def check_against_sdpa(w):
    """The whole decode against SDPA with each KV head repeated for its
    contiguous group of G query heads (the grouping reading)."""
    run = OracleRun(w).run()
    for rec in run.decodes:
        cache = run.q8 if w.dtype == "i8" else run.cache
        q = rec["q"]
        B, Hq, D = q.shape
        G = Hq // w.num_kv_heads
        for b in range(B):
            n = int(rec["lens"][b])
            Kall = np.stack([oracle.gather(cache.K, 0, rec["tables"][b], n, g, cache.scales, 0)
                             for g in range(w.num_kv_heads)])
            Vall = np.stack([oracle.gather(cache.V, 0, rec["tables"][b], n, g, cache.scales, 1)
                             for g in range(w.num_kv_heads)])
            qt = torch.tensor(q[b].astype(np.float64)).reshape(1, Hq, 1, D)
            kt = torch.tensor(Kall).repeat_interleave(G, dim=0).reshape(1, Hq, n, D)
            vt = torch.tensor(Vall).repeat_interleave(G, dim=0).reshape(1, Hq, n, D)
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=w.scale)
            np.testing.assert_allclose(rec["out"][b], ref.reshape(Hq, D).numpy(), rtol=1e-10, atol=1e-12)


def check_against_brute(w):
    run = OracleRun(w).run()
    for rec in run.decodes:
        cache = run.q8 if w.dtype == "i8" else run.cache
        ref = oracle.brute_decode(cache, rec["q"].tolist(), rec["tables"].tolist(),
                                  rec["lens"].tolist(), 0, w.scale)
        np.testing.assert_allclose(rec["out"], np.array(ref), rtol=1e-10, atol=1e-12)


def check_gather_matches_contiguous(seed):
    rng = np.random.default_rng(seed)
    Hkv, D, N = 2, 16, 40
    seqs = [(rng.standard_normal((n, Hkv, D)).astype(np.float16),
             rng.standard_normal((n, Hkv, D)).astype(np.float16)) for n in (1, 15, 16, 17, 70)]
    a, c, sids = fill_sequences(N, Hkv, D, seqs, rng.permutation(N))
    for (k, v), s in zip(seqs, sids):
        for g in range(Hkv):
            np.testing.assert_array_equal(oracle.gather(c.K, 0, a.tables[s], len(k), g),
                                          contiguous_twin(k[:, g]))
            np.testing.assert_array_equal(oracle.gather(c.V, 0, a.tables[s], len(v), g),
                                          contiguous_twin(v[:, g]))


# ---------------------------------------------------------------------------
# brute force and library routine

def test_c1_brute_force():
    check_against_brute(workloads.c1_tiny())


@pytest.mark.parametrize("seed", range(6))
def test_tiny_brute_force(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    check_against_brute(workloads.tiny_random(50 + seed, B=2, Hq=Hkv * G, Hkv=Hkv, D=16, max_len=35))


def test_c1_sdpa():
    check_against_sdpa(workloads.c1_tiny())


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 1), (8, 2), (6, 3)])
def test_mha_mqa_gqa_sdpa(Hq, Hkv):
    # MHA (Hkv == Hq) and MQA (Hkv == 1) are the two ends of GQA ([p2] §4.2)
    check_against_sdpa(workloads.tiny_random(7 + Hq + Hkv, B=3, Hq=Hq, Hkv=Hkv, D=32, max_len=50))


def test_int8_tiny_brute_and_sdpa():
    w = workloads.tiny_random(11, B=2, Hq=4, Hkv=2, D=32, max_len=40, dtype="i8")
    check_against_brute(w)
    check_against_sdpa(w)


# ---------------------------------------------------------------------------
# closed forms

def single_seq_cache(k, v):
    n, Hkv, D = k.shape
    N = -(-n // 16) + 1
    a, c, sids = fill_sequences(N, Hkv, D, [(k, v)], np.arange(N))
    return c, [a.tables[sids[0]]], [n]


def test_one_token_returns_its_value():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 1, 8)).astype(np.float16)
    v = rng.standard_normal((1, 1, 8)).astype(np.float16)
    c, t, n = single_seq_cache(k, v)
    q = rng.standard_normal((1, 1, 8)).astype(np.float16)
    out = oracle.decode(c, q, t, n)
    assert np.array_equal(out[0, 0], v[0, 0].astype(np.float64))


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((37, 1, 8)).astype(np.float16)
    v = rng.standard_normal((37, 1, 8)).astype(np.float16)
    c, t, n = single_seq_cache(k, v)
    out = oracle.decode(c, np.zeros((1, 1, 8), np.float16), t, n)
    np.testing.assert_allclose(out[0, 0], v[:, 0].astype(np.float64).mean(0), rtol=1e-13, atol=1e-14)


def test_equal_keys_give_mean_value():
    rng = np.random.default_rng(5)
    row = rng.standard_normal(8).astype(np.float16)
    k = np.tile(row, (20, 1, 1)).reshape(20, 1, 8)
    v = rng.standard_normal((20, 1, 8)).astype(np.float16)
    c, t, n = single_seq_cache(k, v)
    q = rng.standard_normal((1, 1, 8)).astype(np.float16)
    out = oracle.decode(c, q, t, n)
    np.testing.assert_allclose(out[0, 0], v[:, 0].astype(np.float64).mean(0), rtol=1e-13, atol=1e-14)


def test_peaked_query_selects_one_value():
    rng = np.random.default_rng(6)
    n, D, j = 33, 8, 21
    k = (rng.standard_normal((n, 1, D)) * 0.1).astype(np.float16)
    k[:, 0, 0] = 0
    k[j, 0, 0] = 4.0
    v = rng.standard_normal((n, 1, D)).astype(np.float16)
    c, t, nn = single_seq_cache(k, v)
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, 0] = 100.0
    out = oracle.decode(c, q, t, nn)
    np.testing.assert_allclose(out[0, 0], v[j, 0].astype(np.float64), rtol=0, atol=1e-12)


def test_two_tokens_logistic():
    # with two tokens the weight of token 0 is the logistic of the score gap
    rng = np.random.default_rng(8)
    k = rng.standard_normal((2, 1, 16)).astype(np.float16)
    v = rng.standard_normal((2, 1, 16)).astype(np.float16)
    q = rng.standard_normal((1, 1, 16)).astype(np.float16)
    c, t, n = single_seq_cache(k, v)
    out = oracle.decode(c, q, t, n, scale=0.25)
    qd, kd, vd = (x.astype(np.float64) for x in (q[0, 0], k[:, 0], v[:, 0]))
    gap = 0.25 * (qd @ kd[0] - qd @ kd[1])
    w0 = 1.0 / (1.0 + math.exp(-gap))
    np.testing.assert_allclose(out[0, 0], w0 * vd[0] + (1 - w0) * vd[1], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# paging invariants

@pytest.mark.parametrize("seed", range(4))
def test_gather_matches_contiguous(seed):
    check_gather_matches_contiguous(seed)


def test_output_independent_of_physical_order():
    w1 = workloads.tiny_random(21, B=4, Hq=4, Hkv=2, D=32, max_len=60)
    out1 = OracleRun(w1).run().decodes[0]["out"]
    rng = np.random.default_rng(99)
    for _ in range(3):
        w2 = workloads.tiny_random(21, B=4, Hq=4, Hkv=2, D=32, max_len=60)
        w2.free_order = rng.permutation(w2.num_blocks).astype(np.int32)
        run = OracleRun(w2).run()
        assert not np.array_equal(run.decodes[0]["tables"], OracleRun(w1).run().decodes[0]["tables"])
        assert np.array_equal(run.decodes[0]["out"], out1)


def test_shared_prefix_equals_private_copy():
    rng = np.random.default_rng(12)
    Hkv, D, Hq = 2, 16, 4
    prefix = 40
    pk = rng.standard_normal((prefix, Hkv, D)).astype(np.float16)
    pv = rng.standard_normal((prefix, Hkv, D)).astype(np.float16)
    sk = [rng.standard_normal((n, Hkv, D)).astype(np.float16) for n in (3, 20)]
    sv = [rng.standard_normal((n, Hkv, D)).astype(np.float16) for n in (3, 20)]
    q = rng.standard_normal((2, Hq, D)).astype(np.float16)
    # shared: one prefix, forked, then private suffixes (the first one COWs)
    a = oracle.RefAllocator(32, rng.permutation(32))
    c = oracle.RefCache(1, 32, Hkv, D)
    p = a.seq_create()
    slots, cow = a.seq_reserve(p, prefix)
    c.append(0, pk, pv, slots)
    ch = a.seq_fork(p)
    copies = 0
    for s, k, v in ((p, sk[0], sv[0]), (ch, sk[1], sv[1])):
        slots, cow = a.seq_reserve(s, len(k))
        copies += len(cow)
        c.copy_blocks(cow)
        c.append(0, k, v, slots)
    assert copies == 1  # 40 % 16 != 0: the first writer into the shared tail copies it
    tables, lens = a.block_tables([p, ch], 4)
    shared = oracle.decode(c, q, tables, lens)
    # private: two unrelated sequences with the same token contents
    seqs = [(np.concatenate([pk, sk[i]]), np.concatenate([pv, sv[i]])) for i in range(2)]
    a2, c2, sids = fill_sequences(32, Hkv, D, seqs, rng.permutation(32))
    tables2, lens2 = a2.block_tables(sids, 4)
    private = oracle.decode(c2, q, tables2, lens2)
    assert np.array_equal(shared, private)


def test_append_writes_only_its_slot_and_cow_preserves_parent():
    rng = np.random.default_rng(13)
    a = oracle.RefAllocator(10, rng.permutation(10))
    c = oracle.RefCache(1, 10, 2, 8, fill=np.float16(np.nan))
    p = a.seq_create()
    k = rng.standard_normal((21, 2, 8)).astype(np.float16)
    slots, _ = a.seq_reserve(p, 21)
    before = c.K.copy()
    c.append(0, k, k, slots)
    changed = np.argwhere(~(np.isnan(c.K) & np.isnan(before)) & (c.K != before))
    written = {(int(s) // 16, int(s) % 16) for s in slots}
    assert {(int(b), int(o)) for _, b, _, o, _ in changed} == written
    ch = a.seq_fork(p)
    parent_tail = a.tables[p][1]
    snap = c.K[0, parent_tail].copy()
    slots, cow = a.seq_reserve(ch, 1)
    assert len(cow) == 1 and cow[0][0] == parent_tail
    c.copy_blocks(cow)
    knew = rng.standard_normal((1, 2, 8)).astype(np.float16)
    c.append(0, knew, knew, slots)
    # the parent's block is untouched; the child's copy agrees below the offset
    assert np.array_equal(c.K[0, parent_tail], snap, equal_nan=True)
    new = cow[0][1]
    np.testing.assert_array_equal(c.K[0, new, :, :5], snap[:, :5])
    np.testing.assert_array_equal(c.K[0, new, :, 5], knew[0])
