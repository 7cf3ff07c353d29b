"""The Python binding refuses inputs that do not match the cache before any
library call: shapes, dtypes, counts and devices (the C ABI sees only raw
addresses and cannot check them). CPU only: the cache is made on the host,
where every device call must be refused too."""

import numpy as np
import pytest
import torch

import paged_kv_cache_392_amd as pkv


@pytest.fixture
def cache():
    c = pkv.PagedKVCache(2, 16, 2, 64, device="cpu")
    yield c
    c.close()


def decode_inputs(B=3, Hq=4, D=64, max_blocks=4):
    q = torch.zeros((B, Hq, D), dtype=torch.float16)
    tables = torch.zeros((B, max_blocks), dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    return q, tables, lens


def test_decode_rejects_mismatched_shapes(cache):
    q, t, l = decode_inputs()
    bad = [
        dict(q=torch.zeros((3, 4, 128), dtype=torch.float16)),  # head_dim 128 on a d64 cache
        dict(q=torch.zeros((3, 3, 64), dtype=torch.float16)),  # 3 q heads over 2 KV heads
        dict(block_tables=torch.zeros((2, 4), dtype=torch.int32)),  # rows != batch
        dict(block_tables=torch.zeros((3,), dtype=torch.int32)),  # not 2-D
        dict(context_lens=torch.ones(4, dtype=torch.int32)),  # lengths != batch
        dict(context_lens_host=np.ones(2, np.int32)),  # host copy too short
        dict(out=torch.zeros((3, 4, 32), dtype=torch.float16)),
        dict(out=torch.zeros((3, 4, 64), dtype=torch.float32)),
        dict(layer=2),
        dict(layer=-1),
    ]
    for kw in bad:
        args = dict(q=q, block_tables=t, context_lens=l)
        args.update(kw)
        with pytest.raises(ValueError):
            cache.paged_decode(**args)
    with pytest.raises(TypeError):
        cache.paged_decode(q, t.to(torch.int64), l)


def test_decode_refuses_a_host_cache_and_host_tensors(cache):
    q, t, l = decode_inputs()
    with pytest.raises(ValueError, match="GPU"):
        cache.paged_decode(q, t, l)
    with pytest.raises(ValueError, match="GPU"):
        cache.paged_decode(q, t, l, k_new=torch.zeros((3, 2, 64), dtype=torch.float16),
                           v_new=torch.zeros((3, 2, 64), dtype=torch.float16))


def test_prefill_rejects_mismatched_shapes(cache):
    q = torch.zeros((10, 4, 64), dtype=torch.float16)
    t = torch.zeros((2, 4), dtype=torch.int32)
    l = torch.full((2,), 8, dtype=torch.int32)
    bad = [
        dict(q=torch.zeros((10, 4, 128), dtype=torch.float16)),
        dict(q_lens=[4, 5]),  # does not add up to the rows of q
        dict(q_lens=[12, -2]),
        dict(block_tables=torch.zeros((3, 4), dtype=torch.int32)),
        dict(context_lens=torch.ones(3, dtype=torch.int32)),
        dict(context_lens_host=np.ones(3, np.int32)),
        dict(out=torch.zeros((9, 4, 64), dtype=torch.float16)),
        dict(layer=5),
    ]
    for kw in bad:
        args = dict(q=q, q_lens=[4, 6], block_tables=t, context_lens=l)
        args.update(kw)
        with pytest.raises(ValueError):
            cache.paged_prefill(**args)
    with pytest.raises(ValueError, match="GPU"):
        cache.paged_prefill(q, [4, 6], t, l)


def test_write_rejects_mismatched_inputs(cache):
    k = torch.zeros((3, 2, 64), dtype=torch.float16)
    slots = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError):
        cache.write(0, k, torch.zeros((3, 2, 32), dtype=torch.float16), slots)
    with pytest.raises(ValueError):
        cache.write(0, k, k, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(TypeError):
        cache.write(0, k, k, torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError):
        cache.write(7, k, k, slots)
    with pytest.raises(ValueError, match="GPU"):
        cache.write(0, k, k, slots)


def test_append_kv_rejects_a_sequence_named_twice(cache):
    a, b = cache.create_seq(), cache.create_seq()
    free = cache.num_free()
    k = torch.zeros((2, 3, 2, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="more than once"):
        cache.append_kv([a, b, a], k, k)
    # refused before any reservation: the allocator is untouched
    assert cache.num_free() == free
    assert cache.seq_len(a) == 0 and cache.seq_len(b) == 0


def test_plan_members_follow_the_query_heads():
    """A decode's shared-prefix work-groups hold 128 query rows: planned with
    the decode's query heads, groups hold at most 128 // G members (32 at
    most); planned without them, 32."""
    c = pkv.PagedKVCache(1, 256, 2, 64, device="cpu")
    root = c.create_seq()
    c.reserve([root], [48])  # three full shared blocks
    seqs = [root] + [c.fork(root) for _ in range(39)]
    c.reserve(seqs, [5] * len(seqs))  # a private tail block each
    sizes = lambda plan: sorted(len(members) for _, members in plan.groups())
    assert sizes(c.plan_shared_prefix(seqs)) == [8, 32]
    assert sizes(c.plan_shared_prefix(seqs, num_q_heads=16)) == [8, 16, 16]  # G = 8
    assert sizes(c.plan_shared_prefix(seqs, num_q_heads=10)) == [15, 25]  # G = 5
    assert sizes(c.plan_shared_prefix(seqs, max_members=20)) == [20, 20]
    with pytest.raises(ValueError):
        c.plan_shared_prefix(seqs, num_q_heads=3)
    with pytest.raises(ValueError):
        c.plan_shared_prefix(seqs, max_members=8, num_q_heads=16)
    c.close()
