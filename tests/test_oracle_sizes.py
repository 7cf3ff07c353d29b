"""Pins of the oracle's size formulas to the figures printed on the pages."""

import os

import pytest

import oracle


def load_sizes(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "kv_sizes.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kind, L, H, D, E, n, B, lo, hi, cite = line.rstrip("\n").split("\t")
            rows.append((kind, int(L), int(H), int(D), int(E), int(n), int(B), int(lo), int(hi), cite))
    return rows


def check_printed_sizes(golden_dir):
    rows = load_sizes(golden_dir)
    assert len(rows) == 7
    for kind, L, H, D, E, n, B, lo, hi, cite in rows:
        got = oracle.kv_cache_bytes(L, H, D, E, n, B)
        if kind == "exact":
            assert got == lo, (cite, got, lo)
        else:
            assert lo <= got <= hi, (cite, got)


def test_printed_sizes(golden_dir):
    check_printed_sizes(golden_dir)


def test_per_token_is_128_kib():
    # [p2] §2.3: 32 layers, 8 KV heads, d128, fp16 -> 128 KB per token
    assert oracle.kv_bytes_per_token(32, 8, 128, 2) == 128 * 1024


def test_gqa_quarter_of_mha():
    # [p2] §4.2: 32 query heads sharing 8 KV heads need a quarter of the cache
    mha = oracle.kv_cache_bytes(32, 32, 128, 2, 4096, 16)
    gqa = oracle.kv_cache_bytes(32, 8, 128, 2, 4096, 16)
    assert mha == 4 * gqa


def test_mqa_is_one_kv_head():
    # [p2] §4.2: MQA shares a single KV head across all query heads
    assert oracle.kv_cache_bytes(32, 1, 128, 2, 1, 1) * 8 == oracle.kv_bytes_per_token(32, 8, 128, 2)


@pytest.mark.parametrize("N", [1, 64, 520, 8208])
def test_int8_halves_data_bytes(N):
    # [p2] §4.1: 8-bit K/V halve the cache (scales are the only extra)
    f16 = oracle.pool_bytes(32, N, 8, 128, "f16")
    i8 = oracle.pool_bytes(32, N, 8, 128, "i8")
    scales = 32 * N * 8 * 2 * 2
    assert 2 * (i8 - scales) == f16


def test_pool_is_per_token_times_slots():
    # a pool of N 16-token blocks holds exactly N*16 tokens of [p2] §2.3 size
    for L, N, H, D in [(1, 64, 2, 64), (32, 8208, 8, 128), (3, 7, 1, 128)]:
        assert oracle.pool_bytes(L, N, H, D) == oracle.kv_bytes_per_token(L, H, D, 2) * N * 16


def test_headline_pool_matches_table_row():
    # 16 sequences of 8192 tokens fill 16 * 512 blocks: the 16 GB row of [p2] §2.3
    assert oracle.pool_bytes(32, 16 * 512, 8, 128) == 16 * 2**30
    # int8 with the same shape: 8 GiB of data
    assert oracle.pool_bytes(32, 16 * 512, 8, 128, "i8") - 32 * 16 * 512 * 8 * 4 == 8 * 2**30
