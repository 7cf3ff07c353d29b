"""Pins of the oracle's causal prefill: a library routine (torch
scaled_dot_product_attention in fp64 on the CPU, causal or with an explicit
mask), agreement with the independently pinned decode on every truncated
context, brute force, closed forms and the paging invariant."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle_driver import OracleRun


def sdpa_reference(run, rec, w):
    """SDPA over each sequence's gathered rows, K/V repeated per group; causal
    for a fresh prompt, an explicit boolean mask when the chunk follows
    cached tokens."""
    out = []
    row0 = 0
    G = w.num_q_heads // w.num_kv_heads
    for b, ql in enumerate(rec["q_lens"]):
        n = int(rec["lens"][b])
        Kall = np.stack([oracle.gather(run.cache.K, 0, rec["tables"][b], n, g) for g in range(w.num_kv_heads)])
        Vall = np.stack([oracle.gather(run.cache.V, 0, rec["tables"][b], n, g) for g in range(w.num_kv_heads)])
        qt = torch.tensor(rec["q"][row0:row0 + ql].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        kt = torch.tensor(Kall).repeat_interleave(G, dim=0).unsqueeze(0)
        vt = torch.tensor(Vall).repeat_interleave(G, dim=0).unsqueeze(0)
        if ql == n:
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=w.scale)
        else:
            pos = torch.arange(n - ql, n)
            mask = torch.arange(n)[None, :] <= pos[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=w.scale)
        out.append(ref.squeeze(0).permute(1, 0, 2).numpy())
        row0 += ql
    return np.concatenate(out)


def check_prefill_against_sdpa(w):
    run = OracleRun(w).run()
    for rec in run.prefills:
        np.testing.assert_allclose(rec["out"], sdpa_reference(run, rec, w), rtol=1e-10, atol=1e-12)


def check_prefill_against_decode(w):
    """Every chunk row equals the decode of that token over the context cut
    right after it (the decode is pinned on its own)."""
    run = OracleRun(w).run()
    for rec in run.prefills:
        row0 = 0
        for b, ql in enumerate(rec["q_lens"]):
            n = int(rec["lens"][b])
            for i in range(ql):
                p = n - ql + i
                ref = oracle.decode(run.cache, rec["q"][row0 + i][None], rec["tables"][b:b + 1],
                                    np.array([p + 1]), 0, w.scale)
                np.testing.assert_allclose(rec["out"][row0 + i], ref[0], rtol=1e-11, atol=1e-13)
            row0 += ql


@pytest.mark.parametrize("cached,chunk,Hq,Hkv,D", [
    ([0, 0], [17, 40], 4, 2, 64),  # fresh prompts
    ([5, 33, 0], [12, 1, 30], 8, 2, 64),  # chunks after cached tokens, one of a single token
    ([16, 100], [16, 47], 8, 8, 32),  # MHA, a chunk starting on a block boundary
    ([3], [61], 8, 1, 32),  # MQA
])
def test_prefill_matches_sdpa(cached, chunk, Hq, Hkv, D):
    check_prefill_against_sdpa(workloads.prefill_chunks(11, cached, chunk, Hq, Hkv, D))


@pytest.mark.parametrize("cached,chunk", [([0, 9], [20, 7]), ([40], [25])])
def test_prefill_matches_decode_on_each_prefix(cached, chunk):
    check_prefill_against_decode(workloads.prefill_chunks(12, cached, chunk, 8, 2, 32))


def test_prefill_matches_brute_force():
    w = workloads.prefill_chunks(13, [3, 0], [5, 4], 4, 2, 8)
    run = OracleRun(w).run()
    rec = run.prefills[0]
    row0 = 0
    for b, ql in enumerate(rec["q_lens"]):
        n = int(rec["lens"][b])
        for i in range(ql):
            ref = oracle.brute_decode(run.cache, [rec["q"][row0 + i].tolist()], [rec["tables"][b].tolist()],
                                      [n - ql + i + 1], 0, w.scale)
            np.testing.assert_allclose(rec["out"][row0 + i], np.array(ref[0]), rtol=1e-10, atol=1e-12)
        row0 += ql


def test_first_prompt_token_sees_only_itself():
    """A fresh prompt's first token attends to itself alone: its output is
    its own V row exactly, whatever q and K are."""
    w = workloads.prefill_chunks(14, [0, 0], [9, 30], 8, 2, 32)
    run = OracleRun(w).run()
    rec = run.prefills[0]
    row0 = 0
    for b, ql in enumerate(rec["q_lens"]):
        V0 = np.stack([oracle.gather(run.cache.V, 0, rec["tables"][b], 1, g)[0] for g in range(2)])
        np.testing.assert_array_equal(rec["out"][row0], np.repeat(V0, 4, axis=0))
        row0 += ql


def test_equal_keys_give_running_means():
    """With every key equal, token at position p averages V rows 0..p."""
    w = workloads.prefill_chunks(15, [6], [20], 4, 1, 16)
    k0 = w.steps[1][2][0].copy()
    for st in w.steps:
        if st[0] == "prefill":
            st[2][:] = k0
    run = OracleRun(w).run()
    rec = run.prefills[0]
    n = int(rec["lens"][0])
    Vc = oracle.gather(run.cache.V, 0, rec["tables"][0], n, 0)
    for i in range(20):
        p = n - 20 + i
        np.testing.assert_allclose(rec["out"][i], np.repeat(Vc[:p + 1].mean(axis=0)[None], 4, axis=0),
                                   rtol=1e-12, atol=1e-13)


def test_prefill_is_invariant_to_physical_order():
    outs = []
    for shuffle in (False, True):
        run = OracleRun(workloads.prefill_chunks(16, [21, 0], [30, 18], 8, 2, 32, shuffle=shuffle)).run()
        outs.append(run.prefills[0])
    assert not np.array_equal(outs[0]["tables"], outs[1]["tables"])
    np.testing.assert_array_equal(outs[0]["out"], outs[1]["out"])


def test_bad_lengths_are_rejected():
    w = workloads.prefill_chunks(17, [0], [5], 4, 2, 8)
    run = OracleRun(w).run()
    rec = run.prefills[0]
    with pytest.raises(ValueError):
        oracle.prefill(run.cache, rec["q"], [6], rec["tables"], rec["lens"])
    with pytest.raises(ValueError):
        oracle.prefill(run.cache, rec["q"], [5], rec["tables"], np.array([4]))


def test_empty_chunk_contributes_no_rows():
    """A sequence without new tokens adds no rows; the others are as if it
    were absent."""
    w = workloads.prefill_chunks(18, [3, 9, 0], [7, 0, 5], 4, 2, 8)
    run = OracleRun(w).run()
    rec = run.prefills[0]
    assert rec["out"].shape[0] == 12
    alone = oracle.prefill(run.cache, rec["q"], [7, 5], rec["tables"][[0, 2]], rec["lens"][[0, 2]], 0, w.scale)
    np.testing.assert_array_equal(rec["out"], alone)
