"""Parity at the benchmarked sizes, on an MI355X, through the C ABI.

The decode runs in the launch configuration the benchmark times (automatic
partitions from the host lengths, compact grid for ragged batches) and is
compared with the fp64 oracle on every output row: fp16 within 2e-3 max abs
error, int8 within 2e-2 of the oracle on the dequantised values. Each test
prints its case before touching the GPU.
"""

import numpy as np
import pytest
import torch

import workloads
from lib_driver import LibRun
from oracle_driver import OracleRun

pytestmark = pytest.mark.gpu

F16_TOL = 2e-3
I8_TOL = 2e-2
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu case] {msg}", flush=True)


def compare_all_rows(w, tol, fused_append=False, check=None):
    """Replay w on both sides; every (sequence, head) row of every decode
    must be within tol of the oracle. Returns (lib, oracle run, max err)."""
    o = OracleRun(w).run()
    lib = LibRun(w, device=DEV, poison=True, quantised=o.q8, fused_append=fused_append).run()
    for a, b in zip(lib.reserves, o.reserves):
        assert a == b
    err = 0.0
    for a, b in zip(lib.decodes, o.decodes):
        np.testing.assert_array_equal(a["tables"], b["tables"])
        np.testing.assert_array_equal(a["lens"], b["lens"])
        assert a["out"].dtype == np.float16 and np.isfinite(a["out"]).all()
        err = max(err, float(np.abs(a["out"].astype(np.float64) - b["out"]).max()))
    if check is not None:
        check(lib, o)
    return lib, o, err


def test_headline_full_size_all_rows():
    """Batch 16 at 8192 + 1 tokens, 32 q / 8 KV heads, d128, fp16, the new
    token appended inside the decode launch as the benchmark does: all 512
    output rows against the oracle."""
    w = workloads.headline()
    announce("headline B16 ctx 8192+1, 32q/8kv d128 fp16, fused append, all rows")
    lib, o, err = compare_all_rows(w, F16_TOL, fused_append=True)
    assert lib.decodes[0]["fused"]
    announce(f"headline max abs err {err:.3g}")
    assert err <= F16_TOL
    lib.close()


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_gqa8_batch16_ctx8k(dtype):
    """64 q / 8 KV heads (G = 8) at batch 16 and 8K context: fp16 with the
    appended token (8193), int8 decode-only over block-quantised codes."""
    append = dtype == "f16"
    w = workloads.uniform_decode(61, 16, 8192, Hq=64, Hkv=8, dtype=dtype, append=append)
    announce(f"G=8 B16 ctx 8192{'+1' if append else ''} {dtype}")
    lib, o, err = compare_all_rows(w, F16_TOL if dtype == "f16" else I8_TOL)
    announce(f"G=8 {dtype} max abs err {err:.3g}")
    assert err <= (F16_TOL if dtype == "f16" else I8_TOL)
    lib.close()


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_continuous_batching_mix_stream_k(dtype):
    """The continuous-batching mix (16 sequences at U[128, 8192] + 1 tokens
    over a pool scrambled by churn), fp16 and int8: the ragged batch takes
    the stream-K split; all rows against the oracle, and the plain grid
    (no host lengths) at explicit partitions against the oracle too."""
    w = workloads.c3_mixed(dtype=dtype)
    tol = F16_TOL if dtype == "f16" else I8_TOL
    announce(f"c3 mix {dtype}, stream-K split")
    lib, o, err = compare_all_rows(w, tol)
    announce(f"c3 {dtype} max abs err {err:.3g}")
    assert err <= tol
    rec = lib.decodes[0]
    td = torch.from_numpy(rec["tables"]).to(DEV)
    ld = torch.from_numpy(rec["lens"]).to(DEV)
    qd = torch.from_numpy(rec["q"]).to(DEV)
    width = rec["tables"].shape[1] * 16
    for pt in (1024, 2048):
        announce(f"c3 {dtype} plain grid, partition_tokens={pt}")
        plain = lib.cache.paged_decode(qd, td, ld, max_context=width, partition_tokens=pt).cpu().numpy()
        assert np.abs(plain.astype(np.float64) - o.decodes[0]["out"]).max() <= tol, pt
    lib.close()


def test_gqa8_ragged_stream_k():
    """64 q / 8 KV heads (G = 8) over the continuous-batching mix's ragged
    lengths, fp16: the stream-K split of the eight-head kernel, which the
    launch holds at one work-group per CU; all 1024 rows."""
    w = workloads.c3_mixed(seed=63, Hq=64)
    announce("G=8 ragged 16 x U[128, 8192] + 1, fp16, stream-K split")
    lib, o, err = compare_all_rows(w, F16_TOL)
    announce(f"G=8 ragged max abs err {err:.3g}")
    assert err <= F16_TOL
    lib.close()


def test_two_rounds_of_work_groups_32x8193():
    """32 sequences at 8192 + 1 tokens: more partitions than the device holds
    at once (two rounds of work-groups); all 1024 rows."""
    w = workloads.uniform_decode(62, 32, 8192)
    announce("B32 ctx 8193 fp16 (two rounds)")
    lib, o, err = compare_all_rows(w, F16_TOL)
    announce(f"B32 max abs err {err:.3g}")
    assert err <= F16_TOL
    lib.close()


def test_four_sequences_at_32k():
    """4 sequences at 32768 + 1 tokens: few (sequence, KV head) pairs, many
    partitions each."""
    w = workloads.uniform_decode(63, 4, 32768)
    announce("B4 ctx 32769 fp16")
    lib, o, err = compare_all_rows(w, F16_TOL)
    announce(f"B4 ctx 32K max abs err {err:.3g}")
    assert err <= F16_TOL
    lib.close()


@pytest.mark.parametrize("fused", [False, True])
def test_int8_decode_over_gpu_appended_codes(fused):
    """Long int8 contexts written token by token by the library's int8 append
    (quantise on write; the block scale raised and earlier rows re-rounded
    when needed), the last token appended by the append kernel or inside the
    decode launch: codes and scales bit-exact, every row within the int8
    bar."""
    w = workloads.uniform_decode(64, 3, 0, lens=[4100, 6000, 4097], dtype="i8", i8_write="append")
    announce(f"int8 appended codes, lens 4100/6000/4097 +1, fused={fused}")

    def check(lib, o):
        K = lib.cache.region(0, 0).cpu().numpy()
        V = lib.cache.region(1, 0).cpu().numpy()
        S = lib.cache.scales()[0].cpu().numpy()
        for sid, table in o.alloc.tables.items():
            n = o.alloc.lens[sid]
            for j, blk in enumerate(table):
                rows = min(16, n - 16 * j)
                assert np.array_equal(K[blk, :, :rows], o.cache.K[0, blk, :, :rows]), blk
                assert np.array_equal(V[blk, :, :rows], o.cache.V[0, blk, :, :rows]), blk
                assert np.array_equal(S[blk].view(np.uint16), o.cache.scales[0, blk].view(np.uint16)), blk

    lib, o, err = compare_all_rows(w, I8_TOL, fused_append=fused, check=check)
    assert lib.decodes[0]["fused"] == fused
    announce(f"int8 appended max abs err {err:.3g}")
    assert err <= I8_TOL
    lib.close()
