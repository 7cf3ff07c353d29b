#!/usr/bin/env python3
"""Benchmark of the paged KV cache decode step on one MI355X.

Workload (seeded, synthetic): the 32-query-head / 8-KV-head, head_dim 128,
fp16 decode step at batch 16 and 8K context over 32 layer pools -- every
sequence prefilled to 8192 tokens ([p2] lqnn.cn/news/235768 §2.3 table, the
8192 x 16 row: 16 GB of K/V). One step is the whole hot path for one new
token per sequence: host slot reservation and block-table packing, their
upload, then for each of the 32 layers the KV append and the paged decode
(split-K kernel + log-sum-exp merge). The context grows by one token per
step, as in serving.

Printed: one JSON line. ``value`` is whole-step throughput in GB/s of
algorithmic bytes (K/V read by decode, q, tables, out, appended K/V read and
written); ``decode_tok_s`` is batch / step time (attention only);
``roofline`` is the split-K decode kernel's algorithmic bytes per launch
over its average duration, from HIP events recorded around that kernel on
its launch stream for one decode per timed step (the layer rotating with the
step); ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.
"""

import argparse
import contextlib
import ctypes
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
B, HQ, HKV, D, CTX = 16, 32, 8, 128, 8192


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps (one timed sample of each kernel per step)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every layer directly instead of replaying layers 1.. as one HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--workload", choices=["headline", "c5", "c3", "shape", "prefix", "prefill"],
                    default="headline",
                    help="headline: the fp16 batch-16 8K decode step (the bench line); c5: the int8 "
                         "batch-16 8K decode-only step over 32 int8 layer pools; c3: the decode-only step "
                         "of the continuous-batching mix (16 sequences at seeded U[128, 8192] lengths); "
                         "shape: a decode-only step of the shape given by --batch, --context or --lengths, "
                         "--q-heads, --kv-heads, --dtype; prefix: the decode step "
                         "of 32 sequences sharing a 2048-token prefix, with and without the shared-prefix "
                         "plan; prefill: 4 prompts of 2048 tokens appended and attended causally over 32 "
                         "layer pools (timing and profiling; parity is covered by the GPU tests)")
    ap.add_argument("--batch", type=int, default=16, help="shape workload: sequences")
    ap.add_argument("--context", type=int, default=8192, help="shape workload: tokens per sequence")
    ap.add_argument("--lengths", type=int, nargs=2, metavar=("LO", "HI"),
                    help="shape workload: seeded uniform lengths in [LO, HI] instead of --context")
    ap.add_argument("--context-list", type=str, default=None,
                    help="shape workload: comma-separated context lengths, one per sequence")
    ap.add_argument("--q-heads", type=int, default=32, help="shape workload")
    ap.add_argument("--kv-heads", type=int, default=8, help="shape workload")
    ap.add_argument("--head-dim", type=int, choices=[64, 128], default=128, help="shape workload")
    ap.add_argument("--dtype", choices=["f16", "i8"], default="f16",
                    help="headline: the element type of the 32 layer pools (i8: the same step on int8 K/V, "
                         "each new token quantised on write inside the decode launch); shape workload")
    ap.add_argument("--seed", type=int, default=None,
                    help="shape workload: lengths and block order (default 7); c3: block order (default: "
                         "the config's seed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB three times (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


@contextlib.contextmanager
def no_collections():
    """Python's cyclic collector stays out of a timed loop. The set-up leaves
    ~170K tracked objects, and a full collection of them takes 35-40 ms on
    the host; falling inside the loop it outlasts the few steps the host has
    queued ahead, and the GPU idles (measured: 2.86 ms per headline step
    without it, 3.5-3.6 ms with one such pause in 50 steps). Objects from
    before the loop are collected and frozen, and nothing is collected
    inside it."""
    gc.collect()
    gc.freeze()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()
        gc.unfreeze()


def copy_calibration():
    """A plain elementwise copy kernel (x * 1) of exactly 2**30 bytes in and
    2**30 bytes out, three times, on cuda:0: under rocprofv3 --pmc its
    FETCH_SIZE and WRITE_SIZE per dispatch give the factor between the
    counters and true HBM bytes. (An elementwise kernel rather than
    Tensor.copy_, which may become a DMA transfer that the counters miss.)"""
    import torch
    n = 2**30
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "paged_kv_cache_392_amd", "csrc", "kernels.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    ``profiles/<name>_traffic.json``, if it was taken on the current kernel
    source; else None."""
    if name is None:
        return None
    path = os.path.join(ROOT, "profiles", name + "_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the paged decode path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, ROOT)
    import paged_kv_cache_392_amd as pkv
    from paged_kv_cache_392_amd import _capi as C
    import workloads

    if args.workload == "c5":
        int8_decode_bench(args, torch, pkv, C, workloads)
        return
    if args.workload == "c3":
        c3_decode_bench(args, torch, pkv, C, workloads)
        return
    if args.workload == "shape":
        shape_decode_bench(args, torch, pkv, C, workloads)
        return
    if args.workload == "prefix":
        prefix_decode_bench(args, torch, pkv, C, workloads)
        return
    if args.workload == "prefill":
        prefill_bench(args, torch, pkv, C, workloads)
        return

    dev = torch.device("cuda:0")
    K, W, L = args.steps, args.warmup, args.layers
    total_steps = K + W + 1
    spare = B * (-(-(total_steps + 1) // 16))
    w = workloads.headline(spare_blocks=spare)
    N = w.num_blocks
    max_blocks = -(-(CTX + total_steps + 1) // 16)

    i8 = args.dtype == "i8"
    cache = pkv.PagedKVCache(L, N, HKV, D, args.dtype, w.free_order, dev)
    lib = C.load()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    print(f"[bench] pool {cache.nbytes / 2**30:.2f} GiB, {L} layers, {N} blocks, {args.dtype}", file=sys.stderr,
          flush=True)

    # --- build the cache: layer 0 from the seeded workload through the
    # library's append (int8: quantised on write), layers 1.. with seeded
    # device noise (timing only; int8: random codes and scales)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    for layer in range(1, L):
        for which in (0, 1):
            r = cache.region(which, layer)
            if i8:
                r.copy_(torch.randint(-127, 128, r.shape, dtype=torch.int8, device=dev, generator=gen))
            else:
                r.normal_(generator=gen)
    if i8:
        cache.scales()[1:].uniform_(0.01, 0.03, generator=gen)
    seqs, first_k, first_v, first_q = [], None, None, None
    for step in w.steps:
        if step[0] == "create":
            seqs.append(cache.create_seq())
        elif step[0] == "prefill":
            _, name, k, v = step
            s = seqs[int(name[1:])]
            slots, cow = cache.reserve([s], [len(k)])
            sd = torch.from_numpy(slots).to(dev)
            cache.write(0, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), sd)
        elif step[0] == "append":
            first_k, first_v = step[2], step[3]
        elif step[0] == "decode":
            first_q = step[2]
    torch.cuda.synchronize()

    # per-layer new-token k/v and q; step 0 of layer 0 uses the workload's own
    knew = torch.empty((total_steps, L, B, HKV, D), dtype=torch.float16, device=dev).normal_(generator=gen)
    vnew = torch.empty_like(knew).normal_(generator=gen)
    qall = torch.empty((L, B, HQ, D), dtype=torch.float16, device=dev).normal_(generator=gen)
    knew[0, 0].copy_(torch.from_numpy(first_k))
    vnew[0, 0].copy_(torch.from_numpy(first_v))
    qall[0].copy_(torch.from_numpy(first_q))
    out = torch.empty((L, B, HQ, D), dtype=torch.float16, device=dev)
    ws_bytes = C.pkv_decode_workspace_bytes(cache.cfg, B, HQ, max_blocks * 16, args.partition_tokens)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    # per-step pinned upload buffers (a step's buffer is never reused while its
    # copy may still be queued)
    tables_h = torch.empty((total_steps, B, max_blocks), dtype=torch.int32).pin_memory()
    lens_h = torch.empty((total_steps, B), dtype=torch.int32).pin_memory()
    tables_d = torch.empty((B, max_blocks), dtype=torch.int32, device=dev)
    lens_d = torch.empty((B,), dtype=torch.int32, device=dev)
    seq_arr = np.array(seqs, np.int64)
    cap = max_blocks * 16  # table width in tokens: the graph's max_context

    # prebuilt decode argument blocks, one per layer
    argv = []
    for layer in range(L):
        a = C.pkv_decode_args()
        a.cfg = ctypes.pointer(cache.cfg)
        a.pool_dev = cache.pool.data_ptr()
        a.layer = layer
        a.q_dev = qall[layer].data_ptr()
        a.num_seqs = B
        a.num_q_heads = HQ
        a.block_tables_dev = tables_d.data_ptr()
        a.max_blocks = max_blocks
        a.ctx_lens_dev = lens_d.data_ptr()
        a.out_dev = out[layer].data_ptr()
        a.scale = 1.0 / math.sqrt(D)
        a.workspace_dev = ws.data_ptr()
        a.workspace_bytes = ws.numel()
        a.partition_tokens = args.partition_tokens
        a.timing_events = None
        argv.append(a)

    # timing events around the split and merge kernels of layer 0's decode in
    # every timed step (an event pair costs a few µs of queue time, so the
    # other decodes run without); recorded once so each owns a HIP event
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for group in ev:
        for e in group:
            e.record()
    ev_arrays = [(ctypes.c_void_p * 4)(*[e.cuda_event for e in group]) for group in ev]
    ev_ptrs = [ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)) for arr in ev_arrays]
    torch.cuda.synchronize()

    lib_reserve = lib.pkv_seq_reserve
    slot1 = np.empty(1, np.int32)
    cow = np.empty((1, 2), np.int32)
    ncow = ctypes.c_int32()
    step_lens = []

    def prepare(i):
        """a1: reserve one slot per sequence (host allocator; the kernel finds
        the slot through the table); a2: pack and upload tables and lengths."""
        for b in range(B):
            st = lib_reserve(cache.handle, int(seq_arr[b]), 1, C._i32p(slot1), C._i32p(cow), 1, ctypes.byref(ncow))
            if st != 0 or ncow.value:
                raise RuntimeError(f"reserve failed ({st}) or unexpected copy-on-write")
        th, lh = tables_h[i].numpy(), lens_h[i].numpy()
        C._check(lib.pkv_build_block_tables(cache.handle, seq_arr.ctypes.data_as(C._p_i64), B, max_blocks,
                                            C._i32p(th), C._i32p(lh)))
        step_lens.append(lh.copy())
        # uploaded by the library's kernel, on the compute queue
        C._check(lib.pkv_upload(tables_d.data_ptr(), tables_h[i].data_ptr(), tables_d.numel() * 4, sp))
        C._check(lib.pkv_upload(lens_d.data_ptr(), lens_h[i].data_ptr(), B * 4, sp))
        return lh

    def launch(layer, i, lh, max_context, events=None, stream_handle=None):
        """a4 + a5 (+ a6): one decode launch with the new token's K/V appended
        inside it, and the merge kernel."""
        a = argv[layer]
        a.max_context = max_context
        a.ctx_lens_host = None if lh is None else C._i32p(lh)
        a.k_new_dev = knew[i, layer].data_ptr()
        a.v_new_dev = vnew[i, layer].data_ptr()
        a.timing_events = events
        C._check(lib.pkv_paged_decode(ctypes.byref(a), sp if stream_handle is None else stream_handle))

    def eager_step(i, events=None):
        lh = prepare(i)
        mc = int(lh.max())
        for layer in range(L):
            launch(layer, i, lh, mc, events if layer == 0 else None)

    print(f"[bench] warmup {W} steps", file=sys.stderr, flush=True)
    for i in range(W):
        eager_step(i)
        if i == 0:
            torch.cuda.synchronize()
            first_out = out[0].float().cpu().numpy()
            first_tables = tables_h[0].numpy().copy()
            first_lens = lens_h[0].numpy().copy()
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        # layers 1..L-1 of a step as one HIP graph: grids and partitions sized
        # for the table width (no host lengths: they grow from replay to
        # replay), lengths and tables read from the device buffers at replay;
        # the appended rows come from step 0's buffers (values do not matter
        # for timing; layer 0, which carries the seeded workload, stays eager)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream().cuda_stream
            for layer in range(1, L):
                launch(layer, 0, None, cap, stream_handle=cs)
        torch.cuda.synchronize()

    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K + 1)]

    def graph_step(i, events=None):
        lh = prepare(i)
        launch(0, i, lh, int(lh.max()), events)
        j = i - (W + 1)  # timed step index (the untimed step's events are overwritten)
        if 0 <= j < K:
            gev[j][0].record()
        graph.replay()
        if 0 <= j < K:
            gev[j][1].record()

    step_fn = eager_step if graph is None else graph_step
    step_fn(W)  # one untimed step in the timed mode (first graph replay)
    torch.cuda.synchronize()

    print(f"[bench] timing {K} steps ({'eager' if graph is None else 'layer 0 eager + graph'})",
          file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with no_collections():
        t0.record()
        h0 = time.perf_counter()
        for i in range(K):
            step_fn(W + 1 + i, ev_ptrs[i])
        host_ms = (time.perf_counter() - h0) * 1e3 / K
        t1.record()
        torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / K

    # the last graph step's outputs against eager launches of the same layers
    # with the same arguments (the appended rows are rewritten with the same
    # bytes)
    graph_matches_eager = None
    if graph is not None:
        check_layers = [1, L // 2, L - 1] if L > 2 else list(range(1, L))
        got = {l: out[l].clone() for l in check_layers}
        for l in check_layers:
            launch(l, 0, None, cap)
        torch.cuda.synchronize()
        graph_matches_eager = all(torch.equal(got[l].view(torch.int16), out[l].view(torch.int16))
                                  for l in check_layers)

    split_ms = np.array([g[0].elapsed_time(g[1]) for g in ev])
    # a launch that needed no merge leaves its merge events at their set-up
    # record, from before the timed loop
    merged = all(t0.elapsed_time(g[2]) > 0 for g in ev)
    merge_ms = np.array([g[2].elapsed_time(g[3]) for g in ev]) if merged else None
    timed_lens = step_lens[W + 1:]
    append_us = time_append(torch, C, lib, cache, dev, sp, K, knew, vnew, seq_arr, max_blocks)

    # algorithmic bytes
    E = 1 if i8 else 2
    kv_tok = 2 * HKV * D * E  # K and V of one token, one layer
    def decode_bytes(lens, with_out=True):
        """K/V rows read + q + table entries + lengths (+ out) of one decode."""
        lens = np.asarray(lens, np.int64)
        nb = len(lens)
        nblk = (lens + 15) // 16
        b = int(lens.sum()) * kv_tok + nb * HQ * D * 2 + int(nblk.sum()) * 4 + nb * 4
        if i8:
            b += int(nblk.sum()) * HKV * 4  # the tiles' (K, V) fp16 scales
        return b + (nb * HQ * D * 2 if with_out else 0)
    append_bytes = 2 * (B * HKV * D * 2) + 2 * (B * HKV * D * E)  # the new k and v rows read (fp16), written
    upload_bytes = B * max_blocks * 4 + B * 4  # tables and lengths
    step_bytes = [L * (decode_bytes(l) + append_bytes) + upload_bytes for l in timed_lens]
    split_bytes = np.array([decode_bytes(l, with_out=False) for l in timed_lens])
    value = float(np.sum(step_bytes) / (total_ms * 1e-3) / 1e9)
    split_gbps = float(np.mean(split_bytes) / (np.mean(split_ms) * 1e-3) / 1e9)

    # HBM probe: a plain coalesced read in the same run
    probe = None
    if not args.no_probe:
        nbytes = min(cache.nbytes, 8 * 2**30)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        C.pkv_probe_stream_read(cache.pool.data_ptr(), nbytes, sink.data_ptr(), sp)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        torch.cuda.synchronize()
        p0.record()
        for _ in range(reps):
            C.pkv_probe_stream_read(cache.pool.data_ptr(), nbytes, sink.data_ptr(), sp)
        p1.record()
        torch.cuda.synchronize()
        probe = nbytes * reps / (p0.elapsed_time(p1) * 1e-3) / 1e9

    src_hash = kernel_source_hash()
    traffic = None if i8 or args.partition_tokens else measured_traffic("paged_decode_b16_ctx8k", src_hash)
    result = {
        "metric": "paged decode HBM GB/s (% of peak) + decode tok/s, 32q/8kv d128 " + ("int8" if i8 else "fp16"),
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {
            "workload": "decode step, batch 16, context 8192 (+1 token per step), 32 q heads / 8 KV heads, "
                        "head_dim 128, " + ("int8 K/V with one fp16 scale per (block, KV head), the new token "
                                            "quantised on write" if i8 else "fp16 K/V") +
                        " in 16-token blocks, 32 layer pools",
            "batch": B, "context": CTX, "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "layers": L,
            "block_tokens": 16, "pool_blocks_per_layer": N,
            "partition_tokens": args.partition_tokens or "auto",
        },
        "decode_tok_s": round(B / (ms_per_step * 1e-3), 1),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBPS, 2),
        "split_kernel_us": round(float(np.mean(split_ms)) * 1e3, 2),
        "split_kernel_us_p10_p90": [round(float(np.percentile(split_ms, 10)) * 1e3, 2),
                                    round(float(np.percentile(split_ms, 90)) * 1e3, 2)],
        "merge_kernel_us": round(float(np.mean(merge_ms)) * 1e3, 2) if merged else None,
        "decode_a5_a6": decode_metric(split_ms, merge_ms, split_bytes),
        # graph layers: the decode with its fused append and the merge, sized
        # for the table width (no host lengths)
        "decode_a4_a5_a6_graph": None if graph is None else graph_layer_metric(
            np.array([a.elapsed_time(b) for a, b in gev[:K]]) / (L - 1),
            split_bytes + append_bytes, L - 1),
        "append_kernel_us": append_us,
        "timed_launch_samples": int(len(split_ms)),
        "execution": ("per step: host slot reservation and table packing, table upload, layer 0 "
                      "launched directly (timing events), " +
                      ("layers 1.. directly" if graph is None else f"layers 1..{L - 1} as one HIP graph replay") +
                      "; the append runs inside the decode kernel"),
        "graph_matches_eager_bitwise": graph_matches_eager,
        "host_issue_ms_per_step": round(host_ms, 4),
        "probe_read_GBps": None if probe is None else round(probe, 1),
        "split_kernel_pct_of_probe": None if not probe else round(100.0 * split_gbps / probe, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": f"paged_decode_kernel<128,4,{args.dtype}> (split-K decode)",
            "achieved": round(split_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(split_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": int(np.mean(split_bytes)),
        },
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline and not i8:
        result["cpu_baseline"] = cpu_baseline(w, first_out, first_tables, first_lens, args.cpu_seconds,
                                              decode_bytes)
    print(json.dumps(result), flush=True)


def decode_metric(split_ms, merge_ms, bytes_per_launch):
    """The decode metric over the split-K kernel and the merge together (the
    two launches of one paged decode): per-sample sums of the two kernels'
    HIP-event times, median and p10/p90 in µs, and the algorithmic bytes over
    the median as GB/s and as a fraction of the 8 TB/s peak. Samples whose
    launch needed no merge count the split kernel alone (merge_ms None)."""
    both = np.asarray(split_ms) + (0.0 if merge_ms is None else np.asarray(merge_ms))
    med = float(np.median(both))
    gbps = float(np.mean(bytes_per_launch)) / (med * 1e-3) / 1e9
    return {"median_us": round(med * 1e3, 2), "p10_us": round(float(np.percentile(both, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(both, 90)) * 1e3, 2), "GBps": round(gbps, 1),
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "samples": int(len(both))}


def graph_layer_metric(layer_ms, bytes_per_layer, layers):
    """The same launches as they run back to back in a step: per timed step,
    one HIP-event pair around the replay of the graph of `layers` layers
    (each layer's launches and nothing else), divided by `layers`; median
    and p10/p90 in µs, and the algorithmic bytes of one layer over the
    median as GB/s and as a fraction of the 8 TB/s peak."""
    med = float(np.median(layer_ms))
    gbps = float(np.mean(bytes_per_layer)) / (med * 1e-3) / 1e9
    return {"median_us": round(med * 1e3, 2), "p10_us": round(float(np.percentile(layer_ms, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(layer_ms, 90)) * 1e3, 2), "GBps": round(gbps, 1),
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "layers_per_replay": layers, "samples": int(len(layer_ms))}


def time_append(torch, C, lib, cache, dev, sp, K, knew, vnew, seq_arr, max_blocks):
    """The append step (a4) on its own: the batch's new token (k and v of
    every KV head) written into every layer by one pkv_append_kv launch per
    layer, at slots reserved past the timed steps' tokens. The L launches are
    replayed from one HIP graph (as a two-call decode step would issue them),
    K replays between two events: µs per launch is the replay time over K x L.
    Also the median of per-launch event pairs around single eager launches
    (host-bound: it includes the launch gap). (The decode step itself
    appends inside the decode launch; this is the separate kernel's cost.)"""
    nb = len(seq_arr)
    L = cache.num_layers
    slots = np.empty(nb, np.int32)
    for b in range(nb):
        s, _ = cache.reserve([int(seq_arr[b])], [1])
        slots[b] = s[0]
    sd = torch.from_numpy(slots).to(dev)

    def launch(layer, stream_handle):
        C._check(lib.pkv_append_kv(ctypes.byref(cache.cfg), cache.pool.data_ptr(), layer,
                                   knew[0, layer].data_ptr(), vnew[0, layer].data_ptr(), sd.data_ptr(), nb,
                                   stream_handle))

    for layer in range(L):
        launch(layer, sp)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream().cuda_stream
        for layer in range(L):
            launch(layer, cs)
    torch.cuda.synchronize()
    graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    per_launch = e0.elapsed_time(e1) * 1e3 / (K * L)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        evs[i][0].record()
        launch(0, sp)
        evs[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    return {"graph_us_per_launch": round(per_launch, 2), "eager_event_median_us": round(float(np.median(t)), 2),
            "tokens_per_launch": nb, "launches_per_replay": L}


def decode_only_bench(args, torch, pkv, C, lens, hq, hkv, dtype, free_order, seed, metric, workload,
                      traffic_name=None):
    """Decode-only step (no append) over `args.layers` layer pools: one
    paged decode per layer for sequences of the given context lengths, q
    heads, KV heads and element type (d128). K/V (codes and scales for int8)
    are seeded device noise: values do not change the timing, and parity of
    every shape is covered by the GPU tests. Tables come from the library's
    allocator in the given block order. Layer 0 is launched directly with
    timing events around the split and merge kernels, layers 1.. are
    replayed from one HIP graph and checked against direct launches bit for
    bit."""
    dev = torch.device("cuda:0")
    K, W, L = args.steps, args.warmup, args.layers
    lens = [int(n) for n in lens]
    nb = len(lens)
    N = len(free_order)
    cache = pkv.PagedKVCache(L, N, hkv, D, dtype, free_order, dev)
    lib = C.load()
    sp = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    for layer in range(L):
        for which in (0, 1):
            r = cache.region(which, layer)
            if dtype == "i8":
                r.copy_(torch.randint(-127, 128, r.shape, dtype=torch.int8, device=dev, generator=gen))
            else:
                r.normal_(generator=gen)
    if dtype == "i8":
        cache.scales().uniform_(0.01, 0.03, generator=gen)
    seqs = [cache.create_seq() for _ in range(nb)]
    for s, n in zip(seqs, lens):
        cache.reserve([s], [n])
    ctx = max(lens)
    max_blocks = -(-ctx // 16)
    tables_h, lens_h = cache.block_tables(seqs, max_blocks)
    tables_d = torch.from_numpy(tables_h).to(dev)
    lens_d = torch.from_numpy(lens_h).to(dev)
    q = torch.empty((L, nb, hq, D), dtype=torch.float16, device=dev).normal_(generator=gen)
    out = torch.empty_like(q)
    ws_bytes = C.pkv_decode_workspace_bytes(cache.cfg, nb, hq, ctx, args.partition_tokens)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    argv = []
    for layer in range(L):
        a = C.pkv_decode_args()
        a.cfg = ctypes.pointer(cache.cfg)
        a.pool_dev = cache.pool.data_ptr()
        a.layer = layer
        a.q_dev = q[layer].data_ptr()
        a.num_seqs = nb
        a.num_q_heads = hq
        a.block_tables_dev = tables_d.data_ptr()
        a.max_blocks = max_blocks
        a.ctx_lens_dev = lens_d.data_ptr()
        a.ctx_lens_host = C._i32p(lens_h)
        a.max_context = ctx
        a.out_dev = out[layer].data_ptr()
        a.scale = 1.0 / math.sqrt(D)
        a.workspace_dev = ws.data_ptr()
        a.workspace_bytes = ws.numel()
        a.partition_tokens = args.partition_tokens
        argv.append(a)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for group in ev:
        for e in group:
            e.record()
    ev_ptrs = [ctypes.cast((ctypes.c_void_p * 4)(*[e.cuda_event for e in g]), ctypes.POINTER(ctypes.c_void_p))
               for g in ev]
    keep = list(ev_ptrs)

    def launch(layer, events=None, stream_handle=None):
        a = argv[layer]
        a.timing_events = events
        C._check(lib.pkv_paged_decode(ctypes.byref(a), sp if stream_handle is None else stream_handle))

    for _ in range(W):
        for layer in range(L):
            launch(layer)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream().cuda_stream
        for layer in range(1, L):
            launch(layer, stream_handle=cs)
    torch.cuda.synchronize()
    launch(0)
    graph.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    with no_collections():
        t0.record()
        for i in range(K):
            launch(0, keep[i])
            gev[i][0].record()
            graph.replay()
            gev[i][1].record()
        t1.record()
        torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / K
    layer_ms = np.array([a.elapsed_time(b) for a, b in gev]) / (L - 1)
    check = [1, L // 2, L - 1] if L > 2 else list(range(1, L))
    got = {l: out[l].clone() for l in check}
    for l in check:
        launch(l)
    torch.cuda.synchronize()
    same = all(torch.equal(got[l].view(torch.int16), out[l].view(torch.int16)) for l in check)
    split_ms = np.array([g[0].elapsed_time(g[1]) for g in ev])
    merge_ms = np.array([g[2].elapsed_time(g[3]) for g in ev])
    # a launch with one partition per sequence has no merge: its merge events
    # then still hold their set-up record, from before the timed loop
    merged = all(t0.elapsed_time(g[2]) > 0 for g in ev)
    E = 1 if dtype == "i8" else 2
    nblk = sum(-(-n // 16) for n in lens)
    kernel_bytes = (sum(lens) * 2 * hkv * D * E + (nblk * hkv * 4 if dtype == "i8" else 0)
                    + nb * hq * D * 2 + nblk * 4 + nb * 4)
    step_bytes = L * (kernel_bytes + nb * hq * D * 2)
    achieved = kernel_bytes / (float(np.mean(split_ms)) * 1e-3) / 1e9
    G = hq // hkv
    print(json.dumps({
        "metric": metric,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": workload, "layers": L, "batch": nb, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": D, "context_min": min(lens), "context_max": ctx, "context_sum": sum(lens),
                   "partition_tokens": args.partition_tokens or "auto"},
        "decode_tok_s": round(nb / (ms_per_step * 1e-3), 1),
        "split_kernel_us": round(float(np.mean(split_ms)) * 1e3, 2),
        "split_kernel_us_p10_p90": [round(float(np.percentile(split_ms, 10)) * 1e3, 2),
                                    round(float(np.percentile(split_ms, 90)) * 1e3, 2)],
        "merge_kernel_us": round(float(np.mean(merge_ms)) * 1e3, 2) if merged else None,
        "decode_a5_a6": decode_metric(split_ms, merge_ms if merged else None, [kernel_bytes]),
        "decode_a5_a6_graph": graph_layer_metric(layer_ms, [kernel_bytes], L - 1),
        "graph_matches_eager_bitwise": same,
        "roofline": {"bound": "hbm", "kernel": f"paged_decode_kernel<128,{G},{dtype}> (split-K decode)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(traffic_name, kernel_source_hash()),
                     "bytes_per_launch": int(kernel_bytes)},
        "cpu_baseline": None,
    }), flush=True)


def int8_decode_bench(args, torch, pkv, C, workloads):
    """int8 decode-only step (the int8 long-context config): batch 16 at
    context 8192, 32 q / 8 KV heads, d128, one fp16 scale per (block, KV
    head) for K and V, over 32 layer pools (8 GiB of codes), in the config's
    seeded block order."""
    w = workloads.c5_int8()
    decode_only_bench(args, torch, pkv, C, [8192] * B, HQ, HKV, "i8", w.free_order, w.seed,
                      "paged decode HBM GB/s (% of peak), int8 K/V, 32q/8kv d128",
                      "int8 decode-only step, batch 16, context 8192, 32 q heads / 8 KV heads, head_dim 128, "
                      "int8 K/V with one fp16 scale per (block, KV head), 32 layer pools",
                      traffic_name=None if args.partition_tokens else "paged_decode_int8_b16_ctx8k")


def c3_decode_bench(args, torch, pkv, C, workloads):
    """Decode-only step of the continuous-batching mix: 16 sequences at the
    config's seeded lengths U[128, 8192] + the appended token, fp16, 32 q / 8
    KV heads, over 32 layer pools in a seeded random block order (the
    config's fragmentation: a scrambled pool)."""
    w = workloads.c3_mixed()
    lens = [len(st[2]) + 1 for st in w.steps if st[0] == "prefill"]
    N = sum(-(-n // 16) for n in lens) + 16
    seed = w.seed if args.seed is None else args.seed
    order = np.random.default_rng(seed).permutation(N).astype(np.int32)
    decode_only_bench(args, torch, pkv, C, lens, HQ, HKV, "f16", order, seed,
                      "paged decode HBM GB/s (% of peak), fp16, continuous-batching mix",
                      "decode-only step, 16 sequences at U[128, 8192] + 1 tokens (seeded), 32 q heads / "
                      "8 KV heads, head_dim 128, fp16, scrambled block order, 32 layer pools",
                      traffic_name=None if args.partition_tokens or args.seed is not None
                      else "paged_decode_c3_mix_b16")


def shape_decode_bench(args, torch, pkv, C, workloads):
    """Decode-only step of any shape given on the command line."""
    global D
    D = args.head_dim
    if args.seed is None:
        args.seed = 7
    if args.context_list:
        lens = [int(x) for x in args.context_list.split(",")]
        args.batch = len(lens)
    elif args.lengths:
        lo, hi = args.lengths
        lens = np.random.default_rng(args.seed).integers(lo, hi + 1, args.batch).tolist()
    else:
        lens = [args.context] * args.batch
    N = sum(-(-n // 16) for n in lens) + 16
    order = np.random.default_rng(args.seed).permutation(N).astype(np.int32)
    desc = (f"decode-only step, {args.batch} sequences at "
            + (f"{args.context_list} tokens" if args.context_list
               else f"U[{args.lengths[0]}, {args.lengths[1]}] tokens (seed {args.seed})" if args.lengths
               else f"{args.context} tokens")
            + f", {args.q_heads} q heads / {args.kv_heads} KV heads, head_dim {D}, {args.dtype}, "
            f"{args.layers} layer pools")
    decode_only_bench(args, torch, pkv, C, lens, args.q_heads, args.kv_heads, args.dtype, order, args.seed,
                      f"paged decode HBM GB/s (% of peak), {args.dtype}, decode-only shape", desc)


def prefix_decode_bench(args, torch, pkv, C, workloads):
    """Shared-prefix decode step (the copy-on-write config's shape): one
    sequence prefilled to 2048 tokens and forked 31 times, private suffixes
    of the config's seeded U[64, 1024] lengths, one appended token each
    (fused into the decode launch), 32 q / 8 KV heads, d128, over 32 layer
    pools of seeded fp16 noise. The block state comes from the library's
    allocator (fork, copy-on-write reserve) in the config's block order. The
    step is timed twice, without and with the shared-prefix plan (layer 0
    launched directly with timing events, layers 1.. replayed from a HIP
    graph); the two outputs are compared."""
    dev = torch.device("cuda:0")
    K, W, L = args.steps, args.warmup, args.layers
    w = workloads.c4_prefix()
    prefix = next(len(st[2]) for st in w.steps if st[0] == "prefill")
    suffix = [len(st[2]) for st in w.steps if st[0] == "prefill"][1:]
    nseq = len(suffix)
    cache = pkv.PagedKVCache(L, w.num_blocks, HKV, D, "f16", w.free_order, dev)
    lib = C.load()
    sp = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    cache.pool.view(torch.float16).normal_(generator=gen)
    root = cache.create_seq()
    cache.reserve([root], [prefix])
    seqs = [root] + [cache.fork(root) for _ in range(nseq - 1)]
    cache.reserve(seqs, suffix)
    _, cow = cache.reserve(seqs, [1] * nseq)  # the decode step's token: its slot now, written in the launch
    cache.copy_blocks(cow)
    tables_h, lens_h = cache.block_tables(seqs)
    max_blocks = tables_h.shape[1]
    ctx = int(lens_h.max())
    plan = cache.plan_shared_prefix(seqs, num_q_heads=HQ)
    tables_d = torch.from_numpy(tables_h).to(dev)
    lens_d = torch.from_numpy(lens_h).to(dev)
    q = torch.empty((L, nseq, HQ, D), dtype=torch.float16, device=dev).normal_(generator=gen)
    kv_new = torch.empty((2, L, nseq, HKV, D), dtype=torch.float16, device=dev).normal_(generator=gen)

    def build(use_plan):
        out = torch.empty_like(q)
        if use_plan:
            nb = C.pkv_prefix_decode_workspace_bytes(cache.cfg, nseq, HQ, ctx, max_blocks, args.partition_tokens,
                                                     plan.n_groups)
        else:
            nb = C.pkv_decode_workspace_bytes(cache.cfg, nseq, HQ, ctx, args.partition_tokens)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        argv = []
        for layer in range(L):
            a = C.pkv_decode_args()
            a.cfg = ctypes.pointer(cache.cfg)
            a.pool_dev = cache.pool.data_ptr()
            a.layer = layer
            a.q_dev = q[layer].data_ptr()
            a.num_seqs = nseq
            a.num_q_heads = HQ
            a.block_tables_dev = tables_d.data_ptr()
            a.max_blocks = max_blocks
            a.ctx_lens_dev = lens_d.data_ptr()
            a.ctx_lens_host = C._i32p(lens_h)
            a.max_context = ctx
            a.out_dev = out[layer].data_ptr()
            a.scale = 1.0 / math.sqrt(D)
            a.workspace_dev = ws.data_ptr()
            a.workspace_bytes = ws.numel()
            a.partition_tokens = args.partition_tokens
            a.k_new_dev = kv_new[0, layer].data_ptr()
            a.v_new_dev = kv_new[1, layer].data_ptr()
            if use_plan:
                a.prefix_plan_dev = plan.dev.data_ptr()
                a.prefix_plan_host = C._i32p(plan.host)
                a.prefix_groups = plan.n_groups
            argv.append(a)
        return out, ws, argv

    def run(use_plan):
        out, ws, argv = build(use_plan)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        for group in ev:
            for e in group:
                e.record()
        ptrs = [ctypes.cast((ctypes.c_void_p * 4)(*[e.cuda_event for e in g]), ctypes.POINTER(ctypes.c_void_p))
                for g in ev]

        def launch(layer, events=None, stream_handle=None):
            a = argv[layer]
            a.timing_events = events
            C._check(lib.pkv_paged_decode(ctypes.byref(a), sp if stream_handle is None else stream_handle))

        for _ in range(W):
            for layer in range(L):
                launch(layer)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream().cuda_stream
            for layer in range(1, L):
                launch(layer, stream_handle=cs)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with no_collections():
            t0.record()
            for i in range(K):
                launch(0, ptrs[i])
                graph.replay()
            t1.record()
            torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / K
        split_ms = np.array([g[0].elapsed_time(g[1]) for g in ev])
        merge_ms = np.array([g[2].elapsed_time(g[3]) for g in ev])
        merged = all(t0.elapsed_time(g[2]) > 0 for g in ev)
        return ms, split_ms, merge_ms if merged else None, out

    ms0, split0_ms, merge0_ms, out0 = run(False)
    ms1, split1_ms, merge1_ms, out1 = run(True)
    split0, split1 = float(np.mean(split0_ms)) * 1e3, float(np.mean(split1_ms)) * 1e3
    merge0 = None if merge0_ms is None else float(np.mean(merge0_ms)) * 1e3
    merge1 = None if merge1_ms is None else float(np.mean(merge1_ms)) * 1e3
    diff = float((out0.float() - out1.float()).abs().max())
    kv_tok = 2 * HKV * D * 2
    groups = plan.groups()
    shared = sum(nb * 16 * (len(mem) - 1) for nb, mem in groups)  # tokens read once instead of per member
    logical = int(lens_h.sum())
    unique_bytes = (logical - shared) * kv_tok + nseq * HQ * D * 2 * 2 + tables_h.size * 4
    achieved = unique_bytes / (split1 * 1e-6) / 1e9
    print(json.dumps({
        "metric": "shared-prefix decode step tokens/s (32 sequences over one 2048-token prefix)",
        "value": round(nseq / (ms1 * 1e-3), 1), "unit": "tok/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms1, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"decode step with fused append, {nseq} sequences forked from one "
                               f"{prefix}-token prefix, private suffixes U[64, 1024] + 1, 32 q / 8 KV heads, "
                               f"head_dim 128, fp16, {L} layer pools", "layers": L,
                   "partition_tokens": args.partition_tokens or "auto", "plan_groups": plan.n_groups,
                   "shared_blocks": [nb for nb, _ in groups]},
        "with_plan": {"ms_per_step": round(ms1, 4), "decode_kernel_us": round(split1, 2),
                      "merge_kernel_us": None if merge1 is None else round(merge1, 2),
                      "decode_a5_a6_unique_bytes": decode_metric(split1_ms, merge1_ms, [unique_bytes])},
        "without_plan": {"ms_per_step": round(ms0, 4), "decode_kernel_us": round(split0, 2),
                         "merge_kernel_us": None if merge0 is None else round(merge0, 2),
                         "tok_s": round(nseq / (ms0 * 1e-3), 1)},
        "speedup": round(ms0 / ms1, 3),
        "max_abs_diff_plan_vs_no_plan": diff,
        "logical_kv_bytes": logical * kv_tok, "unique_kv_bytes": (logical - shared) * kv_tok,
        "roofline": {"bound": "hbm", "kernel": "paged_decode_kernel<128,4,f16> with shared-prefix work-groups",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "bytes_per_launch": int(unique_bytes)},
        "cpu_baseline": None,
    }), flush=True)


def prefill_bench(args, torch, pkv, C, workloads):
    """Prefill step: 4 fresh prompts of 2048 tokens, 32 q / 8 KV heads, d128,
    fp16 (or int8 pools with ``--dtype i8``: the append quantises on write),
    over 32 layer pools. Per layer the prompts' K/V rows are appended
    into their blocks (one bulk append of 8192 tokens) and attended
    causally (one prefill launch). The blocks come from the library's
    allocator in a seeded random order; K, V and q are seeded device noise
    (values do not change the timing). The prefill launch of layer 0 is
    bracketed by HIP events in every timed step."""
    dev = torch.device("cuda:0")
    K, W, L = args.steps, args.warmup, args.layers
    Bp, T = 4, 2048
    nblk = T // 16
    N = Bp * nblk
    order = np.random.default_rng(7).permutation(N).astype(np.int32)
    dt = args.dtype
    cache = pkv.PagedKVCache(L, N, HKV, D, dt, order, dev)
    lib = C.load()
    sp = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    seqs = [cache.create_seq() for _ in range(Bp)]
    slots, _ = cache.reserve(seqs, [T] * Bp)
    slots_d = torch.from_numpy(slots).to(dev)
    tables_h, lens_h = cache.block_tables(seqs, nblk)
    tables_d = torch.from_numpy(tables_h).to(dev)
    lens_d = torch.from_numpy(lens_h).to(dev)
    starts_h = (np.arange(Bp + 1) * T).astype(np.int32)
    starts_d = torch.from_numpy(starts_h).to(dev)
    kv = torch.empty((2, L, Bp * T, HKV, D), dtype=torch.float16, device=dev).normal_(generator=gen)
    q = torch.empty((L, Bp * T, HQ, D), dtype=torch.float16, device=dev).normal_(generator=gen)
    out = torch.empty_like(q)
    argv = []
    for layer in range(L):
        a = C.pkv_prefill_args()
        a.cfg = ctypes.pointer(cache.cfg)
        a.pool_dev = cache.pool.data_ptr()
        a.layer = layer
        a.q_dev = q[layer].data_ptr()
        a.num_seqs = Bp
        a.num_q_heads = HQ
        a.q_start_dev = starts_d.data_ptr()
        a.q_start_host = C._i32p(starts_h)
        a.block_tables_dev = tables_d.data_ptr()
        a.max_blocks = nblk
        a.ctx_lens_dev = lens_d.data_ptr()
        a.ctx_lens_host = C._i32p(lens_h)
        a.max_context = T
        a.out_dev = out[layer].data_ptr()
        a.scale = 1.0 / math.sqrt(D)
        argv.append(a)

    def step(ev=None):
        for layer in range(L):
            C._check(lib.pkv_append_kv(ctypes.byref(cache.cfg), cache.pool.data_ptr(), layer, kv[0, layer].data_ptr(),
                                       kv[1, layer].data_ptr(), slots_d.data_ptr(), Bp * T, sp))
            if layer == 0 and ev is not None:
                ev[0].record()
            C._check(lib.pkv_paged_prefill(ctypes.byref(argv[layer]), sp))
            if layer == 0 and ev is not None:
                ev[1].record()

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with no_collections():
        t0.record()
        for i in range(K):
            step(evs[i])
        t1.record()
        torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    pre = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3
    flops = 4.0 * HQ * D * Bp * (T * (T + 1) / 2)
    achieved = flops / (float(np.mean(pre)) * 1e-6) / 1e12
    print(json.dumps({
        "metric": f"paged prefill tokens/s (4 x 2048-token prompts, causal, 32q/8kv d128 {'fp16' if dt == 'f16' else 'int8 pool'})",
        "value": round(Bp * T / (ms * 1e-3), 1), "unit": "tok/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dt, "data": "synthetic",
        "config": {"workload": f"prefill step: {Bp} fresh prompts of {T} tokens appended into 16-token blocks "
                               f"and attended causally, 32 q / 8 KV heads, head_dim 128, "
                               f"{'fp16' if dt == 'f16' else 'int8 pool (quantised on append)'}, {L} layer pools",
                   "layers": L},
        "prefill_kernel_us": round(float(np.mean(pre)), 2),
        "prefill_kernel_us_p10_p90": [round(float(np.percentile(pre, 10)), 2), round(float(np.percentile(pre, 90)), 2)],
        "roofline": {"bound": "mfma", "kernel": f"prefill_kernel<128,4,{'f16' if dt == 'f16' else 'i8'}> (causal paged prefill)",
                     "achieved": round(achieved, 1), "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_MFMA_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": flops},
        "cpu_baseline": None,
    }), flush=True)


def cpu_baseline(w, gpu_out, gpu_tables, gpu_lens, budget_s, decode_bytes):
    """Time the CPU oracle (fp64 NumPy, as it stands) on whole sequences of
    layer 0 of the first decode step until about ``budget_s`` seconds of CPU
    work; report GB/s of the same algorithmic bytes and, for information, the
    GPU's max abs error on that sample."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from oracle_driver import OracleRun

    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    o = OracleRun(w).run(decode=False)
    rec = o.decodes[0]
    assert np.array_equal(rec["tables"], gpu_tables[:, :rec["tables"].shape[1]])
    assert np.array_equal(rec["lens"], gpu_lens)
    # one sequence (all 32 q heads) at a time, cycling over the batch until
    # the budget is spent; the GPU's error is taken on the first pass
    done, err, t_total = 0, 0.0, 0.0
    while t_total < budget_s:
        b = done % B
        t = time.perf_counter()
        ref = oracle.decode(o.cache, rec["q"][b:b + 1], rec["tables"][b:b + 1], rec["lens"][b:b + 1], 0, w.scale)
        t_total += time.perf_counter() - t
        if done < B:
            err = max(err, float(np.abs(gpu_out[b].astype(np.float64) - ref[0]).max()))
        done += 1
    lens = np.resize(rec["lens"], done)
    nbytes = decode_bytes(lens, True)
    return {
        "value": round(nbytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": blas,
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "seconds": round(t_total, 2),
        "sample": f"layer 0 of the first decode step: {done} single-sequence decodes (cycling over the "
                  f"{B} sequences at context {int(rec['lens'][0])}, all 32 q heads each; fp64 NumPy gather "
                  f"through the block table + softmax(qK^T/sqrt(d))V)",
        "gpu_max_abs_err_on_sample": err,
    }


if __name__ == "__main__":
    main()
