"""Seeded synthetic workloads for the paged KV cache.

This module is the only source of randomness for tests and the benchmark and
the only thing the HIP library and the CPU oracle have in common: it draws
request lengths, physical-block orders, churn recipes and fp16 K/V/q values,
and it contains none of the method's arithmetic (no attention, no block
bookkeeping). Each workload is a script of steps that a driver replays
against either implementation.

Step kinds::

    ("create", name)                 new empty sequence
    ("prefill", name, k, v)          append len(k) tokens to one sequence
    ("append", names, k, v)          append one token to each named sequence
    ("fork", parent, child)          child shares parent's blocks
    ("free", name)                   release a sequence
    ("churn", Churn)                 alloc/free traffic of earlier requests
    ("decode", names, q)             one decode step over the named sequences
    ("prefill_attn", names, q_lens, q)  causal attention of each named
                                     sequence's newest q_lens[i] tokens (already
                                     written) over its cache; q is [sum q_lens, Hq, D]

``k``/``v`` are ``[n, Hkv, D]`` fp16 and ``q`` is ``[B, Hq, D]`` fp16, drawn as
``standard_normal(float32).astype(float16)``. Draws follow one fixed order:
physical order / churn, then lengths, then K/V per sequence in order, then
the new token's k/v, then q.
"""

from dataclasses import dataclass, field
import math

import numpy as np


@dataclass
class Churn:
    """Alloc/free traffic of earlier requests that scrambles the free list.

    Replayed by :func:`replay_churn`: request ``i`` asks for ``lengths[i]``
    tokens; while the pool refuses it, a random live request is freed; after
    each admission a coin (p = 0.5) may free one random live request; at the
    end every live request is freed in random order. All random choices come
    from the pre-drawn ``uniforms`` stream.
    """

    lengths: np.ndarray
    uniforms: np.ndarray


def replay_churn(churn, alloc, free):
    """Drive ``alloc(tag, n) -> bool`` and ``free(tag)`` through the churn.

    ``alloc`` returns False when the pool is out of blocks (and must then have
    changed nothing)."""
    it = iter(churn.uniforms)

    def pick(live):
        return live.pop(min(int(next(it) * len(live)), len(live) - 1))

    live = []
    for i, n in enumerate(churn.lengths):
        while not alloc(i, int(n)):
            if not live:
                raise RuntimeError("request larger than the whole pool")
            free(pick(live))
        live.append(i)
        if next(it) < 0.5 and live:
            free(pick(live))
    while live:
        free(pick(live))


@dataclass
class Workload:
    name: str
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f16" or "i8"
    free_order: np.ndarray  # int32 permutation of the block ids
    steps: list = field(default_factory=list)
    seed: int = 0
    layers: int = 1  # layers whose contents come from this script
    # int8 workloads: "bulk" = the fp16 K/V are quantised block by block on
    # the host before decode; "append" = every token is quantised on write
    i8_write: str = "bulk"
    # softmax scale; None: 1 / sqrt(head_dim)
    softmax_scale: float = None

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim) if self.softmax_scale is None else self.softmax_scale

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def _scaled(x, factor):
    return x if factor == 1.0 else (x.astype(np.float32) * np.float32(factor)).astype(np.float16)


def _decode_batch(name, rng, N, Hq, Hkv, D, lens, free_order, dtype="f16", append=True, v_scale=1.0):
    """Shared shape of C1, C2, C5 and the headline: B sequences prefilled to
    ``lens``, one appended token each (unless ``append`` is False), then one
    decode step. ``v_scale`` multiplies every V value (after the same draws)."""
    w = Workload(name, N, Hq, Hkv, D, dtype, free_order)
    names = [f"s{i}" for i in range(len(lens))]
    for s in names:
        w.steps.append(("create", s))
    for s, n in zip(names, lens):
        w.steps.append(("prefill", s, _normal(rng, (n, Hkv, D)), _scaled(_normal(rng, (n, Hkv, D)), v_scale)))
    if append:
        B = len(lens)
        w.steps.append(("append", names, _normal(rng, (B, Hkv, D)), _scaled(_normal(rng, (B, Hkv, D)), v_scale)))
    w.steps.append(("decode", names, _normal(rng, (len(lens), Hq, D))))
    return w


def c1_tiny(seed=1):
    """Tiny one-layer case: 4 sequences at {5,17,33,64} tokens, 4 q heads,
    2 KV heads, head_dim 64, a 64-block pool in random physical order; one
    appended token each, then decode over {6,18,34,65}."""
    rng = np.random.default_rng(seed)
    N = 64
    order = rng.permutation(N).astype(np.int32)
    w = _decode_batch("c1_tiny", rng, N, 4, 2, 64, [5, 17, 33, 64], order)
    w.seed = seed
    return w


def c2_llama_b8(seed=2):
    """Llama-7B-shaped layer (32 q / 8 KV heads, d128): batch 8 at 1024
    tokens, pool of exactly 8 * ceil(1025/16) = 520 blocks in random order,
    one appended token, decode over 1025."""
    rng = np.random.default_rng(seed)
    N = 8 * 65
    order = rng.permutation(N).astype(np.int32)
    w = _decode_batch("c2_llama_b8", rng, N, 32, 8, 128, [1024] * 8, order)
    w.seed = seed
    return w


def c3_mixed(seed=3, batch=16, churn_requests=200, dtype="f16", Hq=32):
    """Continuous-batching mix: 16 sequences of U[128, 8192] tokens, pool
    scrambled by 200 earlier requests of U[1, 8192] tokens. ``dtype="i8"``:
    the same draws, stored block-quantised as int8. ``Hq`` query heads over
    the 8 KV heads (32 by default)."""
    rng = np.random.default_rng(seed)
    N = 16 * 513
    churn = Churn(lengths=rng.integers(1, 8193, churn_requests),
                  uniforms=rng.random(8 * churn_requests + 64))
    lens = rng.integers(128, 8193, batch).tolist()
    w = Workload("c3_mixed", N, Hq, 8, 128, dtype, np.arange(N, dtype=np.int32))
    w.steps.append(("churn", churn))
    names = [f"s{i}" for i in range(batch)]
    for s in names:
        w.steps.append(("create", s))
    for s, n in zip(names, lens):
        w.steps.append(("prefill", s, _normal(rng, (n, 8, 128)), _normal(rng, (n, 8, 128))))
    w.steps.append(("append", names, _normal(rng, (batch, 8, 128)), _normal(rng, (batch, 8, 128))))
    w.steps.append(("decode", names, _normal(rng, (batch, Hq, 128))))
    w.seed = seed
    return w


def c4_prefix(seed=4, sharers=32, prefix=2048, dtype="f16"):
    """Copy-on-write prefix sharing: one 2048-token prefix shared by 32
    sequences, private suffixes of U[64, 1024] tokens, one decode step; then
    the lowest-index sequence whose length is not a multiple of 16 forks, the
    child appends one token (into the shared partial tail block) and
    [parent, child] decode."""
    rng = np.random.default_rng(seed)
    N = 2304
    order = rng.permutation(N).astype(np.int32)
    suffix = rng.integers(64, 1025, sharers).tolist()
    w = Workload("c4_prefix", N, 32, 8, 128, dtype, order)
    w.i8_write = "append"  # int8: the shared prefix and every suffix token quantised on write
    names = [f"s{i}" for i in range(sharers)]
    w.steps.append(("create", names[0]))
    w.steps.append(("prefill", names[0], _normal(rng, (prefix, 8, 128)), _normal(rng, (prefix, 8, 128))))
    for s in names[1:]:
        w.steps.append(("fork", names[0], s))
    for s, n in zip(names, suffix):
        w.steps.append(("prefill", s, _normal(rng, (n, 8, 128)), _normal(rng, (n, 8, 128))))
    w.steps.append(("append", names, _normal(rng, (sharers, 8, 128)), _normal(rng, (sharers, 8, 128))))
    w.steps.append(("decode", names, _normal(rng, (sharers, 32, 128))))
    lengths = [prefix + n + 1 for n in suffix]
    parent = next(i for i, n in enumerate(lengths) if n % 16)
    w.steps.append(("fork", names[parent], "child"))
    w.steps.append(("append", ["child"], _normal(rng, (1, 8, 128)), _normal(rng, (1, 8, 128))))
    w.steps.append(("decode", [names[parent], "child"], _normal(rng, (2, 32, 128))))
    w.seed = seed
    return w


def prefix_forest(seed, groups=((700, 6),), singles=2, Hq=32, Hkv=8, D=128, suffix=(1, 300), N=None,
                  shuffle=True, dtype="f16"):
    """Several shared prefixes in one batch: for each ``(prefix, sharers)`` a
    root prefilled to ``prefix`` tokens and forked ``sharers - 1`` times; every
    member (root included) then prefills a private suffix of U[suffix]
    tokens (0 allowed); ``singles`` unrelated sequences of U[1, max prefix]
    tokens; one appended token each; one decode over all of them in a
    shuffled batch order (members of a group not adjacent). ``dtype="i8"``:
    every token is quantised as it is written."""
    rng = np.random.default_rng(seed)
    sizes = [(int(p), int(n)) for p, n in groups]
    top = max([p for p, _ in sizes] + [1])
    suf = [rng.integers(suffix[0], suffix[1] + 1, n).tolist() for _, n in sizes]
    single_lens = rng.integers(1, top + 1, singles).tolist()
    if N is None:
        need = sum(-(-(p + 1) // 16) + sum(-(-(x + 1) // 16) + 1 for x in sf) for (p, _), sf in zip(sizes, suf))
        need += sum(-(-(n + 1) // 16) for n in single_lens)
        N = need + 8
    order = rng.permutation(N).astype(np.int32)
    w = Workload("prefix_forest", N, Hq, Hkv, D, dtype, order)
    w.i8_write = "append"
    names = []
    for gi, ((p, n), sf) in enumerate(zip(sizes, suf)):
        root = f"g{gi}m0"
        w.steps.append(("create", root))
        w.steps.append(("prefill", root, _normal(rng, (p, Hkv, D)), _normal(rng, (p, Hkv, D))))
        members = [root] + [f"g{gi}m{i}" for i in range(1, n)]
        for m in members[1:]:
            w.steps.append(("fork", root, m))
        for m, x in zip(members, sf):
            if x:
                w.steps.append(("prefill", m, _normal(rng, (x, Hkv, D)), _normal(rng, (x, Hkv, D))))
        names += members
    for i, n in enumerate(single_lens):
        w.steps.append(("create", f"u{i}"))
        w.steps.append(("prefill", f"u{i}", _normal(rng, (n, Hkv, D)), _normal(rng, (n, Hkv, D))))
        names.append(f"u{i}")
    if shuffle:
        names = [names[i] for i in rng.permutation(len(names))]
    B = len(names)
    w.steps.append(("append", names, _normal(rng, (B, Hkv, D)), _normal(rng, (B, Hkv, D))))
    w.steps.append(("decode", names, _normal(rng, (B, Hq, D))))
    w.seed = seed
    return w


def prefill_chunks(seed, cached, chunk, Hq=32, Hkv=8, D=128, N=None, shuffle=True, dtype="f16"):
    """Paged prefill: sequence i holds ``cached[i]`` earlier tokens (0 = a
    fresh prompt), then a chunk of ``chunk[i]`` new tokens is written and
    attended causally over the whole cache. Pool blocks in random order
    (``shuffle``); the earlier tokens and the chunk are written in separate
    steps, so a chunk may start inside a partly filled block. ``dtype="i8"``:
    every token is quantised as it is written."""
    rng = np.random.default_rng(seed)
    B = len(chunk)
    if N is None:
        N = sum(-(-(c + k) // 16) for c, k in zip(cached, chunk)) + 4
    order = rng.permutation(N).astype(np.int32)  # drawn either way: the values that follow stay the same
    if not shuffle:
        order = np.arange(N, dtype=np.int32)
    w = Workload("prefill_chunks", N, Hq, Hkv, D, dtype, order)
    w.i8_write = "append"
    names = [f"s{i}" for i in range(B)]
    for s_ in names:
        w.steps.append(("create", s_))
    for s_, c in zip(names, cached):
        if c:
            w.steps.append(("prefill", s_, _normal(rng, (c, Hkv, D)), _normal(rng, (c, Hkv, D))))
    for s_, k in zip(names, chunk):
        w.steps.append(("prefill", s_, _normal(rng, (k, Hkv, D)), _normal(rng, (k, Hkv, D))))
    w.steps.append(("prefill_attn", names, [int(k) for k in chunk], _normal(rng, (int(sum(chunk)), Hq, D))))
    w.seed = seed
    return w


def c5_int8(seed=5, batch=16, ctx=8192):
    """Long-context int8 KV: 16 sequences at 8192 tokens of N(0,1) fp16 data
    stored as int8 with one fp16 scale per (block, KV head); decode only."""
    rng = np.random.default_rng(seed)
    N = batch * (-(-ctx // 16))
    order = rng.permutation(N).astype(np.int32)
    w = _decode_batch("c5_int8", rng, N, 32, 8, 128, [ctx] * batch, order, dtype="i8", append=False)
    w.seed = seed
    return w


def headline(seed=6, batch=16, ctx=8192, spare_blocks=0):
    """The 32q/8kv d128 fp16 decode step at batch 16 and 8K context: 16
    sequences prefilled to 8192 tokens, one appended token each, decode over
    8193. Pool: 16 * 513 blocks (+ ``spare_blocks`` for longer runs)."""
    rng = np.random.default_rng(seed)
    N = batch * (-(-(ctx + 1) // 16)) + spare_blocks
    order = rng.permutation(N).astype(np.int32)
    w = _decode_batch("headline_b16_ctx8k", rng, N, 32, 8, 128, [ctx] * batch, order)
    w.seed = seed
    return w


def uniform_decode(seed, batch, ctx, Hq=32, Hkv=8, D=128, dtype="f16", append=True, i8_write="bulk",
                   lens=None):
    """``batch`` sequences prefilled to ``ctx`` tokens each (or to ``lens``),
    one appended token each unless ``append`` is False, then one decode step;
    a pool of exactly the blocks needed, in seeded random order."""
    rng = np.random.default_rng(seed)
    lens = [ctx] * batch if lens is None else [int(n) for n in lens]
    N = sum(-(-(n + 1) // 16) for n in lens) + 2
    order = rng.permutation(N).astype(np.int32)
    w = _decode_batch(f"uniform_{seed}", rng, N, Hq, Hkv, D, lens, order, dtype=dtype, append=append)
    w.seed = seed
    w.i8_write = i8_write
    return w


def tiny_random(seed, B=3, Hq=4, Hkv=2, D=64, max_len=40, N=None, dtype="f16", v_scale=1.0, i8_write="bulk"):
    """Small random shapes for brute-force and edge-case checks; ``v_scale``
    stretches the V values (large int8 scales)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, B).tolist()
    if N is None:
        N = sum(-(-(n + 1) // 16) for n in lens) + 4
    order = rng.permutation(N).astype(np.int32)
    w = _decode_batch(f"tiny_{seed}", rng, N, Hq, Hkv, D, lens, order, dtype=dtype, v_scale=v_scale)
    w.seed = seed
    w.i8_write = i8_write
    return w


CONFIGS = {
    "c1": c1_tiny,
    "c2": c2_llama_b8,
    "c3": c3_mixed,
    "c4": c4_prefix,
    "c5": c5_int8,
    "headline": headline,
}


class PrefixHashModel:
    """A stand-in for a model's projections and sampler in serving tests.

    The K, V and q rows of the token at position t are seeded normal draws
    keyed by a rolling hash of tokens 0..t, so they depend on the token
    prefix only (as a model's would, and as prefix caching requires). The
    next token depends on the request and its tokens only, never on the
    attention output, so every schedule is reproducible."""

    def __init__(self, Hq, Hkv, D, vocab=50):
        self.Hq, self.Hkv, self.D, self.vocab = Hq, Hkv, D, vocab

    @staticmethod
    def _hashes(tokens, upto):
        h, out = 0x51ED270B27C35C49, []
        for t in tokens[:upto]:
            h = ((h ^ (int(t) + 0x9E3779B9)) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
            out.append(h)
        return out

    def rows(self, req, tokens, start, count):
        hs = self._hashes(tokens, start + count)[start:]
        k = np.empty((count, self.Hkv, self.D), np.float16)
        v = np.empty_like(k)
        q = np.empty((count, self.Hq, self.D), np.float16)
        for i, h in enumerate(hs):
            rng = np.random.default_rng(h)
            k[i] = _normal(rng, (self.Hkv, self.D))
            v[i] = _normal(rng, (self.Hkv, self.D))
            q[i] = _normal(rng, (self.Hq, self.D))
        return k, v, q

    def next_token(self, req, tokens, out_row=None):
        return (7 * int(req) + 3 * len(tokens) + int(tokens[-1])) % self.vocab


def serving_requests(seed, n_req=12, systems=(40, 100), user=(1, 60), max_new=(1, 24)):
    """Requests for serving tests: each prompt is one of a few shared system
    prompts (lengths ``systems``) followed by U[user] private tokens;
    ``max_new`` ~ U[max_new]. Returns [(req, prompt, max_new)]."""
    rng = np.random.default_rng(seed)
    sys_prompts = [list(range(1000 * (k + 1), 1000 * (k + 1) + n)) for k, n in enumerate(systems)]
    out = []
    for rid in range(1, n_req + 1):
        base = sys_prompts[int(rng.integers(len(sys_prompts)))]
        tail = rng.integers(0, 50, int(rng.integers(user[0], user[1] + 1))).tolist()
        out.append((rid, base + tail, int(rng.integers(max_new[0], max_new[1] + 1))))
    return out
