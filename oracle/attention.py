"""Decode attention by its definition.  Test infrastructure only (see the package header).

The method (paged decode with split-K partitions and an online softmax) is
exact: up to rounding it reaches the plain attention of the new token's query
over every cached token, ``softmax(q K^T / sqrt(d)) V`` ([p2] §1.2). So the
oracle computes that definition directly, in fp64, over the tokens gathered
through the block table in logical order ([p2] §2.2 pseudocode: attend over
the cache up to and including the token just appended; [p2] §3.2: the
block table maps logical blocks to physical blocks).

Readings taken where the pages are silent:

* GQA grouping ([p1] §二, [p2] §4.2 say several query heads share one K/V
  head, not which): query head ``h`` uses KV head ``h // (Hq // Hkv)``,
  i.e. contiguous groups.
* Softmax scale is ``1/sqrt(D)`` unless the caller passes one.
* ``context_len`` counts every token the query attends to, the one just
  appended included.
"""

import math

import numpy as np

from .sizes import BLOCK_TOKENS


def gather(store, layer, table, n, g, scales=None, which=0):
    """The ``n`` cached rows of KV head ``g`` in logical order, as fp64.

    Row ``t`` lives at offset ``t % 16`` of physical block
    ``table[t // 16]`` ([p2] §3.2). For an int8 store the rows are
    dequantised as ``q * scale`` with the block's scale (``which`` = 0 for K,
    1 for V); the product is exact in fp64.
    """
    nblk = -(-n // BLOCK_TOKENS)
    parts = []
    for j in range(nblk):
        blk = int(table[j])
        tile = store[layer, blk, g].astype(np.float64)  # [16, D]
        if scales is not None:
            tile = tile * np.float64(scales[layer, blk, g, which])
        parts.append(tile)
    return np.concatenate(parts)[:n]


def decode_seq_head(Kc, Vc, q, scale):
    """``softmax(q . Kc^T * scale) . Vc`` for one query row, fp64 ([p2] §1.2).

    ``Kc, Vc`` are ``[n, D]``; the max is subtracted before ``exp`` only to
    keep the exponentials finite (it cancels in the ratio)."""
    s = (Kc @ np.asarray(q, np.float64)) * np.float64(scale)
    e = np.exp(s - s.max())
    p = e / e.sum()
    return p @ Vc


def decode(cache, q, block_tables, context_lens, layer=0, scale=None):
    """Paged decode for a batch: ``out[b, h] = attention(q[b, h], K_b, V_b)``.

    ``q`` is ``[B, Hq, D]`` (fp16 values, promoted to fp64), ``block_tables``
    rows list the physical blocks of each sequence in logical order and
    ``context_lens[b]`` is the number of tokens attended. Returns fp64
    ``[B, Hq, D]``.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = cache.kv_heads
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((B, Hq, D), np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n <= 0:
            raise ValueError("context_len must be >= 1")
        for g in range(Hkv):
            Kc = gather(cache.K, layer, block_tables[b], n, g, cache.scales, 0)
            Vc = gather(cache.V, layer, block_tables[b], n, g, cache.scales, 1)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = decode_seq_head(Kc, Vc, q[b, h], scale)
    return out


def brute_decode(cache, q, block_tables, context_lens, layer=0, scale=None):
    """The same attention as ``decode`` in plain Python floats and loops.

    No NumPy arithmetic: each score is a Python sum of products, each weight a
    ``math.exp``. For tiny inputs only; it checks ``decode`` by brute force.
    """
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = cache.kv_heads
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        n = int(context_lens[b])
        for h in range(Hq):
            g = h // G
            qv = [float(x) for x in q[b][h]]
            scores, rows = [], []
            for t in range(n):
                blk = int(block_tables[b][t // BLOCK_TOKENS])
                off = t % BLOCK_TOKENS
                krow = [float(x) for x in cache.K[layer, blk, g, off]]
                vrow = [float(x) for x in cache.V[layer, blk, g, off]]
                if cache.scales is not None:
                    sk = float(cache.scales[layer, blk, g, 0])
                    sv = float(cache.scales[layer, blk, g, 1])
                    krow = [x * sk for x in krow]
                    vrow = [x * sv for x in vrow]
                dot = 0.0
                for d in range(D):
                    dot += qv[d] * krow[d]
                scores.append(dot * scale)
                rows.append(vrow)
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            total = sum(weights)
            for d in range(D):
                acc = 0.0
                for t in range(n):
                    acc += weights[t] * rows[t][d]
                out[b][h][d] = acc / total
    return out


def prefill(cache, q, q_lens, block_tables, context_lens, layer=0, scale=None):
    """Attention of each sequence's newest ``q_lens[b]`` tokens over its cache.

    The prefill phase feeds a prompt's tokens in together ([p1] §二; [p2]
    §1.3) and writes their K/V into the cache ([p2] §2.2); Flash Attention
    tiles this attention without changing its result ([p1] §四). Reading
    taken: the attention is causal. Token ``i`` of the chunk sits at logical
    position ``p = context_lens[b] - q_lens[b] + i`` and attends to tokens
    ``0..p``, itself included, which is what decoding the chunk one token at
    a time would give ([p2] §2.2 pseudocode: attend over ``[:cache_len+1]``
    after appending) and what makes cached K/V reusable ([p1] §二). A chunk
    may follow cached tokens (``p`` starts above 0); a sequence with an empty
    chunk contributes no rows.

    ``q`` is ``[T, Hq, D]`` with sequence ``b``'s tokens at rows
    ``sum(q_lens[:b]) ..``; the cache must already hold each sequence's
    ``context_lens[b]`` tokens, the chunk's own included. Returns fp64
    ``[T, Hq, D]``. Per (sequence, KV head) the scores are one matrix product
    of the gathered rows, positions after ``p`` are excluded before the
    softmax, and the weights multiply V.
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = cache.kv_heads
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if int(np.sum(q_lens)) != T:
        raise ValueError("q_lens must add up to the rows of q")
    out = np.empty((T, Hq, D), np.float64)
    row0 = 0
    for b, ql in enumerate(q_lens):
        ql, n = int(ql), int(context_lens[b])
        if ql < 0 or ql > n or n < 1:
            raise ValueError("need 0 <= q_lens[b] <= context_lens[b] and context_lens[b] >= 1")
        if ql == 0:  # no new tokens in this sequence: no rows
            continue
        pos = np.arange(n - ql, n)  # logical positions of the chunk's tokens
        visible = np.arange(n)[None, :] <= pos[:, None]  # [ql, n]
        for g in range(Hkv):
            Kc = gather(cache.K, layer, block_tables[b], n, g, cache.scales, 0)
            Vc = gather(cache.V, layer, block_tables[b], n, g, cache.scales, 1)
            for h in range(g * G, (g + 1) * G):
                s = (q[row0:row0 + ql, h].astype(np.float64) @ Kc.T) * np.float64(scale)  # [ql, n]
                s = np.where(visible, s, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                out[row0:row0 + ql, h] = (e / e.sum(axis=1, keepdims=True)) @ Vc
        row0 += ql
    return out
