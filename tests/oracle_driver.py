"""Replays a seeded workload script against the CPU oracle.

Test infrastructure: records every host-visible result (slots, copy-on-write
pairs, block tables, lengths, free list) and every decode output, so the
library's results can be compared with them step by step.
"""

import numpy as np

import oracle
from workloads import replay_churn


class OracleRun:
    def __init__(self, w, layer=0, fill=None):
        self.w = w
        self.layer = layer
        self.alloc = oracle.RefAllocator(w.num_blocks, w.free_order)
        # fp16 store; for a bulk-quantised int8 workload this is the
        # unquantised shadow that is quantised just before each decode; an
        # int8 workload written by append quantises every token on write.
        self.i8_append = w.dtype == "i8" and w.i8_write == "append"
        self.cache = oracle.RefCache(1, w.num_blocks, w.num_kv_heads, w.head_dim,
                                     "i8" if self.i8_append else "f16", fill=None if self.i8_append else fill)
        self.q8 = None
        self.seq = {}
        self.reserves = []  # (step index, name, slots, cow pairs)
        self.decodes = []  # dicts: names, tables, lens, q, out
        self.prefills = []  # dicts: names, q_lens, tables, lens, q, out
        self.churn_log = []

    # -- steps -----------------------------------------------------------
    def _reserve(self, idx, name, n):
        slots, cow = self.alloc.seq_reserve(self.seq[name], n)
        self.reserves.append((idx, name, list(slots), list(cow)))
        return slots, cow

    def run(self, decode=True):
        for idx, step in enumerate(self.w.steps):
            kind = step[0]
            if kind == "create":
                self.seq[step[1]] = self.alloc.seq_create()
            elif kind == "prefill":
                _, name, k, v = step
                slots, cow = self._reserve(idx, name, len(k))
                self.cache.copy_blocks(cow)
                self.cache.append(0, k, v, slots)
            elif kind == "append":
                _, names, k, v = step
                all_slots, all_cow = [], []
                for name in names:
                    slots, cow = self._reserve(idx, name, 1)
                    all_slots += slots
                    all_cow += cow
                self.cache.copy_blocks(all_cow)
                self.cache.append(0, k, v, all_slots)
            elif kind == "fork":
                self.seq[step[2]] = self.alloc.seq_fork(self.seq[step[1]])
            elif kind == "free":
                self.alloc.seq_free(self.seq.pop(step[1]))
            elif kind == "churn":
                self._churn(step[1])
            elif kind == "decode":
                self._decode(step[1], step[2], decode)
            elif kind == "prefill_attn":
                self._prefill_attn(step[1], step[2], step[3], decode)
            else:
                raise ValueError(kind)
        return self

    def _churn(self, churn):
        tags = {}

        def alloc(tag, n):
            sid = self.alloc.seq_create()
            try:
                self.alloc.seq_reserve(sid, n)
            except oracle.NoBlocks:
                self.alloc.seq_free(sid)
                self.churn_log.append(("refused", tag, n))
                return False
            tags[tag] = sid
            self.churn_log.append(("alloc", tag, n))
            return True

        def free(tag):
            self.alloc.seq_free(tags.pop(tag))
            self.churn_log.append(("free", tag))

        replay_churn(churn, alloc, free)

    def filled_counts(self):
        """Live slots per physical block (for the int8 quantiser)."""
        filled = np.zeros(self.w.num_blocks, np.int64)
        for sid, table in self.alloc.tables.items():
            n = self.alloc.lens[sid]
            for j, blk in enumerate(table):
                filled[blk] = max(filled[blk], min(16, n - 16 * j))
        return filled

    def quantised_cache(self):
        K8, V8, scales = oracle.quantize_pool_int8(self.cache.K, self.cache.V, self.filled_counts())
        c = oracle.RefCache(1, self.w.num_blocks, self.w.num_kv_heads, self.w.head_dim, "i8")
        c.K[...] = K8
        c.V[...] = V8
        c.scales[...] = scales
        return c

    def _decode(self, names, q, compute):
        sids = [self.seq[n] for n in names]
        max_blocks = max(len(self.alloc.tables[s]) for s in sids)
        tables, lens = self.alloc.block_tables(sids, max_blocks)
        rec = {"names": list(names), "tables": np.array(tables, np.int32),
               "lens": np.array(lens, np.int32), "q": q, "out": None}
        if self.w.dtype == "i8":
            self.q8 = self.cache if self.i8_append else self.quantised_cache()
        if compute:
            cache = self.q8 if self.w.dtype == "i8" else self.cache
            rec["out"] = oracle.decode(cache, q, tables, lens, 0, self.w.scale)
        self.decodes.append(rec)

    def _prefill_attn(self, names, q_lens, q, compute):
        sids = [self.seq[n] for n in names]
        max_blocks = max(len(self.alloc.tables[s]) for s in sids)
        tables, lens = self.alloc.block_tables(sids, max_blocks)
        rec = {"names": list(names), "q_lens": list(q_lens), "tables": np.array(tables, np.int32),
               "lens": np.array(lens, np.int32), "q": q, "out": None}
        if compute:
            rec["out"] = oracle.prefill(self.cache, q, q_lens, tables, lens, 0, self.w.scale)
        self.prefills.append(rec)
