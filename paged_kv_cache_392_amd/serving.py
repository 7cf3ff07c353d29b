"""Continuous batching on one GPU: the library's step planner decides every
step, its kernels do the work.

Per step ([p2] §3.3): the planner (``pkv_sched_step``) grants decode slots,
admits waiting requests from the prefix cache and cuts prefill chunks; the
loop copies any copy-on-write blocks, writes each planned token's K/V into
its slot (``pkv_append_kv``), attends prefill chunks causally
(``pkv_paged_prefill``) and decode tokens (``pkv_paged_decode``), and hands
the planner the next token of every request whose newest token was just
computed (``pkv_sched_commit``), which finishes requests and frees their
blocks at once.

There is no model here: a caller-supplied ``model`` stands in for the
projections and the sampler. ``model.rows(req, tokens, start, count)``
returns fp16 ``k, v [count, Hkv, D]`` and ``q [count, Hq, D]`` for tokens
``start .. start + count - 1`` of a request whose tokens so far are
``tokens``; ``model.next_token(req, tokens, out_row)`` picks the next token
from the attention output of the newest token. K/V rows must depend only on
the token prefix (as a model's do), so blocks shared through the prefix
cache hold the right values.
"""

import numpy as np
import torch

from . import _capi as C
from .cache import _dev_i32


class ServingLoop:
    def __init__(self, cache, num_q_heads, max_running, prefill_budget, model, layer=0):
        """``cache`` may hold fp16 or int8 K/V: on int8 pools every token is
        quantised as it is written (``pkv_append_kv``)."""
        self.cache = cache
        self.Hq = num_q_heads
        self.model = model
        self.layer = layer
        self.max_running, self.prefill_budget = max_running, prefill_budget
        self.sched = C.pkv_sched_create(cache.handle, max_running, prefill_budget)
        self.plan = C.StepPlan(max_running, prefill_budget)
        self.steps = 0

    def close(self):
        if self.sched:
            C.pkv_sched_destroy(self.sched)
            self.sched = None

    def submit(self, req, prompt, max_new):
        C.pkv_sched_submit(self.sched, req, prompt, max_new)

    def tokens(self, req):
        return C.pkv_sched_request(self.sched, req)[0]

    def pending(self):
        waiting, running, _ = C.pkv_sched_counts(self.sched)
        return waiting + running

    def step(self):
        """Plan and run one step. Returns ``(plan, outputs, finished)``:
        ``outputs[i]`` is the fp16 ``[count, Hq, D]`` attention output of
        plan item i; ``plan["attn"][kind]`` records the ``(seqs, tables,
        context_lens)`` each attention call of the step read (host copies)."""
        plan = C.pkv_sched_step(self.sched, self.plan)
        items = plan["items"]
        dev = self.cache.device
        self.cache.copy_blocks(np.array(plan["cow"], np.int32).reshape(-1, 2))
        toks = {it[0]: self.tokens(it[0]) for it in items}
        ks, vs, qs, slots = [], [], [], []
        for req, _seq, _kind, start, count, islots, _c in items:
            k, v, q = self.model.rows(req, toks[req], start, count)
            ks.append(k)
            vs.append(v)
            qs.append(q)
            slots += islots
        outputs = [None] * len(items)
        plan["attn"] = {}
        if items:
            kd = torch.from_numpy(np.ascontiguousarray(np.concatenate(ks))).to(dev)
            vd = torch.from_numpy(np.ascontiguousarray(np.concatenate(vs))).to(dev)
            self.cache.write(self.layer, kd, vd, _dev_i32(np.array(slots, np.int32), dev))
            for kind in (C.PKV_STEP_PREFILL, C.PKV_STEP_DECODE):
                idx = [i for i, it in enumerate(items) if it[2] == kind]
                if not idx:
                    continue
                seqs = [items[i][1] for i in idx]
                ctx = np.array([items[i][3] + items[i][4] for i in idx], np.int32)
                tables, _ = C.pkv_build_block_tables(self.cache.handle, seqs,
                                                     max(len(C.pkv_seq_block_table(self.cache.handle, s))
                                                         for s in seqs))
                plan["attn"][kind] = (seqs, tables.copy(), ctx.copy())
                td = torch.from_numpy(tables).to(dev)
                ld = torch.from_numpy(ctx).to(dev)
                qd = torch.from_numpy(np.ascontiguousarray(np.concatenate([qs[i] for i in idx]))).to(dev)
                if kind == C.PKV_STEP_PREFILL:
                    out = self.cache.paged_prefill(qd, [items[i][4] for i in idx], td, ld, layer=self.layer,
                                                   context_lens_host=ctx)
                else:
                    out = self.cache.paged_decode(qd, td, ld, layer=self.layer, context_lens_host=ctx)
                o = out.cpu().numpy()
                row = 0
                for i in idx:
                    outputs[i] = o[row:row + items[i][4]]
                    row += items[i][4]
        nxt = [self.model.next_token(it[0], toks[it[0]], outputs[i][-1])
               for i, it in enumerate(items) if it[6]]
        finished = C.pkv_sched_commit(self.sched, nxt)
        self.steps += 1
        return plan, outputs, finished

    def run(self, max_steps=100000):
        log = []
        while self.pending() and len(log) < max_steps:
            log.append(self.step())
        return log
