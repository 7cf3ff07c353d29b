"""Reference block allocator.  Test infrastructure only (see the package header).

What the pages fix:

* the KV cache is cut into fixed blocks of 16 tokens and each request keeps a
  block table from logical block to physical block ([p1] §三, [p2] §3.2);
* blocks are taken as needed and handed back the moment a request ends, so
  another request can reuse them at once ([p1] §三, [p2] §3.2, [p3]);
* requests that share a prefix point at the same physical blocks, and a block
  is copied only when one of them forks off, as Unix fork() does ([p1] §三);
* the pool has a cap; a request that does not fit waits instead of running
  the device out of memory ([p2] §5.2).

What the pages leave open, and the reading taken here:

* free-list policy: a LIFO stack seeded from the caller's ``free_order``, so
  the first block handed out is ``free_order[0]``; a freed sequence pushes its
  blocks in reverse logical order;
* order within one reservation: tokens in order, blocks in logical order;
* copy-on-write trigger: a token written at a non-zero offset of a block whose
  refcount is above one; the writer takes a fresh block, the pair
  (old, new) is recorded so the caller copies the whole block, the old
  block's refcount drops by one, and only the writer's table changes. A full
  shared block is never copied because the next token opens a new block;
* a failed reservation changes nothing (all-or-nothing), so the caller can
  queue the request;
* sequence ids count up from 1 in creation order (fork included).
"""

from .sizes import BLOCK_TOKENS


class NoBlocks(Exception):
    """The pool has fewer free blocks than the request needs ([p2] §5.2)."""


class UnknownSeq(Exception):
    """The sequence id is not live."""


class RefAllocator:
    def __init__(self, num_blocks, free_order=None):
        if free_order is None:
            free_order = list(range(num_blocks))
        free_order = [int(b) for b in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        # Stack: the last element is popped first, so reverse the order.
        self.free = list(reversed(free_order))
        self.ref = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self.next_id = 1

    # -- sequences -------------------------------------------------------
    def seq_create(self):
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def _check(self, sid):
        if sid not in self.tables:
            raise UnknownSeq(sid)

    def seq_free(self, sid):
        """Release a finished request: every block loses one reference and a
        block that reaches zero goes straight back to the free list
        ([p1] §三, [p2] §3.2). Blocks are pushed in reverse logical order."""
        self._check(sid)
        for blk in reversed(self.tables[sid]):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
        del self.tables[sid]
        del self.lens[sid]

    def seq_fork(self, parent):
        """A new sequence that shares every block of ``parent`` ([p1] §三)."""
        self._check(parent)
        child = self.seq_create()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1
        return child

    # -- reservation -------------------------------------------------------
    def _blocks_needed(self, sid, n):
        table, length = self.tables[sid], self.lens[sid]
        need = 0
        for pos in range(length, length + n):
            off = pos % BLOCK_TOKENS
            if off == 0:
                need += 1
            elif pos == length and self.ref[table[pos // BLOCK_TOKENS]] > 1:
                need += 1  # copy-on-write of the shared tail block
        return need

    def seq_reserve(self, sid, n):
        """Reserve slots for ``n`` new tokens of ``sid`` (appended at the tail,
        [p2] §2.2).  Returns ``(slots, cow_pairs)`` where
        ``slot = physical_block * 16 + offset`` and ``cow_pairs`` lists
        ``(src, dst)`` blocks the caller must copy before writing."""
        self._check(sid)
        if n < 0:
            raise ValueError("n must be >= 0")
        if self._blocks_needed(sid, n) > len(self.free):
            raise NoBlocks(sid)
        table, length = self.tables[sid], self.lens[sid]
        slots, cow = [], []
        for pos in range(length, length + n):
            lblk, off = divmod(pos, BLOCK_TOKENS)
            if off == 0:
                blk = self.free.pop()
                self.ref[blk] = 1
                table.append(blk)
            else:
                blk = table[lblk]
                if self.ref[blk] > 1:
                    new = self.free.pop()
                    self.ref[new] = 1
                    self.ref[blk] -= 1
                    table[lblk] = new
                    cow.append((blk, new))
                    blk = new
            slots.append(blk * BLOCK_TOKENS + off)
        self.lens[sid] = length + n
        return slots, cow

    # -- introspection -----------------------------------------------------
    def block_tables(self, seqs, max_blocks):
        """Pack tables into ``[B][max_blocks]`` rows padded with -1, and the
        lengths. This is the logical->physical map the decode walks in order
        ([p2] §3.2)."""
        rows, lens = [], []
        for sid in seqs:
            self._check(sid)
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[sid])
        return rows, lens

    def num_free(self):
        return len(self.free)

    def free_list(self):
        """Free blocks, next to be handed out first."""
        return list(reversed(self.free))
