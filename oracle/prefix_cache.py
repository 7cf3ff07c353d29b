"""Reference prefix cache over the reference allocator.  Test infrastructure
only (see the package header).

What the pages fix ([p2] §4.3): the framework keeps K/V cached block by
block and records how blocks follow one another; a new request whose prefix
matches an earlier request's reuses those blocks and computes only the rest.
When to evict, which prefixes are worth keeping and how much memory the
cache may hold are left to tuning; a full pool makes requests wait instead
of overflowing ([p2] §5.2), and finished requests release their blocks at
once ([p2] §3.3).

Readings taken here (the plainest ones; each is pinned by a test):

* Only full blocks are cached. A cached block is identified by its 16 token
  ids and its predecessor: the cached block before it (none for the first
  block of a request). Matching compares the ids themselves, so two
  requests share a block only if every token before and in it is equal.
* A lookup matches a new request's blocks in order and stops at the first
  miss; it takes at most floor((n - 1) / 16) blocks of an n-token prompt, so
  at least the last token is computed.
* The cache holds one reference on each cached block, so a cached block
  outlives the request that filled it. A block is evictable when only the
  cache holds it and no cached block follows it.
* Eviction takes the least recently used evictable block first; a lookup
  hit or an insert marks the blocks of its chain as used, last block first,
  so a block is always marked after every block that follows it.
* A reservation that finds too few free blocks evicts just enough evictable
  blocks first, least recently used first; if free plus evictable blocks are
  still too few, nothing changes (the request waits).
* Insert registers a sequence's full blocks in order and stops at the first
  block whose content is already cached as a different block.
"""

from .allocator import NoBlocks, RefAllocator
from .sizes import BLOCK_TOKENS


class RefPrefixCache(RefAllocator):
    def __init__(self, num_blocks, free_order=None):
        super().__init__(num_blocks, free_order)
        self.entries = {}  # block -> (predecessor block or -1, tuple of 16 token ids)
        self.by_content = {}  # (predecessor, ids) -> block
        self.children = {}  # block -> cached blocks that follow it
        self.used = {}  # block -> last-use tick
        self.tick = 0

    # -- bookkeeping -------------------------------------------------------
    def _touch(self, chain):
        for blk in reversed(chain):
            self.tick += 1
            self.used[blk] = self.tick

    def _evictable(self):
        return [b for b in self.entries if self.ref[b] == 1 and self.children.get(b, 0) == 0]

    def _evict_one(self):
        cands = self._evictable()
        if not cands:
            return None
        blk = min(cands, key=lambda b: self.used[b])
        pred, ids = self.entries.pop(blk)
        del self.by_content[(pred, ids)]
        del self.used[blk]
        if pred >= 0:
            self.children[pred] -= 1
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self.free.append(blk)
        return blk

    def reclaimable(self):
        """Cached blocks only the cache holds: all of them can be evicted,
        followers first (a block held by a sequence has every predecessor
        held by it too)."""
        return sum(1 for b in self.entries if self.ref[b] == 1)

    # -- operations ---------------------------------------------------------
    def seq_create_cached(self, tokens):
        """A new sequence holding the cached blocks that match the prompt's
        leading full blocks; returns ``(seq, cached_tokens)``."""
        tokens = [int(t) for t in tokens]
        sid = self.seq_create()
        chain, pred = [], -1
        for j in range(max(len(tokens) - 1, 0) // BLOCK_TOKENS):
            ids = tuple(tokens[j * BLOCK_TOKENS:(j + 1) * BLOCK_TOKENS])
            blk = self.by_content.get((pred, ids))
            if blk is None:
                break
            chain.append(blk)
            pred = blk
        for blk in chain:
            self.ref[blk] += 1
        self.tables[sid] = list(chain)
        self.lens[sid] = len(chain) * BLOCK_TOKENS
        self._touch(chain)
        return sid, self.lens[sid]

    def insert(self, sid, tokens):
        """Register the sequence's full blocks holding ``tokens`` (its first
        ``len(tokens)`` tokens, K/V written). Returns blocks newly cached."""
        self._check(sid)
        tokens = [int(t) for t in tokens]
        table = self.tables[sid]
        nfull = min(len(tokens), self.lens[sid]) // BLOCK_TOKENS
        chain, pred, added = [], -1, 0
        for j in range(nfull):
            blk = table[j]
            ids = tuple(tokens[j * BLOCK_TOKENS:(j + 1) * BLOCK_TOKENS])
            have = self.by_content.get((pred, ids))
            if have is None:
                if blk in self.entries:  # cached under other content: a stale table
                    break
                self.entries[blk] = (pred, ids)
                self.by_content[(pred, ids)] = blk
                self.ref[blk] += 1
                if pred >= 0:
                    self.children[pred] = self.children.get(pred, 0) + 1
                added += 1
            elif have != blk:
                break
            chain.append(blk)
            pred = blk
        self._touch(chain)
        return added

    def evict(self, max_blocks):
        """Release up to ``max_blocks`` evictable blocks; returns them in
        eviction order."""
        out = []
        while len(out) < max_blocks:
            blk = self._evict_one()
            if blk is None:
                break
            out.append(blk)
        return out

    def seq_reserve(self, sid, n):
        self._check(sid)
        if n < 0:
            raise ValueError("n must be >= 0")
        need = self._blocks_needed(sid, n)
        if need > len(self.free):
            if need > len(self.free) + self.reclaimable():
                raise NoBlocks(sid)
            self.evict(need - len(self.free))
        return super().seq_reserve(sid, n)
