"""Reference paged K/V store.  Test infrastructure only (see the package header).

Layout reading. [p2] §3.2 says only that each block holds a short run of
contiguous K/V data and that blocks need not be contiguous with each other.
The layout taken: K and V in separate regions, each ``[L][N][Hkv][16][D]``,
so one (block, KV head) tile is 16 consecutive token rows of ``D`` elements.
The int8 store adds ``scales[L][N][Hkv][2]`` (K scale, V scale) in fp16.

Cached K/V are written once and never modified afterwards; new tokens only
append at the tail ([p1] §二, [p2] §2.2).
"""

import numpy as np

from .sizes import BLOCK_TOKENS


class RefCache:
    def __init__(self, layers, num_blocks, kv_heads, head_dim, dtype="f16", fill=None):
        shape = (layers, num_blocks, kv_heads, BLOCK_TOKENS, head_dim)
        self.layers, self.num_blocks = layers, num_blocks
        self.kv_heads, self.head_dim = kv_heads, head_dim
        self.dtype = dtype
        if dtype == "f16":
            self.K = np.zeros(shape, np.float16)
            self.V = np.zeros(shape, np.float16)
            self.scales = None
        elif dtype == "i8":
            self.K = np.zeros(shape, np.int8)
            self.V = np.zeros(shape, np.int8)
            self.scales = np.zeros((layers, num_blocks, kv_heads, 2), np.float16)
        else:
            raise ValueError(dtype)
        if fill is not None:
            self.K[...] = fill
            self.V[...] = fill

    def append(self, layer, k, v, slots):
        """Write token i's K/V rows ``k[i], v[i]`` (fp16, shape ``[Hkv, D]``)
        at ``slots[i] = block * 16 + offset`` of ``layer``: the decode-step
        write of the new token's K and V at the cache tail ([p2] §2.2).

        An int8 store quantises on write, token by token in the given order
        (``append_row_int8``; a block may be re-expressed in a larger scale
        when a new row exceeds its range)."""
        from .quant import append_row_int8
        k = np.asarray(k)
        v = np.asarray(v)
        assert k.shape == v.shape == (len(slots), self.kv_heads, self.head_dim)
        for i, slot in enumerate(slots):
            blk, off = divmod(int(slot), BLOCK_TOKENS)
            if self.dtype == "f16":
                self.K[layer, blk, :, off, :] = k[i]
                self.V[layer, blk, :, off, :] = v[i]
                continue
            for g in range(self.kv_heads):
                for which, store, rows in ((0, self.K, k), (1, self.V, v)):
                    codes, sc = append_row_int8(store[layer, blk, g], self.scales[layer, blk, g, which], off,
                                                rows[i, g])
                    store[layer, blk, g] = codes
                    self.scales[layer, blk, g, which] = sc

    def copy_blocks(self, pairs):
        """Copy-on-write: each ``(src, dst)`` copies the whole block (every
        layer, K and V, and the int8 scales) before the fork writes into it
        ([p1] §三)."""
        for src, dst in pairs:
            self.K[:, dst] = self.K[:, src]
            self.V[:, dst] = self.V[:, src]
            if self.scales is not None:
                self.scales[:, dst] = self.scales[:, src]
