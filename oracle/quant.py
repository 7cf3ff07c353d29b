"""int8 K/V quantiser.  Test infrastructure only (see the package header).

[p2] §4.1: K and V may be stored in 8 bits, each short run of cache carrying
its own scale factor so the values come back in roughly the right range; 8
bits halves the cache. The pages do not give the formula. Reading taken:

* one group = one (layer, block, KV head) tile of K, and separately of V
  (each gets its own fp16 scale);
* symmetric absmax over the filled slots of the tile:
  ``scale = fp16(fp32(max|x|) / 127)`` rounded to nearest even;
* ``code = clip(rint(fp32(x) / fp32(scale)), -127, 127)``; the division is
  IEEE fp32 and ``rint`` rounds half to even (tie rounding is parity
  unpinned: the pages do not fix it);
* a tile whose absmax is zero, or whose scale rounds to zero, gets scale 0
  and all-zero codes;
* slots past the tile's filled count are stored as 0.

Dequantisation is ``code * scale`` (exact in fp64).
"""

import numpy as np

from .sizes import BLOCK_TOKENS


def quantize_block_int8(x, filled=BLOCK_TOKENS):
    """Quantise one ``[16, D]`` fp16 tile; only rows ``< filled`` count.

    Returns ``(codes int8 [16, D], scale fp16)``."""
    x = np.asarray(x, np.float16)
    codes = np.zeros(x.shape, np.int8)
    if filled == 0:
        return codes, np.float16(0)
    live = x[:filled].astype(np.float32)
    a = np.float32(np.max(np.abs(live)))
    scale = np.float16(a / np.float32(127.0))
    if scale == 0:
        return codes, np.float16(0)
    q = np.rint(live / np.float32(scale))
    codes[:filled] = np.clip(q, -127, 127).astype(np.int8)
    return codes, scale


def dequantize_int8(codes, scale):
    """``code * scale`` in fp64."""
    return np.asarray(codes, np.float64) * np.float64(scale)


def quantize_pool_int8(K16, V16, filled):
    """Quantise whole fp16 stores ``[L][N][Hkv][16][D]``.

    ``filled[n]`` is the number of live slots of physical block ``n``.
    Returns ``(K8, V8, scales)`` with ``scales[L][N][Hkv][2]`` fp16
    (index 0 = K, 1 = V)."""
    L, N, Hkv = K16.shape[:3]
    K8 = np.zeros(K16.shape, np.int8)
    V8 = np.zeros(V16.shape, np.int8)
    scales = np.zeros((L, N, Hkv, 2), np.float16)
    for l in range(L):
        for n in range(N):
            f = int(filled[n])
            if f == 0:
                continue
            for g in range(Hkv):
                K8[l, n, g], scales[l, n, g, 0] = quantize_block_int8(K16[l, n, g], f)
                V8[l, n, g], scales[l, n, g, 1] = quantize_block_int8(V16[l, n, g], f)
    return K8, V8, scales
