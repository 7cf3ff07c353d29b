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

``append_row_int8`` is the quantise-on-write rule for one new token in a
partly filled block (the int8 append step).
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


def append_row_int8(codes, scale, off, x):
    """Quantise-on-write of one new row ``x [D]`` (fp16) into slot ``off`` of
    a ``[16, D]`` int8 tile whose rows ``< off`` are filled with ``scale``.

    The pages say only that 8-bit K/V carry group scale factors ([p2] §4.1);
    appending one token at a time to a block already holding codes needs a
    rule, and the reading taken is the plainest that keeps every filled row
    within half a step of its value:

    * a token at offset 0 opens the block: its scale comes from its own
      absmax, exactly as the block quantiser does for a one-row tile;
    * a token whose absmax fits the block's range (``a <= 127 * scale``) is
      quantised with the block's scale; earlier codes stay as they are;
    * otherwise the block takes the new row's scale
      ``fp16(fp32(a) / 127)`` and its earlier codes are re-expressed in it,
      ``clip(rint(fp32(code) * fp32(scale) / fp32(new_scale)), -127, 127)``.

    Divisions are IEEE fp32, ``rint`` rounds half to even, and a zero scale
    means zero codes. Returns ``(codes', scale')``; rows past ``off`` are
    left unchanged."""
    codes = np.array(codes, np.int8, copy=True)
    x32 = np.asarray(x, np.float16).astype(np.float32)
    a = np.float32(np.max(np.abs(x32)))
    s = np.float16(scale)
    if off == 0:
        new = np.float16(a / np.float32(127.0))
    elif a <= np.float32(127.0) * np.float32(s):
        new = s
    else:
        new = np.float16(a / np.float32(127.0))
        if new == 0:
            codes[:off] = 0
        else:
            old = codes[:off].astype(np.float32) * np.float32(s)
            codes[:off] = np.clip(np.rint(old / np.float32(new)), -127, 127).astype(np.int8)
    if new == 0:
        codes[off] = 0
    else:
        codes[off] = np.clip(np.rint(x32 / np.float32(new)), -127, 127).astype(np.int8)
    return codes, new


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
