"""KV-cache byte counts.  Test infrastructure only (see the package header).

[p2] §2.3 gives the per-token size: two tensors (K and V) times layers times
KV heads times head dimension times bytes per element. [p1] §二 gives the
same product for a whole sequence with the head count H. [p1] §三 and [p2]
§3.2 fix the page (block) size at 16 tokens.
"""

BLOCK_TOKENS = 16  # tokens per block: the default page size of [p1] §三, [p2] §3.2

F16_BYTES = 2
I8_BYTES = 1
SCALE_BYTES = 2  # one fp16 scale


def kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes):
    """Bytes of K and V one token occupies over all layers ([p2] §2.3).

    Two copies (K and V) of layers x kv_heads x head_dim elements.
    """
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_cache_bytes(layers, kv_heads, head_dim, elem_bytes, seq_len, batch=1):
    """Total K/V bytes of ``batch`` sequences of ``seq_len`` tokens.

    The sequence-level form of [p1] §二 and the batch rows of the table in
    [p2] §2.3: per-token bytes times tokens times batch, no padding.
    """
    return kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes) * seq_len * batch


def pool_bytes(layers, num_blocks, kv_heads, head_dim, dtype="f16"):
    """Bytes of a pool of ``num_blocks`` 16-token blocks.

    The pool holds every layer's K and V for ``num_blocks * 16`` token slots,
    which is the per-token size of [p2] §2.3 times the slot count. The int8
    pool ([p2] §4.1: 8-bit K/V with grouped scale factors) also stores one
    fp16 scale for K and one for V per (layer, block, KV head).
    """
    if dtype == "f16":
        return kv_bytes_per_token(layers, kv_heads, head_dim, F16_BYTES) * num_blocks * BLOCK_TOKENS
    if dtype == "i8":
        data = kv_bytes_per_token(layers, kv_heads, head_dim, I8_BYTES) * num_blocks * BLOCK_TOKENS
        scales = layers * num_blocks * kv_heads * 2 * SCALE_BYTES
        return data + scales
    raise ValueError(f"unknown dtype {dtype!r}")
