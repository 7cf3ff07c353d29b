"""PagedKVCache: the Python face of libpkv.

torch provides the device memory (one uint8 tensor holds the whole pool) and
the stream (the current torch stream); every step of the path runs in the
library: block bookkeeping in its C++ allocator, copies, appends and decode
in its HIP kernels. Nothing here computes attention or touches cache
contents.

The calls follow the pages' statement of the problem: a pool of fixed
16-token blocks with a block table per sequence, blocks allocated on demand
and returned when a sequence ends ([p1] chanyi.net.cn/article/49 §三; [p2]
lqnn.cn/news/235768 §3.2), copy-on-write prefix sharing through fork ([p1]
§三), append of the new token's K/V at the tail ([p2] §2.2) and a decode that
reads the blocks in table order ([p2] §3.2).
"""

import math

import numpy as np
import torch

from . import _capi as C


class PrefixPlan:
    """A shared-prefix plan for one batch of ``num_seqs`` sequences
    (``pkv_plan_shared_prefix``): the host ints, the group count, and the
    same ints on the device."""

    def __init__(self, host, n_groups, num_seqs, device):
        self.host = np.ascontiguousarray(host, np.int32)
        self.n_groups = int(n_groups)
        self.num_seqs = int(num_seqs)
        self.dev = _dev_i32(self.host, device)

    def shared_blocks(self):
        """Shared blocks per sequence (0 for an ungrouped one)."""
        return self.host[:2 * self.num_seqs:2]

    def groups(self):
        """``[(shared_blocks, [batch indices])]`` per group."""
        base, w = 2 * self.num_seqs, C.PKV_PREFIX_GROUP_INTS
        out = []
        for g in range(self.n_groups):
            gd = self.host[base + g * w:base + (g + 1) * w]
            out.append((int(gd[0]), [int(x) for x in gd[2:2 + gd[1]]]))
        return out


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check_on(dev, **tensors):
    """Every tensor must live on ``dev``, the cache's GPU: the library reads
    them through raw device addresses."""
    if dev.type != "cuda":
        raise ValueError(f"the cache's pool is on {dev}: device calls need it on a GPU")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the cache on {dev}")


def _check_host_lens(host, B):
    if host is not None and host.shape != (B,):
        raise ValueError(f"context_lens_host must hold {B} lengths (got shape {host.shape})")


def _check_tables(block_tables, context_lens, B):
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or block_tables.shape[1] < 1:
        raise ValueError(f"block_tables must be [{B}, max_blocks] (got {list(block_tables.shape)})")
    if context_lens.numel() != B:
        raise ValueError(f"context_lens must hold {B} lengths (got {context_lens.numel()})")


def _dev_i32(a, device):
    t = torch.from_numpy(np.ascontiguousarray(a, np.int32))
    if t.numel() == 0:
        return torch.empty(t.shape, dtype=torch.int32, device=device)
    if torch.device(device).type == "cpu":  # a host cache (host-side calls only): no pinned staging
        return t.clone()
    return t.pin_memory().to(device, non_blocking=True)


class PagedKVCache:
    """A pool of ``num_blocks`` blocks for ``num_layers`` layers.

    ``dtype`` is ``"f16"`` or ``"i8"`` (int8 K/V with one fp16 scale per
    (layer, block, KV head) for K and for V). ``free_order`` fixes the order
    in which blocks are handed out (a permutation of the block ids).
    """

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, dtype="f16",
                 free_order=None, device="cuda"):
        self.cfg = C.make_config(num_layers, num_blocks, num_kv_heads, head_dim, dtype)
        self.dtype = dtype
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.num_layers, self.num_blocks = num_layers, num_blocks
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.nbytes = C.pkv_pool_bytes(self.cfg)
        self.pool = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        self.handle = C.pkv_pool_create(self.cfg, free_order)

    def close(self):
        if getattr(self, "handle", None):
            C.pkv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode_workspace(self, nbytes):
        """A device workspace of at least ``nbytes`` for pkv_paged_decode,
        kept and reused by later calls (calls on one cache share one stream)."""
        ws = getattr(self, "_workspace", None)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._workspace = ws
        return ws

    # ---- views of the device pool (for tests and bulk fills) ---------------
    def _region_bytes(self):
        e = 1 if self.dtype == "i8" else 2
        return self.num_layers * self.num_blocks * self.num_kv_heads * 16 * self.head_dim * e

    def region(self, which, layer=None):
        """K (``which=0``) or V (1) region as ``[L, N, Hkv, 16, D]`` (or one layer)."""
        rb = self._region_bytes()
        raw = self.pool[which * rb:(which + 1) * rb]
        t = raw.view(torch.int8 if self.dtype == "i8" else torch.float16)
        t = t.view(self.num_layers, self.num_blocks, self.num_kv_heads, 16, self.head_dim)
        return t if layer is None else t[layer]

    def scales(self):
        """int8 scales ``[L, N, Hkv, 2]`` fp16 (0 = K, 1 = V)."""
        if self.dtype != "i8":
            raise ValueError("fp16 pools have no scales")
        rb = self._region_bytes()
        raw = self.pool[2 * rb:]
        return raw.view(torch.float16).view(self.num_layers, self.num_blocks, self.num_kv_heads, 2)

    # ---- sequences (host) -------------------------------------------------------
    def create_seq(self):
        return C.pkv_seq_create(self.handle)

    def free_seq(self, seq):
        C.pkv_seq_free(self.handle, seq)

    def fork(self, parent):
        return C.pkv_seq_fork(self.handle, parent)

    def seq_len(self, seq):
        return C.pkv_seq_len(self.handle, seq)

    def block_table(self, seq):
        return C.pkv_seq_block_table(self.handle, seq)

    def num_free(self):
        return C.pkv_num_free(self.handle)

    def free_list(self):
        return C.pkv_free_list(self.handle)

    def refcount(self, block):
        return C.pkv_block_refcount(self.handle, block)

    def reserve(self, seqs, counts):
        """Reserve ``counts[i]`` token slots for ``seqs[i]``, in order.

        Returns ``(slots int32[sum(counts)], cow_pairs int32[k, 2])``. A
        NoBlocksError leaves the sequence that failed (and every later one)
        untouched; earlier sequences in the list keep their reservation."""
        all_slots, all_cow = [], []
        for s, n in zip(seqs, counts):
            slots, cow = C.pkv_seq_reserve(self.handle, s, int(n), cow_cap=1)
            all_slots.append(slots)
            all_cow.append(cow)
        slots = np.concatenate(all_slots) if all_slots else np.empty(0, np.int32)
        cow = np.concatenate(all_cow) if all_cow else np.empty((0, 2), np.int32)
        return slots, cow

    # ---- device steps -------------------------------------------------------------
    def copy_blocks(self, pairs):
        """Copy-on-write block copies (host pairs ``[k, 2]``), all layers."""
        pairs = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
        if len(pairs) == 0:
            return
        dev = _dev_i32(pairs, self.device)
        C.pkv_copy_blocks(self.cfg, self.pool.data_ptr(), dev.data_ptr(), len(pairs), _stream())

    def write(self, layer, k, v, slots_dev):
        """Write fp16 ``k, v [n, Hkv, D]`` (device, contiguous) of one layer
        into the reserved device slots."""
        k = k.contiguous()
        v = v.contiguous()
        if k.dtype != torch.float16 or v.dtype != torch.float16:
            raise TypeError("k and v must be float16")
        n = k.shape[0]
        if tuple(k.shape) != (n, self.num_kv_heads, self.head_dim) or v.shape != k.shape:
            raise ValueError(f"k, v must be [n, {self.num_kv_heads}, {self.head_dim}]")
        if slots_dev.numel() != n:
            raise ValueError("one slot per token")
        if slots_dev.dtype != torch.int32 or not slots_dev.is_contiguous():
            raise TypeError("slots must be a contiguous int32 tensor")
        if not 0 <= layer < self.num_layers:
            raise ValueError(f"layer {layer} out of range [0, {self.num_layers})")
        _check_on(self.device, k=k, v=v, slots=slots_dev)
        C.pkv_append_kv(self.cfg, self.pool.data_ptr(), layer, k.data_ptr(), v.data_ptr(),
                        slots_dev.data_ptr(), n, _stream())

    def append_kv(self, seq, k, v):
        """Append new tokens' K/V at the tail ([p2] §2.2).

        ``seq`` is one sequence id with ``k, v [n, Hkv, D]`` (n tokens), or a
        list of B ids with ``k, v [B, Hkv, D]`` (one token each). With a
        leading layer axis ``[L, ...]`` every layer is written; without it
        the pool must have one layer. Returns the device slot tensor."""
        seqs = [seq] if isinstance(seq, (int, np.integer)) else list(seq)
        if len(set(int(x) for x in seqs)) != len(seqs):
            # one token per sequence: a sequence named twice would have two
            # appends racing on its tail block (and, for int8, on its scale)
            raise ValueError("append_kv: a sequence appears more than once in the list")
        per_layer = k.dim() == 4
        n = k.shape[1] if per_layer else k.shape[0]
        counts = [n] if len(seqs) == 1 and isinstance(seq, (int, np.integer)) else [1] * len(seqs)
        if sum(counts) != n:
            raise ValueError("token count does not match the sequences")
        if not per_layer and self.num_layers != 1:
            raise ValueError("pass k, v with a leading layer axis for a multi-layer pool")
        slots, cow = self.reserve(seqs, counts)
        self.copy_blocks(cow)
        slots_dev = _dev_i32(slots, self.device)
        if per_layer:
            for layer in range(k.shape[0]):
                self.write(layer, k[layer], v[layer], slots_dev)
        else:
            self.write(0, k, v, slots_dev)
        return slots_dev

    def upload(self, dst, src_pinned):
        """Copy a pinned host tensor into a device tensor of the same size
        with the library's upload kernel on the current stream (no copy
        engine): the per-step block tables and lengths."""
        if not src_pinned.is_pinned() or dst.device.type != "cuda" or not dst.is_contiguous() \
                or not src_pinned.is_contiguous():
            raise ValueError("upload needs a contiguous pinned host source and a contiguous device target")
        n = src_pinned.numel() * src_pinned.element_size()
        if dst.numel() * dst.element_size() != n:
            raise ValueError("source and target sizes differ")
        C.pkv_upload(dst.data_ptr(), src_pinned.data_ptr(), n, _stream())

    def block_tables(self, seqs, max_blocks=None):
        """Host ``(tables int32[B, max_blocks], ctx_lens int32[B])`` for the
        decode, padded with -1."""
        if max_blocks is None:
            max_blocks = max(len(self.block_table(s)) for s in seqs)
        return C.pkv_build_block_tables(self.handle, seqs, max_blocks)

    def paged_prefill(self, q, q_lens, block_tables, context_lens, layer=0, out=None, scale=None,
                      context_lens_host=None, max_context=None):
        """Causal attention of each sequence's newest ``q_lens[b]`` tokens
        (their K/V already appended) over its cache: ``q`` is fp16
        ``[T, Hq, D]``, sequence after sequence; token i of sequence b's
        chunk sits at position ``context_lens[b] - q_lens[b] + i`` and sees
        tokens up to itself. Returns ``out [T, Hq, D]`` fp16."""
        if q.dtype != torch.float16 or q.dim() != 3:
            raise TypeError("q must be float16 [T, Hq, D]")
        q = q.contiguous()
        T, Hq, D = q.shape
        if D != self.head_dim or Hq % self.num_kv_heads:
            raise ValueError(f"q must be [T, Hq, {self.head_dim}] with Hq a multiple of {self.num_kv_heads}")
        ql = np.ascontiguousarray(q_lens, np.int64)
        if ql.ndim != 1 or ql.sum() != T or (ql < 0).any():
            raise ValueError("q_lens must be non-negative and add up to the rows of q")
        B = len(ql)
        _check_tables(block_tables, context_lens, B)
        block_tables = block_tables.contiguous()
        context_lens = context_lens.contiguous()
        max_blocks = block_tables.shape[1]
        host = None if context_lens_host is None else np.ascontiguousarray(context_lens_host, np.int32)
        _check_host_lens(host, B)
        if out is not None and (tuple(out.shape) != (T, Hq, D) or out.dtype != torch.float16
                                or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous float16 [{T}, {Hq}, {D}] tensor")
        if not 0 <= layer < self.num_layers:
            raise ValueError(f"layer {layer} out of range [0, {self.num_layers})")
        _check_on(self.device, q=q, block_tables=block_tables, context_lens=context_lens, out=out)
        starts = np.zeros(B + 1, np.int32)
        starts[1:] = np.cumsum(ql)
        starts_dev = _dev_i32(starts, self.device)
        if max_context is None:
            max_context = int(host.max()) if host is not None else max_blocks * 16
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        if out is None:
            out = torch.empty((T, Hq, D), dtype=torch.float16, device=q.device)
        a = C.pkv_prefill_args()
        a.cfg = C.ctypes.pointer(self.cfg)
        a.pool_dev = self.pool.data_ptr()
        a.layer = layer
        a.q_dev = q.data_ptr()
        a.num_seqs = B
        a.num_q_heads = Hq
        a.q_start_dev = starts_dev.data_ptr()
        a.q_start_host = starts.ctypes.data_as(C._p_i32)
        a.block_tables_dev = block_tables.data_ptr()
        a.max_blocks = max_blocks
        a.ctx_lens_dev = context_lens.data_ptr()
        a.ctx_lens_host = host.ctypes.data_as(C._p_i32) if host is not None else None
        a.max_context = max_context
        a.out_dev = out.data_ptr()
        a.scale = scale
        C.pkv_paged_prefill(a, _stream())
        return out

    def plan_shared_prefix(self, seqs, min_blocks=1, max_members=None, num_q_heads=None):
        """Group the batch's sequences that share leading blocks so one decode
        reads those blocks once for all of them (the plan is tied to this
        order of ``seqs`` and to the current block tables). A decode takes
        groups of at most 128 query rows (members x query heads per KV head):
        give the decode's ``num_q_heads`` and groups hold at most
        ``128 // (num_q_heads // num_kv_heads)`` members (and at most 32);
        else ``max_members`` (default 32, right up to 4 heads per KV head)."""
        if max_members is None:
            max_members = C.PKV_MAX_SHARERS
            if num_q_heads is not None:
                if num_q_heads < 1 or num_q_heads % self.num_kv_heads:
                    raise ValueError(f"num_q_heads {num_q_heads} is not a multiple of {self.num_kv_heads}")
                max_members = min(max_members, 128 // (num_q_heads // self.num_kv_heads))
        elif num_q_heads is not None:
            raise ValueError("give max_members or num_q_heads, not both")
        host, ng = C.pkv_plan_shared_prefix(self.handle, seqs, min_blocks, max_members)
        return PrefixPlan(host, ng, len(seqs), self.device)

    def paged_decode(self, q, block_tables, context_lens, layer=0, out=None, scale=None,
                     context_lens_host=None, max_context=None, workspace=None, partition_tokens=0,
                     k_new=None, v_new=None, prefix_plan=None):
        """``out[b, h] = softmax(q[b, h] K_b^T * scale) V_b`` over the
        ``context_lens[b]`` tokens of each sequence, read in place through
        ``block_tables`` (device int32 ``[B, max_blocks]``). With ``k_new,
        v_new`` (fp16 ``[B, Hkv, D]``) the kernel first stores them as the
        last token of each sequence (the slot already reserved), so append
        and attention run in one launch. With ``prefix_plan`` (from
        :meth:`plan_shared_prefix` for these sequences in this order) each
        group's shared blocks are read once for all its members."""
        return paged_decode(self, q, block_tables, context_lens, layer, out, scale,
                            context_lens_host, max_context, workspace, partition_tokens, k_new, v_new,
                            prefix_plan)


def paged_decode(cache, q, block_tables, context_lens, layer=0, out=None, scale=None,
                 context_lens_host=None, max_context=None, workspace=None, partition_tokens=0,
                 k_new=None, v_new=None, prefix_plan=None):
    if q.dtype != torch.float16 or q.dim() != 3:
        raise TypeError("q must be float16 [B, Hq, D]")
    q = q.contiguous()
    B, Hq, D = q.shape
    if D != cache.head_dim or Hq % cache.num_kv_heads:
        raise ValueError(f"q must be [B, Hq, {cache.head_dim}] with Hq a multiple of {cache.num_kv_heads}")
    _check_tables(block_tables, context_lens, B)
    block_tables = block_tables.contiguous()
    context_lens = context_lens.contiguous()
    max_blocks = block_tables.shape[1]
    host = None
    if context_lens_host is not None:
        host = np.ascontiguousarray(context_lens_host, np.int32)
    _check_host_lens(host, B)
    if out is not None and (tuple(out.shape) != (B, Hq, D) or out.dtype != torch.float16 or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous float16 [{B}, {Hq}, {D}] tensor")
    if not 0 <= layer < cache.num_layers:
        raise ValueError(f"layer {layer} out of range [0, {cache.num_layers})")
    if k_new is not None and v_new is not None:
        k_new, v_new = k_new.contiguous(), v_new.contiguous()
    _check_on(cache.device, q=q, block_tables=block_tables, context_lens=context_lens, out=out,
              workspace=workspace, k_new=k_new, v_new=v_new,
              prefix_plan=None if prefix_plan is None else prefix_plan.dev)
    if max_context is None:
        max_context = int(host.max()) if host is not None else max_blocks * 16
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=q.device)
    n_groups = prefix_plan.n_groups if prefix_plan is not None else 0
    if n_groups:
        ws_bytes = C.pkv_prefix_decode_workspace_bytes(cache.cfg, B, Hq, max_context, max_blocks,
                                                       partition_tokens, n_groups)
    else:
        ws_bytes = C.pkv_decode_workspace_bytes(cache.cfg, B, Hq, max_context, partition_tokens)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = cache.decode_workspace(ws_bytes)
    args = C.pkv_decode_args()
    args.cfg = C.ctypes.pointer(cache.cfg)
    args.pool_dev = cache.pool.data_ptr()
    args.layer = layer
    args.q_dev = q.data_ptr()
    args.num_seqs = B
    args.num_q_heads = Hq
    args.block_tables_dev = block_tables.data_ptr()
    args.max_blocks = max_blocks
    args.ctx_lens_dev = context_lens.data_ptr()
    args.ctx_lens_host = host.ctypes.data_as(C._p_i32) if host is not None else None
    args.max_context = max_context
    args.out_dev = out.data_ptr()
    args.scale = scale
    args.workspace_dev = workspace.data_ptr()
    args.workspace_bytes = workspace.numel() * workspace.element_size()
    args.partition_tokens = partition_tokens
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        shape = (B, cache.num_kv_heads, D)
        if k_new.dtype != torch.float16 or tuple(k_new.shape) != shape or tuple(v_new.shape) != shape \
                or v_new.dtype != torch.float16:
            raise ValueError(f"k_new, v_new must be float16 {list(shape)}")
        args.k_new_dev = k_new.data_ptr()
        args.v_new_dev = v_new.data_ptr()
    if n_groups:
        if prefix_plan.num_seqs != B:
            raise ValueError("the plan was made for another batch size")
        args.prefix_plan_dev = prefix_plan.dev.data_ptr()
        args.prefix_plan_host = prefix_plan.host.ctypes.data_as(C._p_i32)
        args.prefix_groups = n_groups
    C.pkv_paged_decode(args, _stream())
    return out
