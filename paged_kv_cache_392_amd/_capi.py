"""ctypes binding of libpkv (include/pkv.h): argument marshalling only.

Every function keeps the C name. Host calls take and return Python ints and
NumPy arrays; device calls take raw device addresses (ints) and a stream
handle (int), so any device-memory owner can drive them. A non-zero status
raises :class:`PkvError` carrying the library's message.

torch is imported before the library is opened so that libpkv binds to the
HIP runtime torch already loaded (both carry the soname libamdhip64.so.7);
opening it first would map a second HIP runtime into the process.
"""

import ctypes
import os

import numpy as np

import torch  # noqa: F401  (must precede loading libpkv; see module docstring)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_NO_BLOCKS = -2
PKV_ERR_UNKNOWN_SEQ = -3
PKV_ERR_REFCOUNT = -4
PKV_ERR_UNSUPPORTED = -5
PKV_ERR_HIP = -6

PKV_F16 = 0
PKV_I8 = 1
BLOCK_TOKENS = 16
PKV_MAX_SHARERS = 32
PKV_PREFIX_GROUP_INTS = 34
PKV_NOALLOC_SCRATCH_BYTES = 16 << 20

_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_p_i32 = ctypes.POINTER(ctypes.c_int32)
_p_i64 = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


class pkv_config(ctypes.Structure):
    _fields_ = [("num_layers", _c_i32), ("num_blocks", _c_i32), ("block_size", _c_i32),
                ("num_kv_heads", _c_i32), ("head_dim", _c_i32), ("dtype", _c_i32)]


class pkv_decode_args(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(pkv_config)), ("pool_dev", _vp), ("layer", _c_i32),
                ("q_dev", _vp), ("num_seqs", _c_i32), ("num_q_heads", _c_i32),
                ("block_tables_dev", _vp), ("max_blocks", _c_i32), ("ctx_lens_dev", _vp),
                ("ctx_lens_host", _p_i32), ("max_context", _c_i32), ("out_dev", _vp),
                ("scale", ctypes.c_float), ("workspace_dev", _vp), ("workspace_bytes", _c_i64),
                ("partition_tokens", _c_i32), ("k_new_dev", _vp), ("v_new_dev", _vp),
                ("prefix_plan_dev", _vp), ("prefix_plan_host", _p_i32), ("prefix_groups", _c_i32),
                ("timing_events", ctypes.POINTER(_vp))]


class pkv_prefill_args(ctypes.Structure):
    _fields_ = [("cfg", ctypes.POINTER(pkv_config)), ("pool_dev", _vp), ("layer", _c_i32),
                ("q_dev", _vp), ("num_seqs", _c_i32), ("num_q_heads", _c_i32),
                ("q_start_dev", _vp), ("q_start_host", _p_i32), ("block_tables_dev", _vp),
                ("max_blocks", _c_i32), ("ctx_lens_dev", _vp), ("ctx_lens_host", _p_i32),
                ("max_context", _c_i32), ("out_dev", _vp), ("scale", ctypes.c_float)]


class pkv_step_item(ctypes.Structure):
    _fields_ = [("req", _c_i64), ("seq", _c_i64), ("kind", _c_i32), ("start", _c_i32), ("count", _c_i32),
                ("slot_index", _c_i32), ("completes", _c_i32)]


class pkv_step_plan(ctypes.Structure):
    _fields_ = [("items", ctypes.POINTER(pkv_step_item)), ("item_cap", _c_i32), ("n_items", _c_i32),
                ("slots", _p_i32), ("slot_cap", _c_i32), ("n_slots", _c_i32),
                ("cow_pairs", _p_i32), ("cow_cap", _c_i32), ("n_cow", _c_i32),
                ("preempted", _p_i64), ("preempted_cap", _c_i32), ("n_preempted", _c_i32),
                ("admitted", _p_i64), ("admitted_cached", _p_i32), ("admitted_cap", _c_i32), ("n_admitted", _c_i32)]


PKV_STEP_DECODE = 0
PKV_STEP_PREFILL = 1
PKV_REQ_WAITING, PKV_REQ_RUNNING, PKV_REQ_FINISHED = 0, 1, 2


class PkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"pkv error {status}: {message}")
        self.status = status


class NoBlocksError(PkvError):
    """The pool cannot hold the request; nothing changed (queue it)."""


_SIGS = {
    "pkv_pool_bytes": (_c_i64, [ctypes.POINTER(pkv_config)]),
    "pkv_pool_create": (ctypes.c_int, [ctypes.POINTER(pkv_config), _p_i32, _c_i32, ctypes.POINTER(_vp)]),
    "pkv_pool_destroy": (None, [_vp]),
    "pkv_seq_create": (ctypes.c_int, [_vp, _p_i64]),
    "pkv_seq_free": (ctypes.c_int, [_vp, _c_i64]),
    "pkv_seq_fork": (ctypes.c_int, [_vp, _c_i64, _p_i64]),
    "pkv_seq_reserve": (ctypes.c_int, [_vp, _c_i64, _c_i32, _p_i32, _p_i32, _c_i32, _p_i32]),
    "pkv_seq_len": (ctypes.c_int, [_vp, _c_i64, _p_i32]),
    "pkv_seq_block_table": (ctypes.c_int, [_vp, _c_i64, _p_i32, _c_i32, _p_i32]),
    "pkv_block_refcount": (ctypes.c_int, [_vp, _c_i32, _p_i32]),
    "pkv_num_free": (ctypes.c_int, [_vp, _p_i32]),
    "pkv_free_list": (ctypes.c_int, [_vp, _p_i32, _c_i32, _p_i32]),
    "pkv_build_block_tables": (ctypes.c_int, [_vp, _p_i64, _c_i32, _c_i32, _p_i32, _p_i32]),
    "pkv_seq_create_cached": (ctypes.c_int, [_vp, _p_i32, _c_i32, _p_i64, _p_i32]),
    "pkv_prefix_cache_insert": (ctypes.c_int, [_vp, _c_i64, _p_i32, _c_i32, _p_i32]),
    "pkv_prefix_cache_evict": (ctypes.c_int, [_vp, _c_i32, _p_i32, _p_i32]),
    "pkv_prefix_cache_stats": (ctypes.c_int, [_vp, _p_i32, _p_i32]),
    "pkv_prefix_cache_entry": (ctypes.c_int, [_vp, _c_i32, _p_i32, _p_i32, _p_i32, _p_i64]),
    "pkv_sched_limits": (ctypes.c_int, [_c_i32, _c_i32, _p_i32, _p_i32]),
    "pkv_sched_create": (ctypes.c_int, [_vp, _c_i32, _c_i32, ctypes.POINTER(_vp)]),
    "pkv_sched_destroy": (None, [_vp]),
    "pkv_sched_submit": (ctypes.c_int, [_vp, _c_i64, _p_i32, _c_i32, _c_i32]),
    "pkv_sched_step": (ctypes.c_int, [_vp, ctypes.POINTER(pkv_step_plan)]),
    "pkv_sched_commit": (ctypes.c_int, [_vp, _p_i32, _c_i32, _p_i64, _c_i32, _p_i32]),
    "pkv_sched_request": (ctypes.c_int, [_vp, _c_i64, _p_i32, _c_i32, _p_i32, _p_i32, _p_i64, _p_i32]),
    "pkv_sched_counts": (ctypes.c_int, [_vp, _p_i32, _p_i32, _p_i32]),
    "pkv_plan_ints": (_c_i32, [_c_i32]),
    "pkv_plan_shared_prefix": (ctypes.c_int, [_vp, _p_i64, _c_i32, _c_i32, _c_i32, _p_i32, _c_i32, _p_i32]),
    "pkv_copy_blocks": (ctypes.c_int, [ctypes.POINTER(pkv_config), _vp, _vp, _c_i32, _vp]),
    "pkv_append_kv": (ctypes.c_int, [ctypes.POINTER(pkv_config), _vp, _c_i32, _vp, _vp, _vp, _c_i32, _vp]),
    "pkv_decode_workspace_bytes": (_c_i64, [ctypes.POINTER(pkv_config), _c_i32, _c_i32, _c_i32, _c_i32]),
    "pkv_prefix_decode_workspace_bytes": (_c_i64, [ctypes.POINTER(pkv_config), _c_i32, _c_i32, _c_i32, _c_i32,
                                                   _c_i32, _c_i32]),
    "pkv_paged_decode": (ctypes.c_int, [ctypes.POINTER(pkv_decode_args), _vp]),
    "pkv_paged_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(pkv_decode_args), _vp]),
    "pkv_paged_prefill": (ctypes.c_int, [ctypes.POINTER(pkv_prefill_args), _vp]),
    "pkv_upload": (ctypes.c_int, [_vp, _vp, _c_i64, _vp]),
    "pkv_probe_stream_read": (ctypes.c_int, [_vp, _c_i64, _vp, _vp]),
    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_last_error": (ctypes.c_char_p, []),
}

EXPORTS = tuple(_SIGS)

_lib = None


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load(path=None):
    """Open libpkv (once). Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"libpkv not built: {path} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes mapped in one process: {sorted(runtimes)}")
    _lib = lib
    return lib


def _check(status):
    if status != PKV_OK:
        msg = load().pkv_last_error().decode(errors="replace")
        cls = NoBlocksError if status == PKV_ERR_NO_BLOCKS else PkvError
        raise cls(status, msg)
    return status


def _i32p(a):
    return a.ctypes.data_as(_p_i32)


def make_config(num_layers, num_blocks, num_kv_heads, head_dim, dtype=PKV_F16):
    if isinstance(dtype, str):
        dtype = {"f16": PKV_F16, "i8": PKV_I8}[dtype]
    return pkv_config(num_layers, num_blocks, BLOCK_TOKENS, num_kv_heads, head_dim, dtype)


# ---- host calls -------------------------------------------------------------

def pkv_pool_bytes(cfg):
    n = load().pkv_pool_bytes(ctypes.byref(cfg))
    if n < 0:
        _check(int(n))
    return int(n)


def pkv_pool_create(cfg, free_order=None):
    out = _vp()
    if free_order is None:
        _check(load().pkv_pool_create(ctypes.byref(cfg), None, 0, ctypes.byref(out)))
    else:
        fo = np.ascontiguousarray(free_order, np.int32)
        _check(load().pkv_pool_create(ctypes.byref(cfg), _i32p(fo), len(fo), ctypes.byref(out)))
    return out.value


def pkv_pool_destroy(pool):
    if pool:
        load().pkv_pool_destroy(pool)


def pkv_seq_create(pool):
    s = _c_i64()
    _check(load().pkv_seq_create(pool, ctypes.byref(s)))
    return s.value


def pkv_seq_free(pool, seq):
    _check(load().pkv_seq_free(pool, seq))


def pkv_seq_fork(pool, parent):
    s = _c_i64()
    _check(load().pkv_seq_fork(pool, parent, ctypes.byref(s)))
    return s.value


def pkv_seq_reserve(pool, seq, n, cow_cap=1):
    """Returns ``(slots int32[n], cow_pairs int32[k, 2])``."""
    slots = np.empty(max(n, 1), np.int32)
    cow = np.empty((max(cow_cap, 1), 2), np.int32)
    ncow = _c_i32(0)
    _check(load().pkv_seq_reserve(pool, seq, n, _i32p(slots), _i32p(cow), cow_cap, ctypes.byref(ncow)))
    return slots[:n], cow[:ncow.value]


def pkv_seq_len(pool, seq):
    n = _c_i32()
    _check(load().pkv_seq_len(pool, seq, ctypes.byref(n)))
    return n.value


def pkv_seq_block_table(pool, seq):
    n = _c_i32()
    st = load().pkv_seq_block_table(pool, seq, None, 0, ctypes.byref(n))
    if st != PKV_OK and n.value == 0:
        _check(st)
    out = np.empty(max(n.value, 1), np.int32)
    _check(load().pkv_seq_block_table(pool, seq, _i32p(out), len(out), ctypes.byref(n)))
    return out[:n.value]


def pkv_block_refcount(pool, block):
    r = _c_i32()
    _check(load().pkv_block_refcount(pool, block, ctypes.byref(r)))
    return r.value


def pkv_num_free(pool):
    n = _c_i32()
    _check(load().pkv_num_free(pool, ctypes.byref(n)))
    return n.value


def pkv_free_list(pool):
    n = pkv_num_free(pool)
    out = np.empty(max(n, 1), np.int32)
    cnt = _c_i32()
    _check(load().pkv_free_list(pool, _i32p(out), len(out), ctypes.byref(cnt)))
    return out[:cnt.value]


def pkv_build_block_tables(pool, seqs, max_blocks):
    """Returns ``(tables int32[B, max_blocks], ctx_lens int32[B])``."""
    s = np.ascontiguousarray(seqs, np.int64)
    tables = np.empty((len(s), max(max_blocks, 1)), np.int32)
    lens = np.empty(max(len(s), 1), np.int32)
    _check(load().pkv_build_block_tables(pool, s.ctypes.data_as(_p_i64), len(s), max_blocks,
                                         _i32p(tables), _i32p(lens)))
    return tables[:, :max_blocks], lens[:len(s)]


def pkv_seq_create_cached(pool, tokens):
    """Returns ``(seq, n_cached)``: a new sequence holding the cached blocks
    that match the prompt's leading full blocks."""
    t = np.ascontiguousarray(tokens, np.int32)
    s, nc = _c_i64(), _c_i32()
    _check(load().pkv_seq_create_cached(pool, _i32p(t) if len(t) else None, len(t), ctypes.byref(s), ctypes.byref(nc)))
    return s.value, nc.value


def pkv_prefix_cache_insert(pool, seq, tokens):
    t = np.ascontiguousarray(tokens, np.int32)
    n = _c_i32()
    _check(load().pkv_prefix_cache_insert(pool, seq, _i32p(t) if len(t) else None, len(t), ctypes.byref(n)))
    return n.value


def pkv_prefix_cache_evict(pool, max_blocks):
    out = np.empty(max(max_blocks, 1), np.int32)
    n = _c_i32()
    _check(load().pkv_prefix_cache_evict(pool, max_blocks, _i32p(out), ctypes.byref(n)))
    return [int(x) for x in out[:n.value]]


def pkv_prefix_cache_stats(pool):
    """Returns ``(cached blocks, blocks only the cache holds)``."""
    a, b = _c_i32(), _c_i32()
    _check(load().pkv_prefix_cache_stats(pool, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def pkv_prefix_cache_entry(pool, block):
    """Returns ``(is_cached, predecessor, ids[16], last_use)``."""
    c, p, t = _c_i32(), _c_i32(), _c_i64()
    ids = np.empty(16, np.int32)
    _check(load().pkv_prefix_cache_entry(pool, block, ctypes.byref(c), ctypes.byref(p), _i32p(ids), ctypes.byref(t)))
    return bool(c.value), p.value, [int(x) for x in ids], t.value


def pkv_sched_limits(max_running, prefill_budget):
    a, b = _c_i32(), _c_i32()
    _check(load().pkv_sched_limits(max_running, prefill_budget, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def pkv_sched_create(pool, max_running, prefill_budget):
    out = _vp()
    _check(load().pkv_sched_create(pool, max_running, prefill_budget, ctypes.byref(out)))
    return out.value


def pkv_sched_destroy(sched):
    if sched:
        load().pkv_sched_destroy(sched)


def pkv_sched_submit(sched, req, prompt, max_new):
    t = np.ascontiguousarray(prompt, np.int32)
    _check(load().pkv_sched_submit(sched, req, _i32p(t) if len(t) else None, len(t), max_new))


class StepPlan:
    """Caller-owned arrays of one step plan (sized by pkv_sched_limits)."""

    def __init__(self, max_running, prefill_budget):
        mi, ms = pkv_sched_limits(max_running, prefill_budget)
        self.items = (pkv_step_item * mi)()
        self.slots = np.zeros(ms, np.int32)
        self.cow = np.zeros(2 * mi, np.int32)
        self.pre = np.zeros(mi, np.int64)
        self.adm = np.zeros(mi, np.int64)
        self.adm_hit = np.zeros(mi, np.int32)
        p = pkv_step_plan()
        p.items, p.item_cap = self.items, mi
        p.slots, p.slot_cap = _i32p(self.slots), ms
        p.cow_pairs, p.cow_cap = _i32p(self.cow), mi
        p.preempted, p.preempted_cap = self.pre.ctypes.data_as(_p_i64), mi
        p.admitted, p.admitted_cached, p.admitted_cap = self.adm.ctypes.data_as(_p_i64), _i32p(self.adm_hit), mi
        self.c = p

    def decode(self):
        """``{"items": [(req, seq, kind, start, count, slots, completes)], "cow": [(src, dst)],
        "preempted": [req], "admitted": [(req, cached)]}``."""
        p = self.c
        items = []
        for i in range(p.n_items):
            it = self.items[i]
            items.append((it.req, it.seq, it.kind, it.start, it.count,
                          [int(x) for x in self.slots[it.slot_index:it.slot_index + it.count]], it.completes))
        return {"items": items,
                "cow": [(int(self.cow[2 * i]), int(self.cow[2 * i + 1])) for i in range(p.n_cow)],
                "preempted": [int(x) for x in self.pre[:p.n_preempted]],
                "admitted": [(int(self.adm[i]), int(self.adm_hit[i])) for i in range(p.n_admitted)]}


def pkv_sched_step(sched, plan):
    _check(load().pkv_sched_step(sched, ctypes.byref(plan.c)))
    return plan.decode()


def pkv_sched_commit(sched, next_tokens):
    t = np.ascontiguousarray(next_tokens, np.int32)
    fin = np.zeros(max(len(t), 1), np.int64)
    n = _c_i32()
    _check(load().pkv_sched_commit(sched, _i32p(t) if len(t) else None, len(t), fin.ctypes.data_as(_p_i64),
                                   len(fin), ctypes.byref(n)))
    return [int(x) for x in fin[:n.value]]


def pkv_sched_request(sched, req):
    """Returns ``(tokens, computed, seq, state)``."""
    n, comp, st = _c_i32(), _c_i32(), _c_i32()
    seq = _c_i64()
    _check(load().pkv_sched_request(sched, req, None, 0, ctypes.byref(n), ctypes.byref(comp), ctypes.byref(seq),
                                    ctypes.byref(st)))
    out = np.zeros(max(n.value, 1), np.int32)
    _check(load().pkv_sched_request(sched, req, _i32p(out), len(out), ctypes.byref(n), ctypes.byref(comp),
                                    ctypes.byref(seq), ctypes.byref(st)))
    return [int(x) for x in out[:n.value]], comp.value, seq.value, st.value


def pkv_sched_counts(sched):
    a, b, c = _c_i32(), _c_i32(), _c_i32()
    _check(load().pkv_sched_counts(sched, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def pkv_plan_ints(B):
    return int(load().pkv_plan_ints(B))


def pkv_plan_shared_prefix(pool, seqs, min_blocks=1, max_members=PKV_MAX_SHARERS):
    """Returns ``(plan int32[pkv_plan_ints(B)], n_groups)``."""
    s = np.ascontiguousarray(seqs, np.int64)
    plan = np.full(max(pkv_plan_ints(len(s)), 1), -1, np.int32)
    ng = _c_i32(0)
    _check(load().pkv_plan_shared_prefix(pool, s.ctypes.data_as(_p_i64), len(s), min_blocks, max_members,
                                         _i32p(plan), len(plan), ctypes.byref(ng)))
    return plan[:pkv_plan_ints(len(s))], ng.value


# ---- device calls -------------------------------------------------------------

def pkv_copy_blocks(cfg, pool_dev, pairs_dev, n, stream):
    _check(load().pkv_copy_blocks(ctypes.byref(cfg), pool_dev, pairs_dev, n, stream))


def pkv_append_kv(cfg, pool_dev, layer, k_dev, v_dev, slots_dev, n_tokens, stream):
    _check(load().pkv_append_kv(ctypes.byref(cfg), pool_dev, layer, k_dev, v_dev, slots_dev, n_tokens, stream))


def pkv_decode_workspace_bytes(cfg, num_seqs, num_q_heads, max_context, partition_tokens=0):
    n = load().pkv_decode_workspace_bytes(ctypes.byref(cfg), num_seqs, num_q_heads, max_context,
                                          partition_tokens)
    if n < 0:
        _check(int(n))
    return int(n)


def pkv_prefix_decode_workspace_bytes(cfg, num_seqs, num_q_heads, max_context, max_blocks, partition_tokens=0,
                                      n_groups=0):
    n = load().pkv_prefix_decode_workspace_bytes(ctypes.byref(cfg), num_seqs, num_q_heads, max_context,
                                                 max_blocks, partition_tokens, n_groups)
    if n < 0:
        _check(int(n))
    return int(n)


def pkv_paged_decode(args, stream):
    _check(load().pkv_paged_decode(ctypes.byref(args), stream))


def pkv_paged_decode_noalloc(args, stream):
    _check(load().pkv_paged_decode_noalloc(ctypes.byref(args), stream))


def pkv_paged_prefill(args, stream):
    _check(load().pkv_paged_prefill(ctypes.byref(args), stream))


def pkv_upload(dst_dev, src_host, nbytes, stream):
    _check(load().pkv_upload(dst_dev, src_host, nbytes, stream))


def pkv_probe_stream_read(buf_dev, nbytes, sink_dev, stream):
    _check(load().pkv_probe_stream_read(buf_dev, nbytes, sink_dev, stream))


def pkv_strerror(status):
    return load().pkv_strerror(status).decode()


def pkv_last_error():
    return load().pkv_last_error().decode(errors="replace")
