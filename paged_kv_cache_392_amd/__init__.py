"""Paged KV cache and paged decode attention for AMD Instinct MI355X (gfx950).

The work runs in libpkv (``include/pkv.h``): a C++ block allocator and HIP
kernels for append, copy-on-write block copies, split-K paged decode and the
log-sum-exp merge, and causal paged prefill. This package is its thin Python binding: ``_capi`` keeps
the C names (argument marshalling only) and ``PagedKVCache`` wraps them with
torch tensors for device memory and streams. Importing the package opens
the library and fails loudly if it is not built.
"""

from . import _capi
from ._capi import (  # noqa: F401  (re-exported C names)
    BLOCK_TOKENS, PKV_F16, PKV_I8, PKV_MAX_SHARERS, PKV_PREFIX_GROUP_INTS, PkvError, NoBlocksError, make_config,
    pkv_pool_bytes, pkv_pool_create, pkv_pool_destroy, pkv_seq_create, pkv_seq_free,
    pkv_seq_fork, pkv_seq_reserve, pkv_seq_create_cached, pkv_prefix_cache_insert, pkv_prefix_cache_evict,
    pkv_prefix_cache_stats, pkv_prefix_cache_entry, pkv_sched_limits, pkv_sched_create, pkv_sched_destroy,
    pkv_sched_submit, pkv_sched_step, pkv_sched_commit, pkv_sched_request, pkv_sched_counts, StepPlan,
    PKV_STEP_DECODE, PKV_STEP_PREFILL, pkv_seq_len, pkv_seq_block_table, pkv_block_refcount,
    pkv_num_free, pkv_free_list, pkv_build_block_tables, pkv_plan_ints, pkv_plan_shared_prefix,
    pkv_copy_blocks, pkv_append_kv, pkv_decode_workspace_bytes, pkv_prefix_decode_workspace_bytes, pkv_paged_decode,
    pkv_paged_decode_noalloc, pkv_paged_prefill, pkv_upload, pkv_probe_stream_read, pkv_strerror,
    pkv_last_error,
)
from .cache import PagedKVCache, paged_decode  # noqa: F401

_capi.load()
