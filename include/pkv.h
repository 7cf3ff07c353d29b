/*
 * pkv.h -- C ABI of libpkv: a paged KV cache and paged decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * Source pages cited below:
 *   [p1] KV Cache / PagedAttention / Flash Attention overview,
 *        chanyi.net.cn/article/49, sections 一 to 六
 *   [p2] practitioner notes on KV cache and vLLM, lqnn.cn/news/235768,
 *        sections 1 to 5.3
 *   [p3] course notes "9.1 推理优化：KV Cache、PagedAttention 与 vLLM",
 *        hdu-wiki.cn/courses/inference-kvcache-vllm
 *
 * Conventions
 *   - Every call returns an int status (PKV_OK = 0, negative on error) unless
 *     stated otherwise. No C++ exception crosses this boundary. On error,
 *     pkv_last_error() returns a message for the calling thread.
 *   - The library owns host metadata only. All device memory (the pool, the
 *     tables, q, out, the workspace) belongs to the caller; device calls are
 *     asynchronous on the caller's stream and never allocate.
 *   - A pkv_pool handle is not thread-safe: the caller serialises calls on
 *     one handle.
 *   - Streams are passed as void* and must be a hipStream_t (NULL = the
 *     default stream).
 *
 * Device pool layout (one allocation of pkv_pool_bytes() bytes):
 *   K region   [L][N][Hkv][16][D] elements (fp16 or int8)
 *   V region   same shape, right after K
 *   scales     int8 pools only: [L][N][Hkv][2] fp16 (0 = K scale, 1 = V)
 * One (layer, block, KV head) tile is 16 consecutive token rows of D
 * elements: each block holds a short contiguous run of K/V and blocks need
 * not be contiguous with each other ([p2] §3.2).
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1) /* bad pointer, size, shape or value          */
#define PKV_ERR_NO_BLOCKS (-2)   /* pool exhausted; nothing changed ([p2] §5.2) */
#define PKV_ERR_UNKNOWN_SEQ (-3) /* sequence id not live                        */
#define PKV_ERR_REFCOUNT (-4)    /* block refcount inconsistency                */
#define PKV_ERR_UNSUPPORTED (-5) /* head_dim / dtype / group size not built     */
#define PKV_ERR_HIP (-6)         /* a HIP runtime call failed                   */

/* ---- element types ------------------------------------------------------ */
#define PKV_F16 0 /* IEEE binary16 K/V                                          */
#define PKV_I8 1  /* int8 K/V with one fp16 scale per (block, KV head), [p2] §4.1 */

#define PKV_BLOCK_TOKENS 16 /* tokens per block: the page size of [p1] §三, [p2] §3.2 */

/* Shape of one pool. Validated by every call that takes it:
 * num_layers >= 1, num_blocks >= 1, block_size == 16, num_kv_heads >= 1,
 * head_dim in {64, 128}, dtype in {PKV_F16, PKV_I8}. */
typedef struct pkv_config {
  int32_t num_layers;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
} pkv_config;

typedef struct pkv_pool pkv_pool;

/* Bytes of device memory the pool needs: N*16 token slots of
 * 2*L*Hkv*D*elem_bytes each (the per-token size of [p2] §2.3), plus
 * N*L*Hkv*2 fp16 scales for int8. Returns < 0 (a status) on a bad config. */
int64_t pkv_pool_bytes(const pkv_config* cfg);

/* ---- host block allocator ([p1] §三, [p2] §3.2) --------------------------- */

/* Create the host metadata of a pool of cfg->num_blocks blocks.
 * free_order: a permutation of 0..N-1 giving the order in which blocks are
 * handed out (NULL = 0,1,2,...); n must equal N when free_order is given.
 * The free list is a LIFO stack: a freed sequence pushes its blocks in
 * reverse logical order, and the next allocation takes the last one pushed.
 * *out receives the handle. The library allocates no device memory. */
int pkv_pool_create(const pkv_config* cfg, const int32_t* free_order, int32_t n, pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);

/* A new, empty sequence. Ids count up from 1 in creation order. */
int pkv_seq_create(pkv_pool* pool, int64_t* seq);
/* Release a finished request: each of its blocks loses a reference and a
 * block that reaches zero returns to the free list at once ([p1] §三,
 * [p2] §3.2). */
int pkv_seq_free(pkv_pool* pool, int64_t seq);
/* A new sequence sharing all of parent's blocks (refcount + 1 each); blocks
 * are copied only when one sharer later writes into a shared block, as with
 * Unix fork() ([p1] §三). */
int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t* child);

/* Reserve slots for n new tokens appended at the tail of seq ([p2] §2.2).
 * slots_out[n] receives slot = physical_block*16 + offset for each token in
 * order. A token at offset 0 opens a new block. A token written at a
 * non-zero offset of a block shared with another sequence first moves the
 * writer to a fresh block (copy-on-write): the (src, dst) block pair is
 * appended to cow_pairs_out (int32 [cow_cap][2]) and *n_cow counts them; the
 * caller copies those blocks with pkv_copy_blocks before writing.
 * All or nothing: on PKV_ERR_NO_BLOCKS (or INVALID_ARG for cow_cap too small)
 * no state changes, so the caller may queue the request ([p2] §5.2).
 * slots_out may be NULL only when n == 0. */
int pkv_seq_reserve(pkv_pool* pool, int64_t seq, int32_t n, int32_t* slots_out,
                    int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow);

/* ---- introspection (host) ------------------------------------------------- */
int pkv_seq_len(const pkv_pool* pool, int64_t seq, int32_t* len);
/* Logical -> physical block map of seq; *n = number of blocks. cap < *n is
 * INVALID_ARG (and *n still reports the size). */
int pkv_seq_block_table(const pkv_pool* pool, int64_t seq, int32_t* out, int32_t cap, int32_t* n);
int pkv_block_refcount(const pkv_pool* pool, int32_t block, int32_t* ref);
int pkv_num_free(const pkv_pool* pool, int32_t* n);
/* Free blocks, the next to be handed out first. */
int pkv_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* Pack the tables of B sequences into host buffers for upload:
 * tables_host int32 [B][max_blocks] (unused entries = -1) and
 * ctx_lens_host int32 [B] (tokens held by each sequence). INVALID_ARG if a
 * table is wider than max_blocks. The decode walks these rows in logical
 * order instead of gathering blocks into contiguous memory ([p2] §3.2). */
int pkv_build_block_tables(const pkv_pool* pool, const int64_t* seqs, int32_t B, int32_t max_blocks,
                           int32_t* tables_host, int32_t* ctx_lens_host);

/* ---- prefix cache (host) ([p2] §4.3: K/V kept block by block with the
 * order of the blocks recorded, so a request whose prefix matches an earlier
 * one reuses those blocks and computes only the rest) ------------------------
 * Only full blocks are cached, each identified by its 16 token ids and the
 * cached block before it; matching compares the ids. The cache holds one
 * reference on every cached block. A block that only the cache holds and
 * that no cached block follows is evictable; eviction takes the least
 * recently used one first (a hit or an insert marks its chain used).
 * pkv_seq_reserve evicts just enough cache-only blocks when the free list
 * is short; if free plus cache-only blocks are still too few it returns
 * PKV_ERR_NO_BLOCKS and changes nothing. */

/* Create a sequence for a prompt of n token ids: its leading full blocks
 * are taken from the cache while they match (at most floor((n-1)/16), so
 * the last token is always computed), each gaining a reference. *n_cached
 * receives the tokens the sequence now holds (a multiple of 16); the caller
 * reserves and computes tokens n_cached .. n-1. */
int pkv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int32_t n, int64_t* seq, int32_t* n_cached);

/* Register seq's full blocks holding its first n tokens (token ids, K/V
 * already written) in the cache, in order; stops at the first block whose
 * content is already cached as another block. *n_added (optional) receives
 * the blocks newly cached. */
int pkv_prefix_cache_insert(pkv_pool* pool, int64_t seq, const int32_t* tokens, int32_t n, int32_t* n_added);

/* Evict up to max_blocks evictable blocks, least recently used first;
 * evicted_out (max_blocks ints) receives them in order, *n_evicted their
 * count. The blocks go back to the free list. */
int pkv_prefix_cache_evict(pkv_pool* pool, int32_t max_blocks, int32_t* evicted_out, int32_t* n_evicted);

/* Cached blocks, and how many of them only the cache holds. */
int pkv_prefix_cache_stats(const pkv_pool* pool, int32_t* n_cached, int32_t* n_reclaimable);

/* Introspection for exact tests: whether `block` is cached, its predecessor
 * (-1 for none), its 16 ids (ids[16]) and its last-use tick. */
int pkv_prefix_cache_entry(const pkv_pool* pool, int32_t block, int32_t* is_cached, int32_t* pred, int32_t* ids,
                           int64_t* last_use);

/* ---- continuous batching (host) ([p2] §3.3: finished requests leave the
 * batch after every step and free their blocks, waiting requests come in;
 * [p2] §5.2: a full pool makes requests wait; [p2] §4.3: a request starts
 * from the cached blocks of its prefix) -------------------------------------
 * A request is its token list (prompt, then each generated token); its K/V
 * are computed in order. pkv_sched_step plans one step:
 *   1. decode: every running request with no chunk left whose newest token
 *      still needs its K/V gets one slot, in admission order; if the pool
 *      refuses, the newest running request is preempted (its sequence is
 *      freed, it returns to the front of the queue and is recomputed later,
 *      from whatever the prefix cache still holds), until the slot is
 *      granted or the request itself yielded;
 *   2. admission: while fewer than max_running run, the first waiting
 *      request starts a sequence from the prefix cache and reserves slots
 *      for the rest of its tokens, or stays first and admission stops;
 *   3. prefill: running requests with tokens left get chunks in admission
 *      order, prefill_budget tokens per step in all.
 * The caller writes each item's K/V into its slots (after copying any
 * copy-on-write pairs), attends, and passes pkv_sched_commit the next token
 * of every item that computed its request's newest token (completes = 1),
 * in item order. A request with max_new generated tokens then inserts its
 * computed tokens into the prefix cache and frees its sequence; a request
 * whose prompt is first computed inserts the prompt. */

#define PKV_STEP_DECODE 0
#define PKV_STEP_PREFILL 1
#define PKV_REQ_WAITING 0
#define PKV_REQ_RUNNING 1
#define PKV_REQ_FINISHED 2

typedef struct pkv_sched pkv_sched;

typedef struct pkv_step_item {
  int64_t req;         /* request id                                          */
  int64_t seq;         /* its sequence in the pool                            */
  int32_t kind;        /* PKV_STEP_DECODE or PKV_STEP_PREFILL                 */
  int32_t start;       /* position of the item's first token                  */
  int32_t count;       /* tokens (1 for a decode)                             */
  int32_t slot_index;  /* index of its first slot in the plan's slots         */
  int32_t completes;   /* 1: the item computes the request's newest token     */
} pkv_step_item;

typedef struct pkv_step_plan {  /* caller-owned arrays, capacities from
                                   pkv_sched_limits; decode items come first */
  pkv_step_item* items;
  int32_t item_cap, n_items;
  int32_t* slots;
  int32_t slot_cap, n_slots;
  int32_t* cow_pairs;          /* (src, dst) block pairs to copy first:
                                  2 x cow_cap ints; cow_cap, n_cow in pairs   */
  int32_t cow_cap, n_cow;
  int64_t* preempted;
  int32_t preempted_cap, n_preempted;
  int64_t* admitted;
  int32_t* admitted_cached;    /* tokens each admitted request took from the cache */
  int32_t admitted_cap, n_admitted;
} pkv_step_plan;

/* The plan array sizes a step may need: items (also preempted, admitted and
 * copy-on-write pairs) and slots. */
int pkv_sched_limits(int32_t max_running, int32_t prefill_budget, int32_t* max_items, int32_t* max_slots);
int pkv_sched_create(pkv_pool* pool, int32_t max_running, int32_t prefill_budget, pkv_sched** out);
void pkv_sched_destroy(pkv_sched* sched);
/* Queue a request (ids unique; n >= 1 prompt tokens; max_new >= 1).
 * INVALID_ARG for a request whose n + max_new tokens need more blocks than
 * the whole pool (it could never run). Requests that fit the pool but find
 * it held by sequences outside the scheduler wait until those are freed. */
int pkv_sched_submit(pkv_sched* sched, int64_t req, const int32_t* prompt, int32_t n, int32_t max_new);
/* Plan one step into `plan` (INVALID_ARG, nothing changed, if its arrays
 * are below the limits). */
int pkv_sched_step(pkv_sched* sched, pkv_step_plan* plan);
/* Hand out the next tokens of the last plan's completing items, in item
 * order; finished (at least as many entries as next tokens) receives the
 * requests that finished. */
int pkv_sched_commit(pkv_sched* sched, const int32_t* next_tokens, int32_t n, int64_t* finished, int32_t fin_cap,
                     int32_t* n_finished);
/* A request's tokens (tokens may be NULL to query the count), computed
 * tokens, sequence (0 if none) and PKV_REQ_* state. */
int pkv_sched_request(const pkv_sched* sched, int64_t req, int32_t* tokens, int32_t cap, int32_t* n_tokens,
                      int32_t* computed, int64_t* seq, int32_t* state);
int pkv_sched_counts(const pkv_sched* sched, int32_t* n_waiting, int32_t* n_running, int32_t* n_finished);

/* ---- shared-prefix plan (host) ([p1] §三: requests with a common prefix
 * point at the same physical blocks) -------------------------------------- */

#define PKV_MAX_SHARERS 32         /* sequences per shared-prefix group        */
#define PKV_PREFIX_GROUP_INTS 34   /* ints per group: blocks, members, ids[32]  */

/* Ints a plan for B sequences may need: 2 B + (B / 2) * PKV_PREFIX_GROUP_INTS. */
int32_t pkv_plan_ints(int32_t B);

/* Group the B sequences (batch order) whose block tables begin with the same
 * physical blocks, so one decode reads those blocks once for all of them.
 * Sequences are keyed by their first block; each key's sequences form groups
 * of up to max_members (1..PKV_MAX_SHARERS) in batch order. A group's shared
 * run is the longest run of leading blocks identical in all its members,
 * ending before the block holding each member's last token (so every member
 * keeps a private suffix, and an appended token is never in a shared block);
 * groups of fewer than 2 members or fewer than min_blocks (>= 1) shared
 * blocks are dropped.
 * plan_host (int32, plan_cap >= pkv_plan_ints(B)) receives:
 *   [0, 2B)      per sequence b: [2b] = its shared blocks (0 if ungrouped),
 *                [2b + 1] = group * 64 + member, or -1
 *   then per group g, PKV_PREFIX_GROUP_INTS ints at 2B + g * 34:
 *                [shared blocks, member count, batch index of each member
 *                 (-1 padded)]
 * *n_groups receives the group count. The plan holds batch indices: it is
 * valid for this `seqs` order and these tables. INVALID_ARG on bad sizes,
 * UNKNOWN_SEQ for an unknown id. */
int pkv_plan_shared_prefix(const pkv_pool* pool, const int64_t* seqs, int32_t B, int32_t min_blocks,
                           int32_t max_members, int32_t* plan_host, int32_t plan_cap, int32_t* n_groups);

/* ---- device operations (asynchronous on `stream`) ------------------------ */

/* Copy-on-write block copy ([p1] §三): for each of the n (src, dst) pairs in
 * pairs_dev (int32 [n][2], device), copy the whole block -- every layer, K
 * and V, and the int8 scales -- from src to dst. Pairs with an id outside
 * [0, N) are skipped. n == 0 is a no-op. */
int pkv_copy_blocks(const pkv_config* cfg, void* pool_dev, const int32_t* pairs_dev, int32_t n,
                    void* stream);

/* Append ([p2] §2.2 pseudocode: the new token's k and v go to the cache
 * tail; cached K/V are never modified afterwards, [p1] §二): for token i,
 * write k_dev[i] and v_dev[i] (fp16, contiguous [n_tokens][Hkv][D], device)
 * into slot slots_dev[i] (int32, device) of `layer`. Slots outside [0, 16N)
 * are skipped.
 *   fp16 pools: bit-exact copy.
 *   int8 pools ([p2] §4.1, 8-bit K/V with group scales): quantise on write,
 *   one (block, KV head) scale each for K and V. A token at offset 0 sets
 *   the block's scale from its own absmax (fp16(absmax / 127)); a token
 *   whose absmax fits 127 * scale is coded with that scale; otherwise the
 *   block takes the new token's scale and its earlier codes are re-rounded
 *   into it (the scale never shrinks; earlier rows move by at most half a
 *   step). Codes are rint(x / scale) clipped to [-127, 127]. Tokens that
 *   write one block must be adjacent in the call and in increasing offset,
 *   as pkv_seq_reserve returns them. */
int pkv_append_kv(const pkv_config* cfg, void* pool_dev, int32_t layer, const void* k_dev,
                  const void* v_dev, const int32_t* slots_dev, int32_t n_tokens, void* stream);

/* Arguments of one paged decode step over a batch ([p2] §1.2 attention of
 * the new token's query over all cached tokens; [p2] §3.2 walk through the
 * block table). */
typedef struct pkv_decode_args {
  const pkv_config* cfg;
  const void* pool_dev;           /* the pool, layout above (written only by the
                                     fused append below)                         */
  int32_t layer;                  /* 0 <= layer < L                               */
  const void* q_dev;              /* fp16 [B][Hq][D]                              */
  int32_t num_seqs;               /* B >= 1                                       */
  int32_t num_q_heads;            /* Hq, a multiple of Hkv; G = Hq/Hkv in 1..8     */
  const int32_t* block_tables_dev;/* int32 [B][max_blocks], -1 padded             */
  int32_t max_blocks;             /* row stride of the tables                     */
  const int32_t* ctx_lens_dev;    /* int32 [B], tokens attended (>= 1)            */
  const int32_t* ctx_lens_host;   /* optional host copy of ctx_lens_dev (same
                                     values), validated if non-NULL; with
                                     automatic partitions it also sizes them */
  int32_t max_context;            /* >= every ctx_len; sizes the grid             */
  void* out_dev;                  /* fp16 [B][Hq][D], written by the call         */
  float scale;                    /* softmax scale, usually 1/sqrt(D)             */
  void* workspace_dev;            /* split-K partials, caller owned               */
  int64_t workspace_bytes;        /* >= pkv_decode_workspace_bytes(...)           */
  int32_t partition_tokens;       /* tokens per split-K partition, a multiple of
                                     16 in [16, 4096]; 0 = automatic             */
  const void* k_new_dev;          /* optional fused append (NULL = none, the
                                     default): fp16 [B][Hkv][D] k and v of one new
                                     token per sequence, stored first at logical
                                     position ctx_lens[b] - 1 of sequence b (the
                                     slot pkv_seq_reserve gave that token; any
                                     copy-on-write pairs already copied), then
                                     attended like every other token. Same bytes
                                     as pkv_append_kv (int8 pools: quantised on
                                     write by the same rule).                    */
  const void* v_new_dev;
  const int32_t* prefix_plan_dev; /* optional shared-prefix plan (NULL = none):
                                     pkv_plan_shared_prefix's output for these
                                     sequences in this order, uploaded. Each
                                     group's shared blocks are read once for all
                                     its members (fp16 and int8 pools). Same
                                     result up to rounding.                      */
  const int32_t* prefix_plan_host;/* optional host copy, validated if non-NULL    */
  int32_t prefix_groups;          /* groups in the plan (0 = no plan)             */
  void* const* timing_events;     /* optional (NULL = none): 4 hipEvent_t recorded
                                     around the split kernel ([0] start, [1] stop)
                                     and the merge kernel ([2], [3]; untouched if
                                     the merge is not needed). Instrumentation
                                     only; the result does not depend on it.     */
} pkv_decode_args;

/* Workspace bytes pkv_paged_decode needs for these sizes (0 when every
 * sequence fits one partition). Returns < 0 (a status) on bad arguments.
 * partition_tokens 0 = room for the finest automatic cut (partitions for
 * about 2048 work-groups at max_context; an automatic launch never cuts
 * finer). Layout: fp32 partials m [B][Hq][P], l [B][Hq][P], o [B][Hq][P][D]. */
int64_t pkv_decode_workspace_bytes(const pkv_config* cfg, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_context, int32_t partition_tokens);

/* Paged decode: out[b][h] = softmax(q[b][h] . K_b^T * scale) . V_b over the
 * ctx_lens[b] tokens of sequence b, read in place through its block table
 * (no gather), with query head h using KV head h / (Hq/Hkv) ([p2] §1.2,
 * §3.2, §4.2). Split-K: the context is cut into partitions of
 * partition_tokens (a multiple of 16); each partition runs an online
 * softmax ([p1] §四) and writes a (max, sum, weighted-V) partial, and a
 * second kernel merges the partials by log-sum-exp in partition order
 * (skipped when every sequence fits one partition). Automatic partitions
 * (partition_tokens 0): the fewest rounds of work-groups resident on the
 * device at once, over each sequence's blocks (from ctx_lens_host when
 * given, else every sequence at max_context), and among those the finest
 * cut; 16 to 256 blocks per partition, never finer than the workspace's
 * cut. The partition size changes the result only by rounding. With
 * ctx_lens_host, automatic partitions, no shared-prefix plan and at most 1024
 * sequences, a ragged batch (one whose grid of (sequence, partition) slots
 * at max_context would hold slots past some sequence's last partition) is
 * split stream-K: all sequences' blocks laid end to end, each sequence's
 * led by a few blocks' worth of start-up charge that hold no work, are cut
 * into equal runs, about one round of resident work-groups, a run possibly
 * ending one sequence and starting the next (and then holding fewer real
 * blocks), and each sequence's pieces are merged in order. ctx_lens_host
 * must then equal the device lengths (a mismatch gives wrong output for the
 * sequences it misstates and possibly for those after them, never an
 * access out of bounds).
 * Accumulation is fp32 and
 * the output is rounded to fp16 (nearest even). The result depends only on
 * logical token order, not on physical block ids, and is bitwise
 * reproducible. Slots past ctx_len in a tail block are never used. Block ids
 * outside [0, N) are treated as empty.
 *
 * Workspace: device memory of at least pkv_decode_workspace_bytes() bytes,
 * 16-byte aligned, scratch owned by the caller (no initial contents needed;
 * contents after the call unspecified). Calls sharing one workspace must be
 * ordered on one stream.
 *
 * With a shared-prefix plan (prefix_plan_dev, prefix_groups > 0), extra
 * work-groups of the same launch attend every group's members to the
 * group's shared blocks, reading each K/V tile once for up to 128
 * query rows on the matrix cores; the split work-groups cover each grouped
 * sequence from its first unshared block, and the merge combines prefix and
 * suffix partials in logical order. The workspace must hold
 * pkv_prefix_decode_workspace_bytes() bytes. Members x (Hq/Hkv) must not
 * exceed 128. On int8 pools the shared tiles are dequantised (code x block
 * scale, rounded to fp16) as they are staged for the matrix cores;
 * INVALID_ARG for an inconsistent plan when the host copy is given (without
 * it the plan is trusted: a wrong plan gives wrong results, never an
 * out-of-bounds access). With both host copies (lengths and plan) and
 * automatic partitions, split-K partitions are sized for the longest
 * unshared stretch instead of max_context. With the plan's host copy the
 * launch also cuts shared runs into prefix partitions of about 32 blocks
 * (never more partitions than the workspace holds); without it, into as
 * many as the workspace holds. The output is the same up to rounding.
 *
 * With k_new_dev/v_new_dev set, the call also performs the append step of
 * [p2] §2.2 for every sequence (one token each) before attending: the
 * decode step of the pages in one launch. pool_dev is then written.
 *
 * INVALID_ARG: null pointers, ctx_len == 0 or > 16*max_blocks or >
 * max_context (host copy), workspace too small or misaligned,
 * partition_tokens not a multiple of 16, only one of k_new/v_new given.
 * UNSUPPORTED: head_dim not 64 or 128, or more than 8 query heads per KV
 * head (groups of 3, 5, 6 or 7 run on the kernels built for 4 and 8, their
 * extra heads never written). */
int pkv_paged_decode(const pkv_decode_args* args, void* stream);

/* pkv_paged_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, kernels and results, but the split-K
 * partials go to the library's own scratch, a file-scope device array of
 * PKV_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the library's load
 * until the process ends; workspace_dev and workspace_bytes are ignored. The
 * call allocates no device memory (its first call on a device looks up the
 * array's address there, once). INVALID_ARG, with a message naming the
 * limit, when the decode needs more than that maximum
 * (pkv_decode_workspace_bytes / pkv_prefix_decode_workspace_bytes give the
 * need); every other check and status is pkv_paged_decode's. The scratch
 * needs no initial contents and keeps the last call's partials: all calls on
 * one GPU share it, so calls that may overlap on one GPU (different streams,
 * threads or processes sharing the library) race and must be serialised by
 * the caller, for instance by issuing them on one stream. */
#define PKV_NOALLOC_SCRATCH_BYTES (16 << 20)
int pkv_paged_decode_noalloc(const pkv_decode_args* args, void* stream);

/* Workspace bytes pkv_paged_decode needs with a shared-prefix plan of
 * n_groups groups: the whole workspace, in place of
 * pkv_decode_workspace_bytes() (equal to it when n_groups == 0). Layout:
 * fp32 partial rows m [B][Hq][P], l [B][Hq][P], o [B][Hq][P][D] whose P
 * slots hold a grouped sequence's prefix partials (one per prefix partition
 * of at most 64 shared blocks) followed by its split-K partials. Returns < 0
 * (a status) on bad arguments. */
int64_t pkv_prefix_decode_workspace_bytes(const pkv_config* cfg, int32_t num_seqs, int32_t num_q_heads,
                                          int32_t max_context, int32_t max_blocks, int32_t partition_tokens,
                                          int32_t n_groups);

/* ---- paged prefill ([p1] §二, [p2] §1.3: a prompt's tokens are processed
 * together; [p1] §四: tiled attention with an online softmax) ------------- */

typedef struct pkv_prefill_args {
  const pkv_config* cfg;
  const void* pool_dev;
  int32_t layer;
  const void* q_dev;              /* fp16 [T][Hq][D]: the chunks' queries,
                                     sequence after sequence                     */
  int32_t num_seqs;               /* B, in [1, 65535]                             */
  int32_t num_q_heads;            /* Hq, a multiple of Hkv; Hq/Hkv in 1..8        */
  const int32_t* q_start_dev;     /* int32 [B + 1]: sequence b's rows of q and out
                                     are q_start[b] .. q_start[b + 1] - 1         */
  const int32_t* q_start_host;    /* the same, on the host: required              */
  const int32_t* block_tables_dev;/* int32 [B][max_blocks]                        */
  int32_t max_blocks;
  const int32_t* ctx_lens_dev;    /* int32 [B]: tokens cached, the chunk's own
                                     included (append the chunk's K/V first)      */
  const int32_t* ctx_lens_host;   /* optional host copy, validated if non-NULL    */
  int32_t max_context;            /* >= every ctx_len                             */
  void* out_dev;                  /* fp16 [T][Hq][D]                              */
  float scale;                    /* softmax scale, normally 1/sqrt(D)            */
} pkv_prefill_args;

/* Causal attention of a chunk of new tokens per sequence over its paged
 * cache: token i of sequence b's chunk (qlen_b = q_start[b+1] - q_start[b]
 * tokens) sits at logical position ctx_lens[b] - qlen_b + i and attends to
 * tokens 0..that position, itself included; with ctx_lens[b] > qlen_b the
 * chunk follows cached tokens (chunked prefill). Query head h uses KV head
 * h / (Hq/Hkv). The K/V rows are read in place through the block table.
 * fp32 accumulation, fp16 probabilities in the value product, fp16 output
 * (nearest even). The chunk's K/V must already be in the cache
 * (pkv_append_kv). fp16 or int8 pools (int8 tiles dequantised, code x
 * block scale rounded to fp16, as they are staged); head_dim 64 or 128. No
 * workspace.
 * Any context length: a work-group keeps its block ids in a ring of 1024
 * in LDS, refilled as it walks longer contexts.
 * INVALID_ARG: null pointers, q_start not starting at 0 or decreasing,
 * misalignment, a chunk longer than its context or a context out of range
 * (host copies). UNSUPPORTED: more than 8 query heads per KV head, or
 * head_dim not 64 or 128 (a query tile holds floor(128 / G) tokens).
 * Sequences with qlen_b = 0 are skipped. */
int pkv_paged_prefill(const pkv_prefill_args* args, void* stream);

/* Upload host metadata for the next step (block tables, lengths: the
 * per-step upload of [p2] §3.3's batch that changes every step) from pinned
 * host memory to device memory, with a kernel on `stream` that reads the
 * host buffer through its device mapping. The copy stays on the compute
 * queue: no hand-off to a copy engine between kernels. src_host must be
 * pinned host memory allocated for the device (hipHostMalloc, torch
 * pin_memory); it is read when the kernel runs, so the caller keeps it
 * unchanged until then. dst_dev must be device memory. Both 16-byte aligned.
 * INVALID_ARG (no launch): bytes < 0, null or misaligned pointers, src not
 * pinned host memory, dst not device memory. bytes == 0 is a no-op. */
int pkv_upload(void* dst_dev, const void* src_host, int64_t bytes, void* stream);

/* ---- measurement helper ------------------------------------------------------ */

/* Plain coalesced read of `bytes` (>= 16) bytes at buf_dev (16-byte aligned),
 * the reference for achievable HBM read bandwidth on this device. sink_dev
 * must point to 4 writable device bytes (practically never written). */
int pkv_probe_stream_read(const void* buf_dev, int64_t bytes, void* sink_dev, void* stream);

/* ---- errors ---------------------------------------------------------------- */
const char* pkv_strerror(int status);
const char* pkv_last_error(void); /* thread-local; "" if none */

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
