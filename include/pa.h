/*
 * pa.h — paged KV-cache attention for AMD Instinct MI355X (gfx950). C ABI.
 *
 * What is computed. A sequence's keys and values live in fixed-size physical
 * blocks ("pages") of two pools, k_cache and v_cache, each laid out
 * [num_blocks, block_size, num_kv_heads, head_dim] ("LLM推理优化：技术原理解析
 * 总览", dpshk.com, §3.3 — the page layout, block_size 16 typical). A
 * per-sequence block table maps logical block i to a physical block id
 * ("vLLM的'内存分页'到底多神奇 — PagedAttention原理图解", xxqk.cn, §2: pages,
 * the per-sequence page table, the free-page list). Attention walks the table,
 * reads the pages in logical order as one contiguous K/V, and computes
 * softmax(scale · q·Kᵀ)·V (same page, §3 phase 2).
 *
 * Conventions shared by every call:
 *  - Status: every call returns pa_status (0 = OK) and never throws across the
 *    ABI. On error nothing is launched and no state changes; pa_last_error()
 *    gives a thread-local message for the last non-OK status of this thread.
 *  - Ownership: the library owns only the pool handle and its host-side
 *    bookkeeping. All device buffers (k_cache, v_cache, q, out, tables,
 *    workspace) are allocated and owned by the caller, who keeps them alive
 *    until the stream work that uses them has completed.
 *  - Pointers marked "device" are device (HBM) addresses on the current HIP
 *    device; pointers marked "host" are ordinary host memory.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream). Device
 *    calls are asynchronous: they enqueue work and return.
 *  - Threads: a pool is not thread-safe; callers serialise calls on one pool.
 *  - Supported set: head_dim ∈ {64, 128}; block_size ∈ {8, 16, 32};
 *    dtype ∈ {PA_F32, PA_BF16, PA_FP8_E4M3}; num_q_heads a multiple of
 *    num_kv_heads with group G = num_q_heads / num_kv_heads ∈ {1, 2, 4, 8}.
 *    q, out and the pools share one dtype, except that an FP8 pool takes
 *    bf16 q, out and K/V rows (PA_FP8_E4M3 needs head_dim 128 and is served
 *    by pa_write_kv and pa_decode; pa_prefill returns PA_ERR_UNSUPPORTED).
 *    Anything else returns PA_ERR_UNSUPPORTED.
 *  - Grouped-query attention: q head h reads kv head h / G.
 *  - Block ids in tables are int32. Table contents are not validated on the
 *    device: an id outside [0, num_blocks) is undefined (the kernels clamp it
 *    into range so that it cannot fault, and the result is then meaningless).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument (null pointer, negative size, bad geometry) */
  PA_ERR_NO_BLOCKS = -2,   /* free list cannot cover the request; nothing changed      */
  PA_ERR_UNSUPPORTED = -3, /* valid but outside the supported set                      */
  PA_ERR_HIP = -4,         /* a HIP runtime call failed (launch, device query)         */
  PA_ERR_UNKNOWN_SEQ = -5  /* sequence id not known to the pool                        */
} pa_status;

/* PA_FP8_E4M3: the pools hold 8-bit OCP E4M3 codes (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; 0x7F/0xFF NaN, no infinity, largest finite
 * 448), one code per element, with one scale per pool for K and one for V
 * (pa_pool_set_kv_scales): a code c stands for value(c) · scale. The FP8 KV
 * cache is the remedy "LLM推理优化：技术原理解析总览" (dpshk.com) §5.1 gives
 * for a 16-bit cache next to a quantised model; the page names no format. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Geometry of the two pools. dtype holds a pa_dtype value. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
} pa_kv_layout;

typedef struct pa_pool pa_pool; /* opaque, library-owned */

/* Block accounting ("vLLM的'内存分页'到底多神奇", §5 monitoring: cache usage).
 * used = refcount > 0; shared = refcount > 1; allocated_slots = used ×
 * block_size; filled_slots = slots holding a valid token. The difference is
 * the in-page tail waste, the only fragmentation paging leaves (same page,
 * §2 comparison table). */
typedef struct {
  int32_t free_blocks;
  int32_t used_blocks;
  int32_t shared_blocks;
  int32_t pending_copies;  /* copy-on-write block copies not yet run (see pa_write_kv) */
  int64_t filled_slots;
  int64_t allocated_slots;
} pa_pool_stats_t;

/* ------------------------------------------------------------------------ */
/* Pool and host block manager                                               */
/* ------------------------------------------------------------------------ */

/* Create a pool over caller-owned device buffers k_cache and v_cache: the
 * fixed-size physical pages and the free-page list the scheduler hands them
 * out from ("vLLM的'内存分页'到底多神奇", xxqk.cn, §2), each buffer laid out
 * [num_blocks, block_size, num_kv_heads, head_dim] ("LLM推理优化：技术原理解析
 * 总览", §3.3), sized by the caller to its memory budget (the budget setting
 * of the same xxqk.cn page, §4). Each buffer holds
 * layout->num_blocks × block_size × num_kv_heads × head_dim elements of
 * layout->dtype, row-major in that order. free_order (host, may be NULL) is a
 * permutation of [0, num_blocks) giving the order in which free blocks are
 * handed out (free_order[0] first); NULL means ascending ids. The free list is
 * a LIFO stack: blocks returned by pa_seq_free are reused first.
 * On success *out receives the handle. Errors: PA_ERR_INVALID (null pointers,
 * non-positive sizes, free_order not a permutation), PA_ERR_UNSUPPORTED
 * (geometry outside the supported set). */
pa_status pa_alloc_pool(const pa_kv_layout* layout, void* k_cache, void* v_cache,
                        const int32_t* free_order, pa_pool** out);

/* Destroy a pool handle (host bookkeeping only; device buffers stay the
 * caller's). NULL is ignored. Library addition (no passage): the handle's
 * lifetime. */
void pa_free_pool(pa_pool* pool);

/* Grow sequence seq_id by n_tokens (creating it if unknown), taking new blocks
 * from the free list on demand: a token goes into the sequence's last block
 * until it is full, then a fresh block is taken ("vLLM的'内存分页'到底多神奇",
 * §3 phase 1). All-or-nothing: if the free list cannot cover the new blocks,
 * returns PA_ERR_NO_BLOCKS and changes nothing (admission control, same page,
 * §4). slots_out (host, n_tokens int64, may be NULL when n_tokens == 0)
 * receives the flat slot of each new token, slot = table[pos / block_size] ×
 * block_size + pos % block_size, for pos = old_len .. old_len + n_tokens - 1.
 * Errors: PA_ERR_INVALID (n_tokens < 0, null slots_out, length overflow). */
pa_status pa_seq_append(pa_pool* pool, int64_t seq_id, int32_t n_tokens, int64_t* slots_out);

/* One decode step's bookkeeping in one call: grow each of the n distinct
 * sequences seq_ids[0..n) (host) by n_tokens, exactly as n pa_seq_append
 * calls in that order would, but all-or-nothing over the whole batch: if the
 * free list cannot cover every new block of the batch, returns
 * PA_ERR_NO_BLOCKS and changes nothing (admission control,
 * "vLLM的'内存分页'到底多神奇", §4). slots_out (host, n × n_tokens int64,
 * may be NULL when n_tokens == 0): row i holds seq_ids[i]'s new slots.
 * Errors: PA_ERR_INVALID (negative sizes, null pointers, a sequence id twice
 * in the batch, length overflow). */
pa_status pa_seq_append_batch(pa_pool* pool, const int64_t* seq_ids, int32_t n, int32_t n_tokens,
                              int64_t* slots_out);

/* Append n_tokens tokens whose ids are known (token_ids, host, n_tokens
 * int32), with prefix caching: when several sequences start with the same
 * prompt, they reuse the same physical blocks ("vLLM 生产级落地深剖",
 * musen-ai.com, §2; blocks are found by hashing, §5). Every block that
 * token-aware appends fill completely is registered under a key standing for
 * the ids of all tokens from position 0 to the block's end (a 64-bit FNV-1a
 * chain; a match also compares the block's ids and its parent key). When the
 * append reaches a block boundary, the following full blocks of new tokens
 * are looked up in order; while found, each is shared (refcount + 1; a
 * cached block with refcount 0 is taken back off the free list) instead of
 * allocated, and its tokens get slot -1 in slots_out (host, n_tokens int64):
 * their K/V is already in the pool, and pa_write_kv skips -1. Lookups stop
 * at the first miss. A registered block keeps its key after it is freed,
 * until it is handed out again (then the key is dropped). *n_cached_out
 * (host) receives the number of -1 slots. Admission is all-or-nothing over
 * fresh blocks, copy-on-write and cached blocks taken off the free list.
 * A sequence created or grown by pa_seq_append / pa_seq_append_batch has
 * token ids the pool does not know: it is never keyed, and this call then
 * behaves as pa_seq_append. pa_seq_fork copies the keys of the source.
 * Errors: as pa_seq_append. */
pa_status pa_seq_append_tokens(pa_pool* pool, int64_t seq_id, const int32_t* token_ids, int32_t n_tokens,
                               int64_t* slots_out, int32_t* n_cached_out);

/* Prefix-cache counters: blocks holding a registered key (in use or free),
 * full blocks looked up and found since the pool was created (the cache hit
 * rate the prefix caching of "vLLM 生产级落地深剖", §2, is judged by; the
 * counters themselves are a library addition). Errors: PA_ERR_INVALID (null
 * pointers). */
typedef struct {
  int32_t cached_blocks;
  int64_t lookups;
  int64_t hits;
} pa_prefix_stats_t;
pa_status pa_pool_prefix_stats(const pa_pool* pool, pa_prefix_stats_t* out);

/* Block size for a pool of sequences of the given expected length class,
 * after the tiers of "LLM推理优化：技术原理解析总览" §3.3: 32 below 1024
 * tokens, 16 from 1024 to below 8192, 8 from 8192 on. A deployment keeps
 * one pool per tier and routes each sequence to its tier's pool. */
int32_t pa_tier_block_size(int64_t expected_len);

/* Make dst a new sequence that shares all of src's blocks (prefix sharing:
 * same physical blocks, each block's refcount + 1; "vLLM的'内存分页'到底多神奇",
 * §2 and §3 phase 3), a partly filled last block included. Sharing is
 * copy-on-write (same page, §3 phase 3): when a sequence appends into a
 * partly filled last block that other sequences still share, the append
 * takes a fresh block for it first (before any new tail block; it counts
 * toward the all-or-nothing admission), drops one reference of the shared
 * block, and records a pending copy shared -> fresh. The next pa_write_kv on
 * this pool performs the pending copies, in the order recorded, on its
 * stream before its scatter; a copy sees the block as the device holds it
 * then, so write the rows of an append (pa_write_kv) before forking that
 * sequence. Pending copies are kept across frees of their blocks.
 * Errors: PA_ERR_UNKNOWN_SEQ (src unknown), PA_ERR_INVALID (dst exists or
 * dst == src). */
pa_status pa_seq_fork(pa_pool* pool, int64_t src_seq_id, int64_t dst_seq_id);

/* End a sequence: each of its blocks loses one reference; a block whose count
 * reaches zero goes back on top of the free list, in table order (same page,
 * §3 phase 3; aborting a request frees its pages, §4). Errors:
 * PA_ERR_UNKNOWN_SEQ. */
pa_status pa_seq_free(pa_pool* pool, int64_t seq_id);

/* Export block tables and lengths for n sequences: each sequence's page table
 * mapping logical page i to its physical page ("vLLM的'内存分页'到底多神奇",
 * §2), one row per sequence, as the device calls read them. max_blocks, the
 * row width, bounds the pages one sequence may hold, as the page's
 * longest-sequence setting does (same page, §3 phase 3). Rows follow the
 * order given by seq_ids (host, n). tables_out (host, n × max_blocks int32, row-major) gets
 * each sequence's physical block ids, padded with -1; seq_lens_out (host, n
 * int32) gets each length. Errors: PA_ERR_UNKNOWN_SEQ, PA_ERR_INVALID (a
 * sequence needs more than max_blocks entries, a length above INT32_MAX, or
 * null/negative arguments). Nothing is written on error. */
pa_status pa_block_tables(const pa_pool* pool, const int64_t* seq_ids, int32_t n,
                          int32_t max_blocks, int32_t* tables_out, int32_t* seq_lens_out);

/* The geometry the pool was created with (host *out): a binding checks the
 * shapes and element types of device buffers against it before a call, since
 * the kernels size every access from it. Library addition (no passage).
 * Errors: PA_ERR_INVALID (null pointers). */
pa_status pa_pool_layout(const pa_pool* pool, pa_kv_layout* out);

/* Current block accounting into *out (host): the cache-usage figures the
 * monitoring of "vLLM的'内存分页'到底多神奇", §5, watches (see
 * pa_pool_stats_t). Errors: PA_ERR_INVALID (null pointers). */
pa_status pa_pool_stats(const pa_pool* pool, pa_pool_stats_t* out);

/* The pending copy-on-write block copies (the copy a write into a shared page
 * needs first: "vLLM的'内存分页'到底多神奇", §3 phase 3), in the order they will run:
 * src_out[i] -> dst_out[i] (host, capacity entries each); *n_out receives the
 * count. Errors: PA_ERR_INVALID (null pointers, capacity below the count). */
pa_status pa_pool_pending_copies(const pa_pool* pool, int32_t* src_out, int32_t* dst_out, int32_t capacity,
                                 int32_t* n_out);

/* Per-tensor scales of an FP8 pool: a K code c stands for value(c) · k_scale,
 * a V code for value(c) · v_scale. Both default to 1. pa_write_kv quantises
 * with the scales current at the call, so set them before the first write.
 * Errors: PA_ERR_INVALID (a scale not finite or not > 0),
 * PA_ERR_UNSUPPORTED (the pool is not PA_FP8_E4M3). */
pa_status pa_pool_set_kv_scales(pa_pool* pool, float k_scale, float v_scale);

/* ------------------------------------------------------------------------ */
/* Device operations                                                          */
/* ------------------------------------------------------------------------ */

/* KV append scatter (paging's O(1) append: "LLM推理优化：技术原理解析总览", §2.2).
 * First performs, in order, the pool's pending copy-on-write block copies
 * (see pa_seq_fork), then the scatter, all on `stream`.
 * key, value (device): [T, num_kv_heads, head_dim] of the pool dtype,
 * contiguous. slot_mapping (device): T int64 flat slots from pa_seq_append.
 * Row t is copied bit for bit to k_cache/v_cache[slot / block_size][slot %
 * block_size]. A negative slot is padding and is skipped; a slot ≥
 * num_blocks × block_size is also skipped (no fault). Two rows with the same
 * slot race (undefined which lands). T == 0 launches only pending copies.
 * FP8 pools: key and value are bf16 rows; each element x is stored as the
 * E4M3 code nearest to x / scale (the quotient rounded to fp32 first, then
 * clamped to ±448, ties to the code with an even mantissa; NaN inputs give
 * an unspecified code).
 * Errors: PA_ERR_INVALID (T < 0, null pointers with T > 0), PA_ERR_HIP. */
pa_status pa_write_kv(pa_pool* pool, const void* key, const void* value,
                      const int64_t* slot_mapping, int32_t T, void* stream);

/* Bytes of device workspace pa_decode needs for this shape. Library addition:
 * the pages' decode walks a sequence's pages in one pass
 * ("vLLM的'内存分页'到底多神奇", §3 phase 2); here long contexts
 * are split into KV partitions of partition_tokens tokens, and when a
 * sequence spans more than one, the workspace holds the fp32 partial state
 * (max, sum, Σ weight·V) of every (sequence, q head, partition). 0 when one
 * partition covers max_seq_len. partition_tokens 0 means the library's
 * choice (pa_decode_partition_tokens); the size returned for 0 covers it
 * (that choice is never shorter than 512 tokens unless one partition covers
 * max_seq_len). Returns 0 for invalid arguments. */
size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t partition_tokens);

/* The KV partition pa_decode uses for partition_tokens = 0 when
 * max_seq_len < 8192 (or B > 1024), chosen from the launch shape (the host
 * does not see the lengths); for max_seq_len >= 8192 this is only the
 * starting point: the decode kernel itself then takes the lengths into
 * account, as pa_decode_partition_tokens_for_lengths does on the host (the
 * shape rule stays when every sequence has at least 8192 tokens). Work items are
 * (sequence, group of kv heads, partition), with two kv heads per group
 * when the pool's kv-head count is even. For max_seq_len >= 8192 the
 * partition is the longest that still gives 256 items at max_seq_len (long
 * runs per wave stream fastest). Below that, lengths are taken as uniform in
 * [0, max_seq_len] and the partition is the smallest whose expected item
 * count is at most 480 (672 for an FP8 pool): shorter partitions even out
 * the work of sequences of different lengths while every item still finds a
 * workgroup slot at once on MI355X. It is kept within [640, 8192] tokens
 * and rounded up to a multiple of 64. (The split into
 * partitions merged by log-sum-exp is this library's; the pages' decode
 * walks a sequence's blocks in one pass: "vLLM的'内存分页'到底多神奇",
 * xxqk.cn, §3 phase 2.) Returns 0 for a null pool or negative sizes. */
int32_t pa_decode_partition_tokens(const pa_pool* pool, int32_t B, int32_t max_seq_len);

/* The KV partition pa_append_decode_args uses for partition_tokens = 0, from
 * the lengths themselves (seq_lens_host [B], host): when every sequence has
 * at least 8192 tokens, the shape rule of pa_decode_partition_tokens;
 * otherwise the smallest multiple of 64 tokens, at least 512, for which the
 * launch has at most 480 (sequence, kv-head group, partition) items, so that
 * every item starts at once on MI355X and a long sequence among short ones
 * is split finely (one partition per sequence when no partition gets that
 * low). Returns 0 for a null pool, negative sizes or null lengths with
 * B > 0. */
int32_t pa_decode_partition_tokens_for_lengths(const pa_pool* pool, const int32_t* seq_lens_host, int32_t B,
                                               int32_t max_seq_len);

/* Decode attention: one query token per sequence over its paged cache
 * ("vLLM的'内存分页'到底多神奇", xxqk.cn, §3 phase 2: walk the sequence's page
 * table, read its pages in logical order, attend; GQA head mapping and the
 * scale are this library's readings, see the file header).
 * out (device): [B, num_q_heads, head_dim], pool dtype (bf16 for an FP8
 *   pool), written.
 * q (device): [B, num_q_heads, head_dim], pool dtype (bf16 for an FP8 pool).
 *   An FP8 pool's codes are read as value(code) · k_scale for keys and
 *   value(code) · v_scale for values.
 * block_tables (device): [B, max_blocks] int32, row b = sequence b's table.
 * seq_lens (device): [B] int32, valid cache entries of each sequence at call
 *   time (the new token included, i.e. after pa_write_kv). Entries past
 *   ceil(L / block_size) and slots past L in the last block are never used.
 *   A value outside [0, max_seq_len] is clamped into it.
 * scale: multiplies q·k before the softmax (1/sqrt(head_dim) usually).
 * max_seq_len: an upper bound on seq_lens (sizes the grid); must satisfy
 *   max_seq_len ≤ max_blocks × block_size.
 * partition_tokens: long contexts are split into KV partitions of this many
 *   tokens, each reduced to (max, sum, Σ weight·V), then merged by
 *   log-sum-exp (a second launch, only when some sequence spans more than
 *   one partition). 0 = the library's choice (pa_decode_partition_tokens;
 *   for max_seq_len >= 8192 and B <= 1024 the kernel refines it from the
 *   lengths: the smallest multiple of 64 tokens, at least 512, giving at
 *   most 480 work items, 672 on FP8 pools, unless every sequence has at
 *   least 8192 tokens).
 *   Must be a multiple of 64, at most 2^24, else PA_ERR_UNSUPPORTED.
 * workspace (device, 16-byte aligned, contents irrelevant) of
 *   workspace_bytes ≥ pa_decode_workspace_bytes(...); may be NULL when that
 *   is 0. Calls that may run concurrently (different streams) need separate
 *   workspaces.
 * L = 0 gives a zero output row.
 * Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_decode(pa_pool* pool, void* out, const void* q, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t num_q_heads,
                    float scale, int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Size of the device scratch pa_decode_static keeps its partial states in. */
#define PA_DECODE_STATIC_SCRATCH_BYTES (32u << 20)

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, kernels and output as pa_decode, without the workspace
 * arguments. The split-KV partial states go to a scratch array of
 * PA_DECODE_STATIC_SCRATCH_BYTES bytes that the library holds in each GPU's
 * memory for the life of the process (a static device array; its address on
 * a device is resolved once, when a pool is created or on the first call on
 * that device). This call allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine. Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (each call writes every partial state
 * before it reads it, so nothing needs clearing): calls that overlap on one
 * GPU (different streams, or several threads) race and must be serialised
 * by the caller. partition_tokens = 0 chooses the partition as pa_decode
 * does, except that a long-context launch keeps the shape rule of
 * pa_decode_partition_tokens when the partial states of 512-token
 * partitions would not fit the scratch. Errors: those of pa_decode;
 * PA_ERR_UNSUPPORTED when the partial states of this shape (B × num_q_heads
 * × partitions × (head_dim + 2) × 4 bytes + 16, partitions =
 * ceil(max_seq_len / partition_tokens), 0 when one partition covers
 * max_seq_len) exceed PA_DECODE_STATIC_SCRATCH_BYTES. */
pa_status pa_decode_static(pa_pool* pool, void* out, const void* q, const int32_t* block_tables,
                           int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t num_q_heads,
                           float scale, int32_t max_seq_len, int32_t partition_tokens, void* stream);

/* One decode step with the append fused in: the effect of pa_write_kv with
 * T = B followed by pa_decode, in one launch (plus the log-sum-exp pass).
 * The pages place a generated token's K/V in its page, then attend over the
 * sequence's pages ("vLLM的'内存分页'到底多神奇", xxqk.cn, §3 phases 1-2).
 * For each b with slot_mapping[b] >= 0, row b of key/value ([B, Hkv, D],
 * the pool dtype, device) is sequence b's newest token: it sits at position
 * seq_lens[b] - 1, and slot_mapping[b] is its slot (as pa_seq_append_batch
 * with n_tokens = 1 returns it). The row is written into the pool, and the
 * block_tables entry of the block that holds it (index (seq_lens[b] - 1) /
 * block_size of row b) is set to slot_mapping[b] / block_size, so the caller
 * need not upload tables when a step opens a new block or takes a
 * copy-on-write block; every other entry must already match the pool's
 * table (pa_block_tables). slot_mapping[b] < 0: no new token for b (the
 * decode reads the pool as pa_decode does). Pending copy-on-write copies run
 * first, as in pa_write_kv. The other arguments and the output are those of
 * pa_decode. block_tables is read and written on the device; nothing else
 * is written. bf16 and fp32 pools only. Errors: those of pa_decode;
 * PA_ERR_INVALID (null or unaligned key/value/slot_mapping with B > 0);
 * PA_ERR_UNSUPPORTED (FP8 pool). */
pa_status pa_append_decode(pa_pool* pool, void* out, const void* q, const void* key, const void* value,
                           const int64_t* slot_mapping, int32_t* block_tables, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t B, int32_t num_q_heads, float scale,
                           int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);

/* pa_append_decode for a batch of at most 128 sequences whose slots and
 * lengths are on the host: slot_mapping_host [B] and seq_lens_host [B] are
 * read during the call and travel in the kernels' launch arguments, so a
 * decode step needs no host-to-device copy at all (a copy costs a few
 * microseconds to a few tens of them per step on MI355X, against a decode of
 * about a hundred). Same meaning, output and table update as
 * pa_append_decode; key, value, q, out, block_tables and workspace are
 * device pointers. partition_tokens = 0 takes the partition from the
 * actual lengths (pa_decode_partition_tokens_for_lengths). Errors: those of
 * pa_append_decode; PA_ERR_UNSUPPORTED when B > 128. */
pa_status pa_append_decode_args(pa_pool* pool, void* out, const void* q, const void* key, const void* value,
                                const int64_t* slot_mapping_host, int32_t* block_tables, int32_t max_blocks,
                                const int32_t* seq_lens_host, int32_t B, int32_t num_q_heads, float scale,
                                int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Chunked causal prefill (a long prompt processed in chunks: "LLM推理优化：技术
 * 原理解析总览", §2.3; prefill and decode mixed in one step: "vLLM 生产级落地
 * 深剖", musen-ai.com, §2). The chunk's own K/V must already be in the cache
 * (pa_write_kv). Sequence b's chunk has n_b = cu_q_lens[b+1] - cu_q_lens[b]
 * query rows; its cache holds L_b = seq_lens[b] tokens (chunk included); row i
 * sits at absolute position L_b - n_b + i and attends to tokens 0 ..
 * L_b - n_b + i.
 * out, q (device): [T, num_q_heads, head_dim] bf16, T = cu_q_lens[B].
 * cu_q_lens (device): [B + 1] int32, non-decreasing, cu_q_lens[0] = 0.
 * block_tables (device): [B, max_blocks] int32. seq_lens (device): [B] int32.
 * max_q_len: an upper bound on n_b (sizes the grid); rows past it are not
 *   computed. Rows with a negative position (n_b > L_b) get zeros.
 * seq_lens values are clamped to max_blocks × block_size.
 * Only PA_BF16 pools are supported here (bf16 MFMA); PA_F32 returns
 * PA_ERR_UNSUPPORTED. Errors: PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_HIP. */
pa_status pa_prefill(pa_pool* pool, void* out, const void* q, const int32_t* cu_q_lens,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                     int32_t B, int32_t num_q_heads, int32_t max_q_len, float scale, void* stream);

/* ------------------------------------------------------------------------ */
/* One mixed step, eager or as a replayable HIP graph                         */
/* ------------------------------------------------------------------------ */

/* A serving step mixes the decode of running sequences with prefill chunks
 * of new ones in one batch ("vLLM 生产级落地深剖", musen-ai.com, §2; chunked
 * prefill: "LLM推理优化：技术原理解析总览", §2.3). One step is: the scatter of
 * every new K/V row (decode tokens and prefill chunks together), then decode
 * over the decode sequences, then prefill over the chunk sequences, all on
 * one stream. The fields mean what the same-named arguments of
 * pa_write_kv, pa_decode and pa_prefill mean; a part whose count is 0
 * (num_new_tokens, dec_batch, pre_batch) is skipped and its pointers may be
 * NULL. dec_out and pre_out must not overlap. */
typedef struct {
  /* scatter (pa_write_kv) */
  const void* key;              /* device [num_new_tokens, Hkv, D] */
  const void* value;            /* device [num_new_tokens, Hkv, D] */
  const int64_t* slot_mapping;  /* device [num_new_tokens]; -1 rows are skipped */
  int32_t num_new_tokens;
  /* shared */
  int32_t num_q_heads;
  float scale;
  int32_t max_blocks;           /* row width of both block-table arrays */
  /* decode (pa_decode) */
  void* dec_out;
  const void* dec_q;
  const int32_t* dec_block_tables;
  const int32_t* dec_seq_lens;
  int32_t dec_batch;
  int32_t dec_max_seq_len;
  int32_t partition_tokens;
  void* workspace;
  size_t workspace_bytes;
  /* prefill (pa_prefill) */
  void* pre_out;
  const void* pre_q;
  const int32_t* pre_cu_q_lens;
  const int32_t* pre_block_tables;
  const int32_t* pre_seq_lens;
  int32_t pre_batch;
  int32_t pre_max_q_len;
} pa_step_desc;

/* Enqueue one mixed step ("vLLM 生产级落地深剖", §2) on `stream`: pending copy-on-write copies, the
 * scatter, then decode and prefill. When the step has both, the prefill
 * runs on a stream the pool owns (default priority, made on the first such
 * call on the device current then), forked from `stream` after the scatter
 * and joined back before the call's work on `stream` ends, so the
 * bandwidth-bound decode and the matrix-bound prefill share the GPU; work
 * enqueued on `stream` afterwards sees both outputs. Beside a decode with at
 * least one (sequence, kv-head pair) for every second compute unit, the
 * prefill serves its work with the fewest compute units that keep its span
 * within 1.1 times its longest work item, and leaves the others to the
 * decode (the outputs are the same either way). Steps of one pool
 * share that stream, so calls for one pool from several host threads must be
 * serialised, as for every pool call. Every part is validated before
 * anything is launched. Errors: those of pa_write_kv, pa_decode and
 * pa_prefill. */
pa_status pa_step(pa_pool* pool, const pa_step_desc* desc, void* stream);

typedef struct pa_step_graph pa_step_graph; /* opaque, library-owned */

/* Capture the launches of one mixed step ("vLLM 生产级落地深剖", §2; the capture
 * itself is a library addition) (pa_step without copies) into an
 * instantiated HIP graph. Sizes, grid shapes and every pointer in `desc` are
 * frozen; the device buffers they name are read when the graph runs, so the
 * caller updates their contents (new rows, slots, tables, lengths, queries,
 * cu_q_lens) between launches. Decode rows with length 0 give zero output and
 * slots of -1 skip their rows, so a frozen batch can carry idle entries.
 * A step with both decode and prefill is captured as two branches joined at
 * the end, as pa_step runs them. The pool must have no pending copy-on-write
 * copies at capture. The graph
 * refers to the pool and to the caller's buffers: destroy it before freeing
 * them. Nothing is launched by this call. Errors: those of pa_step;
 * PA_ERR_INVALID when copies are pending; PA_ERR_HIP (capture or
 * instantiation failed). */
pa_status pa_step_graph_create(pa_pool* pool, const pa_step_desc* desc, pa_step_graph** out);

/* Launch the captured step ("vLLM 生产级落地深剖", §2: one engine step mixing
 * prefill and decode) on `stream`, after enqueueing the pool's pending
 * copy-on-write copies (they change from step to step, so they stay outside
 * the graph). Errors: PA_ERR_INVALID (null graph), PA_ERR_HIP. */
pa_status pa_step_graph_launch(pa_step_graph* graph, void* stream);

/* Release the graph (NULL is ignored). Call it once the graph's launches
 * have completed (synchronise their stream first). Library addition (no
 * passage): the graph's lifetime. */
void pa_step_graph_destroy(pa_step_graph* graph);

/* Debug checks of the device calls' integer inputs. Two rows of one scatter
 * with the same slot race, and a block id outside the pool is undefined (the
 * pages leave both open: a slot names one place in one page, "vLLM的'内存分页'
 * 到底多神奇", §3 phase 1; a table maps each logical page to a physical one,
 * §2). With the checks on, pa_write_kv, pa_decode, pa_append_decode,
 * pa_append_decode_args, pa_prefill, pa_step and pa_step_graph_create first
 * copy the slots, block tables and lengths they are given to the host (on
 * their stream, waiting for the copy: slow, for debugging), and return
 * PA_ERR_INVALID, launching nothing, when a slot in the pool appears twice
 * in one call or when a table entry the call reads (logical blocks 0 ..
 * ceil(L / block_size) - 1 of each row, L clamped as the kernels clamp it;
 * for a fused append, not the entry the call fills in itself) is not in
 * [0, num_blocks). enable != 0 turns them on, 0 off, for the whole process;
 * returns the previous setting. The initial setting is on when the
 * environment variable PA_DEBUG_CHECKS is set to a value other than "0". */
int32_t pa_set_debug_checks(int32_t enable);

/* Thread-local text describing the last non-OK status returned on this
 * thread ("" if none). Valid until the next call on this thread. Library
 * addition (no passage): error reporting. */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
