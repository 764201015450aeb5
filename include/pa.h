/*
 * pa.h -- C ABI of the MI355X (gfx950) paged decode-attention library.
 *
 * One hot path: single-token decode attention over a paged KV cache, plus
 * its write side.  Every sequence's keys and values live in fixed-size
 * physical blocks of one shared pool per layer and are reached only through
 * that sequence's block table.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量 PagedAttention 与 KV 缓存分块"
 *        (sheratonhq.com/news/141880): sections "嵌入式轻量 Block 分配器设计"
 *        (pool of fixed-size blocks, free bitmap, lowest free id first, -1 when
 *        exhausted), "注意力寻址：非连续物理块的间接寻址" (logical token ->
 *        logical block and offset -> physical block via the block table) and
 *        "共享前缀块" (several block tables point at the same resident prefix
 *        blocks).
 *   [P2] "Ollama的内存管理策略：从KV Cache Block分配到Prefix-aware内存复用的演进"
 *        (xdnf.cn/news/5086), section "三、KV Cache内存管理的工程实现":
 *        per-block reference counts, release at the last reference, pool
 *        statistics (total / used / shared / free).
 *   [P3] wzjinhao.cn/news/69573 (deferred speculative decoding with a
 *        circular context), section "环形上下文与注意力沉淀机制": the sink +
 *        ring slot equation; section "C++ 环形 KV 缓存管理内核实现": resident
 *        keys in cache order (sinks, then the window oldest first).
 *   [P4] "大模型推理内存优化：从 KV Cache 分页到连续批处理的工程实践"
 *        (pwwt.cn/news/3010209), section "KV Cache 的内存开销与分页机制":
 *        blocks of usually 16 tokens, one block table per request, a new
 *        block when the last one fills, block sharing, and the decode kernel
 *        reading K/V indirectly through the block table.
 *
 * Conventions
 *   - Every int-returning call returns a pa_status (0 = PA_OK, < 0 = error)
 *     unless noted otherwise.  pa_status_str() names a status.
 *   - "device" pointers are HIP device memory owned by the caller (for
 *     example PyTorch tensors); "host" pointers are ordinary host memory.
 *     Device tensors are contiguous, row-major, 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; no call synchronises,
 *     so a fault caused by bad device-resident data (block ids, lengths,
 *     slots) surfaces at the caller's next synchronisation.
 *   - Device-resident contents (block ids in block tables, context lengths,
 *     slots) are a caller contract and are not validated in the fast path.
 *   - Host-side allocator calls are thread-safe (internal mutex).  Decode and
 *     cache writes are re-entrant across streams; concurrent writes to the
 *     same slot have unspecified results.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVAL = -1,       /* invalid argument (shape, pointer, alignment, size) */
  PA_ERR_NOMEM = -2,       /* host allocation failed / workspace too small */
  PA_ERR_STATE = -3,       /* refcount misuse: the block is free */
  PA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_UNSUPPORTED = -5  /* a combination the library has no kernel for */
} pa_status;

/* PA_FP8_E4M3 and PA_FP8_E5M2 are storage types of K/V pools only: such
 * pools are made by pa_create_pool_kv8 (or pa_create_pool_fp8 for E4M3), and
 * pa_create_pool rejects them. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3, PA_FP8_E5M2 = 4 } pa_dtype;

/* Opaque pool handle: host-side state only (shapes, free list, refcounts). */
typedef struct pa_pool pa_pool;

typedef struct {
  int32_t total;  /* blocks in the pool */
  int32_t used;   /* blocks with refcount >= 1 */
  int32_t shared; /* blocks with refcount >= 2 */
  int32_t free;   /* total - used */
} pa_pool_stats;

/* Sink + ring mode [P3].  A stream of logical positions maps into
 * sink + window ring slots; slot r of the ring is then addressed through the
 * block table exactly like logical token r of a plain sequence.  Keys are
 * stored un-rotated; decode rotates (rotate-half pairing: (x_i, x_{i+D/2}))
 * the key at cache index j by j * theta_i and the query by (L - 1) * theta_i,
 * theta_i = rope_base^(-2i/D), L = min(context_len, sink + window).
 * `rope_table` is a device buffer of pa_rope_table_bytes(rope_capacity,
 * rope_head_dim) bytes filled by pa_rope_table_init() with the same
 * (rope_capacity, rope_head_dim, rope_base).  Decode refuses (PA_ERR_INVAL)
 * a table that holds fewer than sink + window positions or was built for
 * another head size than the pool's: the kernels index it by cache position
 * and head size, so a smaller table would be read past its end. */
typedef struct {
  int32_t sink;            /* S >= 0 */
  int32_t window;          /* W >= 1 */
  float rope_base;         /* e.g. 10000 */
  int32_t rope_style;      /* 0 = rotate-half (the only style implemented) */
  const float *rope_table; /* device, float2 (cos, sin) [rope_capacity][rope_head_dim / 2] */
  int32_t rope_capacity;   /* positions the table holds, >= S + W */
  int32_t rope_head_dim;   /* head size the table was built for (= the pool's) */
} pa_ring;

/* ---------------------------------------------------------------- pool --- */

/* Describe one layer's K and V pools, each [num_blocks, block_size,
 * num_kv_heads, head_dim] of `dtype`, in caller-owned device memory
 * (k_cache, v_cache), and create the host-side allocator over its block ids
 * [P1 allocator; P4].  block_size in {16, 64}; head_dim in {64, 128}.
 * The handle never frees k_cache / v_cache.  *out is set on success. */
int pa_create_pool(pa_pool **out, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, pa_dtype dtype, void *k_cache, void *v_cache);

/* Pools of 8-bit K/V [P4, section "工程边界与架构取舍": FP8 storage halves
 * the KV cache].  k_cache / v_cache hold E4M3 codes (OCP 8-bit float: 4
 * exponent bits, bias 7, 3 mantissa bits, largest finite 448, S.1111.111 =
 * NaN), [num_blocks, block_size, num_kv_heads, head_dim] bytes each.  A code
 * c of KV head h stands for k_scale[h] * value(c) (V: v_scale[h]).
 * act_dtype (PA_F16 or PA_BF16) is the dtype of the query, the output and
 * the key/value rows handed to pa_reshape_and_cache, which stores
 * nearest-even E4M3 codes of fp32(x) * fp32(1 / scale[h]), saturating at
 * +-448.  k_scale, v_scale: host float [num_kv_heads], finite and > 0,
 * copied into the handle; num_kv_heads <= 64.  Decode on such a pool needs
 * 1 <= Hq / Hkv <= 16 and no ring (else PA_ERR_UNSUPPORTED).  Other
 * arguments and errors as pa_create_pool.  Same as pa_create_pool_kv8 with
 * kv_dtype = PA_FP8_E4M3. */
int pa_create_pool_fp8(pa_pool **out, int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim, pa_dtype act_dtype,
                       const float *k_scale, const float *v_scale, void *k_cache, void *v_cache);

/* Pools of 8-bit K/V in either OCP 8-bit float format [P4, section
 * "工程边界与架构取舍"; the page names FP8 storage without fixing a
 * format]: kv_dtype PA_FP8_E4M3 (as pa_create_pool_fp8) or PA_FP8_E5M2
 * (5 exponent bits, bias 15, 2 mantissa bits; exponent field 0 subnormal,
 * 31 infinity or NaN; largest finite 57344 = 1.75 * 2^15; the code is the
 * top byte of the IEEE binary16 number it stands for).  pa_reshape_and_cache
 * stores nearest-even codes of fp32(x) * fp32(1 / scale[h]) in that format,
 * magnitudes beyond the largest finite one (infinities too) saturating to
 * it, NaN to 0x7F.  Everything else as pa_create_pool_fp8; PA_ERR_INVAL for
 * any other kv_dtype. */
int pa_create_pool_kv8(pa_pool **out, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_dim, pa_dtype kv_dtype, pa_dtype act_dtype, const float *k_scale,
                       const float *v_scale, void *k_cache, void *v_cache);

/* Free the host-side state (NULL is a no-op).  Device memory is untouched. */
void pa_destroy_pool(pa_pool *pool);

/* Take the lowest free block id and set its refcount to 1 [P1 allocator].
 * Returns the id, or -1 when the pool is exhausted or pool is NULL. */
int32_t pa_alloc_block(pa_pool *pool);

/* Add a reference to an allocated block (prefix sharing [P1 prefix; P2]).
 * PA_ERR_INVAL for an id outside the pool, PA_ERR_STATE for a free block. */
int pa_incref_block(pa_pool *pool, int32_t block_id);

/* Drop a reference; at zero the block returns to the free set [P2].
 * PA_ERR_INVAL for an id outside the pool, PA_ERR_STATE for a free block
 * (double release) or when the one reference left is the prefix index's
 * (only eviction or pa_prefix_clear drops that one). */
int pa_decref_block(pa_pool *pool, int32_t block_id);

/* Current reference count of a block (0 = free), or -1 for a bad id. */
int32_t pa_get_refcount(const pa_pool *pool, int32_t block_id);

/* Pool statistics [P2]. */
int pa_get_stats(const pa_pool *pool, pa_pool_stats *out);

/* ------------------------------------------- prefix reuse, copy-on-write --- */

/* Prefix-aware reuse of cached blocks [P2, sections "三、KV Cache内存管理的
 * 工程实现" and "四、内存管理策略的边界"; P1, section "共享前缀块"].
 * Token ids are uint32.  A full block (block_size ids) is keyed by a 64-bit
 * FNV-1a fold of its ids, one id per step (h ^= id; h *= 0x100000001b3 mod
 * 2^64), continued from the previous block's key (the first block starts
 * from 0xcbf29ce484222325): the key of block i covers every id up to its
 * end.  The index lists blocks whose contents are the K/V of known ids and
 * holds one reference on each; a key hit counts only when the ids match and
 * the entry hangs off the entry matched for the previous block, so hash
 * collisions never join different prefixes.  A partial last block (a
 * "tail", fewer ids than a block) may be listed too and is found under its
 * parent.  Listed blocks are read-only: a caller writes into a block only
 * after pa_cow_block.  Host-only state under the pool's mutex; nothing here
 * touches device memory. */
typedef enum {
  PA_PREFIX_TAIL = 1,     /* also list the partial last block */
  PA_PREFIX_RESIDENT = 2  /* the listed blocks are never evicted */
} pa_prefix_flags;

typedef struct {
  int32_t entries;      /* listed blocks */
  int32_t tail_entries; /* of which partial */
  int32_t resident;     /* of which resident */
  int32_t index_only;   /* listed blocks no caller holds (refcount 1) */
} pa_prefix_stats;

/* Host: keys of the num_tokens / block_size full blocks of `tokens` (host
 * uint32 [num_tokens]) into out (host uint64, one per full block); a
 * trailing partial block gets no key.  block_size >= 1 (any value: this
 * call needs no pool).  PA_ERR_INVAL for num_tokens < 0, block_size < 1 or
 * NULL pointers where a key is due. */
int pa_block_hashes(const uint32_t *tokens, int64_t num_tokens, int32_t block_size,
                    uint64_t *out);

/* Host: the longest cached prefix of `tokens` (host uint32 [num_tokens]).
 * Walks full blocks by key while they verify, then takes the longest tail
 * listed under the last matched entry whose ids all lie within the request.
 * Each returned block gains one reference for the caller (release with
 * pa_decref_block); blocks_out (host int32 [max_blocks]) gets them in
 * logical order, *num_blocks_out their count and *num_tokens_matched the
 * ids they cover (a multiple of block_size unless the last one is a tail).
 * At most max_blocks are returned.  Every entry walked counts as used now
 * for eviction order. */
int pa_prefix_match(pa_pool *pool, const uint32_t *tokens, int64_t num_tokens,
                    int32_t *blocks_out, int32_t max_blocks, int32_t *num_blocks_out,
                    int64_t *num_tokens_matched);

/* Host: list a sequence's blocks: blocks[i] (host int32, allocated, caller
 * holds a reference) holds the K/V of ids [i * block_size, (i+1) *
 * block_size) of `tokens`.  Every full block is listed; with PA_PREFIX_TAIL
 * the partial last block too.  A block whose (previous entry, ids) is listed
 * already is skipped (the caller keeps its own copy); each new entry takes
 * one reference on its block.  PA_PREFIX_RESIDENT marks every entry walked
 * (new or known) as never evicted.  *num_new (may be NULL) = entries made.
 * PA_ERR_INVAL: num_blocks short of the blocks needed, unknown flags, or a
 * new entry's id outside the pool; PA_ERR_STATE: a new entry's block is
 * free, listed already under other ids, or given twice.  On error nothing
 * changes. */
int pa_prefix_insert(pa_pool *pool, const uint32_t *tokens, int64_t num_tokens,
                     const int32_t *blocks, int32_t num_blocks, uint32_t flags, int32_t *num_new);

/* Host: free up to max_blocks blocks that only the index still holds
 * (refcount 1), taking leaf entries (none listed after them), never
 * resident ones, least recently used first (ties: the older entry); a
 * parent whose last child goes becomes a candidate in turn.  freed (host
 * int32 [max_blocks], may be NULL) gets the freed ids in order and
 * *num_freed their count. */
int pa_prefix_evict(pa_pool *pool, int32_t max_blocks, int32_t *freed, int32_t *num_freed);

/* Host: drop every entry, resident ones too, and the index's references. */
int pa_prefix_clear(pa_pool *pool);

/* Host: counts of the prefix index. */
int pa_prefix_get_stats(const pa_pool *pool, pa_prefix_stats *out);

/* Host: copy-on-write [P2, section "三、KV Cache内存管理的工程实现": a
 * shared block is read-only and is copied before it is modified].  The
 * caller holds a reference on block_id and wants to write into it.  With
 * refcount 1 *out_block = block_id and nothing changes.  Otherwise the
 * lowest free block is allocated for the caller (refcount 1), block_id
 * loses the caller's reference, and *out_block = the new id: the caller
 * then enqueues pa_copy_blocks(block_id -> *out_block) before writing and
 * puts the new id in its block table.  PA_ERR_NOMEM (*out_block = -1,
 * nothing changed) when no block is free; PA_ERR_STATE for a free block or
 * one only the index holds; PA_ERR_INVAL for an id outside the pool. */
int pa_cow_block(pa_pool *pool, int32_t block_id, int32_t *out_block);

/* Device: for each pair i, block dst_blocks[i] of both the K and the V pool
 * takes the contents of block src_blocks[i] (every byte: block_size rows
 * of num_kv_heads * head_dim elements, or codes for an 8-bit pool).
 * src_blocks, dst_blocks: device int32 [num_pairs]; a pair with either id
 * outside [0, num_blocks) is skipped (negative ids are padding).
 * Destinations must be distinct and no destination may be a source (caller
 * contract; otherwise the result is unspecified).  num_pairs == 0 is a
 * no-op. */
int pa_copy_blocks(pa_pool *pool, const int32_t *src_blocks, const int32_t *dst_blocks,
                   int32_t num_pairs, void *stream);

/* ------------------------------------------------- continuous batching --- */

/* Host-side continuous-batching driver over a pool [P4, the scheduler of
 * its continuous-batching section]: it decides every iteration which
 * requests run and holds their block tables.  One pa_batcher_schedule call
 * takes three steps in this order:
 *   1. every decoding request stays; when the tokens it holds (prompt +
 *      generated) need more blocks than its table has, it gets one block
 *      (pa_alloc_block), and when none is free it sits this iteration out
 *      ("preempted", keeping its blocks);
 *   2. waiting requests are admitted first come, first served while the
 *      batch is below max_batch and the pool's free blocks cover
 *      ceil(prompt / block_size); the first that does not fit stays at the
 *      head of the queue and admission stops;
 *   3. requests that generated max_tokens tokens leave; their blocks lose
 *      the batcher's reference (pa_decref_block).
 * Decoding requests are visited in admission order.  The admission
 * iteration is the prefill: it writes positions 0 .. prompt - 1.  Every
 * later iteration of a request writes the K/V of its last generated token
 * at position prompt + generated - 1 and attends over prompt + generated
 * positions.  After running an iteration the caller calls pa_batcher_step
 * once per scheduled request.  Host state under the batcher's mutex; other
 * users of the same pool should not allocate while a schedule call runs. */
typedef struct pa_batcher pa_batcher;

typedef struct {
  int32_t scheduled;      /* requests in this iteration's batch */
  int32_t prefill;        /* of which admitted now */
  int32_t preempted;      /* decoding requests left out for want of a block */
  int32_t freed_requests; /* finished requests released at step 3 */
  int32_t freed_blocks;   /* their blocks */
  int32_t waiting;        /* queue length after the call */
  int32_t active;         /* admitted requests after the call */
} pa_batch_info;

/* Create a driver over `pool` with at most max_batch requests per
 * iteration and block tables of max_blocks_per_seq entries. */
int pa_batcher_create(pa_pool *pool, int32_t max_batch, int32_t max_blocks_per_seq, pa_batcher **out);

/* Free the driver and drop its references on every block it holds. */
void pa_batcher_destroy(pa_batcher *batcher);

/* Queue a request.  PA_ERR_INVAL: prompt_len < 1, max_tokens < 1, or
 * prompt_len + max_tokens tokens need more than max_blocks_per_seq blocks;
 * PA_ERR_STATE: the id is waiting or active already. */
int pa_batcher_add(pa_batcher *batcher, uint64_t request_id, int32_t prompt_len, int32_t max_tokens);

/* One scheduling call (the three steps above).  Outputs, host arrays of
 * max_batch entries (block_tables: [max_batch][max_blocks_per_seq], rows
 * padded with -1), filled for the info->scheduled requests in batch order
 * (decoding requests in admission order, then the admitted ones): ids,
 * the table, context_lens (positions attended after this iteration's
 * writes), write_start / write_count (positions written now), prefill
 * (1 for a request admitted now). */
int pa_batcher_schedule(pa_batcher *batcher, uint64_t *ids, int32_t *block_tables, int32_t *context_lens,
                        int32_t *write_start, int32_t *write_count, int32_t *prefill,
                        pa_batch_info *info);

/* Advance a scheduled request by one generated token; at max_tokens it is
 * finished and the next schedule call releases it.  PA_ERR_INVAL for an id
 * that is not active, PA_ERR_STATE for a finished request. */
int pa_batcher_step(pa_batcher *batcher, uint64_t request_id);

/* ------------------------------------------------------------- mapping --- */

/* Ring slot of a logical position [P3 slot equation]:
 * pos if pos < sink, else sink + ((pos - sink) mod window).
 * Returns -1 for pos < 0, sink < 0 or window < 1. */
int32_t pa_ring_slot(int64_t pos, int32_t sink, int32_t window);

/* Host: flat pool slots for (sequence, logical position) pairs [P1
 * addressing; P4 paging]:  r = position (plain) or pa_ring_slot(position)
 * (ring != NULL);  slot = block_tables[seq][r / block_size] * block_size +
 * r % block_size.  block_tables is host int32 [num_seqs][max_blocks_per_seq];
 * seq_ids host int32 [n]; positions host int64 [n]; out host int32 [n].
 * PA_ERR_INVAL if an entry is out of range or the table holds a negative or
 * out-of-pool id where a block is needed. */
int pa_compute_slot_mapping(const pa_pool *pool, const int32_t *block_tables, int32_t num_seqs,
                            int32_t max_blocks_per_seq, const int32_t *seq_ids,
                            const int64_t *positions, int32_t n, const pa_ring *ring,
                            int32_t *out);

/* --------------------------------------------------------- write side --- */

/* Device: copy token i's key and value rows ([num_kv_heads, head_dim] each,
 * pool dtype, no conversion; for an 8-bit pool the rows are in its act_dtype
 * and are stored as scaled E4M3 codes) into flat pool slot slot_mapping[i]
 * (block = slot / block_size, row = slot % block_size).  key, value: device
 * [num_tokens, num_kv_heads, head_dim]; slot_mapping: device int32
 * [num_tokens]; a negative slot is padding and is skipped, and so is a slot
 * at or beyond num_blocks * block_size.  Slots must be distinct (caller
 * contract).  num_tokens == 0 is a no-op. */
int pa_reshape_and_cache(pa_pool *pool, const void *key, const void *value,
                         const int32_t *slot_mapping, int32_t num_tokens, void *stream);

/* ------------------------------------------------------------- decode --- */

/* Bytes of device workspace pa_decode needs for this batch shape (split-K
 * partials).  ring may be NULL.  Returns 0 on invalid arguments. */
size_t pa_decode_workspace_bytes(const pa_pool *pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, const pa_ring *ring);

/* Bytes of the RoPE table for `capacity` = sink + window cached keys. */
size_t pa_rope_table_bytes(int32_t capacity, int32_t head_dim);

/* Device: fill table (float2 [capacity][head_dim / 2]) with
 * (cos, sin)(j * rope_base^(-2i/head_dim)), computed in double precision and
 * rounded to float. */
int pa_rope_table_init(float *table, int32_t capacity, int32_t head_dim, float rope_base,
                       void *stream);

/* Device: single-token decode attention over the paged cache [P4 paging;
 * P1 addressing; P3 ring].  For sequence b and query head h (KV head
 * g = h / (num_q_heads / num_kv_heads)):
 *   out[b,h,:] = sum_t softmax_t(scale * <q[b,h,:], K_t[g,:]>) * V_t[g,:]
 * over the first context_lens[b] logical tokens (plain) or the resident ring
 * keys (ring != NULL), each read through block_tables[b].
 *   out:          device [num_seqs, num_q_heads, head_dim], query dtype
 *                 (= pool dtype), rounded to nearest-even from fp32.
 *   query:        device [num_seqs, num_q_heads, head_dim], pool dtype.
 *   block_tables: device int32 [num_seqs, max_blocks_per_seq].
 *   context_lens: device int32 [num_seqs]; 0 gives an all-zero output row.
 *   max_context_len: host upper bound of context_lens (sizes the split-K
 *                 grid); plain mode needs max_context_len <=
 *                 max_blocks_per_seq * block_size.  Device lengths are
 *                 clamped to [0, max_context_len]; block ids outside the
 *                 pool are clamped into it (no fault; unspecified result).
 *   workspace:    device, >= pa_decode_workspace_bytes(...) bytes, 256-byte
 *                 aligned; its contents need no initialisation.  Concurrent
 *                 calls need distinct workspaces.
 * num_q_heads must be a multiple of the pool's num_kv_heads.  The reduction
 * order depends only on logical positions and lengths, so the result is
 * bit-identical under any relabelling of physical blocks and for shared
 * versus private copies of the same blocks. */
int pa_decode(pa_pool *pool, void *out, const void *query, const int32_t *block_tables,
              int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
              int32_t num_q_heads, int32_t max_context_len, float scale, const pa_ring *ring,
              void *workspace, size_t workspace_bytes, void *stream);

/* Device: one decode step that also stores the step's new token [P4
 * paging; P1 addressing; the write side as in pa_reshape_and_cache].  For
 * each sequence b, key[b] and value[b] ([num_kv_heads, head_dim], pool
 * dtype; for an 8-bit pool its act_dtype) are the new token's rows, stored
 * in flat slot slot_mapping[b]; out[b] is the decode attention over
 * context_lens[b] tokens, the last of which (position context_lens[b] - 1)
 * is that new token.  The result, cache contents and output, is bit for bit
 * that of pa_reshape_and_cache(key, value, slot_mapping, num_seqs) followed
 * by pa_decode (same ring), including padding: a negative slot, or one at
 * or beyond num_blocks * block_size, stores nothing.  Caller contract:
 * slot_mapping[b] is the slot of position context_lens[b] - 1 through
 * block_tables[b] (ring != NULL: of its ring slot Slot(context_lens[b] - 1))
 * (or padding), it is -1 where context_lens[b] == 0, no
 * other sequence of the call reads it, and slots are distinct; otherwise
 * the result is unspecified (no fault).  On f16/bf16 and 8-bit pools with
 * num_q_heads / num_kv_heads <= 16 both happen in the decode launch: the
 * wave that streams the tile holding a sequence's newest token for KV head
 * g (its last tile; ring mode: the tile of its ring slot) stores the new
 * rows of head g (8-bit pools: quantised exactly as pa_reshape_and_cache
 * does) just before it loads that tile.  Other pools (fp32, wider groups)
 * run the two calls in turn.  Other
 * arguments, the workspace size (pa_decode_workspace_bytes with the same
 * ring) and errors are those of pa_decode; key and value must be 16-byte
 * aligned and slot_mapping 4-byte aligned (PA_ERR_INVAL otherwise). */
int pa_decode_append(pa_pool *pool, void *out, const void *query, const void *key, const void *value,
                     const int32_t *slot_mapping, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_context_len, float scale, const pa_ring *ring, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Device: pa_decode_append for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument, and no hipMalloc, hipFree or other
 * allocating call.  The split-K partials and the tile schedule go to a
 * scratch array of pa_decode_noalloc_scratch_bytes() bytes (32 MiB) that
 * the library holds in device memory, one per GPU, from its first use on
 * that GPU until the process ends.  The call needs exactly the workspace
 * that pa_decode_workspace_bytes (same pool, num_seqs, num_q_heads,
 * max_context_len and ring) reports; above the scratch size it returns
 * PA_ERR_NOMEM and enqueues nothing.  Every call on one GPU shares that
 * GPU's array (it keeps the last call's contents; the kernels need no
 * initialised contents): calls that overlap in time on one GPU, on
 * different streams or threads, race on it and give unspecified results.
 * Other arguments, results and errors are those of pa_decode_append. */
int pa_decode_append_noalloc(pa_pool *pool, void *out, const void *query, const void *key,
                             const void *value, const int32_t *slot_mapping, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t max_context_len, float scale, const pa_ring *ring,
                             void *stream);
size_t pa_decode_noalloc_scratch_bytes(void);

/* Device: debug checks of the device-resident inputs that pa_decode,
 * pa_decode_append and pa_reshape_and_cache trust without checking (their
 * caller contract [P1 addressing: a block id must name a block of the
 * pool; P4 paging: the table row maps each logical block]; the fast path
 * clamps instead, so bad data gives an unspecified result but no fault).
 * One small launch on `stream` writes counts (device int32 [4], 4-byte
 * aligned; overwritten, need not be zeroed, no memset, safe to capture in
 * a graph): counts[0] = lengths outside [0, max_context_len]; counts[1] =
 * block-table entries that a decode reads (the first ceil(L / block_size)
 * of row b, L = context_lens[b] clamped into [0, max_context_len], or
 * min(L, sink + window) with ring != NULL) outside [0, num_blocks);
 * counts[2] = slot_mapping entries at or beyond num_blocks * block_size
 * (negative slots are padding, not errors); counts[3] = 0.  slot_mapping
 * may be NULL when num_slot_entries == 0.  PA_ERR_INVAL on NULL or
 * misaligned pointers or negative sizes. */
int pa_check_decode_inputs(const pa_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                           const pa_ring *ring, const int32_t *slot_mapping, int32_t num_slot_entries,
                           int32_t *counts, void *stream);

/* Bytes of device workspace pa_decode_multi needs (tile schedule and
 * stream-K partials); 0 for num_seqs == 0 or invalid arguments. */
size_t pa_decode_multi_workspace_bytes(const pa_pool *pool, int32_t num_seqs, int32_t q_len,
                                       int32_t num_q_heads, int32_t max_context_len);

/* Device: attention of q_len new tokens per sequence over the paged cache,
 * for the batched check of draft tokens in speculative decoding [P3,
 * section "嵌入式流式推理的访存墙与投机瓶颈": a step of draft tokens is scored
 * in one pass] and for chunked prefill [P4, section "工程边界与架构取舍": a
 * long prompt is processed in pieces].  The new tokens' K/V are already in
 * the cache (pa_reshape_and_cache) and counted in context_lens.  New token i
 * of sequence b sits at position p = context_lens[b] - q_len + i and attends
 * causally to positions 0..p; p < 0 gives an all-zero row.  For query head h
 * (KV head h / G):
 *   out[b,i,h,:] = sum_{t<=p} softmax_t(scale * <q[b,i,h,:], K_t>) * V_t
 *   out, query:   device [num_seqs, q_len, num_q_heads, head_dim], pool dtype
 *                 (an 8-bit pool's act_dtype), rounded to nearest-even from
 *                 fp32.
 *   block_tables, context_lens, max_context_len, workspace: as pa_decode
 *                 (workspace >= pa_decode_multi_workspace_bytes).
 *   q_len:        1 .. 4096; q_len * G <= 49152 (D = 128) or 65536 (D = 64),
 *                 else PA_ERR_UNSUPPORTED.
 * q_len = 1 is single-token decode by another kernel (same result within
 * rounding).  Rejecting draft tokens needs no call: lowering context_lens
 * hides their rows, and the next write overwrites them.  8-bit pools are
 * dequantised in registers (k_scale on scores, v_scale on outputs).
 * PA_ERR_UNSUPPORTED for fp32 pools. */
int pa_decode_multi(pa_pool *pool, void *out, const void *query, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                    int32_t q_len, int32_t num_q_heads, int32_t max_context_len, float scale,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Device: speculative verification over the sink + ring cache [P3,
 * "嵌入式流式推理的访存墙与投机瓶颈": the target model scores a step of draft
 * tokens in one pass; "环形上下文与注意力沉淀机制": the sink + ring cache and
 * its cache-order RoPE; "C++ 环形 KV 缓存管理内核实现": drafts that are
 * rejected are rolled back].  Stream b holds its committed positions
 * 0..n_b-1 in the ring (n_b = context_lens[b], clamped to [0,
 * max_context_len]); its q_len draft tokens sit at positions n_b..n_b+q_len-1
 * with query rows query[b, i] ([B, q_len, Hq, D]) and K/V rows
 * draft_key[b, i], draft_value[b, i] ([B, q_len, Hkv, D]), all in the
 * pool's dtype and un-rotated.  out[b, i] ([B, q_len, Hq, D]) is what
 * decoding draft i alone would give after drafts 0..i had been written to
 * their ring slots: the single-token ring decode over that cache.  The
 * drafts are never written: the cache is read only, so after the caller
 * accepts a_b drafts it stores them with pa_reshape_and_cache at the ring
 * slots of positions n_b..n_b+a_b-1 and the rejected ones leave nothing to
 * undo.  1 <= q_len <= 16; ring is required and its RoPE table must cover
 * sink + window + q_len - 1 positions (rope_capacity) at the pool's head
 * size (PA_ERR_INVAL otherwise); f16/bf16 pools only (PA_ERR_UNSUPPORTED
 * otherwise).  workspace: pa_decode_verify_ring_workspace_bytes(pool,
 * num_seqs, q_len, num_q_heads) bytes, 256-byte aligned, no initialisation
 * needed.  Other arguments and errors as pa_decode_multi. */
int pa_decode_verify_ring(pa_pool *pool, void *out, const void *query, const void *draft_key,
                          const void *draft_value, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *context_lens, int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                          int32_t max_context_len, float scale, const pa_ring *ring, void *workspace,
                          size_t workspace_bytes, void *stream);
size_t pa_decode_verify_ring_workspace_bytes(const pa_pool *pool, int32_t num_seqs, int32_t q_len,
                                             int32_t num_q_heads);

/* Device: a streaming-read probe, a measurement aid outside the attention
 * path (the pages define no such operation).  Reads `bytes` (a nonzero
 * multiple of 16) at src (16-byte aligned) with the non-temporal 16-byte
 * loads the decode kernels use for K/V, four work-groups per CU; work-group
 * w stores the XOR of the 32-bit words it read to checksums[w], so the
 * caller-owned checksums array must hold 4096 uint32 (the XOR of all
 * entries is the XOR of every word of the buffer).  Timing it gives the
 * practical read ceiling the decode's HBM fraction is compared against.
 * PA_ERR_INVAL for bad pointers or sizes. */
int pa_read_probe(const void *src, size_t bytes, uint32_t *checksums, void *stream);

/* Name of a status code (static string). */
const char *pa_status_str(int status);

/* Text of the last HIP error seen by this thread in a pa_* call ("" if none). */
const char *pa_last_hip_error(void);

/* Kernel-configuration overrides, for tests and measurements only (not
 * defined by the pages).  Each option starts from the environment variable
 * of the same name (PA_FORCE_VALU, ...), read once when the library is
 * loaded; value 0 means the library's own choice.
 *   PA_OPT_FORCE_VALU        nonzero: decode uses the VALU kernel for every dtype
 *   PA_OPT_PARTITION_TOKENS  VALU kernel partition size (a multiple of 16)
 *   PA_OPT_MULTI_WAVES       multi-token decode: waves per SIMD (1 or 2)
 *   PA_OPT_MULTI_ROW_TILES   multi-token decode: 16-row tiles per wave
 *   PA_OPT_MULTI_PASS_GROUP  multi-token decode: passes per work-group (1, 2, 4)
 *   PA_OPT_MULTI_MIN_RANGE   multi-token decode: shortest stream-K range (tiles)
 *   PA_OPT_DECODE_SEQ_COST   single-token stream-K decode: the extra work a
 *                            sequence brings to the range that holds it, in
 *                            16-token tiles, plus one (1: none)
 *   PA_OPT_MULTI_SEQ_COST    multi-token decode: the same for a (sequence,
 *                            pass group), plus one (1: none)
 *   PA_OPT_YOUNG_SHARE       stream-K kernels that run two work-groups per
 *                            CU: range size of the second work-group of a
 *                            CU relative to the first, in thousandths
 *                            (1000: equal)
 * Options change the kernel choice and the workspace size: set them before
 * pa_*_workspace_bytes and keep them until the matching call has been
 * enqueued.  pa_set_option returns PA_ERR_INVAL for an unknown option or a
 * negative value; pa_get_option returns -1 for an unknown option. */
typedef enum {
  PA_OPT_FORCE_VALU = 0,
  PA_OPT_PARTITION_TOKENS = 1,
  PA_OPT_MULTI_WAVES = 2,
  PA_OPT_MULTI_ROW_TILES = 3,
  PA_OPT_MULTI_PASS_GROUP = 4,
  PA_OPT_MULTI_MIN_RANGE = 5,
  PA_OPT_DECODE_SEQ_COST = 6,
  PA_OPT_MULTI_SEQ_COST = 7,
  PA_OPT_YOUNG_SHARE = 8,
  PA_OPT_COUNT = 9
} pa_option;
int pa_set_option(pa_option opt, int32_t value);
int32_t pa_get_option(pa_option opt);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
