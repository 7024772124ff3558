/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention library.
 *
 * The library implements one decode step of attention over a KV cache cut into
 * fixed 16-token blocks that may sit anywhere in a preallocated physical pool,
 * with per-request block tables mapping logical to physical blocks, blocks
 * shared between requests with reference counts, and copy-on-write when a
 * shared, partially filled block is appended to.  Sources (web pages on vLLM
 * and PagedAttention, cited by title and section):
 *   [ngrok]   techfeed.io summary of "Serving models at scale with vLLM",
 *             sections "PagedAttention", "prefix caching", "the scheduler".
 *   [tcd]     media.tcdigital.jp vLLM article, "paging", "logical and physical
 *             block mapping", "memory sharing for parallel sampling".
 *   [lens]    ta-paperlens "LLM serving from scratch", "prefill and decode",
 *             eq. (1) and the KV-size example, "fragmentation and
 *             PagedAttention", FIG 1, "scheduler skeleton", "in practice".
 *   [sns]     sns.style vLLM overview article, "deep dive".
 *   [yj]      youngju.dev "vLLM inference optimization", "KV Cache problem",
 *             "PagedAttention" (block diagram, PagedAttentionManager listing),
 *             "copy-on-write prefix sharing".
 *
 * Conventions
 *   - Every call returns a pa_status (or a plain value where noted); no C++
 *     exception crosses this boundary.
 *   - Host-side pool calls (pa_pool_*, pa_seq_*, pa_append_slots, ...) touch
 *     host memory only and never call the GPU runtime.  A pool handle is not
 *     thread-safe: one scheduler thread owns it.
 *   - Device calls take raw device pointers owned by the caller and a HIP
 *     stream (hipStream_t passed as void*; NULL = the null stream).  They only
 *     enqueue work, never allocate or free device memory, and never
 *     synchronise.  Arguments are validated on the host before any launch
 *     (PA_ERR_INVALID); a failed launch returns PA_ERR_HIP.
 *   - "fp16" means IEEE-754 binary16, passed as pa_half (its bit pattern).
 *   - block_size is fixed at PA_BLOCK_SIZE = 16 tokens (the usual block size
 *     per [ngrok] "PagedAttention"; [yj] listing example).
 *
 * Device pool layout (one pool per K and per V, one layer): each pool is
 * [num_blocks][num_kv_heads][tile], a tile holding the 16 slots x head_dim
 * fp16 values of one (block, kv head), 16*D*2 bytes contiguous (4 KiB at
 * D = 128).  Inside a tile the values are ordered the way the matrix cores
 * consume them, so that every 16-byte-per-lane load of a 64-lane wavefront
 * reads 1 KiB with lane i at bytes [16i, 16i + 16):
 *   K tile [D/8][16][8]: slot s, dim c at (c/8)*128 + s*8 + c%8
 *   V tile [D/32][4][16][2][4]: slot s, dim c at
 *           (c/32)*512 + (s/4)*128 + (c%16)*8 + ((c/16)%2)*4 + s%4
 * (offsets in fp16 elements within the tile; tile (b, h) starts at element
 * (b*H + h)*16*D).  D must be a multiple of 32.  A slot id is block*16 +
 * offset.
 */
#ifndef PA_H_
#define PA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

/* pa_paged_attention_decode flags. */
#define PA_DECODE_KEEP_KV 1u /* K/V tiles are shared between requests: cache them */

typedef uint16_t pa_half; /* IEEE binary16 bit pattern */

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = 1,        /* bad argument or geometry; nothing changed        */
  PA_ERR_OUT_OF_BLOCKS = 2,  /* free list cannot cover the request; nothing changed */
  PA_ERR_UNKNOWN_SEQ = 3,    /* sequence id not present; nothing changed          */
  PA_ERR_EXISTS = 4,         /* sequence id already present; nothing changed      */
  PA_ERR_CAPACITY = 5,       /* a caller buffer is too small; nothing changed     */
  PA_ERR_HIP = 6,            /* the HIP runtime reported an error                 */
  PA_ERR_INTERNAL = 7        /* an invariant check failed                         */
} pa_status;

/* Text for a status code (static storage). */
const char* pa_status_string(pa_status s);

/* ------------------------------------------------------------------------ */
/* Host block manager                                                        */
/* ------------------------------------------------------------------------ */

typedef struct pa_pool pa_pool;

typedef struct pa_pool_desc {
  int32_t num_blocks;          /* physical blocks in the pool, >= 1, num_blocks*16 < 2^31 */
  int32_t block_size;          /* must be PA_BLOCK_SIZE                                     */
  const int32_t* free_order;   /* NULL, or a permutation of [0, num_blocks): the initial
                                  free stack from bottom to top (allocation pops the top).
                                  NULL = ascending ids, as [yj]'s listing builds it.       */
} pa_pool_desc;

/* One copy-on-write copy: the first n_slots slots of every KV head of block
 * src are copied to block dst, in both pools ([tcd] memory sharing). */
typedef struct pa_copy {
  int32_t src;
  int32_t dst;
  int32_t n_slots;
} pa_copy;

typedef struct pa_pool_stats {
  int32_t num_blocks;
  int32_t num_free;
  int32_t num_seqs;
  int32_t num_shared;  /* blocks referenced by more than one sequence       */
  int64_t allocs;   /* blocks taken off the free list (including CoW targets) */
  int64_t frees;    /* blocks returned to the free list                       */
  int64_t cows;     /* copy-on-write copies planned                          */
  int32_t num_evictable; /* unreferenced cached blocks (reusable, see below)  */
  int32_t num_cached;    /* blocks holding a registered prefix                */
} pa_pool_stats;

/* Create a pool's host metadata ([yj] listing: the whole pool is known up
 * front and every block starts free).  *out is owned by the caller and
 * released with pa_pool_destroy.  PA_ERR_INVALID on bad geometry or a
 * free_order that is not a permutation. */
pa_status pa_pool_create(const pa_pool_desc* desc, pa_pool** out);
void pa_pool_destroy(pa_pool* pool);

/* Register an empty request (no blocks reserved: [ngrok] "PagedAttention").
 * PA_ERR_EXISTS if seq_id is live. */
pa_status pa_seq_add(pa_pool* pool, int64_t seq_id);

/* Child shares all of parent's blocks; each block's reference count + 1
 * ([tcd] memory sharing for parallel sampling).  PA_ERR_UNKNOWN_SEQ /
 * PA_ERR_EXISTS. */
pa_status pa_seq_fork(pa_pool* pool, int64_t parent, int64_t child);

/* Drop the request: each block's count - 1 in logical order; a block reaching
 * zero is pushed on the free stack (request finished or preempted: [ngrok]
 * scheduler; [lens] scheduler skeleton), or, if it is cached (see
 * pa_seq_register), appended to the evictable list instead. */
pa_status pa_seq_free(pa_pool* pool, int64_t seq_id);

/* Preemption by swapping ([lens] scheduler skeleton: a preempted request is
 * either moved out to CPU memory or dropped and recomputed later; [tcd]
 * tuning anti-patterns: swap is the last-resort spill of KV blocks to CPU
 * memory, much slower than staying on the GPU).
 * pa_seq_swap_out: writes the sequence's physical blocks in logical order
 * (ceil(len/16) of them, at most cap) to `blocks` (host) and its length to
 * *seq_len, then releases it exactly as pa_seq_free does.  The caller must
 * enqueue pa_gather_blocks over those blocks before any later launch on the
 * same stream writes into the pool (the blocks may be handed out again at
 * once).  PA_ERR_UNKNOWN_SEQ, or PA_ERR_CAPACITY (nothing changes).
 * Blocks shared with other sequences stay with them; the swapped copy is
 * private. */
pa_status pa_seq_swap_out(pa_pool* pool, int64_t seq_id, int32_t* blocks, int32_t cap,
                          int32_t* n_blocks, int32_t* seq_len);

/* pa_seq_swap_in: creates `seq_id` (which must not exist: PA_ERR_EXISTS)
 * with length seq_len and ceil(seq_len/16) blocks taken from the free list
 * in logical order (written to `blocks`, host), for pa_scatter_blocks to
 * fill.  Atomic: PA_ERR_OUT_OF_BLOCKS or PA_ERR_CAPACITY change nothing. */
pa_status pa_seq_swap_in(pa_pool* pool, int64_t seq_id, int32_t seq_len, int32_t* blocks,
                         int32_t cap, int32_t* n_blocks);

/* Prefix caching ([ngrok] "prefix caching": requests that begin with the same
 * tokens share the KV blocks of that prefix; only the same tokens at the same
 * positions count, one differing token ends the sharing, and a block is known
 * by a hash of the previous block's hash and its own tokens).  Only full
 * 16-token blocks are cached.
 *
 * pa_seq_add_cached: register a new request (PA_ERR_EXISTS if live) whose
 *   table starts with the cached blocks matching tokens[0..n_tokens) block by
 *   block from the first token, stopping at the first block that is not
 *   cached.  Each hit takes one more reference (sharing as pa_seq_fork does;
 *   an evictable block is revived).  *n_cached = 16 * hits = the request's
 *   length; the caller appends and computes the remaining tokens.  A hash hit
 *   counts only if the block's parent hash and tokens match exactly.
 * pa_seq_register: make the request's full blocks within its first n_tokens
 *   tokens (tokens = those token ids, n_tokens <= its length) findable, in
 *   order: block i gets key hash(key of block i-1, its 16 tokens).  A block
 *   that already has a key keeps it, and a key already held by another block
 *   stays there.  *n_registered = blocks newly cached.
 * A cached block whose last reference is dropped is kept as evictable.
 * Allocation (pa_append_slots) takes the free stack first; when it is empty
 * it evicts the block that became evictable longest ago (dropping its key).
 * pa_num_free_blocks and the capacity checks count free + evictable blocks. */
pa_status pa_seq_add_cached(pa_pool* pool, int64_t seq_id, const int32_t* tokens,
                            int32_t n_tokens, int32_t* n_cached);
pa_status pa_seq_register(pa_pool* pool, int64_t seq_id, const int32_t* tokens,
                          int32_t n_tokens, int32_t* n_registered);

/* Blocks pa_append_slots would take off the free list for the same arguments
 * (new blocks + copy-on-write targets).  Pure. */
pa_status pa_can_append(const pa_pool* pool, int32_t n, const int64_t* seq_ids,
                        const int32_t* n_new, int32_t* blocks_needed);

/* Reserve slots for n_new[i] tokens of seq_ids[i], i < n, sequences in the
 * order given (ids must be distinct), tokens in position order.  For a token
 * at position p of its request, o = p % 16:
 *   o == 0          -> pop a block from the free stack and append it to the
 *                      request's table ([ngrok]: a new block only when the
 *                      last one is full; [yj] listing);
 *   o > 0, shared   -> copy-on-write: pop a block, record {old, new, o},
 *                      old's count - 1, table entry := new ([tcd]);
 *   slot = table[p / 16] * 16 + o.
 * slot_mapping receives sum(n_new) slots in (sequence, position) order
 * (capacity slot_cap); copies receives the CoW list (capacity copy_cap,
 * count in *n_copies).  Atomic: on PA_ERR_OUT_OF_BLOCKS ([yj] listing: no free
 * block is an error), PA_ERR_CAPACITY, PA_ERR_UNKNOWN_SEQ or PA_ERR_INVALID
 * the pool is unchanged, so the caller can preempt and retry. */
pa_status pa_append_slots(pa_pool* pool, int32_t n, const int64_t* seq_ids,
                          const int32_t* n_new, int32_t* slot_mapping, int64_t slot_cap,
                          pa_copy* copies, int32_t copy_cap, int32_t* n_copies);

/* Block tables of the listed requests, row-major [n][max_blocks] int32 padded
 * with -1, and their token counts ([tcd]: the table maps logical to physical
 * blocks).  Caller-owned host buffers.  PA_ERR_CAPACITY if a table is longer
 * than max_blocks. */
pa_status pa_block_tables(const pa_pool* pool, int32_t n, const int64_t* seq_ids,
                          int32_t max_blocks, int32_t* tables, int32_t* seq_lens);

/* One request's table (capacity cap) and length. */
pa_status pa_seq_table(const pa_pool* pool, int64_t seq_id, int32_t* table, int32_t cap,
                       int32_t* n_blocks, int32_t* seq_len);

int32_t pa_num_free_blocks(const pa_pool* pool);
pa_status pa_ref_count(const pa_pool* pool, int32_t block, int32_t* ref);
pa_status pa_pool_get_stats(const pa_pool* pool, pa_pool_stats* stats);

/* Free stack contents from bottom to top (capacity cap, count in *n). */
pa_status pa_free_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* Evictable blocks, the next to be evicted first (capacity cap, count in *n). */
pa_status pa_evictable_list(const pa_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* Invariants: free + evictable + referenced = num_blocks; each block's count
 * equals the number of tables holding it; each table has ceil(len/16)
 * entries; the free stack holds distinct unreferenced uncached blocks, the
 * evictable list distinct unreferenced cached ones; the cache map and the
 * blocks' keys agree.  PA_ERR_INTERNAL if violated. */
pa_status pa_pool_check(const pa_pool* pool);

/* Continuous-batching scheduler over a pool ([ngrok] scheduler section;
 * [lens] "scheduler skeleton").  Host only; it drives the pool through the
 * calls above and the caller runs the kernels for each planned step.
 *
 * A request is (prompt_len, output_len).  Its input is the prompt followed by
 * its generated tokens; each step computes a chunk of its not-yet-computed
 * input, and a step that computes its last input token yields one new token.
 * It finishes when output_len tokens are out; its blocks are freed then.
 *
 * pa_sched_schedule plans one step within token_budget tokens:
 *   1. running requests (admission order) with exactly their newest token
 *      left (decode, 1 token) first;
 *   2. then running requests still in prefill: a chunk of
 *      min(remaining input, budget left) (chunked prefill);
 *   3. then waiting requests in queue order while budget is left, fewer than
 *      max_running run and the pool can hold the blocks of their first
 *      chunk (admission);
 *   4. all chunks are reserved with one pa_append_slots in that order; while
 *      it reports PA_ERR_OUT_OF_BLOCKS, the most recently admitted running
 *      request is preempted: its blocks are freed, it returns to the head of
 *      the waiting queue with nothing computed (it recomputes prompt and
 *      generated tokens later) and leaves this step.
 * items[i] = {request, first position, token count, decode?} in reservation
 * order; slot_mapping / copies are pa_append_slots' outputs for them;
 * preempted lists the preempted requests.  Capacities must be at least
 * max_running (items, copies, preempted) and token_budget (slots), else
 * PA_ERR_CAPACITY with nothing changed.  One plan at a time: the next
 * schedule needs a pa_sched_commit.
 * pa_sched_commit: the planned chunks were computed; advance the requests,
 * free the finished ones and list them in finished (capacity >= items).
 * A request whose prompt and output (but the last token) exceed the pool is
 * refused by pa_sched_add_request (PA_ERR_INVALID): it could never finish. */
typedef struct pa_sched pa_sched;

typedef struct pa_sched_item {
  int64_t req_id;
  int32_t start;     /* first input position of the chunk                 */
  int32_t n_tokens;  /* chunk length                                       */
  int32_t decode;    /* 1: the request's single newest token after its prompt */
  int32_t reserved;
} pa_sched_item;

typedef struct pa_sched_stats {
  int32_t n_waiting;
  int32_t n_running;
  int64_t steps;
  int64_t preemptions;
  int64_t finished;
  int32_t n_swapped;  /* swapped-out requests waiting to resume */
  int32_t reserved;
} pa_sched_stats;

pa_status pa_sched_create(pa_pool* pool, int32_t token_budget, int32_t max_running,
                          pa_sched** out);
void pa_sched_destroy(pa_sched* sched);
pa_status pa_sched_add_request(pa_sched* sched, int64_t req_id, int32_t prompt_len,
                               int32_t output_len);
pa_status pa_sched_schedule(pa_sched* sched, pa_sched_item* items, int32_t item_cap,
                            int32_t* n_items, int32_t* slot_mapping, int64_t slot_cap,
                            pa_copy* copies, int32_t copy_cap, int32_t* n_copies,
                            int64_t* preempted, int32_t preempt_cap, int32_t* n_preempted);
pa_status pa_sched_commit(pa_sched* sched, int64_t* finished, int32_t cap,
                          int32_t* n_finished);
pa_status pa_sched_get_stats(const pa_sched* sched, pa_sched_stats* stats);
/* Swap mode ([lens] scheduler skeleton: a preempted request is moved to CPU
 * memory instead of being dropped; [tcd]: swap as the last-resort spill).
 * pa_sched_set_swap(1) before a step: from then on a preempted request that
 * has computed tokens is released with pa_seq_swap_out, keeps its computed
 * count and goes to the head of a swapped queue (one with nothing computed
 * is preempted as in recompute mode).  Each pa_sched_schedule first resumes
 * swapped requests from the head of that queue, before any other work,
 * while fewer than max_running run and the free blocks cover the request's
 * ceil(computed/16) blocks plus one block per running request; a resumed
 * request gets fresh blocks (pa_seq_swap_in) and runs like the others.  A
 * request resumed and preempted again in the same step goes back to the
 * head of the swapped queue with no data movement.  Switching swap mode off
 * while requests are swapped out is PA_ERR_INVALID.
 * pa_sched_swaps (between schedule and commit) lists the step's transfers
 * in the order the caller must run them, before any of the step's own
 * pool writes: swap-outs (gather those blocks' K/V, then keep them on the
 * host), then swap-ins (scatter the saved K/V into the new blocks).  blocks
 * receives every operation's blocks in logical order; op.first is the
 * offset of its first one.  PA_ERR_CAPACITY (with the counts set) when cap
 * or blocks_cap is short. */
typedef struct pa_sched_swap {
  int64_t req_id;
  int32_t kind;      /* 0: swap out, 1: swap in                    */
  int32_t seq_len;   /* tokens held (the request's computed count) */
  int64_t first;     /* offset of its first block in `blocks`      */
  int32_t n_blocks;
  int32_t reserved;
} pa_sched_swap;

pa_status pa_sched_set_swap(pa_sched* sched, int32_t enable);
pa_status pa_sched_swaps(const pa_sched* sched, pa_sched_swap* ops, int32_t cap, int32_t* n_ops,
                         int32_t* blocks, int64_t blocks_cap, int64_t* n_blocks);

/* One request's progress: input tokens computed, outputs so far, preemptions. */
pa_status pa_sched_request(const pa_sched* sched, int64_t req_id, int32_t* computed,
                           int32_t* generated, int32_t* preemptions);

/* Bytes one token's K and V occupy: 2 * layers * kv_heads * head_dim *
 * dtype_bytes ([lens] KV-size example: 131,072 for 32/8/128/fp16). */
uint64_t pa_kv_bytes_per_token(int32_t layers, int32_t num_kv_heads, int32_t head_dim,
                               int32_t dtype_bytes);

/* ------------------------------------------------------------------------ */
/* Device kernels (gfx950)                                                   */
/* ------------------------------------------------------------------------ */

typedef struct pa_kv_view {
  pa_half* k_pool;       /* device, layout above */
  pa_half* v_pool;       /* device, layout above */
  int32_t num_blocks;
  int32_t block_size;    /* must be PA_BLOCK_SIZE */
  int32_t num_kv_heads;  /* >= 1 */
  int32_t head_dim;      /* 64 or 128 */
} pa_kv_view;

/* Store T new tokens' K and V into their slots ([yj] listing, the
 * cache[block, slot] store of append_token).  k, v: device [T][kv_heads][D]
 * fp16, contiguous.  slot_mapping: device int32 [T]; a negative slot skips the
 * token; a slot >= num_blocks*16 is ignored (never written).  Bit copy. */
pa_status pa_reshape_and_cache(const pa_half* k, const pa_half* v, const int32_t* slot_mapping,
                               int32_t num_tokens, pa_kv_view kv, void* stream);

/* Perform n copy-on-write copies (device array of pa_copy, as returned by
 * pa_append_slots).  Entries with an out-of-range block or n_slots outside
 * [0, 16] are skipped.  Bit copy.  Must be ordered before the
 * pa_reshape_and_cache of the same step (same stream). */
pa_status pa_copy_blocks(const pa_copy* copies, int32_t n, pa_kv_view kv, void* stream);

/* Device address of pinned host memory (allocated with hipHostMalloc, e.g. a
 * torch pin_memory tensor), so that kernels can read per-step metadata in
 * place instead of from a device copy: the slot mapping, block tables,
 * lengths and work list that the scheduler rebuilds every step ([lens]
 * scheduler skeleton: blocks are reserved for the running requests before
 * each forward pass).  host: a pointer into such an allocation; *device
 * receives the matching device address.  Reads through it cross the host
 * link, so it suits data that a launch reads a few times.  The caller keeps
 * the memory unchanged until every launch that reads it has completed.
 * PA_ERR_INVALID for a null argument or memory the runtime does not hold as
 * pinned. */
pa_status pa_host_device_pointer(const void* host, void** device);

/* Copy `bytes` from src to dst with one kernel launch on `stream`, for
 * moving a step's metadata (slot mapping, block tables, lengths, work list:
 * [lens] scheduler skeleton) from pinned host memory, through its device
 * address (pa_host_device_pointer), into device memory.  The runtime's own
 * copy from host memory runs as several launches; this is one.  src, dst:
 * device addresses, 16-byte aligned, non-overlapping; bytes: a multiple of
 * 16 (0 does nothing).  PA_ERR_INVALID on a null pointer, misalignment or a
 * size that is not a multiple of 16.  Async on `stream`. */
pa_status pa_stage_copy(const void* src, void* dst, uint64_t bytes, void* stream);

/* pa_stage_copy plus word updates, in one launch: `bytes` from src to dst as
 * pa_stage_copy moves them, and for each of the n_updates int32 pairs
 * (index, value) at `updates`, target[index] = value.  For a device-resident
 * block table refreshed each step ([lens] scheduler skeleton) with only the
 * entries that changed since the previous step (a request that took a new
 * block or a copy-on-write replacement), instead of the whole padded table.
 * src, updates: device addresses (those of pinned host memory included);
 * src, dst 16-byte aligned, bytes a multiple of 16; updates 8-byte aligned;
 * target: device int32 [target_len], 4-byte aligned.  Indices outside
 * [0, target_len) are skipped; the indices should be distinct (a repeated
 * one takes one of its values).  dst and target must not overlap.
 * PA_ERR_INVALID on a null pointer with a nonzero count, misalignment, a
 * negative count or target_len > INT32_MAX.  Async on `stream`. */
pa_status pa_stage_update(const void* src, void* dst, uint64_t bytes, const int32_t* updates,
                          int64_t n_updates, int32_t* target, int64_t target_len, void* stream);

/* Swap transfers: whole K and V tiles (all kv heads) of n blocks between the
 * pools and contiguous buffers [n][num_kv_heads][16*D] fp16 in the pools'
 * tile order (a bit copy; the caller moves the buffers to and from host
 * memory).  blocks: device int32 [n] (entries outside [0, num_blocks) are
 * skipped); buffers: device, 16-byte aligned, n * num_kv_heads * 16 * D
 * values each.  pa_gather_blocks reads the pools, pa_scatter_blocks writes
 * them.  Async on `stream`. */
pa_status pa_gather_blocks(const int32_t* blocks, int32_t n, pa_kv_view kv, pa_half* k_out,
                           pa_half* v_out, void* stream);
pa_status pa_scatter_blocks(const int32_t* blocks, int32_t n, pa_kv_view kv,
                            const pa_half* k_in, const pa_half* v_in, void* stream);

/* Work list for the work-list form of pa_paged_attention_decode (host, pure).
 * Request b of length L is cut into ceil(ceil(L/16) / (partition_size/16))
 * partitions; each (request, partition) becomes one entry (b << 16) | p, and a
 * request of length 0 one entry (b << 16).  Entries are ordered by partition
 * size in blocks, largest first, ties in (request, partition) order, so that
 * the short units are the last ones the GPU starts.  seq_lens: host int32
 * [batch], batch <= 65535.  Returns the number of entries; they are written to
 * items (host) only if that number is <= cap.  Returns -PA_ERR_INVALID on a
 * negative length, a bad partition_size or more than 65535 partitions. */
int32_t pa_decode_work_items(const int32_t* seq_lens, int32_t batch, int32_t partition_size,
                             int32_t* items, int32_t cap);

/* Workspace bytes pa_paged_attention_decode needs (0 when max_seq_len <=
 * partition_size): a partial softmax state for every (request, query head,
 * partition): the normalised partial output in fp16 (head_dim
 * values; |o| <= max |V|, so fp16 cannot overflow) and the running max and sum
 * in fp32 = B * n_q * ceil(max_seq_len/partition) * (2 * head_dim + 8) bytes. */
uint64_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_seq_len, int32_t partition_size);

/* One decode step of attention over the paged cache ([lens] "fragmentation
 * and PagedAttention": the kernel follows the table to gather K and V while
 * computing).  For request i, query head h, kv head g = h / (n_q / kv_heads):
 *   out[i][h] = sum_j softmax_j(scale * q[i][h] . K_j) V_j,  j < seq_lens[i],
 * K_j, V_j the j-th logical token, in block tables[i][j/16] at slot j%16.
 *   out: device [B][n_q][D] fp16 (RNE from fp32).  q: device [B][n_q][D] fp16.
 *   tables: device int32 [B][max_blocks]; seq_lens: device int32 [B], each in
 *   [0, max_seq_len] and <= max_blocks*16 (a request of length 0 gets zeros).
 *   n_q must be a multiple of kv_heads with n_q/kv_heads <= 16.
 *   Requests are split into partitions of partition_size tokens (a multiple
 *   of 16 in [16, 4096], e.g. 512); each (kv head, request, partition) unit is
 *   computed by one workgroup, which writes the request's output directly if
 *   it has one partition and a partial softmax state otherwise; a second
 *   kernel merges the partitions by log-sum-exp.
 *   scale: positive and finite (PA_ERR_INVALID otherwise).
 *   work_items / n_items: NULL / 0 launches one workgroup per unit (grid
 *   form).  Otherwise a device copy of the list pa_decode_work_items built
 *   from the same lengths (n_items <= 2^30): then as many workgroups as stay
 *   resident walk it, workgroup y of a kv head taking entries y, 2W-1-y,
 *   2W+y, ... of W such workgroups (work-list form); entries naming a
 *   request >= batch or a partition the lengths do not contain are skipped.
 *   Both forms give bitwise the same outputs.  In the work-list form the two
 *   wavefronts of a workgroup hand merge slots to each other through LDS
 *   with a bounded wait; should a wait ever exceed its bound (it does not
 *   in a normal run), the workgroup stops and writes NaN to every output
 *   row (or partial) of the units it had not yet written, so the failure
 *   shows in the output instead of leaving stale rows.
 *   workspace: device, 16-byte aligned, >= pa_decode_workspace_bytes(...);
 *   may be NULL when that is 0.  Calls sharing a workspace must not overlap.
 *   A table entry outside [0, num_blocks) or a length above max_blocks*16
 *   makes that request's output NaN (no out-of-bounds access).
 *   flags: 0 or PA_DECODE_KEEP_KV (anything else: PA_ERR_INVALID).  By
 *   default every K/V tile is loaded non-temporally, since without sharing
 *   each is read once per call; pass PA_DECODE_KEEP_KV when requests share
 *   blocks ([tcd] "memory sharing for parallel sampling"; [yj]
 *   "copy-on-write prefix sharing"), e.g. whenever pa_pool_get_stats reports
 *   num_shared > 0, so that a shared tile stays cached for the other
 *   requests.  Results are bitwise the same either way. */
pa_status pa_paged_attention_decode(pa_half* out, const pa_half* q, pa_kv_view kv,
                                    const int32_t* tables, int32_t max_blocks,
                                    const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                    float scale, int32_t partition_size, int32_t max_seq_len,
                                    const int32_t* work_items, int32_t n_items,
                                    void* workspace, uint64_t workspace_bytes, uint32_t flags,
                                    void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pa_paged_attention_decode with the partials kept in a scratch array that
 * the library's code object holds on each GPU, PA_DECODE_SCRATCH_BYTES
 * (64 MiB) per GPU, held until the process ends.  Same arguments, outputs
 * (bitwise) and checks as pa_paged_attention_decode, without workspace.
 *   - Calls no hipMalloc / hipFree or other allocating routine.  The first
 *     call on a device looks the array's address up (hipGetSymbolAddress)
 *     with that device current; `stream` (NULL = the null stream) must
 *     belong to the current device (PA_ERR_INVALID otherwise).
 *   - PA_ERR_CAPACITY, before anything else, when the partials
 *     (pa_decode_workspace_bytes of the same arguments) exceed
 *     PA_DECODE_SCRATCH_BYTES: e.g. 256 requests x 64 query heads at
 *     head_dim 128 fit up to 7,680 tokens with 512-token partitions.
 *   - Every call on one GPU uses the same array, and nothing in it needs
 *     to start at zero (each partial is written before it is read).  Two
 *     calls in flight on one GPU at once (e.g. on different streams) race
 *     on it: the caller orders them. */
#define PA_DECODE_SCRATCH_BYTES (64ull << 20)
pa_status pa_paged_attention_decode_noalloc(pa_half* out, const pa_half* q, pa_kv_view kv,
                                            const int32_t* tables, int32_t max_blocks,
                                            const int32_t* seq_lens, int32_t batch,
                                            int32_t num_q_heads, float scale,
                                            int32_t partition_size, int32_t max_seq_len,
                                            const int32_t* work_items, int32_t n_items,
                                            uint32_t flags, void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 KV cache                                                              */
/* ------------------------------------------------------------------------ */
/* A smaller KV data type as a serving setting ([lens] "in practice": it
 * shrinks K/V, so the same memory holds more tokens and more requests; [sns]
 * "deep dive": FP8 among the supported formats).  The pages fix neither the
 * format nor the scale; this library reads them as:
 *   - each value is one OCP FP8 E4M3 byte (sign, 4 exponent bits with bias 7,
 *     3 mantissa bits; exponent 0 subnormal; 0x7F/0xFF NaN; largest 448);
 *   - one fp32 scale per pool: an fp16 value x is stored as
 *     e4m3(clamp(fp32(x) * fp32(1/k_scale), -448, 448)), the product rounded
 *     to fp32 and then to E4M3 by round-to-nearest-even (NaN stays NaN,
 *     +-inf saturate to +-448); code c stands for value(c) * k_scale (V alike).
 * FP8 pools have the fp16 pools' [num_blocks][num_kv_heads][tile] shape with
 * 16*D one-byte values per tile (tile (b, h) at byte (b*H + h)*16*D), ordered
 * so that each 16-byte-per-lane load brings two MFMA operands:
 *   K tile [D/64][4][16][2][8]: slot s, dim c at byte
 *           (c/64)*1024 + ((c/8)%4)*256 + s*16 + ((c/32)%2)*8 + c%8
 *   V tile [D/64][4][16][2][2][4]: slot s, dim c at byte
 *           (c/64)*1024 + (s/4)*256 + (c%16)*16 + ((c/32)%2)*8 + ((c/16)%2)*4 + s%4
 * (D = 64 or 128). */
typedef struct pa_kv_view_fp8 {
  uint8_t* k_pool;       /* device, E4M3 codes, layout above */
  uint8_t* v_pool;       /* device, E4M3 codes, layout above */
  int32_t num_blocks;
  int32_t block_size;    /* must be PA_BLOCK_SIZE */
  int32_t num_kv_heads;  /* >= 1 */
  int32_t head_dim;      /* 64 or 128 */
  float k_scale;         /* > 0, finite */
  float v_scale;         /* > 0, finite */
} pa_kv_view_fp8;

/* pa_reshape_and_cache into FP8 pools: the same slots and arguments, each
 * value quantised as above (k with k_scale, v with v_scale); the host computes
 * 1/scale in fp32 once per call. */
pa_status pa_reshape_and_cache_fp8(const pa_half* k, const pa_half* v,
                                   const int32_t* slot_mapping, int32_t num_tokens,
                                   pa_kv_view_fp8 kv, void* stream);

/* pa_copy_blocks for FP8 pools (bit copy of slots [0, n_slots) of K and V). */
pa_status pa_copy_blocks_fp8(const pa_copy* copies, int32_t n, pa_kv_view_fp8 kv, void* stream);

/* pa_gather_blocks / pa_scatter_blocks for FP8 pools: the same transfers of
 * 16*D one-byte codes per tile (the pool's scales do not move). */
pa_status pa_gather_blocks_fp8(const int32_t* blocks, int32_t n, pa_kv_view_fp8 kv,
                               uint8_t* k_out, uint8_t* v_out, void* stream);
pa_status pa_scatter_blocks_fp8(const int32_t* blocks, int32_t n, pa_kv_view_fp8 kv,
                                const uint8_t* k_in, const uint8_t* v_in, void* stream);

/* pa_paged_attention_decode over FP8 pools: the same arguments, work list,
 * workspace (pa_decode_workspace_bytes) and flags; K_j and V_j are the values
 * the codes stand for.  The codes are widened to fp16 exactly, k_scale joins
 * the softmax exponent's factor (scale * k_scale) and v_scale multiplies each
 * partition's normalised output; everything else is the fp16 kernels' math. */
pa_status pa_paged_attention_decode_fp8(pa_half* out, const pa_half* q, pa_kv_view_fp8 kv,
                                        const int32_t* tables, int32_t max_blocks,
                                        const int32_t* seq_lens, int32_t batch,
                                        int32_t num_q_heads, float scale, int32_t partition_size,
                                        int32_t max_seq_len, const int32_t* work_items,
                                        int32_t n_items, void* workspace,
                                        uint64_t workspace_bytes, uint32_t flags, void* stream);

/* Workspace bytes pa_paged_attention_prefill needs for a chunk of chunk_len
 * query rows ending at key position q_start + chunk_len. */
uint64_t pa_prefill_workspace_bytes(int32_t chunk_len, int32_t num_q_heads, int32_t head_dim,
                                    int32_t q_start);

/* Causal attention of one prefill chunk over the paged cache ([ngrok]
 * chunked prefill; [lens] FIG 1, prefill grows with the square of the
 * length).  Row r < chunk_len is the query at absolute position q_start + r
 * and attends keys 0..q_start + r of the request whose block table is
 * `table` (device int32, >= ceil((q_start+chunk_len)/16) entries); the
 * chunk's own K/V must already be stored (pa_reshape_and_cache).
 *   out: device [chunk_len][n_q][D] fp16; q: device [chunk_len][n_q][D] fp16.
 *   head_dim 64 or 128; n_q/kv_heads <= 16 and divides 128; scale positive
 *   and finite (PA_ERR_INVALID otherwise).
 *   workspace: device, >= pa_prefill_workspace_bytes(...). */
pa_status pa_paged_attention_prefill(pa_half* out, const pa_half* q, pa_kv_view kv,
                                     const int32_t* table, int32_t table_len, int32_t q_start,
                                     int32_t chunk_len, int32_t num_q_heads, float scale,
                                     void* workspace, uint64_t workspace_bytes, void* stream);

/* pa_paged_attention_prefill over FP8 pools: the same arguments and
 * workspace; K_j and V_j are the values the codes stand for.  The codes are
 * widened to fp16 exactly as the tiles are staged, k_scale joins the softmax
 * exponent's factor (scale * k_scale) and v_scale multiplies the normalised
 * output; everything else is the fp16 kernel's arithmetic.  Scales must be
 * positive and finite (PA_ERR_INVALID). */
pa_status pa_paged_attention_prefill_fp8(pa_half* out, const pa_half* q, pa_kv_view_fp8 kv,
                                         const int32_t* table, int32_t table_len,
                                         int32_t q_start, int32_t chunk_len, int32_t num_q_heads,
                                         float scale, void* workspace, uint64_t workspace_bytes,
                                         void* stream);

/* ------------------------------------------------------------------------ */
/* Mixed step: decode batch + prefill chunk in one launch                    */
/* ------------------------------------------------------------------------ */
/* A scheduler step whose batch holds both decoding requests and one prompt
 * chunk ([lens] "scheduler skeleton": one forward pass over the step's mixed
 * batch; [ngrok] "the scheduler": long prompts are prefilled chunk by chunk
 * alongside decoding requests).  The two parts are the arguments of
 * pa_paged_attention_decode (work-list form) and pa_paged_attention_prefill
 * over the same pool (fp16 here, FP8 E4M3 in pa_paged_attention_mixed_fp8). */
typedef struct pa_decode_batch {
  pa_half* out;              /* device [batch][n_q][D] fp16 */
  const pa_half* q;          /* device [batch][n_q][D] fp16 */
  const int32_t* tables;     /* device int32 [batch][max_blocks] */
  int32_t max_blocks;
  const int32_t* seq_lens;   /* device int32 [batch] */
  int32_t batch;             /* 0: no decode part */
  int32_t partition_size;    /* as for pa_paged_attention_decode */
  int32_t max_seq_len;
  const int32_t* work_items; /* device copy of pa_decode_work_items(seq_lens) */
  int32_t n_items;
} pa_decode_batch;

typedef struct pa_prefill_chunk {
  pa_half* out;              /* device [chunk_len][n_q][D] fp16 */
  const pa_half* q;          /* device [chunk_len][n_q][D] fp16 */
  const int32_t* table;      /* device int32, the chunk's request's block table */
  int32_t table_len;
  int32_t q_start;
  int32_t chunk_len;         /* 0: no prefill part */
} pa_prefill_chunk;

/* Workspace bytes pa_paged_attention_mixed needs: the decode part's
 * pa_decode_workspace_bytes rounded up to 256, then the chunk's
 * pa_prefill_workspace_bytes.  0 for a NULL argument. */
uint64_t pa_mixed_workspace_bytes(const pa_decode_batch* dec, const pa_prefill_chunk* pf,
                                  int32_t num_q_heads, int32_t head_dim);

/* Decode attention for every request of `dec` and causal attention for the
 * chunk `pf`, with the results of pa_paged_attention_decode (bitwise the
 * same outputs) and pa_paged_attention_prefill (bitwise the same outputs),
 * with one attention kernel instead of two: its first workgroups compute the
 * chunk's tiles and the rest, as many as stay resident, walk the decode work
 * list as the decode launch's work-list form does (one walk per wavefront
 * pair, several pairs per workgroup); then the merges of the chunk's key
 * splits and of the decode partitions (two small kernels).  Decode
 * workgroups start on CUs as soon as prefill tiles retire, so memory-bound
 * decode fills the compute-bound chunk's tail.  The decode part's bounded
 * LDS waits behave as in pa_paged_attention_decode: a give-up leaves that
 * walk's remaining rows NaN, never stale.
 *   kv: one fp16 pool; num_q_heads and scale apply to both parts.
 *   dec, pf: host structs (read during the call only); a part with batch 0 /
 *   chunk_len 0 is skipped.  dec->work_items must be non-NULL when batch > 0
 *   and n_items > 0 and must have been built from the same lengths.
 *   workspace: device, 16-byte aligned, >= pa_mixed_workspace_bytes(...).
 *   flags: 0 or PA_DECODE_KEEP_KV (decode loads), as for decode.
 *   Every argument check of both entry points applies (PA_ERR_INVALID before
 *   any launch); a failed launch returns PA_ERR_HIP. */
pa_status pa_paged_attention_mixed(const pa_decode_batch* dec, const pa_prefill_chunk* pf,
                                   pa_kv_view kv, int32_t num_q_heads, float scale,
                                   void* workspace, uint64_t workspace_bytes, uint32_t flags,
                                   void* stream);

/* pa_paged_attention_mixed over an FP8 E4M3 pool (pa_kv_view_fp8, one K and
 * one V scale per pool): the outputs of pa_paged_attention_decode_fp8 and
 * pa_paged_attention_prefill_fp8 on the same arguments, bitwise, from one
 * attention kernel.  Workspace size, flags and error behaviour as for
 * pa_paged_attention_mixed; scales must be positive and finite
 * (PA_ERR_INVALID). */
pa_status pa_paged_attention_mixed_fp8(const pa_decode_batch* dec, const pa_prefill_chunk* pf,
                                       pa_kv_view_fp8 kv, int32_t num_q_heads, float scale,
                                       void* workspace, uint64_t workspace_bytes, uint32_t flags,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
