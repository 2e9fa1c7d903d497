/*
 * pagedkv.h -- C ABI of a gfx950 (MI355X) library for attention over a paged KV cache.
 *
 * The method (pages cited by title and section):
 *   - Serving-engine KV page (ttlab, "LLM KV cache 02"), section 2 "PagedAttention",
 *     subsection "blocks and block table": K/V live in fixed 16-token physical blocks
 *     placed anywhere in a pool; each request maps logical blocks to physical ones
 *     through its block table; a new block is taken when the last one fills; the
 *     attention kernel follows the table and must give the contiguous-cache result.
 *   - Same page, subsection "block sharing": several tables may name one block.
 *   - "How inference engines actually work" page (xiaohu-jiedu), KV-cache section: each
 *     step computes K/V only for the new tokens and reads the rest from the cache;
 *     Chunked Prefill subsection: a long prompt runs as consecutive slices mixed with
 *     other requests' single decode tokens in one step.
 *
 * The GPU entry points are stateless.  The caller (a scheduler) owns every buffer; they
 * never allocate, free or synchronise, and run asynchronously on `stream`.  The block
 * allocator at the end of this header is a host object the caller creates and
 * destroys (it holds only host memory).
 *
 * Common conventions
 *   - All array pointers are DEVICE pointers on the current HIP device, C-contiguous.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - Element type `dtype`: PKV_F32 (float) or PKV_BF16 (bfloat16 stored as 16 bits).
 *     q, k/v pools, new K/V and `out` all use the same element type.
 *   - Pool layout, both pools: [num_blocks][num_kv_heads][16][head_dim].  Each
 *     (block, kv-head) tile is one contiguous run of 16*head_dim elements.
 *   - Flat slot s names pool position (block s / 16, offset s % 16).
 *   - Supported shapes: block_size == 16, head_dim in {64, 128},
 *     num_q_heads % num_kv_heads == 0.  Anything else is PKV_ERR_UNSUPPORTED or
 *     PKV_ERR_INVALID_ARG, returned before any launch.
 *   - Device-resident metadata (slots, table entries, lengths) are trusted
 *     preconditions.  Kernels never access memory outside the buffers whatever their
 *     values, but results for invalid metadata are unspecified;
 *     pkv_validate_metadata() and pkv_validate_fused_metadata() check host copies.
 *   - No exception crosses the ABI.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes   */
  PKV_ERR_UNSUPPORTED = 2, /* block_size != 16, head_dim not 64/128, bad dtype   */
  PKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required         */
  PKV_ERR_LAUNCH = 4,      /* the HIP runtime reported an error at launch        */
  PKV_ERR_OUT_OF_BLOCKS = 5, /* the block allocator has too few free blocks      */
  /* Range markers, not codes: every int32 value is a valid pkv_status, so callers in
   * any language may pass any integer (unknown values are reported as such). */
  PKV_STATUS_RANGE_MIN_ = -2147483647 - 1,
  PKV_STATUS_RANGE_MAX_ = 2147483647
} pkv_status;

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  /* Range markers, not types: any int32 is accepted (others give UNSUPPORTED). */
  PKV_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PKV_DTYPE_RANGE_MAX_ = 2147483647
} pkv_dtype;

#define PKV_BLOCK_SIZE 16

/*
 * paged_kv_write -- store this step's new K/V rows into their pool slots.
 * (Serving-engine KV page, section 2, "blocks and block table"; the inference-engine
 * page's KV-cache section: only the new tokens' K/V are produced each step.)
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim]           (read)
 *   k_pool, v_pool [num_blocks][num_kv_heads][16][head_dim]       (written)
 *   slot_mapping   int32 [num_tokens]; token t goes to flat slot slot_mapping[t];
 *                  a negative slot (or one >= num_blocks*16) skips the token.
 * Each copied row is a bit-exact copy.  Only the named slots change.  Two tokens
 * naming the same slot is a precondition violation (either may win).
 * num_tokens == 0 is a no-op.
 */
pkv_status paged_kv_write(const void *k_new, const void *v_new, void *k_pool,
                          void *v_pool, const int32_t *slot_mapping, int32_t num_tokens,
                          int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, pkv_dtype dtype, void *stream);

/*
 * paged_attention_workspace_size -- bytes of device scratch that
 * paged_attention_varlen needs for the same arguments on the current device.  It
 * holds the partial results of decode segments cut into key ranges (long rows, or too
 * few segments to fill the device) and of prefill chunks split over their keys; it is
 * 0 when nothing is split (e.g. 32 bf16 decode rows with 8 kv heads and up to 4,096
 * keys each, on a 256-CU device), for an empty
 * batch and for invalid shapes.  Its size depends on the device's compute-unit count.
 * For bf16 batches of several sequences with more query rows than sequences (so
 * holding a chunk) it also covers the key ranges of the decode rows when they run in
 * the chunk launch (8-wave workgroups: rows past 4,096 keys are cut into ranges).
 * The shape arguments must match the later call.
 */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t total_q,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      pkv_dtype dtype);

/*
 * paged_attention_varlen -- softmax attention of a varlen batch of query rows over
 * their sequences' paged K/V (run after paged_kv_write of the same step).
 * (Serving-engine KV page, section 2: the kernel walks the block table and must equal
 * attention over a contiguous cache; block sharing; inference-engine page, Chunked
 * Prefill: prefill slices and decode tokens share one step.)
 *
 *   out             [total_q][num_q_heads][head_dim]          (written)
 *   q               [total_q][num_q_heads][head_dim]
 *   k_pool, v_pool  [num_blocks][num_kv_heads][16][head_dim]
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]; entry lb of row s is the
 *                   physical block of sequence s's logical block lb; only entries
 *                   lb < ceil(context_lens[s]/16) are read
 *   context_lens    int32 [num_seqs]; keys of sequence s, this step's tokens included
 *   query_start_loc int32 [num_seqs+1]; rows of sequence s are
 *                   [query_start_loc[s], query_start_loc[s+1]); query_start_loc[0]==0
 *   max_context_len host upper bound of context_lens (sizes the split-K plan)
 *   max_query_len   host upper bound of the per-sequence query counts
 *   scale           multiplier of q.k before the softmax (e.g. 1/sqrt(head_dim))
 *   workspace       device scratch of workspace_bytes >= the size query's answer
 *                   (contents need no initialisation); calls that overlap in time
 *                   need separate workspaces.
 *
 * Row i of a sequence with q query rows and c keys sits at position c-q+i and sees
 * keys 0..c-q+i (a decode token, q == 1, sees all c).  Query head h reads KV head
 * h / (num_q_heads/num_kv_heads).  Rows whose sequence has q > c get zeros.
 * Output precision: bf16 inputs -> fp32 accumulation, bf16 output rounded to nearest
 * even; fp32 inputs -> fp32 throughout.
 */
pkv_status paged_attention_varlen(void *out, const void *q, const void *k_pool,
                                  const void *v_pool, const int32_t *block_tables,
                                  const int32_t *context_lens,
                                  const int32_t *query_start_loc, int32_t num_seqs,
                                  int32_t total_q, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  int32_t max_query_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, float scale, pkv_dtype dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_varlen_with_write -- one launch sequence for a whole step: the slot
 * write of this step's new rows and the attention over the updated pools.
 * (Same passages as paged_kv_write and paged_attention_varlen; the inference-engine
 * page's KV-cache section: each step appends its new tokens' K/V, then attends.)
 *
 * The result (out and both pools) is the same as paged_kv_write(k_new, v_new, k_pool,
 * v_pool, slot_mapping, total_q, ...) followed by paged_attention_varlen(...) with the
 * same arguments, under one extra precondition: new row t (a query row, [total_q]) is
 * the token at position context_len - q_len + i of its sequence (i its index among the
 * sequence's rows), and slot_mapping[t] is that position's table slot
 * (block_tables[s][pos / 16] * 16 + pos % 16).  With that, the first bf16 attention
 * launch stores all new rows itself and reads this step's keys and values straight
 * from k_new / v_new, saving the separate write launch: the decode kernel (decode
 * rows read their newest key and value there) and, for a batch of one chunk sequence,
 * the chunk kernel (its tiles read every new position there).  Other cases run the
 * write kernel first: fp32, and bf16 batches of several sequences with more query rows
 * than sequences, whose chunk tiles and decode rows then share one attention launch
 * (the decode rows in the workgroups after the chunk tiles, filling the compute units
 * that the chunk's shorter row tiles free).  Arguments as for the two calls above
 * (k_new, v_new [total_q][Hkv][D]).
 */
pkv_status paged_attention_varlen_with_write(
    void *out, const void *q, const void *k_new, const void *v_new, void *k_pool,
    void *v_pool, const int32_t *slot_mapping, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int32_t total_q, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
    pkv_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Shared-prefix attention (cascade).  Serving-engine KV page, section 2, "block
 * sharing", and section 4 (prefix cache): requests with a common prompt prefix name
 * the same physical blocks at the start of their tables.  Attention over a row's whole
 * context is the log-sum-exp combination of attention over those shared blocks and
 * attention over the row's own blocks, so the shared keys and values can be read once
 * for every row of the batch instead of once per row.
 *
 * paged_attention_varlen_shared_prefix -- paged_attention_varlen (k_new, v_new and
 * slot_mapping all NULL) or paged_attention_varlen_with_write (all three given, same
 * positional-slot precondition) for a batch of decode rows whose tables all begin with
 * the same `shared_blocks` physical blocks.  Same layouts and result.
 *   shared_blocks  block_tables[s][lb] == block_tables[0][lb] for lb < shared_blocks
 *                  and every s, and every sequence's cached context covers them:
 *                  context_lens[s] - q_len_s >= shared_blocks * 16 (so every row sees
 *                  every shared key, and no new row falls into a shared block);
 *                  pkv_validate_shared_prefix() checks host copies.  0 = nothing
 *                  shared: the call is the plain one (its workspace rules apply).
 *   workspace      at least paged_attention_shared_prefix_workspace_size(...) bytes
 *                  (contents need no initialisation).
 * Supported: bf16, one query row per sequence (max_query_len == 1, total_q ==
 * num_seqs); other shapes give PKV_ERR_UNSUPPORTED before any launch (use the plain
 * entry points).  The workspace query takes the call's max_context_len.  Two
 * launches on `stream`: one of the MFMA chunk kernel, whose first workgroups run the
 * shared blocks with every row as a column (partial results per key split; these also
 * store a fused call's new rows, which no part of the launch reads from the pools) and
 * whose other workgroups run the decode work over each row's own blocks (partial
 * results), then a merge per (row, query head).
 */
size_t paged_attention_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_context_len,
                                                    int32_t shared_blocks, pkv_dtype dtype);
pkv_status paged_attention_varlen_shared_prefix(
    void *out, const void *q, const void *k_new, const void *v_new, void *k_pool,
    void *v_pool, const int32_t *slot_mapping, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int32_t total_q, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_query_len, int32_t shared_blocks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    float scale, pkv_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_varlen_with_write_noalloc -- paged_attention_varlen_with_write for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, result and
 * precondition as paged_attention_varlen_with_write, without the workspace: the
 * split-K partials go to a scratch array of PKV_NOALLOC_SCRATCH_BYTES (32 MiB) that
 * the library keeps on each GPU it runs on for the life of the process.  The call
 * allocates and frees nothing.
 *   - A call whose workspace need (paged_attention_workspace_size for its shapes, with
 *     the chunk part only when max_query_len > 1) exceeds the scratch size returns
 *     PKV_ERR_WORKSPACE before any launch; use the workspace entry point then.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in time on
 *     one GPU (different streams, or different host threads) race and give undefined
 *     results; serialise them (one stream) or use the workspace entry point.  Nothing
 *     in the scratch needs to start at zero, so no call depends on what the previous
 *     one left there.
 *   - The scratch's device address is looked up on the first call on each device
 *     (make that first call outside graph capture); a runtime failure of that lookup
 *     returns PKV_ERR_LAUNCH.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status paged_attention_varlen_with_write_noalloc(
    void *out, const void *q, const void *k_new, const void *v_new, void *k_pool,
    void *v_pool, const int32_t *slot_mapping, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int32_t total_q, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
    pkv_dtype dtype, void *stream);

/*
 * Block bookkeeping (serving-engine KV page, section 2: "blocks and block table" -- a
 * request takes a new 16-token block when its current one fills; "block sharing" --
 * requests sharing a prompt name the same blocks, each block has a reference count,
 * and a shared block is copied only when a holder appends into it).
 *
 * pkv_block_allocator is a host object over physical blocks 0..num_blocks-1 of one
 * pool pair.  Tables passed to it are HOST int32 arrays (a request's logical->physical
 * block list, the row that goes into block_tables).  Not thread-safe.  The lowest
 * free block is always taken first.  Every call either succeeds or changes nothing.
 */
typedef struct pkv_block_allocator pkv_block_allocator;

/* Create an allocator with every block free (1 <= num_blocks <= INT32_MAX / 16, so
 * every flat slot fits in int32).  *out receives the handle. */
pkv_status pkv_allocator_create(int32_t num_blocks, pkv_block_allocator **out);
void pkv_allocator_destroy(pkv_block_allocator *alloc);
/* Free blocks (-1 for a NULL handle); reference count of a block (-1 if out of range). */
int32_t pkv_allocator_num_free(const pkv_block_allocator *alloc);
int32_t pkv_allocator_refcount(const pkv_block_allocator *alloc, int32_t block);

/*
 * pkv_allocator_fork -- another request now shares the num_used blocks of `table`
 * (one more reference each; the caller copies the table row for the new request).
 * INVALID_ARG if an entry is not a held block.
 */
pkv_status pkv_allocator_fork(pkv_block_allocator *alloc, const int32_t *table,
                              int32_t num_used);

/*
 * pkv_allocator_release -- a request is done with the num_used blocks of `table`: one
 * reference fewer each; a block with none left is free again.
 */
pkv_status pkv_allocator_release(pkv_block_allocator *alloc, const int32_t *table,
                                 int32_t num_used);

/*
 * pkv_allocator_append -- make room for num_new tokens after context_len cached ones
 * of the request whose table is `table` (ceil(context_len/16) used entries, room for
 * max_blocks_per_seq; updated in place).  Writes the flat pool slot of every new
 * token to slots[num_new] (the slot_mapping for paged_kv_write).  If the request's
 * partly filled last block is shared, the request first moves to a private copy:
 * the (source, destination) pair is written to copies[0..1], *num_copies = 1, and
 * the caller must run paged_kv_copy_blocks on it before writing the new tokens.
 * Errors: OUT_OF_BLOCKS if the pool cannot hold the append; INVALID_ARG for bad
 * arguments, a table entry that is not a held block, more blocks than
 * max_blocks_per_seq, or max_copies == 0 when a copy is needed.
 */
pkv_status pkv_allocator_append(pkv_block_allocator *alloc, int32_t *table,
                                int32_t max_blocks_per_seq, int32_t context_len,
                                int32_t num_new, int32_t *slots, int32_t *copies,
                                int32_t max_copies, int32_t *num_copies);

/*
 * paged_kv_copy_blocks -- copy-on-write copies on the GPU: for each pair i, every row
 * (all kv heads and offsets) of physical block copies[2i] is copied bit for bit to
 * block copies[2i+1], in both pools.
 *
 *   k_pool, v_pool  [num_blocks][num_kv_heads][16][head_dim]    (device, written)
 *   copies          int32 [num_copies][2] (source, destination) (device)
 * Pairs with an id outside [0, num_blocks) are skipped.  Destinations must be
 * distinct and not also sources in the same call (as the allocator produces them).
 * num_copies == 0 is a no-op.  Asynchronous on `stream`.
 */
pkv_status paged_kv_copy_blocks(void *k_pool, void *v_pool, const int32_t *copies,
                                int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                                void *stream);

/*
 * Prefix caching (host only).  (Serving-engine KV page (ttlab), section 4 "prefix
 * cache": a key per full block hashed from the previous block's key, the block's token
 * ids and extra inputs, SHA-256; freed blocks keep their contents in an eviction
 * queue, entered tail first and evicted least recently used first.  Inference-engine
 * page (xiaohu-jiedu), agent-traffic section: a request whose prefix matches points
 * its table at the blocks already in memory, so only its new tail is prefilled.)
 */
#define PKV_KEY_BYTES 32

/*
 * pkv_block_keys -- keys of the full blocks of a token sequence (host arrays).
 *   tokens[num_tokens]  int32 token ids; block b = tokens[16b .. 16b+15]
 *   extras[extras_len]  bytes hashed into every key (adapter id, multimodal hashes,
 *                       cache salt); may be NULL when extras_len == 0
 *   parent_key          32 bytes: key of the block before tokens[0], or NULL at the
 *                       start of a sequence (then 32 zero bytes)
 *   keys                [max_keys][32] out: key b = SHA-256(key b-1 || the 16 ids as
 *                       little-endian int32 || extras_len as little-endian uint32 ||
 *                       extras); *num_keys = num_tokens / 16 (a partial block has none)
 * INVALID_ARG if max_keys < num_tokens / 16 or an argument is missing.
 */
pkv_status pkv_block_keys(const int32_t *tokens, int32_t num_tokens, const void *extras,
                          int32_t extras_len, const uint8_t *parent_key, uint8_t *keys,
                          int32_t max_keys, int32_t *num_keys);

/*
 * pkv_allocator_enable_prefix_cache -- from now on, a block whose last reference goes
 * keeps its content if it was registered (it becomes evictable instead of free).  A
 * new block is a free one (lowest id first) while any is left, else the least
 * recently used evictable one, whose key is then forgotten.  pkv_allocator_num_free
 * counts free plus evictable blocks, and pkv_allocator_release drops a table's
 * blocks last first, so a finished request's tail is evicted before its head.
 */
pkv_status pkv_allocator_enable_prefix_cache(pkv_block_allocator *alloc);

/*
 * pkv_prefix_match -- the longest run of leading keys[0..num_keys) that are cached:
 * their blocks go to table[0..*num_hit) and each gains a reference (an evictable one
 * leaves the eviction queue).  The request then has *num_hit * 16 tokens cached.
 */
pkv_status pkv_prefix_match(pkv_block_allocator *alloc, const uint8_t *keys, int32_t num_keys,
                            int32_t *table, int32_t *num_hit);

/*
 * pkv_prefix_register -- cache the FULL held blocks table[i] under keys[i], i <
 * num_keys (call once their K/V are written).  A key already cached keeps its block;
 * a block already cached keeps its key.  INVALID_ARG if a block is not held.
 */
pkv_status pkv_prefix_register(pkv_block_allocator *alloc, const int32_t *table,
                               const uint8_t *keys, int32_t num_keys);

/* Cached blocks (held or evictable) and evictable blocks; -1 for a NULL handle. */
int32_t pkv_prefix_num_cached(const pkv_block_allocator *alloc);
int32_t pkv_prefix_num_evictable(const pkv_block_allocator *alloc);

/*
 * Step planning for chunked prefill (host only, no device access).
 * ("How inference engines actually work" page (xiaohu-jiedu), Chunked Prefill
 * subsection: each step has a token budget, long prompts run as consecutive slices and
 * the decoding requests' single tokens ride along in every step; serving-engine KV page
 * (ttlab), section 3, "the new problem": decode tokens fill the step first, and the
 * per-step token limit counts every token of the step.)
 *
 * pkv_plan_step -- how many tokens each of num_requests requests runs this step.
 *   prompt_len[r], num_computed[r]  host int32: prompt length; tokens whose K/V are
 *                   cached.  num_computed >= prompt_len > 0 means decoding.
 *   query_len[r]    host int32, written: 0 = not scheduled.
 * Decoding requests get 1 token each, in request order, while the budget lasts; the
 * rest of token_budget goes to requests still prefilling, in request order, each
 * taking min(prompt_len - num_computed, tokens left).  A zero-length prompt is never
 * scheduled.  INVALID_ARG for negative sizes or NULL arrays (num_requests > 0).
 */
pkv_status pkv_plan_step(int32_t num_requests, const int32_t *prompt_len,
                         const int32_t *num_computed, int32_t token_budget,
                         int32_t *query_len);

/*
 * pkv_build_step -- the varlen batch of one planned step, with its blocks.
 *   tables        host int32 [num_requests][max_blocks_per_seq], updated in place:
 *                 each scheduled request's row gains the blocks its new tokens need
 *                 (and moves to a private copy of a shared, partly filled last block),
 *                 exactly as pkv_allocator_append does, requests in order.
 *   num_computed, query_len   host int32 [num_requests] (query_len from pkv_plan_step).
 * Outputs (host int32; sequence s = the s-th request with query_len > 0):
 *   seq_request     [num_requests]           request index of sequence s
 *   block_tables    [num_requests][max_blocks_per_seq]  row s = the request's table,
 *                   entries past ceil(context_len/16) set to -1
 *   query_start_loc [num_requests + 1]       prefix sums of the query lengths
 *   context_lens    [num_requests]           num_computed + query_len
 *   slot_mapping    [max_tokens]             flat slot of each new token, in batch order
 *   copies          [num_requests][2]        (source, destination) block copies to run
 *                                            (paged_kv_copy_blocks) before the write
 *   *num_seqs, *num_copies
 * The whole step is checked before anything changes: OUT_OF_BLOCKS if the pool cannot
 * hold it, INVALID_ARG for bad arguments, a used table entry that is not a held
 * block, a row that would outgrow max_blocks_per_seq, or more tokens than max_tokens.
 * On error no table, count or output is changed except *num_seqs = *num_copies = 0.
 */
pkv_status pkv_build_step(pkv_block_allocator *alloc, int32_t num_requests, int32_t *tables,
                          int32_t max_blocks_per_seq, const int32_t *num_computed,
                          const int32_t *query_len, int32_t *seq_request,
                          int32_t *block_tables, int32_t *query_start_loc,
                          int32_t *context_lens, int32_t *slot_mapping, int32_t max_tokens,
                          int32_t *copies, int32_t *num_seqs, int32_t *num_copies);

/*
 * KV swap between the pools and host memory.  ("How inference engines actually work"
 * page (xiaohu-jiedu), agent-traffic section: a request idle during a tool call has
 * its KV cache moved to CPU memory and moved back for its next turn; serving-engine
 * KV page (ttlab), section 5: preemption, dropping the KV and prefilling again, is
 * the alternative.)
 *
 * Host image of n blocks: the K rows of blocks[0..n) then their V rows, each block
 * as it lies in a pool (num_kv_heads*16*head_dim elements); paged_kv_swap_bytes(n,
 * ...) bytes.  `staging` is a DEVICE buffer of the same size (caller-owned).  `host`
 * should be pinned (hipHostMalloc) for the copy to be asynchronous; it must stay
 * valid and, for a swap-in, unmodified until `stream` has passed the call.
 *   blocks  int32 [n] DEVICE array of physical block ids; an id outside [0,
 *           num_blocks) gathers zeros (swap-out) or is skipped (swap-in).
 * Swap-out: gathers the blocks into staging, then one device-to-host copy.  The
 * blocks may be reused once the copy has been issued (stream order).  Swap-in: one
 * host-to-device copy into staging, then a scatter into the (typically different)
 * blocks.  n == 0 is a no-op.  Asynchronous on `stream`.
 */
size_t paged_kv_swap_bytes(int32_t n, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, pkv_dtype dtype);
pkv_status paged_kv_swap_out(const void *k_pool, const void *v_pool, const int32_t *blocks,
                             int32_t n, void *staging, void *host, int32_t num_blocks,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             pkv_dtype dtype, void *stream);
pkv_status paged_kv_swap_in(void *k_pool, void *v_pool, const int32_t *blocks, int32_t n,
                            void *staging, const void *host, int32_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            pkv_dtype dtype, void *stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char *pkv_status_string(pkv_status status);

/*
 * pkv_validate_metadata -- host-side check of HOST copies of the metadata (no device
 * access).  Returns PKV_OK, or PKV_ERR_INVALID_ARG and, if `bad_index` is non-NULL,
 * the offending sequence (or token, for slot errors) index.  Checks:
 * query_start_loc non-decreasing from 0 to total_q; 0 <= q_len <= context_len and
 * context_len <= max_blocks_per_seq*16 per sequence; table entries in
 * [0, num_blocks) for every used logical block; slots < num_blocks*16 and no slot
 * named twice (slot_mapping may be NULL to skip the slot checks).
 */
pkv_status pkv_validate_metadata(const int32_t *block_tables, const int32_t *context_lens,
                                 const int32_t *query_start_loc,
                                 const int32_t *slot_mapping, int32_t num_seqs,
                                 int32_t total_q, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t *bad_index);

/*
 * pkv_validate_fused_metadata -- the checks of pkv_validate_metadata (slot_mapping
 * required) plus the extra precondition of paged_attention_varlen_with_write: new row
 * t, the i-th of sequence s with q rows and c keys, is position p = c - q + i, and
 * slot_mapping[t] == block_tables[s][p / 16] * 16 + p % 16 (the slot a scheduler that
 * appends tokens in order gives it; serving-engine KV page, section 2, "blocks and
 * block table": a block fills before the next one is taken).  HOST copies, no device
 * access.  On failure returns PKV_ERR_INVALID_ARG with *bad_index = the offending
 * sequence (base checks) or row (slot checks).  Metadata that fails only the extra
 * check is still valid for paged_kv_write followed by paged_attention_varlen.
 */
pkv_status pkv_validate_fused_metadata(const int32_t *block_tables,
                                       const int32_t *context_lens,
                                       const int32_t *query_start_loc,
                                       const int32_t *slot_mapping, int32_t num_seqs,
                                       int32_t total_q, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t *bad_index);

/*
 * pkv_validate_shared_prefix -- the extra precondition of
 * paged_attention_varlen_shared_prefix on HOST copies: every table row's first
 * shared_blocks entries equal row 0's, and context_lens[s] - q_len_s >=
 * shared_blocks * 16.  On failure returns PKV_ERR_INVALID_ARG with *bad_index = the
 * offending sequence (-1 for bad sizes or null pointers).  The base checks are
 * pkv_validate_metadata's.
 */
pkv_status pkv_validate_shared_prefix(const int32_t *block_tables,
                                      const int32_t *context_lens,
                                      const int32_t *query_start_loc, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, int32_t shared_blocks,
                                      int32_t *bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
