/*
 * pkv.h -- paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer argument named as a
 * device buffer is a device pointer that the caller allocated and owns; the
 * library never allocates, frees or synchronises.  Work is enqueued on
 * `stream` (a hipStream_t; NULL = the default stream), so the return value
 * reports host-side argument checks and launch status only.
 *
 * Layouts (row-major, fp16 = IEEE binary16 bit patterns):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim] fp16
 *                      A sequence's logically contiguous tokens live in
 *                      fixed-size physical blocks; logical token t of a
 *                      sequence sits in block block_tables[seq][t / block_size]
 *                      at offset t % block_size ("LLM 推理引擎 Continuous
 *                      Batching 与 PagedAttention：从 vLLM 原理到生产级部署实战",
 *                      §3.1 and §3.3; "动态批处理算法：连续批处理、In-flight
 *                      请求管理与 PagedAttention", §4.3).  For one KV head a
 *                      block is the [block_size][head_dim] tile that the
 *                      first page's kernel comment describes.
 *   block_tables     : [num_seqs][max_blocks_per_seq] int32; entries at or
 *                      beyond ceil(seq_len / block_size) are never read.
 *   seq_lens         : [num_seqs] int32, tokens held after this step's append.
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Supported instances: head_dim 64 or 128; block_size 1, 8, 16 or 32 for
 * the decode, 8, 16 or 32 for the prefill, any for kv_append; any
 * num_q_heads that is a multiple of num_kv_heads.
 *
 * Device-side contents cannot be checked without a synchronisation, so the
 * kernels guard them instead: a slot outside the pool is skipped; a sequence
 * whose length or block-table entries are out of range gets NaN in every
 * output element of its rows.  No kernel reads or writes outside the buffers
 * described by the size arguments.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PKV_OK = 0,
    PKV_ERR_INVALID = 1,     /* null pointer, bad size, misaligned buffer */
    PKV_ERR_UNSUPPORTED = 2, /* no compiled instance for this shape */
    PKV_ERR_HIP = 3,         /* the HIP runtime reported an error */
    PKV_ERR_NO_BLOCKS = 4,   /* block manager: not enough free blocks */
    PKV_ERR_SCRATCH = 5      /* no-allocation decode: partials exceed its scratch */
};

/* Static description of a status code. */
const char *pkv_status_string(int status);

/*
 * kv append: copies each new token's K and V rows into its physical slot
 * ("LLM 推理引擎 …", §3.2 BlockManager.append_token: a token goes into the
 * last block while it has room, otherwise into a newly taken block; the
 * slot = block * block_size + offset names that place).
 *
 *   key, value   : [num_tokens][num_kv_heads][head_dim] fp16, device
 *   k_cache, v_cache : the pools, device, written in place
 *   slot_mapping : [num_tokens] int32, device; slot < 0 marks a padding row
 *                  that is skipped; slots must be distinct (two rows with
 *                  one slot race); a slot >= num_blocks * block_size is
 *                  skipped.
 * The fp16 bit patterns are copied unchanged.  num_tokens may be 0.
 * Buffers must be 16-byte aligned.
 */
int pkv_kv_append(const void *key, const void *value, void *k_cache,
                  void *v_cache, const int32_t *slot_mapping,
                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks, void *stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these
 * arguments (0 when the sequences are not split).  Same meaning of the
 * arguments as below.
 */
size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size);

/*
 * Tokens per partition the decode uses for these arguments (the library's
 * choice when partition_size is 0).
 */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_seq_len,
                                  int32_t partition_size);

/*
 * Paged attention decode: one query token per sequence attends to all
 * seq_lens[s] tokens of its sequence through the block table
 * ("LLM 推理引擎 …", §3.3: block-table indirection, tokens_in_block bound,
 * running max and sum of exponentials; the V weighting the page leaves out is
 * out = sum_t softmax(q.k_t * scale)_t v_t).  Softmax and the weighted sum
 * accumulate in fp32.
 *
 *   out          : [num_seqs][num_q_heads][head_dim] float32, device
 *   q            : [num_seqs][num_q_heads][head_dim] fp16, device
 *   seq_lens     : each in 1 .. min(max_seq_len, max_blocks_per_seq*block_size)
 *   max_seq_len  : host-side upper bound of seq_lens (sizes the split)
 *   scale        : score scale, finite and > 0, normally 1/sqrt(head_dim)
 *   partition_size : tokens per split-sequence partition, a positive
 *                  multiple of block_size and at most 256 * block_size
 *                  (64 * block_size when block_size < 8), else
 *                  PKV_ERR_INVALID; 0 = library's choice.  Partitions are merged with the
 *                  log-sum-exp identity of the running max / sum recurrence
 *                  (a second kernel, enqueued by the same call).
 *   seq_order    : host, [num_seqs] int32, may be NULL: the order in which
 *                  the sequences' workgroups are dispatched (a permutation
 *                  of 0 .. num_seqs-1, else PKV_ERR_INVALID).  A hint only:
 *                  outputs are identical for every order.  Longest first
 *                  keeps long sequences from running on alone at the end.
 *                  Used for batches of at most 256 sequences (it travels in
 *                  the kernel arguments), ignored above.
 *   workspace    : device, at least pkv_decode_workspace_size(...) bytes,
 *                  16-byte aligned, owned by the caller (may be NULL when
 *                  that size is 0).  Its contents on entry do not matter and
 *                  nothing in it survives a call; calls that share a
 *                  workspace must not run concurrently.
 * Up to 8 query heads that share a KV head are served by one workgroup, so
 * each K/V row is read once for all of them (16 when 16 divide the group
 * and block_size >= 8).  With 4 or more query heads per KV head (a multiple
 * of 4) and block_size >= 8, the scores and the weighted
 * sum run as fp16 matrix-core products with fp32 accumulation; the weights
 * enter them as an fp16 high part plus an fp16 low part, so the result
 * keeps fp32-level accuracy.
 */
int pkv_paged_attention_decode(float *out, const void *q, const void *k_cache,
                               const void *v_cache,
                               const int32_t *block_tables,
                               const int32_t *seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_seq_len, float scale,
                               int32_t partition_size, const int32_t *seq_order,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * The decode above for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels
 * and results.  Split partials go to a device array of the library,
 * PKV_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends; the call itself allocates nothing.
 *   Returns PKV_ERR_SCRATCH, before enqueueing anything, when the partials
 *   of the call (pkv_decode_workspace_size of its arguments) exceed that
 *   size; otherwise as pkv_paged_attention_decode.
 *   Every call on one GPU shares that GPU's array: calls that may overlap
 *   on one GPU (different streams, or different host threads) race and
 *   must be ordered by the caller.  Nothing in the array needs to start at
 *   zero: each call writes the partials it reads.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int pkv_paged_attention_decode_noalloc(float *out, const void *q, const void *k_cache,
                                       const void *v_cache,
                                       const int32_t *block_tables,
                                       const int32_t *seq_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, float scale,
                                       int32_t partition_size, const int32_t *seq_order,
                                       void *stream);

/*
 * Paged attention prefill of causal chunks whose prefix already sits in
 * paged blocks ("LLM 推理引擎 …", §4.3 Chunked Prefill and §1.1: the prompt
 * is processed in chunks; a chunk's query at absolute position p attends to
 * keys 0..p).  Chunk c owns query rows cu_q_lens[c] .. cu_q_lens[c+1]-1;
 * its sequence holds seq_lens[c] tokens including the chunk (already
 * appended with pkv_kv_append), so row j of the chunk sits at position
 * seq_lens[c] - chunk_len + j.  QK^T and PV run on MFMA (fp16 inputs, fp32
 * accumulation); the softmax weights enter PV as fp16.
 *
 *   out          : [total_q_tokens][num_q_heads][head_dim] float32, device
 *   q            : [total_q_tokens][num_q_heads][head_dim] fp16, device
 *   cu_q_lens    : [num_chunks + 1] int32, device, cu_q_lens[0] = 0,
 *                  non-decreasing, cu_q_lens[num_chunks] = total_q_tokens
 *   block_tables : [num_chunks][max_blocks_per_seq] int32, device
 *   seq_lens     : [num_chunks] int32, device, chunk_len <= seq_len
 *   max_q_len    : host-side upper bound of the chunk lengths (rows past
 *                  it are not computed)
 *   max_seq_len  : host-side upper bound of seq_lens, at most
 *                  max_blocks_per_seq * block_size; a chunk whose seq_len
 *                  exceeds it gets NaN rows
 *   scale        : as for the decode
 *   workspace    : device scratch of at least pkv_prefill_workspace_size()
 *                  bytes, 16-byte aligned (may be NULL when that size is 0).
 *                  When the grid of query tiles is small, a query tile's key
 *                  range is cut into parts run by different workgroups; the
 *                  parts leave partial outputs here and a second kernel
 *                  combines them.  Contents on entry do not matter; calls
 *                  sharing one workspace must be ordered (same stream).
 * Errors: PKV_ERR_INVALID for bad sizes, misaligned pointers or a missing
 * or short workspace; PKV_ERR_UNSUPPORTED for head_dim / block_size without
 * an instance.
 */
size_t pkv_prefill_workspace_size(int32_t num_chunks, int32_t total_q_tokens,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  int32_t head_dim, int32_t max_seq_len);
int pkv_paged_attention_prefill(float *out, const void *q,
                                const int32_t *cu_q_lens, const void *k_cache,
                                const void *v_cache,
                                const int32_t *block_tables,
                                const int32_t *seq_lens, int32_t num_chunks,
                                int32_t total_q_tokens, int32_t max_q_len,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Host-side checks of the preconditions above that the kernels cannot check
 * without a synchronisation (plain host code; all pointers are host
 * pointers, read only).  They follow the cache layout of "LLM 推理引擎 …":
 * §3.2 (a token's place is slot / block_size, slot % block_size, one token
 * per place), §3.3 (every logical block below seq_len maps to a physical
 * block of the pool) and §4.3 (a chunk ends its sequence).  Each returns
 * PKV_OK, or PKV_ERR_INVALID with *bad_index (may be NULL) set to the first
 * offending entry, or to -1 when the sizes themselves are invalid.
 *
 * pkv_validate_slots  : every slot >= 0 lies below num_blocks * block_size
 *                       and no two rows share one; negative slots are
 *                       padding.  bad_index = the row (for a shared slot,
 *                       the later of the two rows).
 * pkv_validate_tables : 1 <= seq_lens[s] <= max_blocks_per_seq * block_size
 *                       and the first ceil(seq_lens[s] / block_size) entries
 *                       of row s lie in [0, num_blocks).  bad_index =
 *                       s * max_blocks_per_seq + j (j = 0 for a bad length).
 * pkv_validate_chunks : cu_q_lens[0] = 0, 0 <= chunk_len <= seq_lens[c],
 *                       cu_q_lens[num_chunks] = total_q_tokens.  bad_index =
 *                       the chunk (num_chunks for a wrong total).
 */
int pkv_validate_slots(const int32_t *slot_mapping, int32_t num_tokens,
                       int32_t num_blocks, int32_t block_size, int64_t *bad_index);
int pkv_validate_tables(const int32_t *block_tables, const int32_t *seq_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq,
                        int32_t num_blocks, int32_t block_size, int64_t *bad_index);
int pkv_validate_chunks(const int32_t *cu_q_lens, const int32_t *seq_lens,
                        int32_t num_chunks, int32_t total_q_tokens, int64_t *bad_index);

/*
 * Host-side block manager (plain host code, no device calls, not
 * thread-safe): the free list and per-request block tables that produce the
 * block_tables / seq_lens / slot_mapping arguments above ("LLM 推理引擎 …",
 * §3.2 BlockManager: the free list starts as block ids 0 .. N-1 and blocks
 * are taken from its end; a request of n tokens takes ceil(n / block_size)
 * blocks or, when too few are free, none; a new token goes into the last
 * block while it has room, otherwise into a newly taken block; freed blocks
 * are appended to the free list.  §4.1: a shared prefix is whole blocks
 * referenced by several tables, returned to the free list when the last
 * reference goes).  Request ids are caller-chosen 64-bit integers.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* NULL when the arguments are invalid or memory runs out. */
pkv_block_manager *pkv_bm_create(int32_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_block_manager *bm);
/* Free blocks, or -1 for a NULL manager. */
int32_t pkv_bm_num_free(const pkv_block_manager *bm);
/* The block size the manager was created with; -1 for NULL. */
int32_t pkv_bm_block_size(const pkv_block_manager *bm);
/* A new request holding num_tokens tokens (e.g. a prompt to prefill).
 * PKV_ERR_INVALID if the id exists; PKV_ERR_NO_BLOCKS (nothing taken) if
 * fewer than ceil(num_tokens / block_size) blocks are free. */
int pkv_bm_allocate(pkv_block_manager *bm, int64_t request_id, int32_t num_tokens);
/* Adds one token to a request; *slot = block * block_size + offset of the
 * new token.  PKV_ERR_NO_BLOCKS (no change) if a block is needed and none
 * is free. */
int pkv_bm_append_token(pkv_block_manager *bm, int64_t request_id, int32_t *slot);
/* One token for each of count distinct requests (a decode step's
 * slot_mapping); all or nothing. */
int pkv_bm_append_tokens(pkv_block_manager *bm, const int64_t *request_ids,
                         int32_t count, int32_t *slots);
/* A new request whose table starts with the parent's blocks that lie wholly
 * inside its first prefix_tokens tokens (shared, reference-counted); it
 * holds those blocks' tokens. */
int pkv_bm_fork(pkv_block_manager *bm, int64_t parent_id, int64_t child_id,
                int32_t prefix_tokens);
/* Drops a request; blocks no other table references return to the free list. */
int pkv_bm_free(pkv_block_manager *bm, int64_t request_id);
/* Tokens held by a request, or -1 if unknown. */
int32_t pkv_bm_seq_len(const pkv_block_manager *bm, int64_t request_id);
/* Copies up to capacity block ids of a request (host memory); returns the
 * table's length, or -1 if unknown. */
int32_t pkv_bm_block_table(const pkv_block_manager *bm, int64_t request_id,
                           int32_t *blocks, int32_t capacity);
/* Host arrays for the kernels: block_tables [count][max_blocks_per_seq]
 * (unused entries = pad_block) and seq_lens [count]. */
int pkv_bm_build_tables(const pkv_block_manager *bm, const int64_t *request_ids,
                        int32_t count, int32_t max_blocks_per_seq,
                        int32_t pad_block, int32_t *block_tables,
                        int32_t *seq_lens);
/* Slots of positions first_pos .. first_pos+count-1 of a request (which
 * must already hold them), e.g. the slot_mapping of a prompt's prefill. */
int pkv_bm_slots(const pkv_block_manager *bm, int64_t request_id,
                 int32_t first_pos, int32_t count, int32_t *slots);
/* Moves a request from one manager to another ("LLM 推理引擎 …", §4.4 Swap:
 * a preempted request's KV goes from GPU blocks to CPU blocks and later
 * back).  The target takes ceil(len / block_size) blocks for the request's
 * tokens (its length carries over), the source releases the request's
 * blocks (a block shared with another request stays held by it).
 * src_blocks[i] -> dst_blocks[i], i < *count, is the copy the caller must
 * enqueue (pkv_copy_blocks / pkv_copy_blocks_dma) before anything reuses the
 * released source blocks.  Both managers must have the same block_size;
 * capacity must cover the request's block count.  PKV_ERR_NO_BLOCKS (and
 * nothing changed) when the target has too few free blocks. */
int pkv_bm_swap(pkv_block_manager *from, pkv_block_manager *to, int64_t request_id,
                int32_t *src_blocks, int32_t *dst_blocks, int32_t capacity,
                int32_t *count);

/*
 * Iteration-level scheduler (continuous batching) over a block manager
 * ("LLM 推理引擎 …", §2.2 ContinuousBatchingScheduler, §4.3 Chunked
 * Prefill, §5.4 Preemption; plain host code, not thread-safe).  Each call of
 * pkv_sched_step closes the previous step (its prefill chunks and decode
 * tokens count as written) and plans the next one:
 *   1. requests that have written their prompt and run max_new_tokens
 *      decode steps finish and free their blocks;
 *   2. waiting requests are admitted in arrival order while fewer than
 *      max_batch_size run and ceil(prompt / block_size) blocks can be taken
 *      (the first that does not fit stays at the head);
 *   3. while the decode rows of the step need more new blocks than are
 *      free, the most recently admitted running request is preempted: its
 *      blocks are freed, it goes back to the head of the waiting queue and
 *      its generated tokens join its prompt (recomputed on readmission);
 *   4. the batch: prompt chunks of the running requests still prefilling,
 *      in admission order, within max_num_tokens new tokens (a prompt that
 *      does not fit the rest of the budget is cut, its remainder comes next
 *      step), then one decode row per request that has written its prompt,
 *      while the batch has fewer than max_batch_size rows.
 * The plan's arrays are the kernels' inputs: cu_q_lens / prefill_tables /
 * prefill_lens (seq_len = the prompt tokens written so far plus this chunk)
 * for pkv_paged_attention_prefill; decode_tables / decode_lens for
 * pkv_paged_attention_decode; slot_mapping (the chunks' positions in
 * cu_q_lens order, then one new slot per decode row) for pkv_kv_append.
 * Capacities the caller provides: max_batch_size rows (ids, lens,
 * cu_q_lens + 1), max_batch_size * max_blocks_per_seq table entries,
 * max_num_tokens + max_batch_size slots, max_batch_size finished and
 * preempted ids (those two may be NULL).  max_blocks_per_seq * block_size
 * must cover max_seq_len, and a request's prompt plus max_new_tokens must
 * not exceed max_seq_len (checked when it is added).
 */
typedef struct pkv_scheduler pkv_scheduler;
typedef struct {
  int32_t num_prefill;        /* prefill rows (chunks) */
  int32_t num_prefill_tokens; /* their new tokens = cu_q_lens[num_prefill] */
  int32_t num_decode;         /* decode rows */
  int32_t num_new_tokens;     /* slot_mapping entries */
  int32_t num_finished;       /* requests that finished at this boundary */
  int32_t num_preempted;      /* requests preempted by this step */
} pkv_step_plan;
pkv_scheduler *pkv_sched_create(pkv_block_manager *bm, int32_t max_batch_size,
                                int32_t max_num_tokens, int32_t max_seq_len);
void pkv_sched_destroy(pkv_scheduler *s);
int pkv_sched_add_request(pkv_scheduler *s, int64_t request_id, int32_t prompt_len,
                          int32_t max_new_tokens);
int32_t pkv_sched_num_waiting(const pkv_scheduler *s);
int32_t pkv_sched_num_running(const pkv_scheduler *s);
int pkv_sched_step(pkv_scheduler *s, int32_t max_blocks_per_seq, int32_t pad_block,
                   pkv_step_plan *plan, int64_t *prefill_ids, int32_t *cu_q_lens,
                   int32_t *prefill_tables, int32_t *prefill_lens, int64_t *decode_ids,
                   int32_t *decode_tables, int32_t *decode_lens, int32_t *slot_mapping,
                   int64_t *finished_ids, int64_t *preempted_ids);

/*
 * Native step executor over a scheduler (continuous batching, "LLM 推理引擎
 * …", §2.2: each forward step runs the recomposed batch, prefill chunks and
 * decode rows together).  pkv_server_create allocates, once: two pinned
 * staging buffers and two device copies of a step's plan, the attention
 * workspace for max_batch_size rows of up to max_seq_len tokens, and a
 * copy stream of its own (default priority).  max_batch_size,
 * max_num_tokens and max_seq_len must equal the scheduler's; the pools are
 * the caller's device buffers ([num_blocks][Hkv][bs][D] fp16, bs = the
 * block manager's).  NULL on invalid arguments or a failed allocation.
 *   pkv_server_plan: runs pkv_sched_step into the staging buffer not used
 *     by the previous step (after waiting for its copy of two steps ago)
 *     and enqueues its host-to-device copy on the copy stream, after the
 *     kernels of the step that last read that device buffer; `stream` is
 *     not used.
 *   pkv_server_plan_arrays: host views of the last plan's request ids,
 *     cu_q_lens, prefill_lens, decode_lens, finished and preempted ids
 *     (valid until the next plan), for the caller to produce the step's rows.
 *   pkv_server_execute: makes `stream` wait for the plan's copy, then
 *     enqueues on it the kv append of the plan's new rows, the prefill of
 *     its chunks and the decode of its decode rows.  new_k / new_v [num_new_tokens][Hkv][D] and q
 *     [num_new_tokens][Hq][D] fp16, device, in slot_mapping order (the
 *     chunks' tokens, then one row per decode request); out_prefill
 *     [num_prefill_tokens][Hq][D] and out_decode [num_decode][Hq][D] fp32,
 *     device (may be NULL when the step has no such rows).
 * Use one stream for all calls of a server.
 */
typedef struct pkv_server pkv_server;
pkv_server *pkv_server_create(pkv_scheduler *sched, pkv_block_manager *bm, void *k_cache,
                              void *v_cache, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_blocks, int32_t pad_block,
                              int32_t max_batch_size, int32_t max_num_tokens,
                              int32_t max_seq_len, float scale);
void pkv_server_destroy(pkv_server *s);
int pkv_server_plan(pkv_server *s, pkv_step_plan *plan, void *stream);
int pkv_server_plan_arrays(const pkv_server *s, const int64_t **prefill_ids,
                           const int32_t **cu_q_lens, const int32_t **prefill_lens,
                           const int64_t **decode_ids, const int32_t **decode_lens,
                           const int64_t **finished_ids, const int64_t **preempted_ids);
int pkv_server_execute(pkv_server *s, const void *new_k, const void *new_v, const void *q,
                       float *out_prefill, float *out_decode, void *stream);

/*
 * Block copies between two KV pools ("LLM 推理引擎 …", §4.4 Swap: the
 * device-to-host copy of a swapped-out request's blocks and the
 * host-to-device copy that brings it back).  For i < count, block
 * src_blocks[i] of (src_k, src_v) is copied, bit for bit, to block
 * dst_blocks[i] of (dst_k, dst_v); a block is num_kv_heads * block_size *
 * head_dim fp16 of K and as many of V, contiguous in either pool (the cache
 * layout above).  A pool is device memory or pinned host memory (allocated
 * pinned, e.g. hipHostMalloc; a pool in pinned host memory is read and
 * written over the host link).  Ownership stays with the caller.
 * Destination blocks must be distinct and must not be source blocks of the
 * same call in the same pool (such copies race).
 *
 * pkv_copy_blocks: one kernel launch; src_blocks / dst_blocks are device or
 * pinned host arrays, read by the kernel; a pair with an id outside its
 * pool is skipped.  Pageable host memory anywhere -> PKV_ERR_INVALID.
 * pkv_copy_blocks_dma: src_blocks / dst_blocks are host arrays read before
 * return; runs of blocks consecutive on both sides become one
 * hipMemcpyAsync each for K and for V (the DMA engines); any id outside its
 * pool -> PKV_ERR_INVALID before anything is enqueued.
 * Both: head_dim a multiple of 8, 16-byte aligned pools (kernel path).
 */
int pkv_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                    const int32_t *src_blocks, const int32_t *dst_blocks,
                    int32_t count, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t src_num_blocks,
                    int32_t dst_num_blocks, void *stream);
int pkv_copy_blocks_dma(const void *src_k, const void *src_v, void *dst_k,
                        void *dst_v, const int32_t *src_blocks,
                        const int32_t *dst_blocks, int32_t count,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t src_num_blocks, int32_t dst_num_blocks,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
