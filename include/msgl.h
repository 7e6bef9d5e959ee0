/*
 * msgl.h - C ABI of the paged-KV attention step for AMD Instinct MI355X (gfx950).
 *
 * One transformer layer's attention step as the Mini-SGLang engine runs it:
 * the new tokens' K/V are written into a paged KV pool at out_loc, then every
 * request attends (causal, grouped-query) over its history, gathered through
 * its page-table row.  Sources: "mini-sglang from Scratch, Engine and sampler"
 * (sections on initialisation order and the hand-driven engine), "Stage 4
 * milestone" (section 'What it prints' and the table 'What each chapter
 * adds'), and the Mini-SGLang Engine article's per-layer pipeline (the KV
 * write precedes attention).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers named *_pool, q, q_out, out, lse, k_new, v_new, page_table, table_idx,
 * seq_lens, cached_lens, cu_q, positions, out_loc, weight, ids, group_start,
 * prefix_lens, workspace, result and seen are DEVICE pointers owned
 * by the caller; the library never frees or retains them (except a captured
 * graph, which records them; see msgl_decode_graph_create).  `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).  Calls only enqueue
 * work: they never allocate device memory, never synchronise with the host
 * and never copy between host and device, so they may be recorded into a HIP
 * graph.  Device faults therefore surface at the caller's next synchronisation.
 *
 * Layouts:
 *   k_pool, v_pool  [num_slots, kv_heads, head_dim], contiguous; the engine's
 *                   per-layer pool (num_pages + 1, page_size, kv_heads,
 *                   head_dim) flattened, slot = page * page_size + offset;
 *                   the last page belongs to the dummy request.
 *   page_table      int32 [rows, row_stride] row-major; entry [r, j] is the
 *                   slot of token j of the request in row r (token-level slot
 *                   ids at every page size).
 *   q, out          [tokens, q_heads, head_dim]; k_new, v_new [tokens,
 *                   kv_heads, head_dim]; all contiguous.
 *   lse             float32 [tokens, q_heads], natural-log log-sum-exp of the
 *                   scaled logits; optional (NULL skips it).
 *   dtype           storage type of q, pools, new rows and out; accumulation
 *                   is always float32.
 * Grouped-query mapping: q head h reads kv head h / (q_heads / kv_heads).
 * Causal mask: the query at position p sees keys 0..p.
 *
 * Preconditions on device-array contents are not checked by the compute calls
 * (checking them would need a host synchronisation); msgl_validate_batch
 * checks host copies, and msgl_check_batch checks the device arrays
 * themselves, asynchronously, into a device result (a debug step that can run
 * or be captured before the attention calls).  Only host scalars and pointer
 * presence are validated;
 * a bad value returns a status and enqueues nothing.  The kernels clamp the
 * slot ids and lengths they read into range, but table_idx is a pure
 * precondition (0 <= table_idx[b] < the page table's rows, a count the
 * attention calls do not receive): an id out of range reads outside the
 * page table.
 *
 * Supported: dtype F32 or BF16; head_dim 64 or 128; q_heads / kv_heads in
 * {1, 2, 4, 8}; kv_heads <= 64; page_size >= 1.  Others return
 * MSGL_UNSUPPORTED.  Thread-safety: calls may be made from several threads;
 * msgl_last_error is per thread.
 */
#ifndef MSGL_H
#define MSGL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSGL_OK = 0,
    MSGL_INVALID_ARG = 1,          /* NULL pointer, negative size, inconsistent scalars */
    MSGL_UNSUPPORTED = 2,          /* valid but not implemented (dtype, head_dim, group) */
    MSGL_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the *_workspace_bytes query */
    MSGL_HIP_ERROR = 4             /* a HIP runtime call or launch failed */
} msgl_status;

typedef enum { MSGL_F32 = 0, MSGL_BF16 = 1 } msgl_dtype;

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *msgl_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int msgl_version(void);

/*
 * msgl_store_kv - write the step's new K/V rows into the pools.
 * For t in [0, num_tokens): k_pool[out_loc[t]] = k_new[t] and
 * v_pool[out_loc[t]] = v_new[t], each a [kv_heads, head_dim] row, copied bit
 * for bit.  This is the KV-write custom kernel of the Stage 4 milestone's
 * table; it runs before attention in the layer.
 * out_loc entries must lie in [0, num_slots) and be distinct, except the
 * dummy request's slot, which padded rows may share (its contents are then
 * unspecified).  num_tokens == 0 is a no-op.
 */
msgl_status msgl_store_kv(void *k_pool, void *v_pool, int64_t num_slots, int32_t kv_heads,
                          int32_t head_dim, msgl_dtype dtype, const void *k_new,
                          const void *v_new, const int32_t *out_loc, int32_t num_tokens,
                          void *stream);

/*
 * msgl_rope_store_kv - rotary position embedding of the new q and k rows,
 * fused with the KV write (the layer's RoPE and KV-write steps, in that
 * order, from the Mini-SGLang Engine article's per-layer pipeline).
 * For every new token t at position p = positions[t] and every head, element
 * i < head_dim/2 pairs with element i + head_dim/2 and the pair turns by
 * a_i = p * rope_base^(-2 i / head_dim) (RoFormer, section 3.2, general form,
 * half-split pairing as in the GPT-NeoX and Qwen models):
 *   y[i] = x[i] cos a_i - x[i + d/2] sin a_i,
 *   y[i + d/2] = x[i + d/2] cos a_i + x[i] sin a_i.
 * Writes q_out[t] = rotated q[t] ([q_heads, head_dim] per token; q_out may
 * equal q for an in-place update), k_pool[out_loc[t]] = rotated k_new[t], and
 * v_pool[out_loc[t]] = v_new[t] bit for bit.  k_new is not modified.  The
 * angles are computed in double precision and the rotation in float32, then
 * rounded once (round to nearest even) to the storage type.
 * positions[t] is normally cached_len + i for the request's i-th new token.
 * out_loc follows msgl_store_kv's rules; a token whose out_loc lies outside
 * [0, num_slots) still has its q rotated but writes no pool row.
 * rope_base must be positive and finite (Qwen3 uses 1e6).  q_heads in
 * [1, 256]; kv_heads, head_dim and dtype as for msgl_store_kv.
 * num_tokens == 0 is a no-op.
 */
msgl_status msgl_rope_store_kv(void *q_out, const void *q, void *k_pool, void *v_pool,
                               int64_t num_slots, int32_t q_heads, int32_t kv_heads,
                               int32_t head_dim, msgl_dtype dtype, const void *k_new,
                               const void *v_new, const int32_t *positions, const int32_t *out_loc,
                               int32_t num_tokens, double rope_base, void *stream);

/*
 * msgl_vocab_embed - vocabulary indexing: the embedding rows of the step's
 * token ids (the small custom kernel the Stage 4 milestone's table names next
 * to the KV write).  `weight` [vocab_rows, hidden] holds the rows of the
 * vocabulary ids vocab_start .. vocab_start + vocab_rows - 1 (one rank's
 * shard under tensor parallelism; vocab_start 0 and the whole table on one
 * GPU).  For t in [0, num_tokens): out[t] = weight[ids[t] - vocab_start],
 * copied bit for bit, when the id lies in the shard, else a row of zeros, so
 * the ranks' outputs sum to the full table's rows.  out is [num_tokens,
 * hidden].  hidden * element size must be a multiple of 16 bytes (else
 * MSGL_UNSUPPORTED); vocab_rows >= 1 and vocab_start >= 0 (else
 * MSGL_INVALID_ARG).  Any int32 id is allowed.  num_tokens == 0 is a no-op.
 */
msgl_status msgl_vocab_embed(void *out, const void *weight, int64_t vocab_start, int64_t vocab_rows,
                             int32_t hidden, msgl_dtype dtype, const int32_t *ids, int32_t num_tokens,
                             void *stream);

/*
 * Decode attention: one query token per request, at position seq_lens[b] - 1
 * (the token just written by msgl_store_kv, so a request attends to itself).
 * The keys of request b are page_table[table_idx[b], 0 .. seq_lens[b]-1].
 * Defined by: "mini-sglang from Scratch, Engine and sampler" (the page-table
 * section: one row per request holding each token's KV location; the
 * hand-driven decode step: positions cached_len .. device_len - 1 and out_loc
 * the row's entries there) and the Mini-SGLang tag page's KV-cache article
 * (section 1: the query of step t attends the keys and values of positions
 * 0..t) and Engine article (section 1: the KV write precedes attention).
 *
 * The key sequences of all requests, laid end to end (each request counted as
 * its keys plus a fixed cost of 32 key-equivalents, so runs of very short
 * requests spread out), are cut into equal contiguous shares, one per block of
 * a grid sized to the device; `chunk` (a multiple of 64; 0 picks the library
 * default, 64) is the least number of such units a share holds, so small
 * batches do not split below it.  The
 * pieces' partial softmax states are merged afterwards; the result does not
 * depend on the split beyond float32 rounding.  max_seq_len bounds every seq_lens[b]
 * and sizes the workspace; it may exceed the actual lengths (a graph captured
 * once serves any batch whose lengths stay within it).
 *
 * msgl_decode_workspace_bytes returns the workspace size for these scalars.
 * seq_lens[b] must lie in [1, min(max_seq_len, row_stride)].  Calls with
 * batch * (max_seq_len + 32) >= 2^31 return MSGL_UNSUPPORTED (the split
 * counts work units in 32 bits).
 */
size_t msgl_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t head_dim,
                                   int32_t max_seq_len, int32_t chunk);

msgl_status msgl_decode_attn(void *out, float *lse, const void *q, const void *k_pool,
                             const void *v_pool, int64_t num_slots, const int32_t *page_table,
                             int32_t row_stride, const int32_t *table_idx,
                             const int32_t *seq_lens, int32_t batch, int32_t q_heads,
                             int32_t kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t max_seq_len, int32_t chunk, float sm_scale,
                             msgl_dtype dtype, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * msgl_decode_attn_noalloc - msgl_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and result (the
 * same kernels) with no workspace argument.  The workspace is a fixed device
 * array of MSGL_NOALLOC_SCRATCH_BYTES inside the library, one per device,
 * set up at the first call on a device (its address is looked up once, with
 * that device current) and held until the process ends; the call itself
 * allocates nothing.  A call whose msgl_decode_workspace_bytes exceeds it
 * returns MSGL_WORKSPACE_TOO_SMALL and enqueues nothing: at head_dim 128 it
 * serves up to 944 requests with 32 q heads, 5983 with 16, none with 64.  `stream` must belong to the
 * current device (else MSGL_INVALID_ARG).  Every call on a device shares that
 * device's array: calls that overlap on one device (on different streams, or
 * from several threads without ordering) race and give wrong results.  Other
 * arguments and preconditions as for msgl_decode_attn.
 * msgl_noalloc_scratch_bytes returns MSGL_NOALLOC_SCRATCH_BYTES.
 */
#define MSGL_NOALLOC_SCRATCH_BYTES (80u << 20)

size_t msgl_noalloc_scratch_bytes(void);

msgl_status msgl_decode_attn_noalloc(void *out, float *lse, const void *q, const void *k_pool,
                                     const void *v_pool, int64_t num_slots, const int32_t *page_table,
                                     int32_t row_stride, const int32_t *table_idx,
                                     const int32_t *seq_lens, int32_t batch, int32_t q_heads,
                                     int32_t kv_heads, int32_t head_dim, int32_t page_size,
                                     int32_t max_seq_len, int32_t chunk, float sm_scale,
                                     msgl_dtype dtype, void *stream);

/*
 * Cascade decode over shared radix prefixes.  The requests of a group (batch
 * rows group_start[g] .. group_start[g+1]-1, consecutive) share the first
 * prefix_lens[b] keys of their page-table rows: the same slot ids, as the
 * radix prefix cache hands them out (Mini-SGLang's RadixPrefixCache; "Stage 4
 * milestone", table 'What each chapter adds').  The result is exactly the
 * decode attention of msgl_decode_attn (same out and lse, within float32
 * rounding); the shared keys' K/V rows are read once per group instead of
 * once per request.  The group's queries meet the shared keys on matrix cores
 * (split along the keys to fill the GPU); each request's own keys
 * prefix_lens[b] .. seq_lens[b]-1 go through the split-K decode; the partial
 * results are merged by the log-sum-exp rule.
 *
 * group_start [num_groups + 1] and prefix_lens [batch] are device arrays.
 * Preconditions (msgl_validate_shared_prefix checks host copies):
 * group_start[0] == 0, groups non-empty and increasing, at most
 * max_group_size requests each; prefix_lens equal within a group, in
 * [0, min(seq_len - 1, max_prefix_len)] (the new token is never shared), and
 * 0 for a request in no group; page-table entries 0 .. prefix_len-1 equal
 * across a group's rows.  num_groups <= min(batch, 1024); 0 <= max_prefix_len
 * < max_seq_len.  Other arguments as for msgl_decode_attn.  bf16 with
 * head_dim 128 only (else MSGL_UNSUPPORTED).  The workspace holds the decode
 * workspace plus float32 partial results; size it with
 * msgl_decode_shared_prefix_workspace_bytes.
 */
size_t msgl_decode_shared_prefix_workspace_bytes(int32_t batch, int32_t q_heads, int32_t head_dim,
                                                 int32_t max_seq_len, int32_t chunk);

msgl_status msgl_decode_attn_shared_prefix(void *out, float *lse, const void *q, const void *k_pool,
                                           const void *v_pool, int64_t num_slots, const int32_t *page_table,
                                           int32_t row_stride, const int32_t *table_idx,
                                           const int32_t *seq_lens, int32_t batch,
                                           const int32_t *group_start, const int32_t *prefix_lens,
                                           int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
                                           int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                           int32_t page_size, int32_t max_seq_len, int32_t chunk,
                                           float sm_scale, msgl_dtype dtype, void *workspace,
                                           size_t workspace_bytes, void *stream);

/*
 * Prefill / extend attention over a cached prefix (ragged batch).
 * Request b has seq_lens[b] tokens of which the first cached_lens[b] are
 * already in the pool from earlier steps; its new tokens are q rows
 * cu_q[b] .. cu_q[b+1]-1 at positions cached_lens[b] .. seq_lens[b]-1, and
 * each sees the keys at positions 0..its own position (the causal mask is
 * offset by the cached length).  Defined by: "mini-sglang from Scratch,
 * Engine and sampler" (the hand-driven prefill: positions from cached_len to
 * device_len, a batch of several requests concatenated), the Mini-SGLang tag
 * page's KV-cache article (section 1: the query at position t attends
 * positions 0..t; the radix prefix cache supplies the cached prefix) and its
 * scheduler article (chunked prefill: a request's prompt may arrive in
 * pieces on top of what is cached).  Requires
 * cu_q[b+1] - cu_q[b] == seq_lens[b] - cached_lens[b] >= 1, cu_q[0] == 0,
 * cu_q[batch] == total_q, and max_extend in [1, total_q] (the longest extend
 * length; the grid is sized from total_q, so an understated value changes
 * nothing).  bf16 runs on matrix cores (MFMA); fp32 runs on the vector ALUs.
 * The prefill call needs no workspace.
 */
msgl_status msgl_prefill_attn(void *out, float *lse, const void *q, const void *k_pool,
                              const void *v_pool, int64_t num_slots, const int32_t *page_table,
                              int32_t row_stride, const int32_t *table_idx,
                              const int32_t *seq_lens, const int32_t *cached_lens,
                              const int32_t *cu_q, int32_t batch, int32_t total_q,
                              int32_t max_extend, int32_t q_heads, int32_t kv_heads,
                              int32_t head_dim, int32_t page_size, float sm_scale,
                              msgl_dtype dtype, void *stream);

/*
 * Host plan / run split of the prefill call, after the plan and run steps of
 * the FlashInfer attention backend ("Stage 4 milestone": the table 'What each
 * chapter adds' and the stage checkpoint, which asks what each step does): the
 * block list that msgl_prefill_attn derives on the device from the lengths
 * (every (request, query block) pair, the most key tiles first, ties in
 * request order, one launch block per entry and kv head) is made on the host
 * instead, from host copies of the batch metadata, before the step.  The run
 * reads its work item from that list, so no block enumerates the batch, and
 * the batch may exceed the 1024 requests the device enumeration serves on the
 * matrix-core path.  The results equal msgl_prefill_attn's bit for bit.
 * bf16 and head_dim 128 only (else MSGL_UNSUPPORTED).
 *
 * msgl_prefill_plan_bytes: the plan buffer size that suffices for any batch of
 * these sizes (0 for invalid sizes).
 *
 * msgl_prefill_plan: every pointer is HOST memory.  seq_lens, cached_lens,
 * table_idx [batch] and cu_q [batch + 1] mean what they mean in
 * msgl_prefill_attn; rows is the page table's row count.  Checks the batch
 * (cu_q[0] == 0, cu_q[batch] == total_q, cu_q[b+1] - cu_q[b] >= 1 ==
 * seq_lens[b] - cached_lens[b], cached_lens[b] >= 0, seq_lens[b] <= row_stride,
 * 0 <= table_idx[b] < rows) and writes the plan: a header of 8 int32 (a magic
 * number, the layout, query tokens per block, the entry count, batch, total_q,
 * q_heads, kv_heads), then 8 int32 per entry (request, query block, new tokens,
 * cached tokens, first q row, table row, key tiles, 0).  MSGL_INVALID_ARG on a
 * malformed batch, MSGL_WORKSPACE_TOO_SMALL when plan_bytes is short; nothing
 * is written on error except possibly the buffer's contents.
 *
 * msgl_prefill_attn_planned: plan_host is the plan as written (read on the
 * host for the launch size and layout); plan_dev a device copy of the same
 * bytes that the kernels read, which must stay unchanged until the launch has
 * run.  The plan's heads must equal q_heads and kv_heads.  The other arguments
 * are those of msgl_prefill_attn; the device arrays of the batch (seq_lens,
 * cached_lens, cu_q, table_idx) are not needed: the plan carries them.
 */
size_t msgl_prefill_plan_bytes(int32_t batch, int32_t total_q, int32_t q_heads, int32_t kv_heads);

msgl_status msgl_prefill_plan(int32_t *plan, size_t plan_bytes, const int32_t *seq_lens,
                              const int32_t *cached_lens, const int32_t *cu_q,
                              const int32_t *table_idx, int32_t batch, int32_t total_q,
                              int32_t rows, int32_t row_stride, int32_t q_heads, int32_t kv_heads,
                              int32_t head_dim, msgl_dtype dtype);

msgl_status msgl_prefill_attn_planned(void *out, float *lse, const void *q, const void *k_pool,
                                      const void *v_pool, int64_t num_slots,
                                      const int32_t *page_table, int32_t row_stride,
                                      int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                      int32_t page_size, float sm_scale, msgl_dtype dtype,
                                      const int32_t *plan_host, const int32_t *plan_dev,
                                      size_t plan_bytes, void *stream);

/*
 * Decode step as a captured HIP graph (the KV write, then decode attention),
 * for one padded batch size, after the CUDA-Graph runner of the Stage 4 milestone:
 * every input lives in a fixed buffer whose address is recorded at capture;
 * before each replay the caller writes the step's values into those buffers
 * (rows beyond the real batch use the dummy request: seq_len 1, table row =
 * the dummy row, out_loc = the dummy slot) and launches.  The buffers must
 * stay allocated, at the same addresses, for the graph's lifetime.
 * `stream` must not be the null stream (capture needs a real stream).
 * Arguments mean what they mean in msgl_store_kv and msgl_decode_attn with
 * num_tokens == batch == padded_batch.  In the graph the KV write rides in the
 * decode kernel: the wave that reads a request's last key (its new token,
 * out_loc[b] == page_table[table_idx[b], seq_lens[b] - 1]) writes that row
 * first, so a replay runs two kernels instead of three.
 */
typedef struct msgl_graph msgl_graph;

msgl_status msgl_decode_graph_create(msgl_graph **graph, void *k_pool, void *v_pool,
                                     int64_t num_slots, const void *k_new, const void *v_new,
                                     const int32_t *out_loc, void *out, float *lse,
                                     const void *q, const int32_t *page_table,
                                     int32_t row_stride, const int32_t *table_idx,
                                     const int32_t *seq_lens, int32_t padded_batch,
                                     int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t max_seq_len, int32_t chunk,
                                     float sm_scale, msgl_dtype dtype, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Enqueue one replay of the captured step on `stream`. */
msgl_status msgl_graph_launch(msgl_graph *graph, void *stream);

/* Release the graph (NULL is ignored).  Does not touch the recorded buffers. */
void msgl_graph_destroy(msgl_graph *graph);

/*
 * msgl_validate_batch - check a batch's metadata on HOST copies (no GPU use).
 * Checks, for b < batch: 0 <= table_idx[b] < rows; 1 <= seq_lens[b] <=
 * min(max_seq_len, row_stride); 0 <= cached_lens[b] < seq_lens[b]; when cu_q
 * is given, cu_q[0] == 0 and cu_q[b+1] - cu_q[b] == seq_lens[b] - cached_lens[b];
 * every page-table entry a request uses lies in [0, num_slots); when
 * page_size > 1, the entries of each page are consecutive and the page's
 * first entry is a multiple of page_size; when out_loc is given (num_tokens
 * entries), it lists page_table[table_idx[b], cached_lens[b] .. seq_lens[b]-1]
 * for b in order (one entry per new token; the captured decode step relies on
 * it), its entries lie in [0, num_slots) and no slot other than `dummy_slot`
 * repeats (pass -1 to allow no repeats).
 * cached_lens and cu_q may be NULL (decode: cached = seq_len - 1).
 * Returns MSGL_OK or MSGL_INVALID_ARG with the first violation in
 * msgl_last_error.
 */
msgl_status msgl_validate_batch(const int32_t *page_table, int32_t rows, int32_t row_stride,
                                const int32_t *table_idx, const int32_t *seq_lens,
                                const int32_t *cached_lens, const int32_t *cu_q, int32_t batch,
                                int32_t max_seq_len, int64_t num_slots, int32_t page_size,
                                const int32_t *out_loc, int32_t num_tokens, int64_t dummy_slot);

/*
 * msgl_check_batch - the checks of msgl_validate_batch, run on the DEVICE
 * arrays as kernels on `stream`: no host copy, no allocation, no
 * synchronisation, so a debug build of an engine can run (or capture) it right
 * before its attention calls.  The invariants are those of the engine's
 * per-batch metadata (Mini-SGLang tag page, Engine article, the metadata
 * step: keys page_table[table_idx[b], 0 .. seq_lens[b]-1], new tokens the
 * entries from cached_lens[b] on, out_loc listing them in request order;
 * KV-cache article: pages of page_size consecutive slots).
 * Arguments as for msgl_validate_batch, all arrays in device memory, plus:
 *   result  device int32 [4], written by the call: [0] the OR of the
 *           MSGL_CHECK_* codes found (0: none), [1] the number of requests
 *           with a violation, [2] the first such request, [3] the first new
 *           token whose out_loc entry fails (INT32_MAX when none);
 *   seen    NULL, or device uint32 scratch of ceil(num_slots / 32) words for
 *           the repeat check of out_loc (cleared by the call; NULL skips it).
 * out_loc with cached_lens needs cu_q (the new tokens' offsets); without
 * cached_lens (decode) out_loc must have batch entries, one per request.
 * Every kernel read stays in bounds whatever the metadata hold.  The result is
 * ready when the stream reaches it; a call that overlaps another one sharing
 * `result` or `seen` races with it.  Returns MSGL_INVALID_ARG for NULL
 * required pointers or bad scalars, MSGL_UNSUPPORTED for num_slots >= 2^31.
 */
#define MSGL_CHECK_TABLE_IDX 1     /* table_idx[b] outside [0, rows) */
#define MSGL_CHECK_SEQ_LEN 2       /* seq_lens[b] outside [1, min(max_seq_len, row_stride)] */
#define MSGL_CHECK_CACHED_LEN 4    /* cached_lens[b] outside [0, seq_lens[b]) */
#define MSGL_CHECK_CU_Q 8          /* cu_q[0] != 0, or cu_q[b+1] - cu_q[b] != seq_lens[b] - cached_lens[b] */
#define MSGL_CHECK_SLOT 16         /* a page-table entry the request uses outside [0, num_slots) */
#define MSGL_CHECK_PAGE 32         /* page_size > 1: a page not made of consecutive slots from a multiple of page_size */
#define MSGL_CHECK_OUT_LOC 64      /* out_loc[t] outside [0, num_slots) or not page_table[row, position] */
#define MSGL_CHECK_REPEAT 128      /* out_loc repeats a slot other than dummy_slot */
#define MSGL_CHECK_TOKEN_COUNT 256 /* cu_q[batch] != num_tokens, or a new token indexed outside out_loc */
msgl_status msgl_check_batch(const int32_t *page_table, int32_t rows, int32_t row_stride,
                             const int32_t *table_idx, const int32_t *seq_lens, const int32_t *cached_lens,
                             const int32_t *cu_q, int32_t batch, int32_t max_seq_len, int64_t num_slots,
                             int32_t page_size, const int32_t *out_loc, int32_t num_tokens, int64_t dummy_slot,
                             int32_t *result, uint32_t *seen, void *stream);

/*
 * msgl_validate_shared_prefix - check the group metadata of
 * msgl_decode_attn_shared_prefix on HOST copies (the preconditions listed
 * there).  Returns MSGL_OK or MSGL_INVALID_ARG with the first violation in
 * msgl_last_error.
 */
msgl_status msgl_validate_shared_prefix(const int32_t *page_table, int32_t rows, int32_t row_stride,
                                        const int32_t *table_idx, const int32_t *seq_lens, int32_t batch,
                                        const int32_t *group_start, const int32_t *prefix_lens,
                                        int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len);

#ifdef __cplusplus
}
#endif

#endif /* MSGL_H */
