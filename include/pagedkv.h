/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV-cache attention library.
 *
 * What the library computes, and where the pages describe it:
 *
 *  - KV cache in fixed-size blocks of 16 tokens held in one physical pool and
 *    reached through a per-sequence block table ("vLLM — PagedAttention and
 *    Continuous Batching", §2.2; "vLLM and PagedAttention", §2, block-table figure
 *    and bullets; "How vLLM Works?", section 03).
 *  - Cache tensor layout [num_blocks, block_size, num_kv_heads, head_dim], the
 *    layout of the simplified kernel sketch in "vLLM and PagedAttention", §2, with
 *    its head count read as the number of KV heads.  A block is therefore one
 *    contiguous slab and one token's K (or V) row is one contiguous
 *    num_kv_heads*head_dim vector.
 *  - Decode attention that walks the table block by block and accumulates the
 *    per-block results ("vLLM and PagedAttention", §2 "Reworking the Attention
 *    Computation"; "vLLM — PagedAttention and Continuous Batching", §2.4).
 *  - Copy-on-write sharing of prefix blocks ("vLLM and PagedAttention", §2 bullets;
 *    "How vLLM Works?", section 03), automatic prefix caching ("How vLLM
 *    Works?", section 05), chunked prefill batched with decode ("How vLLM
 *    Works?", section 04), preemption by swapping blocks to host memory ("vLLM
 *    and PagedAttention", §3), and a decode step captured as one graph ("vLLM
 *    and PagedAttention", §6).
 *
 * Conventions for every call below:
 *  - Device buffers are allocated and owned by the caller; the library keeps no
 *    device memory (a graph handle holds only the HIP runtime's graph objects).  Pointers named "device" must be device-accessible, 16-byte
 *    aligned and contiguous in the stated layout.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *    and never synchronize.
 *  - Every call returns PKV_OK or a negative code.  On an error nothing is
 *    launched and no buffer is touched.  pkv_last_error() gives a message for the
 *    last failing call on the calling thread.
 *  - Device data (tables, lengths, slots) is trusted for values but never for
 *    memory safety: kernels do not dereference block ids outside [0, num_blocks)
 *    or table entries past max_blocks_per_seq.
 *  - dtype: PKV_F32 (IEEE float) or PKV_BF16 (bfloat16 bit patterns).  Queries,
 *    caches and outputs share one dtype; accumulation is fp32.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,       /* bad argument (null pointer, bad shape, misalignment) */
  PKV_EUNSUPPORTED = -2, /* valid but not built: block_size != 16, head_dim, GQA group */
  PKV_ENOMEM = -3,       /* allocator: not enough free blocks (state unchanged) */
  PKV_ELAUNCH = -4,      /* the HIP runtime rejected a launch */
  PKV_ENOSEQ = -5,       /* allocator: unknown sequence id */
  PKV_EWORKSPACE = -6,   /* workspace missing or smaller than the query says */
  PKV_ESWAPPED = -7      /* allocator: the sequence is swapped out (or, for a swap-in, is not) */
};

#define PKV_BLOCK_SIZE 16        /* tokens per block; the only size built */
#define PKV_PARTITION_TOKENS 512 /* tokens per split-context partition */

/* Message for the last failing call on this thread ("" if none).  Static storage. */
const char* pkv_last_error(void);
/* Short name of a status code. */
const char* pkv_strerror(int code);

/* ------------------------------------------------------------------------ */
/* KV write: store each new token's K and V row into its slot.
 *
 * The cache keeps every token's key and value for reuse on later steps ("How vLLM
 * Works?", section 01); a token's slot is block_table[pos / 16] * 16 + pos % 16,
 * decided by the allocator below.
 *
 *   key_cache, value_cache  device, [num_blocks, block_size, num_kv_heads, head_dim], dtype dt
 *   k, v                    device, [num_tokens, num_kv_heads, head_dim], dtype dt
 *   slot_mapping            device int32 [num_tokens]; slot s -> block s / 16,
 *                           offset s % 16.  Slots < 0 or >= num_blocks*16 are skipped.
 *                           Duplicate slots in one call race (caller error).
 * Bit copy: the written rows equal the inputs byte for byte; nothing else changes.
 * num_tokens == 0 launches nothing.  Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ELAUNCH. */
int pkv_write(void* key_cache, void* value_cache, const void* k, const void* v,
              const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
              int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dt,
              void* stream);

/* ------------------------------------------------------------------------ */
/* Decode attention for one new token per sequence, over the paged cache.
 *
 *   out[s, h, :] = softmax_j(scale * q[s, h, :] . K_s[j, h / G, :]) . V_s[j, h / G, :]
 *
 * where K_s, V_s are sequence s's first context_lens[s] tokens gathered through
 * block_tables[s] ("vLLM and PagedAttention", §2: attention computed per block
 * through the block table and accumulated), and G = num_q_heads / num_kv_heads
 * (consecutive q heads share a KV head).  Contexts longer than
 * PKV_PARTITION_TOKENS are split into partitions whose softmax statistics
 * (max, sum, normalized partial output) are merged by log-sum-exp; the result is
 * the same softmax up to fp32 rounding.  context_lens[s] == 0 gives zeros.
 *
 *   out, q               device, [num_seqs, num_q_heads, head_dim], dtype dt
 *   key_cache, value_cache  as for pkv_write
 *   block_tables         device int32 [num_seqs, max_blocks_per_seq] row-major;
 *                        entries past ceil(context_len/16) are never read
 *   context_lens         device int32 [num_seqs]; must be <= max_context_len
 *                        (larger values are clamped, never faulted on)
 *   max_context_len      host-known bound on context_lens (no device sync);
 *                        must be <= max_blocks_per_seq * 16
 *   scale                softmax scale (e.g. 1/sqrt(head_dim)); finite and > 0,
 *                        else PKV_EINVAL (every attention call below checks this)
 *   workspace            device, >= pkv_decode_workspace_bytes(...) bytes, 256-byte
 *                        aligned.  Scratch only: a work list the call builds on the
 *                        device from context_lens, and the partition partials.
 *                        Contents undefined between calls; calls sharing one
 *                        workspace must be ordered on one stream.
 * Supported: block_size 16; head_dim 64 or 128; G in {1, 2, 4, 8}; num_seqs <= 65535.
 * bf16 runs on the matrix cores as a persistent kernel fed from that work list;
 * fp32 runs on the vector ALUs.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_ELAUNCH. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len);
int pkv_attention_decode(void* out, const void* q, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, int32_t block_size,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                         int32_t max_context_len, pkv_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream);

/* pkv_attention_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that may not call hipMalloc, harnesses
 * that forbid allocation.  The workspace is a library-owned device array of
 * PKV_STATIC_WORKSPACE_BYTES on each GPU the library runs on (its address is
 * taken at the first call on a device; the array is held until the process
 * ends); the call allocates nothing.  The arguments are those of
 * pkv_attention_decode without the workspace.  A call whose workspace
 * (pkv_decode_workspace_bytes) exceeds PKV_STATIC_WORKSPACE_BYTES returns
 * PKV_EWORKSPACE and launches nothing.  Every call on one GPU uses that GPU's
 * one array, whose contents the previous call left: calls that overlap on one
 * GPU (on different streams or threads) race; order them on one stream.
 * Errors: those of pkv_attention_decode, PKV_ELAUNCH if the array's address
 * cannot be taken. */
#define PKV_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int pkv_attention_decode_noalloc(void* out, const void* q, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, float scale, int32_t block_size,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t max_context_len, pkv_dtype dt, void* stream);

/* The three launches pkv_attention_decode makes, callable one at a time with the
 * same arguments (so each can be timed or overlapped on its own).
 * _plan: builds the work list in the workspace from context_lens (reads nothing
 * else, writes only the workspace), so it may run on another stream -- e.g.
 * beside pkv_write -- if the caller orders it before _partitions.  It launches
 * nothing for fp32 when max_context_len <= PKV_PARTITION_TOKENS (the fp32
 * kernel reads no work list, and there is nothing to merge).
 * _partitions: computes every work item of the planned list (a sequence, a KV
 * head, one or two 512-token partitions); writes `out` for sequences whose
 * context one item covers and partial results (max, sum, normalized output)
 * of the others to the workspace (bf16: one per item; fp32: one per partition).
 * _merge: log-sum-exp merge of those partials into `out` (launches nothing when
 * max_context_len <= PKV_PARTITION_TOKENS).
 * All three take the same workspace; run them in this order.  Errors as
 * pkv_attention_decode. */
int pkv_attention_decode_plan(void* out, const void* q, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, int32_t block_size,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                              int32_t max_context_len, pkv_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream);
/* _plan_upload: the plan of a step whose metadata the host has just written to
 * page-locked memory, fused with the copy of that metadata to the device, in
 * one launch on `stream` (no copy engine, no second stream).  Workgroup 0 builds
 * the work list from host_context_lens (page-locked, mapped for the device;
 * num_seqs values); the others copy upload_bytes (a multiple of 16) from
 * upload_src (page-locked) to upload_dst (device), typically the step's slots,
 * context lengths and tables, so that context_lens / block_tables of the later
 * launches point into upload_dst.  The work list equals _plan's for the same
 * lengths.  Decode (one query row per sequence) only; num_seqs > 0.  The host
 * must not rewrite the page-locked buffers until the stream has passed this
 * launch.  Pointers are checked with the HIP runtime: PKV_EINVAL for pageable
 * or device memory where page-locked host memory is required, and the other
 * way round.  Other errors as pkv_attention_decode.
 * host_block_tables (NULL, or page-locked [num_seqs, max_blocks_per_seq]): the
 * launch also copies, for each sequence s, the first
 * ceil(min(host_context_lens[s], max_context_len) / 16) entries of row s into
 * block_tables (device); the entries after them are not sent (no launch reads
 * them), so the upload region then only needs the rest of the metadata.
 * merge_out, merge_workspace (both NULL, or both given): the same launch also
 * runs _merge for the previous step -- one whose _partitions wrote its partials
 * to merge_workspace with the same shapes, max_context_len and workspace size,
 * and whose output is merge_out -- so a decode loop is
 *   _plan_upload(step i, merging step i-1) ; _partitions(step i)
 * with a plain _merge after the last step.  merge_workspace must not be
 * `workspace` (PKV_EINVAL): step i's plan writes its own workspace while step
 * i-1's partials are read. */
int pkv_attention_decode_plan_upload(void* out, const void* q, const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,
                                     int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void* workspace,
                                     size_t workspace_bytes, const int32_t* host_context_lens,
                                     const void* upload_src, void* upload_dst, size_t upload_bytes,
                                     const int32_t* host_block_tables, void* merge_out,
                                     const void* merge_workspace, void* stream);
int pkv_attention_decode_partitions(void* out, const void* q, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, float scale, int32_t block_size,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t num_seqs, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, int32_t max_context_len, pkv_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream);
int pkv_attention_decode_merge(void* out, const void* q, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, int32_t block_size,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                               int32_t max_context_len, pkv_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Decode step with the cache append in the same launch (bf16).
 *
 * Same result as pkv_write of each sequence's new token followed by
 * pkv_attention_decode, byte for byte, in one launch fewer: the new token is
 * the last of the context (position context_lens[s] - 1, slot
 * block_tables[s][(ctx - 1) / 16] * 16 + (ctx - 1) % 16, the slot the allocator
 * hands out for a decode append); the partition launch reads its K/V from
 * k_new / v_new instead of the cache and writes them to that slot.  The pages
 * write new K/V into the cache first and read them back ("How vLLM Works?",
 * section 01; "vLLM and PagedAttention", §2); this folds the write into the
 * work item that reads that block.
 *
 *   k_new, v_new          device [num_seqs, num_kv_heads, head_dim] bf16, 16-byte aligned
 *   key_cache, value_cache  written at the new tokens' slots only
 *   other arguments       as pkv_attention_decode (dt must be PKV_BF16)
 * A sequence with context_lens[s] == 0 appends nothing; one whose context exceeds
 * max_context_len (clamped) appends nothing.  The slot's block id must lie in
 * [0, num_blocks), else nothing is written there.
 * _partitions_append is the partition launch of this form (after
 * pkv_attention_decode_plan, before pkv_attention_decode_merge, same workspace).
 * Errors as pkv_attention_decode; PKV_EUNSUPPORTED for dt other than bf16. */
int pkv_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                void* key_cache, void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, float scale, int32_t block_size,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                                int32_t max_context_len, pkv_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream);
int pkv_attention_decode_partitions_append(void* out, const void* q, const void* k_new,
                                           const void* v_new, void* key_cache, void* value_cache,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           float scale, int32_t block_size, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t num_seqs,
                                           int32_t max_blocks_per_seq, int32_t num_blocks,
                                           int32_t max_context_len, pkv_dtype dt, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Variable-length attention over the paged cache: decode rows and chunked
 * prefill rows in one call (bf16 only).
 *
 * Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1 of q
 * and out.  With q_s rows and ctx_s = context_lens[s] keys (the rows' own
 * tokens included: write them with pkv_write first), row r attends causally to
 * keys 0 .. ctx_s - q_s + r:
 *   out[row, h, :] = softmax_j(scale * q[row, h, :] . K_s[j, h / G, :]) . V_s[j, h / G, :]
 * A long prompt split into chunks and batched with decode steps is the pages'
 * chunked prefill ("How vLLM Works?", section 04; "vLLM and PagedAttention",
 * key engineering optimizations); a sequence with one row is a decode step.
 * One-row sequences run the decode kernels; longer ones run work items of
 * 256/G rows x the G q heads of one KV head on the matrix cores, over one or
 * two 512-token partitions each.  Keys are split into 512-token partitions
 * whose partial results are merged by log-sum-exp.  A row that sees no key
 * (q_s > ctx_s) gets zeros.
 *
 *   out, q            device [num_tokens, num_q_heads, head_dim] bf16
 *   query_start_loc   device int32 [num_seqs + 1], non-decreasing, values in
 *                     [0, num_tokens] (out-of-range values are clamped)
 *   max_query_len     host bound on rows per sequence (>= 1)
 *   max_context_len   host bound on context_lens, <= max_blocks_per_seq * 16
 *   workspace         device, >= pkv_varlen_workspace_bytes(...) bytes, 256-byte aligned
 * Other arguments as pkv_attention_decode.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED (fp32, shapes), PKV_EWORKSPACE, PKV_ELAUNCH. */
size_t pkv_varlen_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                  int32_t max_context_len);
int pkv_attention_varlen(void* out, const void* q, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                         float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,
                         int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream);
/* pkv_attention_varlen in two calls, for a step whose metadata the host has just
 * written to page-locked memory ("How vLLM Works?", section 04: the scheduler
 * batches a prefill chunk with decode rows every step, so the step's launches
 * should cost little beside the kernels):
 * _plan_upload: the plan (decode and prefill work lists from host_context_lens,
 * page-locked, num_seqs values, and from query_start_loc, device) fused with
 * the upload of the step's metadata in one launch on `stream`, as
 * pkv_attention_decode_plan_upload does for decode (upload_src -> upload_dst,
 * upload_bytes a multiple of 16; host_block_tables NULL or page-locked
 * [num_seqs, max_blocks_per_seq], of which each row's used entries go to
 * block_tables).  The uploaded slots can feed a pkv_write on the same stream
 * before _partitions.  num_seqs and num_tokens must be > 0.
 * _partitions: the launches after the plan (decode partitions, prefill tiles,
 * log-sum-exp merge), same arguments and workspace.
 * Results equal pkv_attention_varlen's byte for byte.  Errors as
 * pkv_attention_varlen, and PKV_EINVAL for host or device buffers of the wrong
 * kind (checked with the HIP runtime). */
int pkv_attention_varlen_plan_upload(void* out, const void* q, const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                                     float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,
                                     int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void* workspace,
                                     size_t workspace_bytes, const int32_t* host_context_lens,
                                     const void* upload_src, void* upload_dst, size_t upload_bytes,
                                     const int32_t* host_block_tables, void* stream);
int pkv_attention_varlen_partitions(void* out, const void* q, const void* key_cache, const void* value_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                                    float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,
                                    int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void* workspace,
                                    size_t workspace_bytes, void* stream);
/* pkv_attention_varlen's four launches one by one, for callers that place
 * them themselves (time them, or put the decode partitions and the prefill
 * tiles on different streams; "How vLLM Works?", section 04: a step batches
 * the memory-bound decode rows with the compute-bound prefill chunk).
 * _plan: the work lists from context_lens and query_start_loc (device); it
 * also resets the ticket counters, so each step's launches need their own
 * plan.  _decode_partitions: the one-row sequences' partitions.
 * _prefill_tiles: the chunk rows' matrix-core tiles.  _merge: the log-sum-exp
 * merge of every row with more than one partial.  Arguments and workspace as
 * pkv_attention_varlen; call them in this order on one workspace (the two
 * middle launches in either order, or concurrently on two streams that meet
 * before _merge).  Together they equal pkv_attention_varlen byte for byte
 * (pkv_attention_varlen_partitions is the last three).  Errors as
 * pkv_attention_varlen.  Ownership: nothing is kept; the caller owns every
 * buffer. */
int pkv_attention_varlen_plan(void* out, const void* q, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_tokens,
    int32_t max_query_len, float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    pkv_dtype dt, void* workspace, size_t workspace_bytes, void* stream);
int pkv_attention_varlen_decode_partitions(void* out, const void* q, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_tokens,
    int32_t max_query_len, float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    pkv_dtype dt, void* workspace, size_t workspace_bytes, void* stream);
int pkv_attention_varlen_prefill_tiles(void* out, const void* q, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_tokens,
    int32_t max_query_len, float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    pkv_dtype dt, void* workspace, size_t workspace_bytes, void* stream);
int pkv_attention_varlen_merge(void* out, const void* q, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_tokens,
    int32_t max_query_len, float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
    pkv_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Log-sum-exp merge of partial softmax results, one output row per input row.
 *
 * The accumulation of separately computed attention pieces ("vLLM and
 * PagedAttention", §2 "Reworking the Attention Computation"): with maxima m_p in
 * base-2 units (scores already multiplied by log2(e)), sums l_p and normalized
 * partial outputs o_p,
 *   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
 * Partials with m_p = -inf or l_p = 0 weigh 0; a row with no live partial is 0.
 *
 *   out        device [rows, head_dim], dtype out_dt
 *   part_m, part_l  device float [rows, max_parts]
 *   part_o     device float [rows, max_parts, head_dim]
 *   num_parts  device int32 [rows]; row r merges its first num_parts[r] partials
 *              (clamped to [0, max_parts])
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED (head_dim not 64/128), PKV_ELAUNCH. */
int pkv_lse_merge(void* out, const float* part_m, const float* part_l, const float* part_o,
                  const int32_t* num_parts, int32_t rows, int32_t max_parts, int32_t head_dim,
                  pkv_dtype out_dt, void* stream);

/* ------------------------------------------------------------------------ */
/* Copy-on-write block copies: for each pair (src, dst), block dst of both caches
 * becomes a byte copy of block src ("vLLM and PagedAttention", §2 shareable
 * prefixes with copy-on-write).  Run the pairs returned by pkv_alloc_append before
 * writing new tokens.
 *
 *   pairs   device int32 [num_pairs, 2]; pairs whose ids fall outside
 *           [0, num_blocks) are skipped.  A dst that is also a src in the same call
 *           races (caller error).
 * num_pairs == 0 launches nothing.  Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ELAUNCH. */
int pkv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                    int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dt, void* stream);

/* ------------------------------------------------------------------------ */
/* Block copies between two pools of the same block shape, for preemption by
 * swapping ("vLLM and PagedAttention", §3 continuous batching: under memory
 * pressure the scheduler moves some requests' KV to CPU memory and brings it
 * back once memory frees up).  For each pair (src, dst), block dst of the
 * destination pool (both caches) becomes a byte copy of block src of the source
 * pool.  One launch moves every pair; run the pairs of pkv_alloc_swap_out
 * (device pool -> host pool) or pkv_alloc_swap_in (host pool -> device pool).
 *
 *   dst_*_cache, src_*_cache  [num_blocks, 16, num_kv_heads, head_dim] of dtype dt,
 *              each either device memory or page-locked host memory allocated
 *              mapped for the device (hipHostMalloc; torch pin_memory), which the
 *              kernel reads or writes across the host link.  The library checks
 *              each pointer with the HIP runtime: pageable memory, or a buffer
 *              shorter than its num_blocks blocks, is PKV_EINVAL.
 *   pairs      device int32 [num_pairs, 2] of (src block, dst block); pairs whose
 *              ids fall outside [0, src_num_blocks) x [0, dst_num_blocks) are
 *              skipped.  Two pairs with one dst race (caller error).
 * Enqueued on stream; the caller keeps a host pool alive and unread until the
 * stream passes the copy.  num_pairs == 0 launches nothing.
 * Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ELAUNCH. */
int pkv_swap_blocks(void* dst_key_cache, void* dst_value_cache, const void* src_key_cache,
                    const void* src_value_cache, const int32_t* pairs, int32_t num_pairs,
                    int32_t src_num_blocks, int32_t dst_num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dt, void* stream);

/* ------------------------------------------------------------------------ */
/* One decode step as a HIP graph ("vLLM and PagedAttention", §6 version
 * evolution, key engineering optimizations: a generation step's kernel
 * sequence is recorded into a graph and launched as one instead of one launch
 * per kernel).  pkv_decode_graph_create records the launches of one step on a
 * private stream of the current device and instantiates them:
 *
 *   slot_mapping != NULL: pkv_write(k_new, v_new, slot_mapping, num_new_tokens)
 *                         (skipped when num_new_tokens == 0), then
 *                         pkv_attention_decode (plan, partitions, merge);
 *   slot_mapping == NULL: pkv_attention_decode_append (bf16 only; k_new, v_new
 *                         are [num_seqs, Hkv, D], one new row per sequence).
 *
 * Every pointer and every size is fixed into the graph; device data (q, the new
 * K/V rows, slots, tables, context lengths) is read when the graph runs, so the
 * caller updates those buffers in place between launches (on the stream it
 * launches on, or with the ordering it needs).  max_context_len is the bound the
 * graph was made for: every later context must stay at or below it.  The
 * workspace is the graph's own: two graphs (or a graph and a direct call) that
 * run at the same time need separate workspaces.  Argument errors as for the
 * captured calls; nothing runs at creation.  pkv_decode_graph_launch enqueues the
 * whole step with one call on stream (NULL = the default stream).
 * No node of the graph is a memset (the plan kernel clears its own counters). */
typedef struct pkv_graph pkv_graph;
int pkv_decode_graph_create(pkv_graph** graph_out, void* out, const void* q, const void* k_new,
                            const void* v_new, const int32_t* slot_mapping, int32_t num_new_tokens,
                            void* key_cache, void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, float scale, int32_t block_size,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                            pkv_dtype dt, void* workspace, size_t workspace_bytes);
int pkv_decode_graph_launch(pkv_graph* graph, void* stream);
void pkv_decode_graph_destroy(pkv_graph* graph);

/* ------------------------------------------------------------------------ */
/* Host-side debug checks (no device access).
 * pkv_check_tables: every entry a sequence uses (the first ceil(context_lens[s]/16)
 * of its row) lies in [0, num_blocks), and context_lens are in [0, max_blocks*16].
 * pkv_check_slots: no two non-negative slots are equal (a duplicate is a write race)
 * and all lie below num_blocks*16.  Both return PKV_OK or PKV_EINVAL. */
int pkv_check_tables(const int32_t* host_block_tables, const int32_t* host_context_lens,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks);
int pkv_check_slots(const int32_t* host_slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size);
/* The check pkv_swap_blocks makes of each pool, on its own (asks the HIP runtime,
 * launches nothing): PKV_OK if [pool, pool + bytes) is device memory or
 * page-locked host memory mapped for the device, within one allocation;
 * PKV_EINVAL otherwise (pageable memory, unknown addresses, a range running past
 * its allocation). */
int pkv_check_pool(const void* pool, size_t bytes);

/* ------------------------------------------------------------------------ */
/* Host block allocator (no device memory; not thread-safe; one pool per object).
 *
 * A sequence takes a new block only when its last block is full, so only the last
 * block can be partly empty ("How vLLM Works?", section 03; "vLLM and
 * PagedAttention", §2 on-demand allocation bullet).  Sequences forked from a parent
 * share its blocks with reference counts; appending into a shared, partly filled
 * last block first copies it (copy-on-write) and reports the (src, dst) pair for
 * pkv_copy_blocks ("vLLM and PagedAttention", §2; "vLLM — PagedAttention and
 * Continuous Batching", §2.3).  Full shared blocks are never copied.
 *
 * The free list is shuffled once at creation with the splitmix64 generator seeded
 * by shuffle_seed (seed 0 keeps ids in order 0, 1, 2, ...), which scatters each
 * sequence's blocks through the pool.  Every operation is all-or-nothing: on
 * PKV_ENOMEM nothing changes. */
typedef struct pkv_allocator pkv_allocator;

/* NULL on bad arguments (num_blocks <= 0, block_size != 16) or allocation failure. */
pkv_allocator* pkv_alloc_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed);
void pkv_alloc_destroy(pkv_allocator* a);
/* New empty sequence.  PKV_EINVAL if the id exists. */
int pkv_alloc_add_seq(pkv_allocator* a, int64_t seq_id);
/* child shares all of parent's blocks and length.  PKV_ENOSEQ / PKV_EINVAL (child exists). */
int pkv_alloc_fork(pkv_allocator* a, int64_t parent, int64_t child);
/* Reserve n_tokens slots at the end of seq_id.  slots_out[n_tokens] receives each
 * new token's slot; cow_pairs_out (capacity 2 ints) receives at most one (src, dst)
 * pair, *num_cow_out its count (0 or 1).  The token ids are not known, so a
 * sequence made with pkv_alloc_add_seq_tokens stops caching its blocks here. */
int pkv_alloc_append(pkv_allocator* a, int64_t seq_id, int32_t n_tokens, int32_t* slots_out,
                     int32_t* cow_pairs_out, int32_t* num_cow_out);
/* Batched append, all-or-nothing over the batch.  seq_ids must be distinct.
 * slots_out receives sum(n_tokens) slots in batch order (capacity slots_cap);
 * cow_pairs_out receives up to cow_cap pairs (2 ints each), *num_cow_out the count. */
int pkv_alloc_append_batch(pkv_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                           int32_t num_seqs, int32_t* slots_out, int64_t slots_cap,
                           int32_t* cow_pairs_out, int32_t cow_cap, int32_t* num_cow_out);
/* Drop a sequence; blocks whose count reaches 0 return to the free list, or, if
 * cached, to the released list (below). */
int pkv_alloc_free_seq(pkv_allocator* a, int64_t seq_id);
/* Copy seq_id's table into out (capacity cap); *len_out = its block count. */
int pkv_alloc_block_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                          int32_t* len_out);
/* Dense row-major [num_seqs, max_blocks] tables (unused entries = fill) and lengths. */
int pkv_alloc_block_tables(const pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                           int32_t* tables_out, int32_t max_blocks, int32_t fill,
                           int32_t* context_lens_out);
/* Tokens held by seq_id, or PKV_ENOSEQ. */
int64_t pkv_alloc_seq_len(const pkv_allocator* a, int64_t seq_id);
/* Blocks an allocation can take: free blocks plus released cached ones. */
int32_t pkv_alloc_num_free(const pkv_allocator* a);
int32_t pkv_alloc_num_blocks(const pkv_allocator* a);
/* Reference count of a block (number of table entries holding it); -1 if out of range. */
int32_t pkv_alloc_refcount(const pkv_allocator* a, int32_t block_id);

/* Automatic prefix caching ("How vLLM Works?", section 05; "vLLM and
 * PagedAttention", section 4; "vLLM — PagedAttention and Continuous Batching",
 * §5).  A sequence made with its token ids keys every full block by (the key of
 * the block before it, a salt, the block's 16 token ids); a full block whose key
 * is new is cached.  A block that is not full is never cached.  A cached block
 * whose last user is freed goes on a released list: a later hit revives it, and
 * when no free block is left an allocation takes over the least recently
 * released one (a freed sequence's cached blocks join that list from its last
 * block to its first).  Different salts never share blocks (tenant isolation).
 *
 * pkv_alloc_add_seq_tokens: new sequence seq_id holding tokens[n_tokens].  Its
 * longest prefix of whole cached blocks (looked up block by block from the
 * start, stopping at the first key not found) is taken from the cache: those
 * *num_cached_out tokens get slot -1 in slots_out[n_tokens] (their K/V is in the
 * pool already; pkv_write skips negative slots), the others get new slots.
 * PKV_EINVAL (bad arguments, id exists), PKV_ENOMEM (all-or-nothing: the blocks
 * a hit revives are counted out of the released list first). */
int pkv_alloc_add_seq_tokens(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                             uint64_t salt, int32_t* slots_out, int32_t* num_cached_out);
/* pkv_alloc_append with the new tokens' ids, for a sequence made by
 * pkv_alloc_add_seq_tokens (or forked from one): blocks that become full are
 * keyed and cached.  PKV_EINVAL for a sequence without token ids. */
int pkv_alloc_append_tokens(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                            int32_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out);
/* Released cached blocks (count 0, reusable by a hit; included in num_free). */
int32_t pkv_alloc_num_cached(const pkv_allocator* a);

/* Preemption by swapping ("vLLM and PagedAttention", §3 continuous batching, on
 * the scheduler's preemption; "How vLLM Works?", section 04, where recompute is
 * the other mode: pkv_alloc_free_seq now, pkv_alloc_add_seq_tokens again later).
 *
 * pkv_alloc_set_host_pool: a pool of num_host_blocks host block ids (the caller
 * owns the memory: a page-locked [num_host_blocks, 16, Hkv, D] pair of caches).
 * Ids are handed out lowest first; freed ids are reused last-freed first.
 * PKV_ESWAPPED while any sequence is swapped out.
 *
 * pkv_alloc_swap_out: moves the distinct sequences seq_ids[num_seqs] (all on the
 * device) to host blocks.  pairs_out (capacity pairs_cap pairs of 2 ints)
 * receives one (device block, host block) pair per distinct device block of the
 * group, in order of first appearance (sequences in the given order, each table
 * in order); *num_pairs_out their count.  A block held several times inside the
 * group gets one host block, so sharing inside the group survives.  The group's
 * device references are dropped as pkv_alloc_free_seq drops them; a block still
 * held by a sequence outside the group stays where it is.  Run the pairs with
 * pkv_swap_blocks before anything is written into the released blocks.
 *
 * pkv_alloc_swap_in: brings swapped sequences back to new device blocks; pairs
 * are (host block, device block), one per distinct host block of the group.
 *
 * A swapped sequence can only be swapped in, freed (its host blocks return) or
 * queried for its length and host table: append, fork and the table calls
 * return PKV_ESWAPPED.  Both calls are all-or-nothing: PKV_ENOMEM when the
 * target pool is short of blocks, PKV_EINVAL when pairs_out is too small,
 * PKV_ENOSEQ / PKV_EINVAL (duplicate id) / PKV_ESWAPPED (wrong pool) for a bad
 * group; nothing changes on an error. */
int pkv_alloc_set_host_pool(pkv_allocator* a, int32_t num_host_blocks);
int pkv_alloc_swap_out(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs, int32_t* pairs_out,
                       int32_t pairs_cap, int32_t* num_pairs_out);
int pkv_alloc_swap_in(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs, int32_t* pairs_out,
                      int32_t pairs_cap, int32_t* num_pairs_out);
/* 1 if seq_id is swapped out, 0 if on the device; PKV_ENOSEQ if unknown. */
int pkv_alloc_is_swapped(const pkv_allocator* a, int64_t seq_id);
/* A swapped sequence's table of host block ids (as pkv_alloc_block_table). */
int pkv_alloc_host_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap, int32_t* len_out);
int32_t pkv_alloc_num_free_host(const pkv_allocator* a);
/* Host table entries holding a host block; -1 if out of range. */
int32_t pkv_alloc_host_refcount(const pkv_allocator* a, int32_t host_block);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
