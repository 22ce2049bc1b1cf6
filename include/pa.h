/*
 * pa.h -- paged KV attention for AMD Instinct MI355X (gfx950): the C ABI.
 *
 * The operation ("Attention Backends", infra.riteshsonawane.com, section
 * "What paged attention requires of a kernel"): for a flat batch of T tokens
 * from N requests,
 *   1. store the T new keys and values in the shared block-pool cache at
 *      slot_mapping[t]  (slot = physical_block * block_size + offset);
 *   2. for each request, attend from its queries over its first seq_len
 *      cached tokens, fetching them block by block through its row of
 *      block_table (position p lives at block block_table[r][p / block_size],
 *      offset p % block_size).
 * The result is softmax(scale * Q K^T + M) V ("第 1 章 注意力后端", §2.1), M the
 * causal mask, plus the natural-log log-sum-exp of each softmax row.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer argument is DEVICE memory owned by the caller:
 *   caches, metadata, inputs, outputs and workspaces.  The library allocates
 *   and frees nothing and keeps no per-call state.
 * Streams.  All work is enqueued on `stream` (0 = the null stream) in the
 *   order described, and the call returns without synchronising.  A new-token
 *   write that an entry point performs is ordered before the attention that
 *   reads it.
 * Errors.  Each call returns a pa_status_t.  Host-side argument checks run
 *   before anything is enqueued: on any error nothing is launched.
 *   pa_last_error() returns a description of the calling thread's last error.
 *   Device-side metadata (block ids, slots, lengths) is not validated; values
 *   outside the documented ranges give undefined results, but the kernels
 *   clamp every index they derive from it so that they never read or write
 *   outside the buffers whose sizes the call describes.
 * Types.  q, k, v, cache and out share one storage dtype (pa_dtype_t);
 *   accumulation is fp32; lse and workspaces are fp32.  bf16 results are
 *   rounded to nearest-even.  block_table, seq_lens and query_start_loc are
 *   int32; slot_mapping is int64, and a negative slot means "do not write".
 * Alignment.  Device pointers must be 16-byte aligned.
 * Shapes.  The GQA cache is [num_blocks, 2, block_size, num_kv_heads,
 *   head_dim] (index 0 = K, 1 = V) and the MLA latent cache is [num_blocks,
 *   block_size, kv_lora_rank + rope_dim] ("AttentionBackend：注意力后端抽象层",
 *   设计动机).  block_size must be a multiple of 16 ("AttentionBackend", 边界与
 *   失败).  All tensors are dense, row-major, in the shapes given, unless a
 *   stride argument says otherwise.
 * Scale.  The softmax scale multiplies Q K^T; it must be finite and >= 0.
 * Query-to-KV head map.  Query head h reads KV head h / (num_q_heads /
 *   num_kv_heads) ("第 1 章 注意力后端", §3.2: groups of query heads share a
 *   KV head).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* an argument is out of range or a pointer is null */
  PA_ERR_UNSUPPORTED = 2, /* a valid configuration this build does not implement */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  PA_ERR_HIP = 4          /* the HIP runtime reported an error (launch, device query) */
} pa_status_t;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype_t;

typedef enum {
  PA_LAYOUT_KV = 0,  /* [num_blocks, 2, block_size, num_kv_heads, head_dim] */
  PA_LAYOUT_MLA = 1  /* [num_blocks, block_size, kv_lora_rank + rope_dim]   */
} pa_layout_t;

/* ---------------------------------------------------------------------------
 * Host helpers (no device work).
 * ------------------------------------------------------------------------- */

/* Number of KV splits for split-KV decode: ceil(max_seq_len / 512), at least
 * 1 and at most 2 * num_cus ("Triton 與 MLA", 關鍵檔案, _compute_num_kv_splits:
 * max_seq_len / 512, capped at twice the compute-unit count; rounding up is
 * this library's reading).  num_cus <= 0 is treated as 1. */
int pa_num_kv_splits(int max_seq_len, int num_cus);

/* Split count pa_decode (and pa_plan_mixed's decode group) uses when called
 * with num_splits = 0.  It starts from pa_num_kv_splits(max_seq_len,
 * num_cus); when that rule splits at all (n > 1) and the batch has fewer
 * than 2 * num_cus (request, KV head) pairs, it is raised until
 * num_seqs * num_kv_heads * n reaches 2 * num_cus, with no split shorter
 * than 64 keys (n <= ceil(max_seq_len / 64)) and n <= 2 * num_cus.  The
 * pages' rule sizes splits from the sequence length only, which leaves most
 * compute units idle for a batch of a few requests; a larger batch keeps the
 * rule's count.  Non-positive num_seqs, num_kv_heads or num_cus count as 1.
 * Size the workspace with it (or call pa_decode_workspace_size). */
int pa_decode_num_kv_splits(int num_seqs, int num_kv_heads, int max_seq_len, int num_cus);

/* Bytes of fp32 workspace pa_decode / pa_mla_decode need for num_splits
 * splits: num_seqs * num_q_heads * num_splits * (head_dim_v + 1) * 4 (the
 * "+1" holds each split's lse, "Triton 與 MLA", 資料流).  Returns 0 if any
 * argument is negative or the product overflows. */
size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim_v,
                                 int num_splits);

/* Split count pa_mla_decode uses when called with num_splits = 0: enough
 * splits of whole 64-token pages that num_seqs * splits work units cover the
 * device's compute units about twice, and never more than
 * pa_num_kv_splits(max_seq_len, num_cus).  Size the workspace with it. */
int pa_mla_num_kv_splits(int num_seqs, int max_seq_len, int num_cus);

/* Compute units of the current HIP device, or -1 if it cannot be queried. */
int pa_device_num_cus(void);

/* Workspace bytes pa_decode needs when called with these sizes: the
 * schedule it picks ("Triton 與 MLA", 邊界與失敗: the split count used to
 * reserve the workspace must be the one the forward pass uses) decides
 * between no workspace (one split covers max_seq_len), the split partials
 * (pa_decode_workspace_bytes for n splits) and the token-balanced ranges
 * (pa_decode_balanced_workspace_bytes).  partials_only != 0 means out =
 * NULL (the two-stage form).  num_splits = 0 queries the current device's
 * compute units, as pa_decode does.  On success *bytes holds the size (0 =
 * none needed).  Errors: PA_ERR_INVALID for a null bytes pointer or sizes
 * pa_decode would reject on their face (negative counts, block_size not a
 * positive multiple of 16); PA_ERR_HIP if the device cannot be queried. */
pa_status_t pa_decode_workspace_size(pa_dtype_t dtype, int num_seqs, int max_seq_len,
                                     int block_size, int num_q_heads, int num_kv_heads,
                                     int head_dim, int num_splits, int partials_only,
                                     size_t* bytes);

/* The same query for pa_mla_decode (bf16 latent cache); head_dim_v is
 * kv_lora_rank. */
pa_status_t pa_mla_decode_workspace_size(int num_seqs, int max_seq_len, int block_size,
                                         int num_heads, int kv_lora_rank, int num_splits,
                                         int partials_only, size_t* bytes);

/* Thread-local description of the last error ("" if none). */
const char* pa_last_error(void);

/* ---------------------------------------------------------------------------
 * pa_cache_write -- step 1 of the contract: store new rows at their slots.
 *
 * PA_LAYOUT_KV:  k, v are [num_tokens, num_kv_heads, head_dim] with a token
 *   stride of k_token_stride / v_token_stride ELEMENTS (heads contiguous);
 *   row t goes to cache[slot / block_size][0 or 1][slot % block_size].
 * PA_LAYOUT_MLA: num_kv_heads must be 1 and head_dim = kv_lora_rank +
 *   rope_dim with rope_dim = 64; k is kv_c [num_tokens, head_dim - 64]
 *   and v is k_pe [num_tokens, 64] (token strides as above); the stored row
 *   is kv_c followed by k_pe ("Triton 與 MLA", 資料流).  bf16 only.
 * slot_mapping: [num_tokens] int64 in [0, num_blocks * block_size), or
 *   negative to skip the token.  Two tokens must not share a slot.
 * The copy is bit-exact.  num_tokens = 0 is a no-op.
 * ------------------------------------------------------------------------- */
pa_status_t pa_cache_write(pa_layout_t layout, pa_dtype_t dtype,
                           const void* k, int64_t k_token_stride,
                           const void* v, int64_t v_token_stride,
                           void* kv_cache, int64_t num_blocks, int block_size,
                           int num_kv_heads, int head_dim,
                           const int64_t* slot_mapping, int num_tokens,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * pa_decode -- GQA decode: one query token per request, split-KV partials
 * merged by log-sum-exp ("第 1 章 注意力后端", §3.1 split-KV; "Triton 與 MLA",
 * 資料流: workspace (B, H, num_kv_splits, D + 1), stage 2 merges by lse).
 *
 * q:           [num_seqs, num_q_heads, head_dim]
 * k, v:        [num_seqs, num_kv_heads, head_dim] new rows, or both NULL
 * slot_mapping:[num_seqs] int64, or NULL (then k, v must be NULL too)
 * kv_cache:    GQA layout, num_blocks blocks of block_size tokens
 * block_table: [num_seqs, max_blocks_per_seq] int32
 * seq_lens:    [num_seqs] int32, each in [1, max_seq_len] and at most
 *              max_blocks_per_seq * block_size; includes the new token, which
 *              is the request's last position.
 * max_seq_len: host copy of max(seq_lens) (sets the split partition).
 * scale:       multiplies Q K^T before the softmax (1/sqrt(head_dim) usually).
 * num_splits:  0 = automatic: with n = pa_decode_num_kv_splits(num_seqs,
 *              num_kv_heads, max_seq_len, pa_device_num_cus()), n == 1
 *              runs one unsplit pass; n > 1 with PA_BF16, out != NULL and
 *              num_kv_heads 1, 2, 4 or a multiple of 8 runs the
 *              token-balanced schedule (pa_decode_balanced +
 *              pa_decode_balanced_merge), whose reduction order depends on
 *              the whole batch's lengths; otherwise n splits.
 *              1 = no split (each request reduced by one work unit, in an
 *              order independent of the rest of the batch); n > 1 = n splits.
 *              Split s of a request covers positions [s*P, (s+1)*P) with
 *              P = ceil(max_seq_len / n) rounded up to a multiple of
 *              block_size; splits past the request's end are empty.
 * workspace:   fp32 scratch of at least pa_decode_workspace_size(...) bytes
 *              (that is pa_decode_workspace_bytes(num_seqs, num_q_heads,
 *              head_dim, n) for n splits, or, for the balanced schedule,
 *              pa_decode_balanced_workspace_bytes(num_seqs, num_q_heads, 128,
 *              pa_decode_balanced_num_ranges(num_kv_heads,
 *              pa_device_num_cus()))), 16-byte aligned; may be NULL when one
 *              split covers max_seq_len (then no partials are formed).
 * out:         [num_seqs, num_q_heads, head_dim], storage dtype; or NULL for
 *              the two-stage form: only stage 1 runs and the workspace holds
 *              the partials [num_seqs, num_q_heads, n, head_dim + 1] (empty
 *              splits have lse = -inf), ready for pa_lse_merge.
 * lse:         [num_seqs, num_q_heads] fp32 natural-log LSE, or NULL (must be
 *              NULL when out is NULL).
 * Supported: head_dim 128; num_q_heads / num_kv_heads in {1, 2, 4, 8};
 * PA_F32 and PA_BF16.
 * Enqueues: the write (if k/v given), the split (or balanced) kernel, and
 * the merge kernel unless one split covers every request or out is NULL.
 * ------------------------------------------------------------------------- */
pa_status_t pa_decode(pa_dtype_t dtype,
                      const void* q, const void* k, const void* v,
                      void* kv_cache, int64_t num_blocks, int block_size,
                      const int32_t* block_table, int max_blocks_per_seq,
                      const int64_t* slot_mapping,
                      const int32_t* seq_lens, int num_seqs, int max_seq_len,
                      int num_q_heads, int num_kv_heads, int head_dim,
                      float scale, int num_splits,
                      void* workspace, size_t workspace_bytes,
                      void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the arguments of pa_decode without the workspace, which
 * is taken from a device array the library owns instead.
 *
 * The array holds PA_NOALLOC_SCRATCH_BYTES (64 MiB) on every device the
 * library runs on, from the first call there until the process ends.  A call
 * needing more (pa_decode_workspace_size with partials_only = 0 larger than
 * that, e.g. a few hundred requests with many splits) fails with
 * PA_ERR_WORKSPACE and launches nothing; out must be non-NULL (the
 * partial-only form is PA_ERR_INVALID here).  Nothing in the array needs to
 * start at any value: every partial is written before it is read.  Every
 * call on one device shares that device's array: calls that overlap on one
 * device (on different streams, or from different threads without ordering)
 * race and give wrong results; calls in one stream's order are safe.  This
 * entry point calls no allocator.  Other arguments, supported
 * configurations, errors and what is enqueued are those of pa_decode.
 * ------------------------------------------------------------------------- */
#define PA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

pa_status_t pa_decode_noalloc(pa_dtype_t dtype,
                              const void* q, const void* k, const void* v,
                              void* kv_cache, int64_t num_blocks, int block_size,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int64_t* slot_mapping,
                              const int32_t* seq_lens, int num_seqs, int max_seq_len,
                              int num_q_heads, int num_kv_heads, int head_dim,
                              float scale, int num_splits,
                              void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Token-balanced decode: the split-KV reduction of pa_decode ("第 1 章
 * 注意力后端", §3.1: partial softmax states over pieces of a request's keys,
 * merged by log-sum-exp) with the pieces cut for an even load instead of at
 * fixed positions.  The 32-token chunks of all requests (request r has
 * ceil(seq_lens[r] / 32) of them) are concatenated into one list of T
 * chunks; with nr = min(num_ranges, T), range j = 0..nr-1 is chunks
 * [floor(j T / nr), floor((j+1) T / nr)).  Each range is one work-group.
 * A request wholly inside one range is written to out / lse by
 * pa_decode_balanced; for the others every range they touch leaves one
 * partial (normalised output + lse) in the workspace, and
 * pa_decode_balanced_merge combines them.  Both run on the caller's stream
 * and use the same workspace; the merge must follow the first call.
 *
 * pa_decode_balanced_num_ranges: ranges that keep 8 waves on each of num_cus
 *   compute units (num_cus * 8 / (min(num_kv_heads, 8) * ceil(num_kv_heads /
 *   8)), at least 1); what pa_decode uses.
 * pa_decode_balanced_workspace_bytes: bytes of workspace: 4 (num_seqs + 1)
 *   rounded up to 256, plus (num_ranges + num_seqs) * num_heads *
 *   (head_dim_v + 4) * 4 (head_dim_v = 128 for GQA, 512 for MLA).  Returns 0
 *   for negative sizes or num_ranges < 1.
 *
 * pa_decode_balanced arguments are those of pa_decode (no new-token write:
 * call pa_cache_write first), with:
 * num_ranges:  [1, 2^24]; the workspace must hold
 *              pa_decode_balanced_workspace_bytes(num_seqs, num_q_heads, 128,
 *              num_ranges) bytes, 16-byte aligned (PA_ERR_WORKSPACE if not).
 * out, lse:    as pa_decode; after this call only the requests inside one
 *              range are final.
 * Supported: PA_BF16 storage, head_dim 128, num_q_heads / num_kv_heads in
 * {1, 2, 4, 8}, num_kv_heads 1, 2, 4 or a multiple of 8 (a work-group loads
 * whole rows of up to 8 heads), num_seqs * ceil(max_blocks_per_seq *
 * block_size / 32) < 2^31.
 * pa_decode_balanced_merge completes out / lse (a request with no keys gets
 * out = 0, lse = -inf) after pa_decode_balanced (head_dim_v 128) or
 * pa_mla_decode_balanced (head_dim_v = kv_lora_rank, 512 or 256; head_dim_v
 * also tells it which of the two partitions cut the ranges); its num_seqs,
 * num_heads, num_ranges and workspace must be those of the preceding call.
 * ------------------------------------------------------------------------- */
int pa_decode_balanced_num_ranges(int num_kv_heads, int num_cus);

size_t pa_decode_balanced_workspace_bytes(int num_seqs, int num_heads, int head_dim_v,
                                          int num_ranges);

pa_status_t pa_decode_balanced(const void* q, const void* kv_cache, int64_t num_blocks,
                               int block_size, const int32_t* block_table,
                               int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                               int num_q_heads, int num_kv_heads, int head_dim, float scale,
                               int num_ranges, void* workspace, size_t workspace_bytes,
                               void* out, float* lse, hipStream_t stream);

pa_status_t pa_decode_balanced_merge(void* workspace, size_t workspace_bytes, int num_seqs,
                                     int num_heads, int head_dim_v, int num_ranges, void* out,
                                     float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * pa_prefill_varlen -- varlen prefill / chunked-prefill extend over the paged
 * cache ("第 1 章 注意力后端", §3.1: prefill has many query rows per request,
 * possibly in chunks; §4.1: tiled attention with an online softmax).
 *
 * q:              [num_tokens, num_q_heads, head_dim]
 * k, v:           [num_tokens, num_kv_heads, head_dim] new rows, or both NULL
 * slot_mapping:   [num_tokens] int64, or NULL (then k, v must be NULL too)
 * query_start_loc:[num_seqs + 1] int32; request r owns query rows
 *                 query_start_loc[r] .. query_start_loc[r+1]-1, which are its
 *                 LAST L_r positions (L_r = query_start_loc[r+1] -
 *                 query_start_loc[r] <= max_query_len, L_r <= seq_lens[r]).
 * seq_lens:       [num_seqs] int32 (<= max_seq_len and <= max_blocks_per_seq *
 *                 block_size), including the L_r new positions.
 * causal:         1 = query i of request r sees keys j <= seq_len - L_r + i
 *                 (bottom-right aligned); 0 = every query sees all seq_len keys.
 * out:            [num_tokens, num_q_heads, head_dim]; lse: [num_tokens,
 *                 num_q_heads] fp32 or NULL.  A query that sees no key gets
 *                 out = 0 and lse = -inf.
 * Supported: PA_BF16, head_dim 128, num_q_heads / num_kv_heads in
 * {1, 2, 4, 8}.
 * Enqueues: the write (if k/v given), then the attention kernel.
 * ------------------------------------------------------------------------- */
pa_status_t pa_prefill_varlen(pa_dtype_t dtype,
                              const void* q, const void* k, const void* v,
                              void* kv_cache, int64_t num_blocks, int block_size,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int64_t* slot_mapping,
                              const int32_t* query_start_loc,
                              const int32_t* seq_lens, int num_seqs,
                              int num_tokens, int max_query_len, int max_seq_len,
                              int num_q_heads, int num_kv_heads, int head_dim,
                              float scale, int causal,
                              void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * pa_mla_decode -- MLA decode: the latent cache row [kv_c | k_pe] is read as
 * ONE key head shared by every query head; the query is [q_nope | q_pe]; V is
 * the first kv_lora_rank columns of the same row ("Triton 與 MLA", 設計動機 and
 * 資料流).
 *
 * q_nope: [num_seqs, num_heads, kv_lora_rank] with strides qn_stride_b /
 *         qn_stride_h (elements, last dim contiguous)
 * q_pe:   [num_seqs, num_heads, rope_dim] with strides qp_stride_b / _h
 * kv_c, k_pe: [num_seqs, kv_lora_rank] / [num_seqs, rope_dim] new rows
 *         (dense), or both NULL; slot_mapping [num_seqs] or NULL.
 * kv_cache: MLA layout [num_blocks, block_size, kv_lora_rank + rope_dim].
 * block_table, seq_lens, max_seq_len, scale: as in pa_decode.
 * num_splits: 0 = automatic: with n = pa_mla_num_kv_splits(num_seqs,
 *         max_seq_len, CUs), n == 1 runs one unsplit pass; n > 1 with out !=
 *         NULL runs the token-balanced schedule (pa_mla_decode_balanced with
 *         num_ranges = CUs, then pa_decode_balanced_merge), whose reduction
 *         order depends on the whole batch's lengths; otherwise n splits as
 *         in pa_decode (P rounded up to a multiple of block_size).
 * workspace: pa_decode_workspace_bytes(num_seqs, num_heads, kv_lora_rank, n)
 *         bytes for n splits, or for the balanced schedule
 *         pa_decode_balanced_workspace_bytes(num_seqs, num_heads, 512, CUs)
 *         bytes (16-byte aligned), as in pa_decode.
 * out:    [num_seqs, num_heads, kv_lora_rank], or NULL for the two-stage form
 *         (partials [num_seqs, num_heads, n, kv_lora_rank + 1] in the
 *         workspace); lse [num_seqs, num_heads] or NULL (NULL if out is).
 * Supported: PA_BF16 only (no dtype argument), kv_lora_rank 512 or 256 with
 * rope_dim 64 (the latent head sizes 576 and 320 of "Triton 與 MLA",
 * 邊界與失敗), num_heads a multiple of 16 up to 128, block_size a multiple of
 * 16.
 * Enqueues: the write (if given), the split (or balanced) kernel, the merge
 * kernel.
 * ------------------------------------------------------------------------- */
pa_status_t pa_mla_decode(const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                          const void* q_pe, int64_t qp_stride_b, int64_t qp_stride_h,
                          const void* kv_c, const void* k_pe,
                          void* kv_cache, int64_t num_blocks, int block_size,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int64_t* slot_mapping,
                          const int32_t* seq_lens, int num_seqs, int max_seq_len,
                          int num_heads, int kv_lora_rank, int rope_dim,
                          float scale, int num_splits,
                          void* workspace, size_t workspace_bytes,
                          void* out, float* lse, hipStream_t stream);

/* pa_mla_decode_balanced -- pa_mla_decode's reduction cut into token-balanced
 * ranges, one work-group each.  As in pa_decode_balanced the batch's 32-key
 * chunks form one list, but each request with keys is entered as 5 units of
 * overhead followed by its chunks (a request without keys adds nothing): a
 * request that starts inside a range costs that range about as much as five
 * chunks (its partial is written and the next query loaded).  With T units
 * and nr = min(num_ranges, T), range j holds the chunks whose units lie in
 * [floor(j T / nr), floor((j+1) T / nr)); a range of overhead units only does
 * nothing.  The workspace's prefix sums are of units.  Sizes: num_seqs *
 * (ceil(max_blocks_per_seq * block_size / 32) + 5) < 2^31
 * (PA_ERR_UNSUPPORTED otherwise).
 * Arguments as in pa_mla_decode (no latent write: call pa_cache_write
 * first), with num_ranges in [1, 2^24] and a 16-byte aligned workspace of
 * pa_decode_balanced_workspace_bytes(num_seqs, num_heads, 512, num_ranges)
 * bytes.  Requests inside one range are final in out / lse afterwards;
 * pa_decode_balanced_merge(..., head_dim_v = 512, ...) completes the rest. */
pa_status_t pa_mla_decode_balanced(const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                                   const void* q_pe, int64_t qp_stride_b, int64_t qp_stride_h,
                                   const void* kv_cache, int64_t num_blocks, int block_size,
                                   const int32_t* block_table, int max_blocks_per_seq,
                                   const int32_t* seq_lens, int num_seqs, int num_heads,
                                   int kv_lora_rank, int rope_dim, float scale, int num_ranges,
                                   void* workspace, size_t workspace_bytes, void* out,
                                   float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * pa_lse_merge -- merge split-KV partials by log-sum-exp ("第 1 章 注意力后端",
 * §3.1 and §4.1 Figure 5c).
 *
 * part: [num_rows, num_heads, num_splits, head_dim_v + 1] fp32; element
 *       head_dim_v of each split is that split's natural-log lse, the first
 *       head_dim_v its normalised partial output.  A split with lse = -inf
 *       weighs nothing (its output values are not read).
 * out:  [num_rows, num_heads, head_dim_v] in out_dtype:
 *       out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M), M = max lse_s.
 * lse:  [num_rows, num_heads] fp32 = M + ln sum_s exp(lse_s - M), or NULL.
 * All splits -inf: out = 0, lse = -inf.
 * Supported: head_dim_v <= 1024, num_splits >= 1.
 * ------------------------------------------------------------------------- */
pa_status_t pa_lse_merge(const float* part, int num_rows, int num_heads,
                         int num_splits, int head_dim_v, pa_dtype_t out_dtype,
                         void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Mixed batches: plan once, run per layer.
 *
 * Prefill and decode stress a kernel differently (long query chunks are a
 * matrix product, single-token decode is a bandwidth-bound gather), so a
 * backend splits a mixed batch into its decode requests and the rest, and
 * the runner orders the batch decode-first so that the two groups are
 * contiguous ("Attention Backends", section "Two kernels inside one attention
 * call").  The split and the decode group's work partition depend only on
 * the request lengths, so they are worked out once per batch and reused by
 * every layer, whose run then only reads its own q / k / v and cache
 * ("第 1 章 注意力后端", §4.2: Plan and Run, the plan reused across layers).
 *
 * pa_plan_mixed (host only, no device work) reads HOST copies of
 * query_start_loc [num_seqs + 1] and seq_lens [num_seqs] and fills *plan:
 * the decode group is the longest leading run of requests with exactly one
 * query row (later one-row requests are computed with the prefill group,
 * which gives the same result); the prefill group is every request after it.
 * Checks: query_start_loc[0] = 0 and non-decreasing; L_r <= seq_lens[r] <=
 * max_blocks_per_seq * block_size; the head configuration is one that
 * pa_decode and pa_prefill_varlen support (head_dim 128, num_q_heads /
 * num_kv_heads in {1, 2, 4, 8}); block_size a multiple of 16.
 * num_cus: compute units the decode group's schedule is sized for (as
 * pa_decode's automatic choice: one pass, n splits, or token-balanced
 * ranges); 0 = the current device's.  The run follows the plan's schedule
 * whatever device it is on.  plan->workspace_bytes is the device scratch
 * pa_mixed_attention needs (16-byte aligned).  On error *plan is all zero.
 *
 * pa_mixed_attention enqueues, in order: the new-token write of all
 * plan->num_tokens rows (if k, v, slot_mapping are given), the decode group
 * (pa_decode with the plan's split count, or pa_decode_balanced + its merge
 * with the plan's ranges), and the prefill group as pa_prefill_varlen
 * (causal) does it.  Every argument is checked before anything is enqueued.  Arguments as in pa_prefill_varlen
 * (q, k, v, out [num_tokens, ...], lse [num_tokens, num_q_heads] or NULL),
 * with num_seqs, num_tokens, head counts, block_size, max_blocks_per_seq and
 * the length maxima taken from the plan, which must have been made from the
 * same batch.  Supported: PA_BF16.
 * ------------------------------------------------------------------------- */
typedef struct {
  int num_seqs;            /* requests in the batch */
  int num_tokens;          /* query rows: query_start_loc[num_seqs] */
  int num_decode;          /* leading requests with one query row each */
  int max_decode_seq_len;  /* max seq_lens over the decode group */
  int prefill_tokens;      /* query rows of the prefill group */
  int max_query_len;       /* max L_r over the prefill group */
  int max_seq_len;         /* max seq_lens over the prefill group */
  int num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int decode_ranges;       /* token-balanced ranges of the decode group, 0 if unsplit or split */
  int decode_splits;       /* split count of the decode group (1 = one pass) */
  size_t workspace_bytes;  /* device scratch of pa_mixed_attention */
} pa_mixed_plan_t;

pa_status_t pa_plan_mixed(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                          int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                          int block_size, int max_blocks_per_seq, int num_cus,
                          pa_mixed_plan_t* plan);

pa_status_t pa_mixed_attention(const pa_mixed_plan_t* plan, pa_dtype_t dtype,
                               const void* q, const void* k, const void* v,
                               void* kv_cache, int64_t num_blocks,
                               const int32_t* block_table, const int64_t* slot_mapping,
                               const int32_t* query_start_loc, const int32_t* seq_lens,
                               float scale, void* workspace, size_t workspace_bytes,
                               void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Cascade (shared-prefix) attention.
 *
 * When every request of a batch starts with the same pages (a common system
 * prompt), attention over those pages is computed once for all query rows and
 * combined with each request's attention over the rest of its keys
 * ("Attention Backends", section "Cascade attention": the scheduler counts
 * the leading blocks common to all running requests; the shared part is
 * processed once and the per-request parts separately; it applies only when
 * every request shares the prefix).  The combination is the exact
 * log-sum-exp merge of two disjoint key sets ("第 1 章 注意力后端", §3.1
 * split-KV, §4.1 Figure 5c), so the result is the ordinary attention's up to
 * rounding.
 *
 * pa_plan_cascade (host only) reads HOST copies of query_start_loc and
 * seq_lens.  num_common_prefix_blocks = P: the first P entries of every
 * block_table row are the same pages (the caller guarantees it; the prefix is
 * read through row 0).  Checks, besides pa_plan_mixed's: every request's
 * queries lie after the prefix (seq_lens[r] - L_r >= P * block_size, so
 * every query row sees all of it) and P < max_blocks_per_seq.  The plan
 * holds the mixed-batch plan of the suffixes (seq_lens - P * block_size, same
 * rows), the prefix's key ranges and the workspace size.  P = 0 plans a
 * plain mixed batch.
 *
 * pa_cascade_attention enqueues: the new-token write of all rows (if k, v,
 * slot_mapping are given); the suffix lengths (a small kernel into the
 * workspace); the suffix pass (pa_mixed_attention's kernels over block_table
 * + P, out holding its result); the prefix pass (every query row against
 * the prefix's keys, fp32 partials into the workspace); the merge into out
 * and lse.  Arguments as in pa_mixed_attention.  Supported: PA_BF16,
 * head_dim 128, num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 * ------------------------------------------------------------------------- */
typedef struct {
  pa_mixed_plan_t suffix;      /* the batch with the prefix's keys removed */
  int prefix_blocks;           /* P */
  int prefix_len;              /* P * block_size */
  int prefix_splits;           /* key ranges of the prefix pass: about one work-group
                                  per compute unit over (KV head, 128-row tile of the
                                  num_tokens * G (token, group head) rows, range) */
  int split_keys;              /* keys per range: a multiple of 64, at least 256 unless
                                  the prefix is shorter */
  size_t workspace_bytes;      /* device scratch of pa_cascade_attention */
} pa_cascade_plan_t;

pa_status_t pa_plan_cascade(const int32_t* query_start_loc_host, const int32_t* seq_lens_host,
                            int num_seqs, int num_common_prefix_blocks, int num_q_heads,
                            int num_kv_heads, int head_dim, int block_size,
                            int max_blocks_per_seq, int num_cus, pa_cascade_plan_t* plan);

pa_status_t pa_cascade_attention(const pa_cascade_plan_t* plan, pa_dtype_t dtype,
                                 const void* q, const void* k, const void* v,
                                 void* kv_cache, int64_t num_blocks,
                                 const int32_t* block_table, const int64_t* slot_mapping,
                                 const int32_t* query_start_loc, const int32_t* seq_lens,
                                 float scale, void* workspace, size_t workspace_bytes,
                                 void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * FP8 KV cache with per-tensor scales.
 *
 * The cache holds one E4M3 byte per element instead of a bf16 pair: a key
 * element is stored as code = E4M3(k / k_scale) and read back as
 * E4M3(code) * k_scale (values likewise with v_scale); the query and the
 * output stay bf16 ("Triton 與 MLA", 資料流: the layer's k_scale / v_scale are
 * passed to the kernel, v_scale = k_scale for the latent cache; 邊界與失敗:
 * with an FP8 cache the kernel dequantises and the query is not quantised).
 * Format: OCP FP8 E4M3 (bias 7, 3 mantissa bits, largest finite 448, no
 * infinities).  Quantisation: the quotient in fp32 (correctly rounded), then
 * the nearest E4M3 value, ties to even, magnitudes above 448 saturated.
 * Layouts are the bf16 ones with 1-byte elements: GQA [num_blocks, 2,
 * block_size, num_kv_heads, head_dim] uint8, MLA [num_blocks, block_size,
 * kv_lora_rank + rope_dim] uint8.  Scales: finite and > 0.
 *
 * pa_cache_write_fp8: pa_cache_write with bf16 inputs quantised on the way
 * in (layout PA_LAYOUT_KV: k with k_scale, v with v_scale; PA_LAYOUT_MLA:
 * k = kv_c, v = k_pe, the whole row with k_scale, v_scale unused).
 *
 * pa_decode_fp8: GQA decode (one query row per request, as pa_decode) over
 * an FP8 cache, on the token-balanced schedule: num_ranges = 0 picks
 * pa_decode_balanced_num_ranges(num_kv_heads, pa_device_num_cus());
 * workspace of pa_decode_balanced_workspace_bytes(num_seqs, num_q_heads,
 * head_dim, num_ranges) bytes, 16-byte aligned.  Enqueues the write (if k,
 * v, slot_mapping are given), the decode kernel and the segment merge.
 * q [num_seqs, num_q_heads, 128] bf16, out the same, lse [num_seqs,
 * num_q_heads] fp32 or NULL.  Supported: head_dim 128, num_q_heads /
 * num_kv_heads in {1, 2, 4, 8}, num_kv_heads 1, 2, 4 or a multiple of 8.
 * ------------------------------------------------------------------------- */
pa_status_t pa_cache_write_fp8(pa_layout_t layout,
                               const void* k, int64_t k_token_stride,
                               const void* v, int64_t v_token_stride,
                               void* kv_cache, int64_t num_blocks, int block_size,
                               int num_kv_heads, int head_dim,
                               const int64_t* slot_mapping, int num_tokens,
                               float k_scale, float v_scale, hipStream_t stream);

/* pa_mla_decode_fp8: MLA decode (as pa_mla_decode) over an FP8 latent cache
 * [num_blocks, block_size, kv_lora_rank + rope_dim] uint8 with one scale for
 * the row (kv_scale: keys and values alike), on the token-balanced schedule
 * of pa_mla_decode_balanced (the same ranges, 5 overhead units per request;
 * num_ranges = 0: one range per compute unit of the current device),
 * workspace of pa_decode_balanced_workspace_bytes(num_seqs, num_heads,
 * kv_lora_rank, num_ranges) bytes.  Enqueues the write of kv_c / k_pe (if
 * given, quantised with kv_scale), the decode kernel and the segment merge.
 * q_nope / q_pe bf16 with the strides of pa_mla_decode; out [num_seqs,
 * num_heads, kv_lora_rank] bf16; lse fp32 or NULL.  Supported: kv_lora_rank
 * 512, rope_dim 64, num_heads a multiple of 16 up to 128. */
pa_status_t pa_mla_decode_fp8(const void* q_nope, int64_t qn_stride_b, int64_t qn_stride_h,
                              const void* q_pe, int64_t qp_stride_b, int64_t qp_stride_h,
                              const void* kv_c, const void* k_pe,
                              void* kv_cache, int64_t num_blocks, int block_size,
                              const int32_t* block_table, int max_blocks_per_seq,
                              const int64_t* slot_mapping, const int32_t* seq_lens, int num_seqs,
                              int num_heads, int kv_lora_rank, int rope_dim,
                              float scale, float kv_scale, int num_ranges,
                              void* workspace, size_t workspace_bytes,
                              void* out, float* lse, hipStream_t stream);

/* pa_prefill_varlen_fp8: pa_prefill_varlen over an FP8 GQA cache
 * [num_blocks, 2, block_size, num_kv_heads, head_dim] uint8 with per-tensor
 * k_scale / v_scale; q, new k / v rows (quantised on the write) and out are
 * bf16.  Same arguments otherwise; head_dim 128, num_q_heads / num_kv_heads
 * in {1, 2, 4, 8}. */
pa_status_t pa_prefill_varlen_fp8(const void* q, const void* k, const void* v,
                                  void* kv_cache, int64_t num_blocks, int block_size,
                                  const int32_t* block_table, int max_blocks_per_seq,
                                  const int64_t* slot_mapping,
                                  const int32_t* query_start_loc,
                                  const int32_t* seq_lens, int num_seqs,
                                  int num_tokens, int max_query_len, int max_seq_len,
                                  int num_q_heads, int num_kv_heads, int head_dim,
                                  float scale, float k_scale, float v_scale, int causal,
                                  void* out, float* lse, hipStream_t stream);

pa_status_t pa_decode_fp8(const void* q, const void* k, const void* v,
                          void* kv_cache, int64_t num_blocks, int block_size,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int64_t* slot_mapping, const int32_t* seq_lens, int num_seqs,
                          int num_q_heads, int num_kv_heads, int head_dim,
                          float scale, float k_scale, float v_scale, int num_ranges,
                          void* workspace, size_t workspace_bytes,
                          void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * MLA prefill: the multi-head form over the latent cache.
 *
 * Decode reads the latent rows directly (pa_mla_decode: one key head of
 * kv_lora_rank + rope dims); prefill has many queries per key, and the
 * multi-head form is cheaper there: every key's latent part is projected by
 * kv_b_proj into per-head keys and values, and each head attends as ordinary
 * causal attention ("Triton 與 MLA", 設計動機 and 關鍵檔案: the layer holds
 * kv_b_proj, qk_nope_head_dim, qk_rope_head_dim, kv_lora_rank and has a
 * separate multi-head entry point; "Attention Backends", latent attention:
 * prefill and decode use different formulations of the same mathematics).
 * Per head h: key_j = [W_k[h] kv_c_j | k_pe_j], value_j = W_v[h] kv_c_j, with
 * the weight stored as a linear layer stores it.
 *
 * q:           [num_tokens, num_heads, qk_nope_dim + rope_dim] bf16 at element
 *              strides (q_stride_t, q_stride_h), last dim contiguous
 * kv_c, k_pe:  new latent rows [num_tokens, kv_lora_rank], [num_tokens,
 *              rope_dim] bf16 written at slot_mapping first, or all NULL
 * kv_cache:    latent cache [num_blocks, block_size, kv_lora_rank + rope_dim]
 * query_start_loc, seq_lens, block_table: as pa_prefill_varlen (causal,
 *              bottom-right aligned)
 * total_keys:  host copy of the sum of seq_lens (every key is projected once)
 * w_kv_b:      [num_heads * (qk_nope_dim + v_head_dim), kv_lora_rank] bf16:
 *              head h's rows h * 256 .. h * 256 + 127 expand keys, the next 128
 *              values
 * workspace:   pa_mla_prefill_workspace_bytes(num_seqs, total_keys, num_heads)
 *              bytes, 256-byte aligned: key offsets, the attention's work
 *              list (one entry per 128-query tile, longest first; sized for
 *              num_seqs + total_keys / 128 + 1 tiles, which holds whenever every
 *              seq_lens[r] counts request r's queries), and the projected keys
 *              [total_keys, num_heads, 192] and values [total_keys, num_heads,
 *              128], bf16 (the projection's output dtype)
 * out:         [num_tokens, num_heads, v_head_dim] bf16; lse [num_tokens,
 *              num_heads] fp32 or NULL
 * Supported: kv_lora_rank 512, rope_dim 64, qk_nope_dim 128, v_head_dim 128.
 * Enqueues: the latent write (if given), the key offsets and work list, the
 * projection and the attention.
 * ------------------------------------------------------------------------- */
size_t pa_mla_prefill_workspace_bytes(int num_seqs, int total_keys, int num_heads);

pa_status_t pa_mla_prefill(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                           const void* kv_c, const void* k_pe,
                           void* kv_cache, int64_t num_blocks, int block_size,
                           const int32_t* block_table, int max_blocks_per_seq,
                           const int64_t* slot_mapping,
                           const int32_t* query_start_loc, const int32_t* seq_lens, int num_seqs,
                           int num_tokens, int max_query_len, int total_keys,
                           const void* w_kv_b, int num_heads, int kv_lora_rank, int rope_dim,
                           int qk_nope_dim, int v_head_dim, float scale,
                           void* workspace, size_t workspace_bytes,
                           void* out, float* lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
