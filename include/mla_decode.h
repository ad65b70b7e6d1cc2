/*
 * mla_decode.h — C ABI of the MI355X (gfx950) dense MLA decode library.
 *
 * Computes weight-absorbed Multi-head Latent Attention decode over a paged
 * KV cache, as defined on the "[DeepSeek-3] FlashMLA" overview page
 * (xutianle.me), sections 3 and 4:
 *
 *   for every request b, query token s < s_q, head h < h_q:
 *     L       = cache_seqlens[b]
 *     K_b[t]  = kv_cache[block_table[b][t / 64], t % 64, 0, 0:576]   (t < L)
 *     score_t = softmax_scale * dot(q[b,s,h,0:576], K_b[t])
 *     out[b,s,h,c] = sum_t softmax(score)_t * K_b[t][c]               (c < 512)
 *     lse[b,h,s]   = log(sum_t exp(score_t))                         (natural log)
 *
 * Work is cut into split-KV pieces by a tile planner (FlashMLA new-kernel
 * deep-dive page, nxmr.cn, section "Tile Scheduler"), each piece is reduced
 * with online softmax, and pieces of one request are merged with the
 * log-sum-exp rule (attention-kernel page, online-softmax section).
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense, row-major, with exactly the shapes given.
 *   - bf16 data is passed as raw 16-bit patterns (void* / uint16_t*).
 *   - "device" pointers are HIP device memory owned by the caller; the
 *     library never frees or retains them past the call.
 *   - Entry points return 0 on success or a negative MLA_ERR_* code; the
 *     message for the last failure on the calling thread is returned by
 *     mla_last_error().  Nothing is launched when an argument check fails.
 *   - Query row r = s * h_q + h (the pages' s_q*h_q rows per KV head).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_INVALID = -1,    /* bad dimension, null pointer, negative length */
  MLA_ERR_CAPACITY = -2,   /* an output buffer is too small */
  MLA_ERR_WORKSPACE = -3,  /* workspace smaller than mla_workspace_bytes() */
  MLA_ERR_HIP = -4         /* a HIP runtime call or kernel launch failed */
};

/* Rows of the per-part schedule table: 8 int32 per part,
 *   [begin_req, end_req (inclusive), begin_block (within begin_req),
 *    end_block (exclusive, within end_req), begin_piece, max_pieces,
 *    first_page, 0]
 * begin_piece is the index, among begin_req's pieces, of the piece this part
 * holds; max_pieces (equal in every row) is the largest number of pieces of
 * any request, which the merge kernel uses to pick its work layout;
 * first_page is 0, or 1 + the block id of the part's first page once the
 * block table is attached (mla_plan_attach_pages, or mla_get_metadata_device
 * given the table).  num_splits is an exclusive prefix sum of pieces per request,
 * length batch + 1: request b owns partial slots [num_splits[b], num_splits[b+1]). */
#define MLA_SCHED_INTS 8

/*
 * mla_plan — split/tile planner (host only, no GPU call).
 *
 * Follows the tile-scheduler description on the new-kernel deep-dive page:
 * n_b = ceil(L_b / 64) KV blocks per request; payload =
 * ceil(sum_b (n_b + F) / num_parts) + F; requests are walked in order and
 * each part is filled up to the payload, a request that does not fit being
 * cut at a block boundary (every piece costs its blocks plus F).  The last
 * part takes whatever remains.  Then (a step of our own, not the page's)
 * each run of consecutive parts that hold one request alone shares that run's
 * blocks evenly, earlier parts one block longer; parts, piece indices and
 * split counts stay the walk's.  force_splits > 0 instead cuts every request
 * into min(force_splits, n_b) (at least 1) page-aligned pieces, one part each.
 *
 *   cache_seqlens  host int32 [batch], each >= 0
 *   num_parts      > 0, number of parts the walk may fill
 *   fixed_overhead F >= 0, per-piece overhead in blocks
 *   sched_out      host int32 [max_parts * 8]
 *   num_splits_out host int32 [batch + 1]
 *   num_parts_out  parts actually written (<= num_parts, or pieces when forced)
 * Errors: MLA_ERR_INVALID (batch <= 0, a length < 0, null pointer),
 *         MLA_ERR_CAPACITY (more parts than max_parts).
 */
int mla_plan(const int32_t* cache_seqlens, int batch, int num_parts, int fixed_overhead,
             int force_splits, int32_t* sched_out, int max_parts, int32_t* num_splits_out,
             int* num_parts_out);

/*
 * mla_get_metadata — plan one decode step (the pages' get_mla_metadata).
 *
 * Chooses num_parts and the fixed overhead from the CU count, the
 * query-row count R = s_q * h_q and the cache format, then calls mla_plan.
 * The plan stays valid for every call (e.g. every layer of one decode step)
 * with the same batch, s_q, h_q, cache format and cache_seqlens
 * ("[DeepSeek-3] FlashMLA", section 5, whose get_mla_metadata also takes the
 * FP8 flag: the launch geometry depends on it).
 *
 *   cache_seqlens  host int32 [batch]
 *   is_fp8         0: bf16 cache, 1: FP8 records (see MLA_FP8_RECORD); must
 *                  match the is_fp8 of the mla_decode_fwd calls the plan
 *                  serves (another plan is still correct, only slower)
 *   num_cus        CUs to fill; 0 = query the current HIP device
 *   force_splits   0 = greedy planner, k > 0 = k pieces per request (testing)
 *   sched_out      host int32 [max_parts * 8]; max_parts >= mla_max_parts(...)
 *   num_splits_out host int32 [batch + 1]
 *   num_parts_out, total_splits_out  parts written, partial slots needed
 * Errors: MLA_ERR_INVALID, MLA_ERR_CAPACITY, MLA_ERR_HIP (device query).
 */
int mla_get_metadata(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int is_fp8, int num_cus,
                     int force_splits, int32_t* sched_out, int max_parts,
                     int32_t* num_splits_out, int* num_parts_out, int* total_splits_out);

/*
 * mla_plan_attach_pages — write into a host plan the block id of every part's
 * first page (column 6: 1 + block_table[begin_req][begin_block], or 0 when
 * the part has no work or its first piece holds no page).  The small-row
 * split-KV kernel then issues that page's copy (and the query rows') as soon
 * as it has read its plan row, one dependent round trip earlier than through
 * the block table (the pages' tile scheduler hands each CTA its start the same
 * way, "FlashMLA new-kernel deep dive", Tile Scheduler).  An attached plan is
 * valid for the calls whose block table holds the same ids at those
 * positions (within one decode step the table is shared by every layer);
 * results are bitwise those of the plain plan.
 *
 *   sched          host int32 [num_parts * 8], from mla_get_metadata
 *   cache_seqlens  host int32 [batch], the lengths the plan was made for
 *   block_table    host int32 [batch, max_blocks_per_seq], the decode calls' table
 *   num_blocks     the pool's block count (ids must lie in [0, num_blocks))
 * Errors: MLA_ERR_INVALID (null pointers, sizes <= 0, a row naming requests
 *         outside [0, batch), a first page past max_blocks_per_seq, an id
 *         outside the pool).
 */
int mla_plan_attach_pages(int32_t* sched, int num_parts, const int32_t* cache_seqlens, int batch,
                          const int32_t* block_table, int max_blocks_per_seq, int num_blocks);

/*
 * mla_get_metadata_device — the same plan as mla_get_metadata (greedy walk,
 * no force_splits) computed on the GPU from device lengths, enqueued on
 * `stream` (the pages run their tile scheduler as a one-warp kernel,
 * "FlashMLA new-kernel deep dive", Tile Scheduler), so that a captured
 * decode step (planner + mla_decode_fwd) replans whenever the lengths in
 * device memory change, with no host round trip.
 *
 *   cache_seqlens_dev device int32 [batch] (read when the kernel runs;
 *                     negative lengths count as 0)
 *   is_fp8            the cache format, as for mla_get_metadata
 *   num_cus           CUs to fill; 0 = query the current HIP device
 *   sched_dev         device int32 [max_parts * 8]; max_parts >= the policy's
 *                     part count (mla_max_parts(..., force_splits = 0))
 *   num_splits_dev    device int32 [batch + 1]
 *   block_table_dev   device int32 [batch, max_blocks_per_seq] or NULL: with
 *                     a table the plan carries each part's first page
 *                     (column 6, as mla_plan_attach_pages writes it; ids
 *                     outside [0, num_blocks) are left unattached), read
 *                     when the kernel runs
 *   num_parts_out     host: the rows written = the policy's part count, the
 *                     num_parts to pass to mla_decode_fwd; rows after the
 *                     walk's last part are empty (begin_req 1 > end_req 0)
 *   stream            hipStream_t (NULL = the null stream)
 * A plan's partial slots never exceed num_parts + batch - 1, so a workspace of
 * mla_workspace_bytes(num_parts + batch - 1, h_q, s_q) fits any lengths.
 * Allocates nothing, does not synchronise; batch <= 65536 and the policy's
 * part count <= 4096 (one workgroup; LDS holds where each part begins).
 * Errors: MLA_ERR_INVALID (also for the limits above, and a table with
 *         max_blocks_per_seq or num_blocks <= 0), MLA_ERR_CAPACITY,
 *         MLA_ERR_HIP.
 */
int mla_get_metadata_device(const int32_t* cache_seqlens_dev, int batch, int h_q, int s_q, int is_fp8,
                            int num_cus, int32_t* sched_dev, int max_parts, int32_t* num_splits_dev,
                            const int32_t* block_table_dev, int max_blocks_per_seq, int num_blocks,
                            int* num_parts_out, void* stream);

/* Upper bound on the parts mla_get_metadata can emit for these sizes. */
int mla_max_parts(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int is_fp8, int num_cus,
                  int force_splits);

/*
 * mla_workspace_bytes — device scratch needed by mla_decode_fwd for a plan
 * with total_splits partial slots, R = s_q * h_q: fp32 partial outputs
 * [total_splits, R, 512] (row-major: one query row's 512 values contiguous)
 * and fp32 base-2 partial lse [total_splits, R], each region 256-byte aligned
 * (the split-KV workspace of the split-KV blog, 0539edu.com, section 3.1).
 * Any plan has total_splits <= num_parts + batch - 1.  The caller allocates
 * it; its contents need no initialisation and are scratch after the call.
 */
size_t mla_workspace_bytes(int total_splits, int h_q, int s_q);

/*
 * mla_decode_fwd — dense MLA decode forward (the pages' flash_mla_with_kvcache,
 * dense path, bf16, one KV head, head_dim_v = 512).
 *
 *   q             device bf16 [batch, s_q, h_q, 576]
 *   kv_cache      device bf16 [num_blocks, 64, 1, 576]; K = all 576 dims,
 *                 V = the first 512 dims of the same rows
 *   block_table   device int32 [batch, max_blocks_per_seq]; entries for
 *                 logical pages >= ceil(L/64) are never read
 *   cache_seqlens device int32 [batch]; must equal the lengths the plan was
 *                 made from, and L <= 64 * max_blocks_per_seq
 *   softmax_scale multiplies the q.k scores; finite and >= 0
 *   is_fp8        0: kv_cache is bf16 as above; 1: kv_cache holds FP8
 *                 records, uint8 [num_blocks, 64, 1, 656] (see MLA_FP8_RECORD)
 *   causal        0: every query token sees all L keys (the dense path);
 *                 1: the s_q query tokens are the last s_q positions of the
 *                 sequence (multi-token prediction), so token s sees keys
 *                 0 .. L - s_q + s (the pages' is_causal flag, "FlashMLA
 *                 new-kernel deep dive", API section); a token that sees no
 *                 key gets out = 0, lse = -inf
 *   sched         device int32 [num_parts, 8] from mla_get_metadata/mla_plan
 *                 (or mla_get_metadata_device); if it carries first pages
 *                 (mla_plan_attach_pages), block_table must hold the same
 *                 ids at those positions
 *   num_splits    device int32 [batch + 1] from the same plan
 *   workspace     device, >= mla_workspace_bytes(num_parts + batch - 1, h_q, s_q)
 *                 bytes (the bound on partial slots of any plan with num_parts)
 *   out           device bf16 [batch, s_q, h_q, 512] (written)
 *   lse           device fp32 [batch, h_q, s_q] (written; -inf when L = 0)
 *   stream        hipStream_t to enqueue on (NULL = the null stream)
 *
 * Enqueues the split-KV kernel (one of three, by R: <= 16, < 128, >= 128;
 * with an FP8 cache every R above 16 takes the 128-row kernel),
 * then the combine kernel (which returns at once when no request is split,
 * and skips the rows of requests that are not); returns without
 * synchronising and allocates nothing.  Block-table
 * entries must lie in [0, num_blocks) and the device lengths must match the
 * plan: neither is checked on the device (undefined behaviour otherwise).
 * Errors: MLA_ERR_INVALID, MLA_ERR_WORKSPACE, MLA_ERR_HIP.
 */
int mla_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table,
                   const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_blocks,
                   int max_blocks_per_seq, float softmax_scale, int causal, int is_fp8,
                   const int32_t* sched, int num_parts, const int32_t* num_splits, void* workspace,
                   size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * mla_decode_fwd_noalloc — mla_decode_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, computation and
 * results, without the workspace.  The split partials live in a
 * library-owned device array of MLA_NOALLOC_SCRATCH_BYTES per GPU, placed
 * when the library's code object is loaded on that GPU and held until the
 * process ends.  The caller still passes (and owns) inputs and outputs.
 *
 *   Sizes: a plan fits iff mla_workspace_bytes(num_parts + batch - 1, h_q,
 *   s_q) <= MLA_NOALLOC_SCRATCH_BYTES (e.g. batch 16 x 16 heads on 256
 *   parts: 8.9 MB; batch 64 x 128 heads: 84 MB; batch 128 x 2 x 128 rows:
 *   134 MB, too large); larger plans return MLA_ERR_WORKSPACE and launch
 *   nothing.
 *   Allocates nothing: no hipMalloc / hipFree or allocating library call.
 *   The first call on a device (with that device current; the stream must
 *   belong to it) looks up the array's device address once.
 *   Sharing: every call on one GPU uses that GPU's one array, so calls that
 *   overlap on a GPU (several streams or threads) race on it; serialise
 *   them.  Nothing in the array needs to start at any value (every partial
 *   slot a call reads was written earlier in the same call).
 * Errors: as mla_decode_fwd, and MLA_ERR_WORKSPACE for plans that do not fit.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (128u << 20)
int mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                           const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_blocks,
                           int max_blocks_per_seq, float softmax_scale, int causal, int is_fp8, const int32_t* sched,
                           int num_parts, const int32_t* num_splits, void* out, float* lse, void* stream);

/*
 * FP8 cache ("[DeepSeek-3] FlashMLA", section 12), accepted by both decode
 * entry points when is_fp8 = 1: each token is a 656-byte record
 *   bytes   0 .. 511  latent dims 0 .. 511 as float8 e4m3 (OCP e4m3fn)
 *   bytes 512 .. 527  four fp32 scales, scale i for dims 128 i .. 128 i + 127
 *   bytes 528 .. 655  RoPE dims 512 .. 575 as bf16
 * and a 64-token page is 64 consecutive records (41,984 bytes).  The method
 * computes with the dequantized cache: latent value =
 * bf16_rne(fp32(e4m3 * scale)), RoPE as stored (the pages dequantize to
 * bf16 and run bf16 matrix products with fp32 accumulation).
 */
#define MLA_FP8_RECORD 656

/*
 * Sparse (top-k) decode ("[DeepSeek-3] FlashMLA", section 11): query token s
 * of request b attends only to the cache rows its index list names,
 *
 *   indices[b][s][i] = page_id * 64 + offset   (cache row `offset` of block
 *                                               `page_id`; no block table)
 *
 * with the dense path's score, softmax and output definitions.  Readings of
 * points the pages leave open: the list is a multiset (a row named twice is
 * two keys); only the first topk_length[b] entries of request b's lists
 * count (all topk when topk_length is NULL; values are clamped to
 * [0, topk]); an entry outside [0, num_blocks * 64), -1 padding for
 * example, names no key and is never dereferenced; a query token left with
 * no key gets out = 0 and lse = -inf.  There is no causal mask (the
 * selector decides what each token sees).
 *
 * The split-KV kernels treat each (request, query token) as one request of
 * h_q query rows whose 64-token "pages" are consecutive runs of its list, so
 * the planner walks batch * s_q lengths.
 */

/* Part count of the sparse planner policy (the max_parts a plan needs). */
int mla_max_parts_sparse(int batch, int s_q, int h_q, int num_cus);

/*
 * mla_get_metadata_sparse — plan one sparse decode step (host only).
 *
 *   topk_length    host int32 [batch] or NULL
 *   topk           entries per index list (> 0)
 *   num_cus        CUs to fill; 0 = query the current HIP device
 *   sched_out      host int32 [max_parts * 8]; max_parts >= mla_max_parts_sparse(...)
 *   num_splits_out host int32 [batch * s_q + 1]: prefix of pieces over
 *                  (request, query token) pairs in the order b * s_q + s
 *   num_parts_out, total_splits_out  parts written, partial slots needed
 * Errors: MLA_ERR_INVALID, MLA_ERR_CAPACITY, MLA_ERR_HIP (device query).
 */
int mla_get_metadata_sparse(const int32_t* topk_length, int batch, int s_q, int h_q, int topk, int num_cus,
                            int32_t* sched_out, int max_parts, int32_t* num_splits_out, int* num_parts_out,
                            int* total_splits_out);

/*
 * mla_decode_sparse_fwd — sparse MLA decode forward (the pages'
 * flash_mla_with_kvcache with indices, bf16 cache, head_dim_v = 512).
 *
 *   q             device bf16 [batch, s_q, h_q, 576]
 *   kv_cache      device bf16 [num_blocks, 64, 1, 576], or with is_fp8 = 1 the
 *                 FP8 records uint8 [num_blocks, 64, 1, 656]; num_blocks <= 2^24
 *   indices       device int32 [batch, s_q, topk]
 *   topk_length   device int32 [batch] or NULL
 *   softmax_scale finite and >= 0
 *   is_fp8        0 or 1 (the cache format, as above)
 *   sched, num_parts, num_splits  from mla_get_metadata_sparse with the same
 *                 batch, s_q, h_q, topk and topk_length
 *   workspace     device, >= mla_workspace_bytes(num_parts + batch * s_q - 1, h_q, 1)
 *   out           device bf16 [batch, s_q, h_q, 512] (written)
 *   lse           device fp32 [batch, h_q, s_q] (written)
 *   stream        hipStream_t (NULL = the null stream)
 * Enqueues the split-KV kernel (gathered copies; h_q <= 16 rows in one
 * workgroup, otherwise 128-row workgroups) and the combine kernel; returns
 * without synchronising and allocates nothing.  The device topk_length must
 * match the plan (not checked on the device).
 * Errors: MLA_ERR_INVALID, MLA_ERR_WORKSPACE, MLA_ERR_HIP.
 */
int mla_decode_sparse_fwd(const void* q, const void* kv_cache, const int32_t* indices, const int32_t* topk_length,
                          int batch, int s_q, int h_q, int num_blocks, int topk, float softmax_scale, int is_fp8,
                          const int32_t* sched, int num_parts, const int32_t* num_splits, void* workspace,
                          size_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * Kernel timing for benchmarks.  mla_profile_start(max_calls) makes the next
 * max_calls mla_decode_fwd calls (any thread) record HIP events on their
 * stream around the split-KV kernel and around the combine kernel.
 * mla_profile_stop waits for the last recorded event and returns the summed
 * device milliseconds of each kernel and the number of calls recorded, then
 * releases the events.  Errors: MLA_ERR_INVALID (max_calls <= 0, null
 * outputs, start while started), MLA_ERR_HIP.
 */
int mla_profile_start(int max_calls);
int mla_profile_stop(float* main_ms, float* combine_ms, int* calls);

/* Message for the last non-zero return on this thread ("" if none). */
const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H */
