/*
 * msa_indexer.h -- C ABI of the decode-time sparse-attention block indexer
 * for AMD Instinct MI355X (gfx950).
 *
 * The library runs one decode step of a sparse-attention block indexer on one
 * GPU. There are three stream-ordered steps (steps 1 and 2 can also run as
 * one launch, msa_score_select, and so can steps 2 and 3,
 * msa_top16_select_merge):
 *
 *   1. msa_score_decode: the score plane. Each decode token's 4 fp8 index
 *      heads are scored against the paged fp8 index-K cache, with one column
 *      per 128-token (B128) block.
 *   2. msa_top16_select: per (token, head) row, or per column range of the
 *      row, the forced blocks at both ends plus the best remaining blocks;
 *      each kept block contributes its unscaled score and its id, and the
 *      ids increase along the row.
 *   3. msa_top16_merge: merges the per-range Top16 lists of a row into one.
 *
 * The operations follow the FlashInfer msa_ops API pages:
 *   "flashinfer.msa_ops.msa_icp_decode_index_score_sharded"  (step 1)
 *   "flashinfer.msa_ops.msa_icp_topk_select_publish"         (step 2, row format)
 *   "flashinfer.msa_ops.prepare_msa_icp_indexer"             (the decode chain
 *       score -> select -> merge; forced init/local blocks)
 * By default one GPU holds every page's full rows. Three entry points serve
 * one rank's share of a cache whose pages are split by rows over 2 or 4
 * ranks (the pages' sharded layout): msa_score_decode_sharded,
 * msa_top16_select_mapped and msa_top16_merge_dedup. There is no peer
 * publish or receive row: the rows stay on this GPU.
 *
 * Conventions for every entry point:
 *  - Pointers named as device buffers are device memory that the caller
 *    allocates and owns. The library never allocates, frees or synchronises.
 *    It enqueues its kernels on `stream` and returns before they run.
 *    Inputs are only read.
 *  - Return value: MSA_OK (0) on success. MSA_ERR_INVALID_ARG (-1) if a
 *    host-checkable precondition fails; nothing is launched in that case and
 *    msa_last_error() describes the failed check. MSA_ERR_LAUNCH (-2) if the
 *    HIP runtime refuses a launch.
 *  - `errors` (nullable, device int32[>= 1]) counts violations of conditions
 *    that only the device can see, by atomic increments. Examples are a
 *    block_table entry outside [0, num_pages), or num_valid_pages outside
 *    [0, cols]. The kernel then clamps or skips the offending input and
 *    writes a defined result. It never traps. The counter is not reset.
 *  - Inputs must not hold e4m3fn NaN codes (0x7F, 0xFF). Results are then
 *    unspecified.
 */
#ifndef MSA_INDEXER_H
#define MSA_INDEXER_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1)
#define MSA_ERR_LAUNCH (-2)

#define MSA_NUM_HEADS 4          /* index heads (prepare_msa_icp_indexer: num_index_heads) */
#define MSA_HEAD_DIM 128         /* index head dim (index_q / index_k last dimension)      */
#define MSA_BLOCK_TOKENS 128     /* tokens per B128 block = one score-plane column          */
#define MSA_TOPK 16              /* entries per Top16 row                                  */
#define MSA_MAX_SCORE_COLS 8192  /* score_out: 0 < cols <= 8192, cols % 4 == 0             */
#define MSA_MAX_SELECT_COLS 12287 /* select scores: 0 < K < 12288                          */
#define MSA_MAX_RANGES 768       /* column ranges per row (16 * 768 = 12288 merge entries) */
#define MSA_STREAM_PROBE_SINK_WORDS 1024   /* uint32 words of msa_stream_read_probe's sink */
#define MSA_STREAM_PROBE_PERSISTENT 0      /* msa_stream_read_probe's persistent shape     */
#define MSA_PREFILL_WINDOW_TOKENS 64       /* query tokens per prefill window              */
#define MSA_PREFILL_PLAN_HEADER_WORDS 8    /* int32 words before a prefill plan's items    */
#define MSA_PREFILL_ITEM_WORDS 8           /* int32 words per prefill plan item            */
#define MSA_PREFILL_MAX_BATCH 8192         /* requests one prefill plan takes              */
#define MSA_NOALLOC_SCRATCH_WORDS (4 * 1024 * 1024) /* int32 words (16 MiB per device) of
                                                       msa_score_select_noalloc's workspace */

/*
 * One Top16 row (128 bytes). score[i] is the score-plane value of block
 * id[i], unscaled. Ids ascend. Unused slots hold (score -inf, id -1) and
 * follow the used ones. Source: "msa_icp_topk_select_publish", description
 * (the row carries sixteen scores and sixteen increasing block ids). The
 * page's row also has a ready flag or generation tags; those belong to the
 * cross-GPU publish, which this library does not have.
 */
typedef struct msa_top16_row {
    float score[MSA_TOPK];
    int32_t id[MSA_TOPK];
} msa_top16_row;

/*
 * Step 1: the score plane.
 * Source: "msa_icp_decode_index_score_sharded" (description; parameters
 * index_q, index_k, block_table, seq_lens, score_out, page_size,
 * decode_query_len).
 *
 * index_q      device, e4m3fn bytes [batch * decode_query_len, 4, 128], contiguous,
 *              16-byte aligned. Token j of request b is row b*decode_query_len + j.
 *              Its position is seq_lens[b] - decode_query_len + j.
 * index_k      device, e4m3fn bytes [num_pages, page_size, 128], contiguous,
 *              16-byte aligned. Key p of request b is row p % page_size of page
 *              block_table[b, p / page_size].
 * block_table  device int32, read as [batch, block_table_stride] rows with unit last
 *              stride. Request b uses entries [0, ceil(seq_len/page_size)). An entry it
 *              needs at or past the row stride, or outside [0, num_pages), is counted
 *              in `errors`, and that block scores -inf.
 * seq_lens     device int32 [batch]. A request with seq_len <= 0 writes nothing.
 * page_size    128 or 256.
 * decode_query_len  1 <= len and 4*len <= 32.
 * score_out    device float32 [batch*decode_query_len, 4, cols], contiguous,
 *              16-byte aligned, 0 < cols <= 8192, cols % 4 == 0.
 *
 * Writes score_out[t, h, c] for every token t of request b and every column
 * c < W_b = min(roundup4(ceil(seq_len_b / 128)), cols). A W_b that cols cuts
 * short is counted in `errors`. Columns c >= W_b are not touched. The value
 * is the maximum, over keys p of block c (128c <= p < 128c + 128) with
 * p < seq_len and p <= the token's position, of the dot product of the
 * token's head row with key p's row (fp8 products, fp32 accumulation). It is
 * -inf if no key of the block qualifies, which includes the padding columns
 * [ceil(seq_len/128), W_b).
 */
int msa_score_decode(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                     const int32_t* block_table, int64_t block_table_stride,
                     const int32_t* seq_lens, int32_t batch, int32_t page_size,
                     int32_t decode_query_len, float* score_out, int32_t cols, int32_t* errors,
                     hipStream_t stream);

/*
 * Step 1 on one rank of a row-sharded cache.
 * Source: "msa_icp_decode_index_score_sharded" (description: the written
 * columns, and the global block a column stands for at page_size 256;
 * index_k: the [pages, page_size / world_size, 128] shard; rank, world_size;
 * Layout: world_size 2 or 4).
 *
 * Arguments are those of msa_score_decode, except:
 * index_k_shard  device, e4m3fn bytes [num_pages, page_size / world_size, 128], contiguous,
 *                16-byte aligned: rows [rank*R, rank*R + R) of every page,
 *                R = page_size / world_size.
 * rank, world_size  world_size 2 or 4, 0 <= rank < world_size.
 *
 * Column c of request b is the request's page c (block_table[b, c]). Its keys
 * on this rank are the positions p = c*page_size + rank*R + i, i < R: part of
 * global B128 block c at page_size 128, part of global block
 * 2c + rank*2/world_size at 256. Writes columns c < min(roundup4(ceil(seq_len /
 * page_size)), cols) (a W cut short by cols is counted in `errors`); other
 * columns are not touched. The value is the maximum, over those keys with
 * p < seq_len and p <= the token's position, of the dot product (fp8 products,
 * fp32 accumulation), or -inf if there is none. The maximum over the ranks that
 * hold a block's rows is that block's msa_score_decode column.
 */
int msa_score_decode_sharded(const uint8_t* index_q, const uint8_t* index_k_shard,
                             int64_t num_pages, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                             int32_t page_size, int32_t decode_query_len, int32_t rank,
                             int32_t world_size, float* score_out, int32_t cols, int32_t* errors,
                             hipStream_t stream);

/*
 * int32 words of msa_score_select's workspace for these sizes (host only):
 * one 128-byte counter line per (request, column range), per-(token, head)
 * merge tickets, and, with with_pool != 0 (score_out == NULL), the pool plane
 * of batch * decode_query_len * 4 * cols floats. Returns MSA_ERR_INVALID_ARG for
 * sizes msa_score_select would reject.
 */
int64_t msa_score_select_workspace_words(int32_t batch, int32_t decode_query_len, int32_t cols,
                                         int32_t num_ranges, int32_t with_pool);

/*
 * Steps 1 and 2 in one launch (and step 3 when `merged` is given): the score
 * plane, Top16 select per (token, head, column range), and the merge of each
 * (token, head)'s range rows.
 * Source: "prepare_msa_icp_indexer", decode: the chain score plane -> Top16
 * select -> merge, whose first two steps a fused scorer
 * (msa_icp_decode_score_publish) can replace with caller-owned pool storage,
 * its scores then unused. Here the rows stay on this GPU (no publish).
 *
 * Arguments are those of msa_score_decode, except that score_out may be NULL:
 * the scores then go to the pool in the workspace and are not returned. Then:
 * num_valid_pages  device int32 [batch * decode_query_len], as for msa_top16_select.
 *                  With score_out NULL, values above the request's written columns
 *                  are counted in `errors` and clamped to them (the pool holds no other).
 * init_blocks, local_blocks  >= 0, sum <= 16.
 * num_ranges       R, 1 <= R <= min(cols, 768), with ceil(cols / R) <= 2048 (and
 *                  R <= 64 with a merged output). Larger spans use the separate calls.
 * out              device [batch * decode_query_len, 4, R] rows.
 * merged           device [batch * decode_query_len, 4] rows, or NULL.
 * workspace        device int32 [workspace_words], 16-byte aligned, caller-owned,
 *                  workspace_words >= msa_score_select_workspace_words(...). It must
 *                  hold zeros (the pool excepted) when the call is made; the launch
 *                  leaves them zero, unless it counted a timed-out wait in `errors`
 *                  (then the caller zeroes it again). Launches that share a workspace
 *                  must not overlap.
 *
 * score_out (when given) receives exactly what msa_score_decode writes, out
 * exactly what msa_top16_select(plane, ..., num_ranges) then writes, and merged
 * exactly what msa_top16_merge of out writes. The waves that score the plane
 * count each range's stored columns; a fixed subset of them (at most half of
 * the waves the device holds at once) then runs the select jobs, each waiting
 * until its range is complete. Scoring never waits, so every wave of the
 * launch finds a slot and every wait ends.
 */
int msa_score_select(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                     const int32_t* block_table, int64_t block_table_stride,
                     const int32_t* seq_lens, int32_t batch, int32_t page_size,
                     int32_t decode_query_len, float* score_out, int32_t cols,
                     const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                     int32_t num_ranges, msa_top16_row* out, msa_top16_row* merged,
                     int32_t* workspace, int64_t workspace_words, int32_t* errors,
                     hipStream_t stream);

/*
 * msa_score_select without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The workspace is a device array of
 * MSA_NOALLOC_SCRATCH_WORDS int32 words inside the library (16 MiB; one copy
 * per device, held from the library's load until the process ends; its
 * address is looked up on the first call on each device). The call allocates
 * nothing: it clears the array's counter words with a small kernel on
 * `stream` (no memset node, so it can be captured), then launches
 * msa_score_select's kernel on the array.
 *
 * Arguments, outputs and errors are those of msa_score_select. Sizes whose
 * msa_score_select_workspace_words(batch, decode_query_len, cols, num_ranges,
 * score_out == NULL) exceeds MSA_NOALLOC_SCRATCH_WORDS return
 * MSA_ERR_INVALID_ARG with nothing launched (with score_out NULL that is
 * about batch * decode_query_len * 4 * cols <= 4 Mi pool floats). Every call
 * on a device shares that device's array, which keeps the last call's
 * contents (with score_out NULL, its pool scores): calls that overlap on one
 * device (several streams or host threads) race, and the caller orders them.
 */
int msa_score_select_noalloc(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                             const int32_t* block_table, int64_t block_table_stride,
                             const int32_t* seq_lens, int32_t batch, int32_t page_size,
                             int32_t decode_query_len, float* score_out, int32_t cols,
                             const int32_t* num_valid_pages, int32_t init_blocks,
                             int32_t local_blocks, int32_t num_ranges, msa_top16_row* out,
                             msa_top16_row* merged, int32_t* errors, hipStream_t stream);

/*
 * Step 2: Top16 select per (token, head, column range).
 * Source: "msa_icp_topk_select_publish" (description: the row format, and
 * that each call writes all rows including padding rows; scores;
 * num_valid_pages, which counts global B128 blocks) and
 * "prepare_msa_icp_indexer" (init_blocks, local_blocks: the blocks forced
 * in at the start and at the end of a row; at most 16 together).
 *
 * scores           device float32 [num_tokens, 4, cols], contiguous, 0 < cols < 12288.
 * num_valid_pages  device int32 [num_tokens]: valid block ids of token t are [0, n),
 *                  n = num_valid_pages[t]. A value outside [0, cols] is counted in
 *                  `errors` and clamped.
 * init_blocks, local_blocks  >= 0, sum <= 16.
 * num_ranges       R, 1 <= R <= min(cols, 768). Range r is the columns
 *                  [r*w, min((r+1)*w, cols)) with w = ceil(cols / R).
 * out              device [num_tokens, 4, R] rows. Every row is written on every call.
 *
 * Row (t, h, r) keeps the forced ids of its range, [0, init) and [n - local, n)
 * within [0, n). It then takes the best 16 - |forced| of the range's other
 * valid ids, ranked by score descending and then lower id (-0 == +0). All
 * kept entries are listed by ascending id.
 */
int msa_top16_select(const float* scores, int32_t num_tokens, int32_t cols,
                     const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                     int32_t num_ranges, msa_top16_row* out, int32_t* errors, hipStream_t stream);

/*
 * Step 2 on a plane whose column c stands for global block id
 * index_scale * c + index_offset.
 * Source: "msa_icp_topk_select_publish" (index_scale, index_offset: the page
 * defers their meaning to a page that is not available, and this library
 * reads them as that linear map) and "msa_icp_decode_index_score_sharded"
 * (at page_size 256 a rank's column c is global block 2c + rank*2/world_size:
 * index_scale 2, index_offset rank*2/world_size; at 128 the identity).
 *
 * Arguments are those of msa_top16_select, and index_scale >= 1, index_offset >= 0,
 * index_scale*cols + index_offset < 2^31. Every id-based step is taken on global ids:
 * validity (id < n), the forced ids [0, init) and [n - local, n), the tie order, and
 * the ids written. num_valid_pages outside [0, index_scale*cols + index_offset] is
 * counted in `errors` and clamped. With index_scale 1 and index_offset 0 this is
 * msa_top16_select.
 */
int msa_top16_select_mapped(const float* scores, int32_t num_tokens, int32_t cols,
                            const int32_t* num_valid_pages, int32_t init_blocks,
                            int32_t local_blocks, int32_t num_ranges, int32_t index_scale,
                            int32_t index_offset, msa_top16_row* out, int32_t* errors,
                            hipStream_t stream);

/*
 * Step 3: merge of the R per-range rows of each (token, head).
 * Source: "prepare_msa_icp_indexer" (decode: score plane -> Top16 select ->
 * merge). On one GPU the merge reduces the split-column lists of a row.
 *
 * partial          device [num_tokens, 4, R] rows from msa_top16_select over disjoint
 *                  column ranges in ascending order, so that valid ids ascend along the
 *                  concatenated rows. A descending consecutive pair is counted in `errors`.
 * num_valid_pages  device int32 [num_tokens], as given to msa_top16_select.
 * init_blocks, local_blocks  as given to msa_top16_select.
 * num_ranges       R, 1 <= R <= 768.
 * out              device [num_tokens, 4] rows. Every row is written on every call.
 *
 * Applies the select rule to the union of the R rows. Forced ids are
 * recomputed over [0, n). A forced id missing from the union is counted in
 * `errors`. The result equals msa_top16_select with R = 1 on the same scores.
 */
int msa_top16_merge(const msa_top16_row* partial, int32_t num_tokens, int32_t num_ranges,
                    const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                    msa_top16_row* out, int32_t* errors, hipStream_t stream);

/*
 * Step 3 for partial rows in any order that may name the same id: the rows of
 * ranks that each hold part of every page's rows (msa_score_decode_sharded at
 * page_size 128, or at 256 with world_size 4) carry each rank's partial
 * maximum of a block.
 * Source: "prepare_msa_icp_indexer" (decode: the owner merge of the ranks'
 * rows) and "msa_icp_decode_index_score_sharded" (index_k shard).
 *
 * partial          device [num_tokens, 4, R] rows, 1 <= R <= 64, in any order.
 * Other arguments as for msa_top16_merge.
 *
 * Applies the select rule to the union of the rows' entries, an id met more than
 * once keeping its highest score (a block's maximum over its rows is the maximum
 * of its shards' maxima). Forced ids are recomputed over [0, n); one missing from
 * the union is counted in `errors`. Every row of out is written on every call.
 */
int msa_top16_merge_dedup(const msa_top16_row* partial, int32_t num_tokens, int32_t num_ranges,
                          const int32_t* num_valid_pages, int32_t init_blocks,
                          int32_t local_blocks, msa_top16_row* out, int32_t* errors,
                          hipStream_t stream);

/*
 * Steps 2 and 3 in one launch: Top16 select over R column ranges, then the
 * merge of each (token, head) row's R range rows.
 * Source: "prepare_msa_icp_indexer" (decode: score plane -> Top16 select ->
 * merge); the select and merge rules are those of msa_top16_select and
 * msa_top16_merge above.
 *
 * Arguments are as for msa_top16_select, and additionally:
 * num_ranges  R, 1 <= R <= min(cols, 16), with ceil(cols / R) <= 2048. Larger
 *             splits use the two separate calls.
 * partial     device [num_tokens, 4, R] rows, or NULL. When given it receives
 *             exactly what msa_top16_select writes.
 * out         device [num_tokens, 4] rows. It receives exactly what
 *             msa_top16_merge of those R rows writes.
 *
 * One workgroup per (token, head). Wave r selects range r and keeps its row in
 * LDS, then one wave merges the R rows, so no partial rows go through memory
 * between the two steps.
 */
int msa_top16_select_merge(const float* scores, int32_t num_tokens, int32_t cols,
                           const int32_t* num_valid_pages, int32_t init_blocks,
                           int32_t local_blocks, int32_t num_ranges, msa_top16_row* partial,
                           msa_top16_row* out, int32_t* errors, hipStream_t stream);

/*
 * The prefill chain: window plan -> local scoring and Top16 select -> merge.
 * Source: "prepare_msa_icp_indexer", prefill bullet (prefill_window_plan once
 * per query window and step; prefill_local per query chunk into the score
 * scratch and the carrier rows; the exchange; prefill_merge of the received
 * rows). The pages give the chain's shape, not its rule (the select page
 * defers its parameters to msa_icp_topk_select_prefill(), which is not among
 * them). This library reads it as the decode chain with a chunk of query
 * tokens per request:
 *   - request b's chunk is rows [qo_indptr[b], qo_indptr[b+1]) of index_q
 *     ([num_tokens, 4, 128] e4m3fn), token j at position
 *     seq_len_b - q_len_b + j (q_len_b = qo_indptr[b+1] - qo_indptr[b]), as a
 *     decode token sits at seq_len - decode_query_len + j;
 *   - the score scratch is a plane [num_tokens, 4, cols] with msa_score_decode's
 *     element and written columns (block max over keys at or before the
 *     token's position, -inf for a block with none, columns
 *     c < min(roundup4(ceil(seq_len_b / 128)), cols), the rest untouched);
 *   - the carrier rows are msa_top16_select's rows of that plane over R column
 *     ranges, and the merge is msa_top16_merge (on one GPU the carrier is the
 *     received set: there is no exchange).
 *
 * A window is at most MSA_PREFILL_WINDOW_TOKENS consecutive tokens of one
 * chunk. The plan lists the windows' work items (a window and a range of its
 * visible columns); it is built once per step on the device and serves every
 * layer of that step.
 */

/*
 * int32 words of a prefill plan able to hold any step of at most num_tokens
 * query tokens over batch requests on a plane of cols columns (host only):
 * MSA_PREFILL_PLAN_HEADER_WORDS + MSA_PREFILL_ITEM_WORDS * capacity. Returns
 * MSA_ERR_INVALID_ARG for num_tokens < 1, batch outside
 * [1, MSA_PREFILL_MAX_BATCH] or cols outside (0, 8192].
 */
int64_t msa_prefill_plan_words(int64_t num_tokens, int32_t batch, int32_t cols);

/*
 * Builds the plan of one prefill step (one workgroup, on `stream`).
 * qo_indptr   device int32 [batch + 1]: chunk boundaries, qo_indptr[0] = 0,
 *             non-decreasing, qo_indptr[batch] <= num_tokens.
 * seq_lens    device int32 [batch]: keys of each request, its chunk's own keys
 *             included. A request with seq_len <= 0 or an empty chunk writes
 *             nothing.
 * batch       1 <= batch <= MSA_PREFILL_MAX_BATCH.
 * num_tokens  rows of index_q and of the score scratch (>= 1).
 * cols        plane width, 0 < cols <= 8192, cols % 4 == 0.
 * plan        device int32 [plan_words], caller-owned; plan_words from
 *             msa_prefill_plan_words (at least header + one item).
 * Device-side problems are counted in `errors`: a malformed chunk (skipped),
 * a request whose columns the plane cuts short (clamped), items past the
 * plan's capacity (dropped).
 */
int msa_prefill_window_plan(const int32_t* qo_indptr, const int32_t* seq_lens, int32_t batch,
                            int32_t num_tokens, int32_t cols, int32_t* plan, int64_t plan_words,
                            int32_t* errors, hipStream_t stream);

/*
 * Scores one prefill step and selects its Top16 rows.
 * index_q, index_k, num_pages, block_table, block_table_stride, page_size
 *             as for msa_score_decode, index_q holding num_tokens query rows.
 * batch       rows of block_table (>= 1); a plan item of a request at or past
 *             it is counted in `errors` and skipped.
 * plan        the step's plan, made for the same num_tokens and cols (a plan
 *             made for others is counted in `errors` and nothing is written).
 * score_scratch  device float32 [num_tokens, 4, cols], 16-byte aligned: the
 *             plane (written columns as above; other columns untouched).
 * num_valid_pages, init_blocks, local_blocks, num_ranges
 *             as for msa_top16_select on that plane (num_valid_pages [num_tokens]).
 * carrier     device [num_tokens, 4, R] rows: msa_top16_select's rows of the plane.
 * Block-table entries outside [0, num_pages) or past the row stride are counted
 * in `errors` and their blocks score -inf.
 */
int msa_prefill_local(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                      const int32_t* block_table, int64_t block_table_stride, int32_t batch,
                      int32_t page_size,
                      const int32_t* plan, int64_t plan_words, float* score_scratch,
                      int32_t num_tokens, int32_t cols, const int32_t* num_valid_pages,
                      int32_t init_blocks, int32_t local_blocks, int32_t num_ranges,
                      msa_top16_row* carrier, int32_t* errors, hipStream_t stream);

/*
 * Merges each (token, head)'s R carrier rows into one row: msa_top16_merge
 * over num_tokens tokens. received [num_tokens, 4, R], output [num_tokens, 4].
 */
int msa_prefill_merge(const msa_top16_row* received, int32_t num_tokens, int32_t num_ranges,
                      const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                      msa_top16_row* output, int32_t* errors, hipStream_t stream);

/*
 * Score-plane width for requests of up to max_seq_len tokens:
 * roundup4(ceil(max_seq_len / 128)).
 * Source: "msa_icp_decode_index_score_sharded", score_out (which refers to
 * msa_icp_decode_score_columns()). Returns MSA_ERR_INVALID_ARG if
 * max_seq_len < 1 or the width would exceed 8192. Host only, no device call.
 */
int32_t msa_score_columns(int64_t max_seq_len);

/*
 * Loads every kernel of the library into the current device's context, so
 * that no later launch waits on module loading, for example inside a timed
 * region or a graph capture.
 * Source: "prepare_msa_icp_indexer", the paragraph on warmup().
 * Returns MSA_OK or MSA_ERR_LAUNCH.
 */
int msa_warmup(void);

/*
 * Measurement aid, not a step of the indexer: no page defines it. It reads
 * `bytes` of device memory at `src` once, with no other work (non-temporal
 * 16-byte loads, a whole 16 KiB block in flight per wave), so its rate is the
 * streaming ceiling that msa_score_decode's rate can be read against.
 * Benchmarks time it beside the scorer over as many index-K bytes, and over
 * a buffer large enough that a launch's ramp and tail weigh little.
 *
 * src              device, 16-byte aligned; bytes a positive multiple of 16384.
 * blocks_per_wave  the read's shape:
 *                  MSA_STREAM_PROBE_PERSISTENT (0): a grid of one wave per
 *                    SIMD of the device, each wave reading one contiguous run
 *                    of blocks, one block in flight;
 *                  2, 4, 8 or 16: a grid that covers the buffer at once, each
 *                    wave reading that many consecutive 16 KiB blocks.
 *                  The fastest shape depends on the size and the device, so
 *                  a ceiling is the best of them (measured on MI355X: the
 *                  persistent shape at 512 MiB and at 4 GiB).
 * sink             device uint32[MSA_STREAM_PROBE_SINK_WORDS]. The probe xors
 *                  every dword of the buffer into these words (each wave's
 *                  share into one of them), so a caller that zeroes them
 *                  first can check that the xor of all words is the xor of
 *                  the buffer, i.e. that every byte was read.
 * Returns MSA_OK, MSA_ERR_INVALID_ARG (null pointer, misaligned src, bad
 * size or blocks_per_wave; nothing launched) or MSA_ERR_LAUNCH.
 */
int msa_stream_read_probe(const void* src, int64_t bytes, int32_t blocks_per_wave,
                          uint32_t* sink, hipStream_t stream);

/*
 * Measurement aid, not a step of the indexer: no page defines it. The pages
 * give fp8 inputs and fp32 scores ("msa_icp_decode_index_score_sharded",
 * index_q / index_k / score_out); this call measures how three gfx950 MFMA
 * forms accumulate 128-dim fp8 dot products, which decides the form the
 * scorer contracts in:
 *   MSA_PROBE_BF16             the scorer's form: codes converted exactly to
 *                              bf16, four v_mfma_f32_16x16x32_bf16 chained;
 *   MSA_PROBE_FP8_16X16X32     four v_mfma_f32_16x16x32_fp8_fp8 chained;
 *   MSA_PROBE_F8F6F4_16X16X128 one v_mfma_f32_16x16x128_f8f6f4 (e4m3, unscaled).
 *
 * q, k   device, e4m3fn bytes [tiles, 16, 128], contiguous, 16-byte aligned.
 * out    device float32 [tiles, 16, 16]: out[t, i, j] = q[t, i, :] . k[t, j, :].
 * Returns MSA_OK, MSA_ERR_INVALID_ARG (null or misaligned pointer, tiles outside
 * [1, 2^31), unknown form; nothing launched) or MSA_ERR_LAUNCH.
 */
#define MSA_PROBE_BF16 0
#define MSA_PROBE_FP8_16X16X32 1
#define MSA_PROBE_F8F6F4_16X16X128 2
int msa_contraction_probe(const uint8_t* q, const uint8_t* k, int64_t tiles, int32_t form,
                          float* out, hipStream_t stream);

/*
 * Text of the last failed check or launch of the calling thread. The string
 * is empty if there was none. It stays valid until the thread's next call
 * into the library.
 */
const char* msa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_INDEXER_H */
