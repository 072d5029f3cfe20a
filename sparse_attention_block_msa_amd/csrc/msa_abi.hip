// C-ABI entry points: host-side argument checks, then one kernel launch each
// on the caller's stream (msa_score_select_noalloc: two). Nothing here
// allocates or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "contraction_probe.h"
#include "msa_internal.h"
#include "stream_probe.h"

// The workspace of msa_score_select_noalloc: counters and, for calls
// without a plane, the pool. One copy per device, from the library's load
// until the process ends. Host code uses only the device address that
// hipGetSymbolAddress returns for it (scratch_address), never this name.
static __device__ __align__(256) int32_t scratch[MSA_NOALLOC_SCRATCH_WORDS];

namespace {

thread_local char g_last_error[512];

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

int launch_result(hipError_t e, const char* what)
{
    if (e != hipSuccess)
        return fail(MSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return MSA_OK;
}

bool aligned(const void* ptr, uintptr_t a)
{
    return ((uintptr_t)ptr % a) == 0;
}

#define MSA_CHECK(cond, ...)                                   \
    do {                                                       \
        if (!(cond))                                           \
            return fail(MSA_ERR_INVALID_ARG, __VA_ARGS__);     \
    } while (0)

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
int32_t* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current.
int scratch_address(const char* fn, int32_t** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(MSA_ERR_LAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MSA_ERR_INVALID_ARG, "%s: device %d is past the %d this library tracks", fn,
                    dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(MSA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s",
                        fn, dev, hipGetErrorString(e));
        g_scratch[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch[dev];
    return MSA_OK;
}

int check_forced(const char* fn, int32_t init_blocks, int32_t local_blocks)
{
    MSA_CHECK(init_blocks >= 0 && local_blocks >= 0,
              "%s: init_blocks (%d) and local_blocks (%d) must be >= 0", fn, init_blocks,
              local_blocks);
    MSA_CHECK(init_blocks + local_blocks <= MSA_TOPK,
              "%s: init_blocks + local_blocks = %d exceeds %d", fn, init_blocks + local_blocks,
              MSA_TOPK);
    return MSA_OK;
}

// Host checks of the score-plane arguments shared by msa_score_decode and
// msa_score_select; fills *p on success.
int score_params(const char* fn, const uint8_t* index_q, const uint8_t* index_k,
                 int64_t num_pages, const int32_t* block_table, int64_t block_table_stride,
                 const int32_t* seq_lens, int32_t batch, int32_t page_size,
                 int32_t decode_query_len, float* score_out, int32_t cols, int32_t* errors,
                 msa::ScoreParams* p)
{
    MSA_CHECK(index_q && index_k && block_table && seq_lens && score_out,
              "%s: null pointer argument", fn);
    MSA_CHECK(aligned(index_q, 16) && aligned(index_k, 16) && aligned(score_out, 16),
              "%s: index_q, index_k and score_out must be 16-byte aligned", fn);
    MSA_CHECK(aligned(block_table, 4) && aligned(seq_lens, 4) && aligned(errors, 4),
              "%s: int32 arrays must be 4-byte aligned", fn);
    MSA_CHECK(page_size == 128 || page_size == 256, "%s: page_size (%d) must be 128 or 256", fn,
              page_size);
    MSA_CHECK(decode_query_len >= 1 && 4 * decode_query_len <= 32,
              "%s: decode_query_len (%d) must satisfy 1 <= len and 4*len <= 32", fn,
              decode_query_len);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SCORE_COLS && cols % 4 == 0,
              "%s: cols (%d) must satisfy 0 < cols <= %d and cols %% 4 == 0", fn, cols,
              MSA_MAX_SCORE_COLS);
    MSA_CHECK(batch >= 1 && batch <= (1 << 22), "%s: batch (%d) must be in [1, 2^22]", fn,
              batch);
    MSA_CHECK(num_pages >= 1, "%s: num_pages (%lld) must be >= 1", fn, (long long)num_pages);
    MSA_CHECK(block_table_stride >= 1, "%s: block_table_stride (%lld) must be >= 1", fn,
              (long long)block_table_stride);
    p->q = index_q;
    p->k = index_k;
    p->num_pages = num_pages;
    p->bt = block_table;
    p->bt_stride = block_table_stride;
    p->seq_lens = seq_lens;
    p->out = score_out;
    p->errors = errors;
    p->batch = batch;
    p->page_size = page_size;
    p->dql = decode_query_len;
    p->cols = cols;
    p->rank = 0;
    p->world_size = 1;
    return MSA_OK;
}

int select_impl(const char* fn, const float* scores, int32_t num_tokens, int32_t cols,
                const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                int32_t num_ranges, int32_t index_scale, int32_t index_offset,
                msa_top16_row* out, int32_t* errors, hipStream_t stream)
{
    MSA_CHECK(scores && num_valid_pages && out, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(scores, 4) && aligned(num_valid_pages, 4) && aligned(out, 4) &&
                  aligned(errors, 4),
              "%s: arrays must be 4-byte aligned", fn);
    MSA_CHECK(num_tokens >= 1 && (int64_t)num_tokens * MSA_NUM_HEADS * num_ranges <= 0x7FFFFFFF,
              "%s: num_tokens (%d) must be >= 1 and tokens*4*ranges < 2^31", fn, num_tokens);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SELECT_COLS,
              "%s: cols (%d) must satisfy 0 < cols <= %d", fn, cols, MSA_MAX_SELECT_COLS);
    MSA_CHECK(num_ranges >= 1 && num_ranges <= cols && num_ranges <= MSA_MAX_RANGES,
              "%s: num_ranges (%d) must be in [1, min(cols, %d)]", fn, num_ranges,
              MSA_MAX_RANGES);
    MSA_CHECK(index_scale >= 1 && index_offset >= 0,
              "%s: index_scale (%d) must be >= 1 and index_offset (%d) >= 0", fn, index_scale,
              index_offset);
    MSA_CHECK((int64_t)index_scale * cols + index_offset <= 0x7FFFFFFF,
              "%s: index_scale * cols + index_offset must be < 2^31", fn);
    int rc = check_forced(fn, init_blocks, local_blocks);
    if (rc != MSA_OK)
        return rc;

    msa::SelectParams p;
    p.scores = scores;
    p.nvp = num_valid_pages;
    p.out = out;
    p.errors = errors;
    p.num_tokens = num_tokens;
    p.cols = cols;
    p.init_blocks = init_blocks;
    p.local_blocks = local_blocks;
    p.num_ranges = num_ranges;
    p.width = (cols + num_ranges - 1) / num_ranges;
    p.index_scale = index_scale;
    p.index_offset = index_offset;
    return launch_result(msa::launch_top16_select(p, stream), fn);
}

int merge_impl(const char* fn, const msa_top16_row* partial, int32_t num_tokens,
               int32_t num_ranges, int32_t max_ranges, const int32_t* num_valid_pages,
               int32_t init_blocks, int32_t local_blocks, msa_top16_row* out, int32_t* errors,
               msa::MergeParams* p)
{
    MSA_CHECK(partial && num_valid_pages && out, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(partial, 4) && aligned(num_valid_pages, 4) && aligned(out, 4) &&
                  aligned(errors, 4),
              "%s: arrays must be 4-byte aligned", fn);
    MSA_CHECK(num_tokens >= 1 && (int64_t)num_tokens * MSA_NUM_HEADS <= 0x7FFFFFFF,
              "%s: num_tokens (%d) must be >= 1 and tokens*4 < 2^31", fn, num_tokens);
    MSA_CHECK(num_ranges >= 1 && num_ranges <= max_ranges,
              "%s: num_ranges (%d) must be in [1, %d]", fn, num_ranges, max_ranges);
    int rc = check_forced(fn, init_blocks, local_blocks);
    if (rc != MSA_OK)
        return rc;
    p->partial = partial;
    p->nvp = num_valid_pages;
    p->out = out;
    p->errors = errors;
    p->num_tokens = num_tokens;
    p->num_ranges = num_ranges;
    p->init_blocks = init_blocks;
    p->local_blocks = local_blocks;
    return MSA_OK;
}


// Zeroes n int32 words (a kernel, so that a captured graph records no memset
// node).
__global__ void clear_words_kernel(int32_t* p, int64_t n)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
        p[i] = 0;
}

hipError_t launch_clear_words(int32_t* p, int64_t n, hipStream_t stream)
{
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
    if (blocks == 0)
        return hipSuccess;
    void* args[] = {&p, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&clear_words_kernel),
                           dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

// Workspace words of msa_score_select for these sizes, or MSA_ERR_INVALID_ARG
// (message set) for sizes it rejects.
int64_t score_select_words(const char* fn, int32_t batch, int32_t decode_query_len,
                           int32_t cols, int32_t num_ranges, bool with_pool)
{
    MSA_CHECK(batch >= 1 && batch <= (1 << 22), "%s: batch (%d) must be in [1, 2^22]", fn, batch);
    MSA_CHECK(decode_query_len >= 1 && 4 * decode_query_len <= 32,
              "%s: decode_query_len (%d) must satisfy 1 <= len and 4*len <= 32", fn,
              decode_query_len);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SCORE_COLS && cols % 4 == 0,
              "%s: cols (%d) must satisfy 0 < cols <= %d and cols %% 4 == 0", fn, cols,
              MSA_MAX_SCORE_COLS);
    MSA_CHECK(num_ranges >= 1 && num_ranges <= cols && num_ranges <= MSA_MAX_RANGES,
              "%s: num_ranges (%d) must be in [1, min(cols, %d)]", fn, num_ranges,
              MSA_MAX_RANGES);
    const int64_t rows = (int64_t)batch * decode_query_len * MSA_NUM_HEADS;
    if (with_pool)  // the pool starts 16-byte aligned
        return msa::fused_pool_offset(batch, decode_query_len, num_ranges) + rows * cols;
    return msa::fused_counter_words(batch, decode_query_len, num_ranges);
}

// msa_score_select on `workspace`; with clear_counters, the workspace's
// counter words are first cleared by a kernel on `stream` (after every check
// has passed).
int score_select_impl(const char* fn, const uint8_t* index_q, const uint8_t* index_k,
                      int64_t num_pages, const int32_t* block_table, int64_t block_table_stride,
                      const int32_t* seq_lens, int32_t batch, int32_t page_size,
                      int32_t decode_query_len, float* score_out, int32_t cols,
                      const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                      int32_t num_ranges, msa_top16_row* out, msa_top16_row* merged,
                      int32_t* workspace, int64_t workspace_words, bool clear_counters,
                      int32_t* errors, hipStream_t stream)
{
    MSA_CHECK(workspace && aligned(workspace, 16), "%s: workspace must be non-null and 16-byte "
              "aligned", fn);
    const bool pool = score_out == nullptr;
    MSA_CHECK(num_ranges >= 1 && num_ranges <= cols && num_ranges <= MSA_MAX_RANGES,
              "%s: num_ranges (%d) must be in [1, min(cols, %d)]", fn, num_ranges,
              MSA_MAX_RANGES);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SCORE_COLS && cols % 4 == 0,
              "%s: cols (%d) must satisfy 0 < cols <= %d and cols %% 4 == 0", fn, cols,
              MSA_MAX_SCORE_COLS);
    MSA_CHECK(batch >= 1 && batch <= (1 << 22), "%s: batch (%d) must be in [1, 2^22]", fn, batch);
    MSA_CHECK(decode_query_len >= 1 && 4 * decode_query_len <= 32,
              "%s: decode_query_len (%d) must satisfy 1 <= len and 4*len <= 32", fn,
              decode_query_len);
    const int64_t need = score_select_words(fn, batch, decode_query_len, cols, num_ranges, pool);
    MSA_CHECK(workspace_words >= need, "%s: workspace_words (%lld) must be >= %lld", fn,
              (long long)workspace_words, (long long)need);
    float* plane = score_out;
    if (pool) {
        plane = reinterpret_cast<float*>(
            workspace + msa::fused_pool_offset(batch, decode_query_len, num_ranges));
    }
    msa::ScoreSelectParams q;
    int rc = score_params(fn, index_q, index_k, num_pages, block_table, block_table_stride,
                          seq_lens, batch, page_size, decode_query_len, plane, cols, errors,
                          &q.score);
    if (rc != MSA_OK)
        return rc;
    MSA_CHECK(num_valid_pages && out, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(num_valid_pages, 4) && aligned(out, 4) && aligned(merged, 4),
              "%s: arrays must be 4-byte aligned", fn);
    const int64_t tokens = (int64_t)batch * decode_query_len;
    MSA_CHECK(tokens * MSA_NUM_HEADS * num_ranges <= 0x7FFFFFFF,
              "%s: tokens*4*num_ranges must be < 2^31", fn);
    const int32_t width = (cols + num_ranges - 1) / num_ranges;
    MSA_CHECK(width <= msa::kMaxFusedWidth,
              "%s: ceil(cols / num_ranges) = %d exceeds %d; use msa_score_decode + "
              "msa_top16_select", fn, width, msa::kMaxFusedWidth);
    MSA_CHECK(merged == nullptr || num_ranges <= msa::kMaxFusedMergeRanges,
              "%s: a merged output needs num_ranges <= %d (got %d); use msa_top16_merge", fn,
              msa::kMaxFusedMergeRanges, num_ranges);
    rc = check_forced(fn, init_blocks, local_blocks);
    if (rc != MSA_OK)
        return rc;
    q.nvp = num_valid_pages;
    q.out = out;
    q.merged = merged;
    q.workspace = workspace;
    q.init_blocks = init_blocks;
    q.local_blocks = local_blocks;
    q.num_ranges = num_ranges;
    q.width = width;
    q.pool = pool ? 1 : 0;
    q.helpers = 0;
    if (clear_counters) {
        const int64_t n = msa::fused_counter_words(batch, decode_query_len, num_ranges);
        rc = launch_result(launch_clear_words(workspace, n, stream), fn);
        if (rc != MSA_OK)
            return rc;
    }
    return launch_result(msa::launch_score_select(q, stream), fn);
}

}  // namespace

extern "C" {

const char* msa_last_error(void)
{
    return g_last_error;
}

int32_t msa_score_columns(int64_t max_seq_len)
{
    g_last_error[0] = '\0';
    MSA_CHECK(max_seq_len >= 1, "msa_score_columns: max_seq_len (%lld) must be >= 1",
              (long long)max_seq_len);
    const int64_t blocks = (max_seq_len + MSA_BLOCK_TOKENS - 1) / MSA_BLOCK_TOKENS;
    const int64_t cols = (blocks + 3) / 4 * 4;
    MSA_CHECK(cols <= MSA_MAX_SCORE_COLS, "msa_score_columns: %lld columns exceed %d",
              (long long)cols, MSA_MAX_SCORE_COLS);
    return (int32_t)cols;
}

int msa_score_decode(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                     const int32_t* block_table, int64_t block_table_stride,
                     const int32_t* seq_lens, int32_t batch, int32_t page_size,
                     int32_t decode_query_len, float* score_out, int32_t cols, int32_t* errors,
                     hipStream_t stream)
{
    g_last_error[0] = '\0';
    msa::ScoreParams p;
    const int rc = score_params("msa_score_decode", index_q, index_k, num_pages, block_table,
                                block_table_stride, seq_lens, batch, page_size, decode_query_len,
                                score_out, cols, errors, &p);
    if (rc != MSA_OK)
        return rc;
    return launch_result(msa::launch_score_decode(p, stream), "msa_score_decode");
}

int msa_score_decode_sharded(const uint8_t* index_q, const uint8_t* index_k_shard,
                             int64_t num_pages, const int32_t* block_table,
                             int64_t block_table_stride, const int32_t* seq_lens, int32_t batch,
                             int32_t page_size, int32_t decode_query_len, int32_t rank,
                             int32_t world_size, float* score_out, int32_t cols, int32_t* errors,
                             hipStream_t stream)
{
    g_last_error[0] = '\0';
    const char* fn = "msa_score_decode_sharded";
    msa::ScoreParams p;
    const int rc = score_params(fn, index_q, index_k_shard, num_pages, block_table,
                                block_table_stride, seq_lens, batch, page_size, decode_query_len,
                                score_out, cols, errors, &p);
    if (rc != MSA_OK)
        return rc;
    MSA_CHECK(world_size == 2 || world_size == 4, "%s: world_size (%d) must be 2 or 4", fn,
              world_size);
    MSA_CHECK(rank >= 0 && rank < world_size, "%s: rank (%d) must be in [0, world_size)", fn,
              rank);
    p.rank = rank;
    p.world_size = world_size;
    return launch_result(msa::launch_score_decode(p, stream), fn);
}

int64_t msa_score_select_workspace_words(int32_t batch, int32_t decode_query_len, int32_t cols,
                                         int32_t num_ranges, int32_t with_pool)
{
    g_last_error[0] = '\0';
    return score_select_words("msa_score_select_workspace_words", batch, decode_query_len, cols,
                              num_ranges, with_pool != 0);
}

int msa_score_select(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                     const int32_t* block_table, int64_t block_table_stride,
                     const int32_t* seq_lens, int32_t batch, int32_t page_size,
                     int32_t decode_query_len, float* score_out, int32_t cols,
                     const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                     int32_t num_ranges, msa_top16_row* out, msa_top16_row* merged,
                     int32_t* workspace, int64_t workspace_words, int32_t* errors,
                     hipStream_t stream)
{
    g_last_error[0] = '\0';
    return score_select_impl("msa_score_select", index_q, index_k, num_pages, block_table,
                             block_table_stride, seq_lens, batch, page_size, decode_query_len,
                             score_out, cols, num_valid_pages, init_blocks, local_blocks,
                             num_ranges, out, merged, workspace, workspace_words, false, errors,
                             stream);
}

int msa_score_select_noalloc(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                             const int32_t* block_table, int64_t block_table_stride,
                             const int32_t* seq_lens, int32_t batch, int32_t page_size,
                             int32_t decode_query_len, float* score_out, int32_t cols,
                             const int32_t* num_valid_pages, int32_t init_blocks,
                             int32_t local_blocks, int32_t num_ranges, msa_top16_row* out,
                             msa_top16_row* merged, int32_t* errors, hipStream_t stream)
{
    g_last_error[0] = '\0';
    const char* fn = "msa_score_select_noalloc";
    const int64_t need =
        score_select_words(fn, batch, decode_query_len, cols, num_ranges, score_out == nullptr);
    if (need < 0)
        return MSA_ERR_INVALID_ARG;  // message set by score_select_words
    MSA_CHECK(need <= MSA_NOALLOC_SCRATCH_WORDS,
              "%s: these sizes need %lld workspace words (counters%s), more than the %d of "
              "the library's scratch array; use msa_score_select with a workspace",
              fn, (long long)need, score_out == nullptr ? " and the pool plane" : "",
              MSA_NOALLOC_SCRATCH_WORDS);
    int32_t* ws = nullptr;
    const int rc = scratch_address(fn, &ws);
    if (rc != MSA_OK)
        return rc;
    return score_select_impl(fn, index_q, index_k, num_pages, block_table, block_table_stride,
                             seq_lens, batch, page_size, decode_query_len, score_out, cols,
                             num_valid_pages, init_blocks, local_blocks, num_ranges, out, merged,
                             ws, MSA_NOALLOC_SCRATCH_WORDS, true, errors, stream);
}

int msa_top16_select(const float* scores, int32_t num_tokens, int32_t cols,
                     const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                     int32_t num_ranges, msa_top16_row* out, int32_t* errors, hipStream_t stream)
{
    g_last_error[0] = '\0';
    return select_impl("msa_top16_select", scores, num_tokens, cols, num_valid_pages, init_blocks,
                       local_blocks, num_ranges, 1, 0, out, errors, stream);
}

int msa_top16_select_mapped(const float* scores, int32_t num_tokens, int32_t cols,
                            const int32_t* num_valid_pages, int32_t init_blocks,
                            int32_t local_blocks, int32_t num_ranges, int32_t index_scale,
                            int32_t index_offset, msa_top16_row* out, int32_t* errors,
                            hipStream_t stream)
{
    g_last_error[0] = '\0';
    return select_impl("msa_top16_select_mapped", scores, num_tokens, cols, num_valid_pages,
                       init_blocks, local_blocks, num_ranges, index_scale, index_offset, out,
                       errors, stream);
}

int msa_top16_merge(const msa_top16_row* partial, int32_t num_tokens, int32_t num_ranges,
                    const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                    msa_top16_row* out, int32_t* errors, hipStream_t stream)
{
    g_last_error[0] = '\0';
    msa::MergeParams p;
    const int rc = merge_impl("msa_top16_merge", partial, num_tokens, num_ranges, MSA_MAX_RANGES,
                              num_valid_pages, init_blocks, local_blocks, out, errors, &p);
    if (rc != MSA_OK)
        return rc;
    return launch_result(msa::launch_top16_merge(p, stream), "msa_top16_merge");
}

int msa_top16_merge_dedup(const msa_top16_row* partial, int32_t num_tokens, int32_t num_ranges,
                          const int32_t* num_valid_pages, int32_t init_blocks,
                          int32_t local_blocks, msa_top16_row* out, int32_t* errors,
                          hipStream_t stream)
{
    g_last_error[0] = '\0';
    msa::MergeParams p;
    const int rc = merge_impl("msa_top16_merge_dedup", partial, num_tokens, num_ranges,
                              msa::kMaxDedupRanges, num_valid_pages, init_blocks, local_blocks,
                              out, errors, &p);
    if (rc != MSA_OK)
        return rc;
    return launch_result(msa::launch_top16_merge_dedup(p, stream), "msa_top16_merge_dedup");
}

int msa_top16_select_merge(const float* scores, int32_t num_tokens, int32_t cols,
                           const int32_t* num_valid_pages, int32_t init_blocks,
                           int32_t local_blocks, int32_t num_ranges, msa_top16_row* partial,
                           msa_top16_row* out, int32_t* errors, hipStream_t stream)
{
    g_last_error[0] = '\0';
    const char* fn = "msa_top16_select_merge";
    MSA_CHECK(scores && num_valid_pages && out, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(scores, 4) && aligned(num_valid_pages, 4) && aligned(out, 4) &&
                  aligned(partial, 4) && aligned(errors, 4),
              "%s: arrays must be 4-byte aligned", fn);
    MSA_CHECK(num_tokens >= 1 && (int64_t)num_tokens * MSA_NUM_HEADS <= 0x7FFFFFFF,
              "%s: num_tokens (%d) must be >= 1 and tokens*4 < 2^31", fn, num_tokens);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SELECT_COLS,
              "%s: cols (%d) must satisfy 0 < cols <= %d", fn, cols, MSA_MAX_SELECT_COLS);
    MSA_CHECK(num_ranges >= 1 && num_ranges <= cols && num_ranges <= msa::kMaxFusedRanges,
              "%s: num_ranges (%d) must be in [1, min(cols, %d)]", fn, num_ranges,
              msa::kMaxFusedRanges);
    const int32_t width = (cols + num_ranges - 1) / num_ranges;
    MSA_CHECK(width <= msa::kMaxFusedWidth,
              "%s: ceil(cols / num_ranges) = %d exceeds %d; use msa_top16_select + "
              "msa_top16_merge", fn, width, msa::kMaxFusedWidth);
    int rc = check_forced(fn, init_blocks, local_blocks);
    if (rc != MSA_OK)
        return rc;

    msa::SelectMergeParams p;
    p.scores = scores;
    p.nvp = num_valid_pages;
    p.partial = partial;
    p.out = out;
    p.errors = errors;
    p.num_tokens = num_tokens;
    p.cols = cols;
    p.init_blocks = init_blocks;
    p.local_blocks = local_blocks;
    p.num_ranges = num_ranges;
    p.width = width;
    return launch_result(msa::launch_top16_select_merge(p, stream), fn);
}

int msa_stream_read_probe(const void* src, int64_t bytes, int32_t blocks_per_wave,
                          uint32_t* sink, hipStream_t stream)
{
    static const char* fn = "msa_stream_read_probe";
    g_last_error[0] = '\0';
    MSA_CHECK(src && sink, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(src, 16), "%s: src must be 16-byte aligned", fn);
    MSA_CHECK(bytes > 0 && bytes % msa::kProbeBlockBytes == 0,
              "%s: bytes (%lld) must be a positive multiple of %lld", fn, (long long)bytes,
              (long long)msa::kProbeBlockBytes);
    MSA_CHECK(blocks_per_wave == MSA_STREAM_PROBE_PERSISTENT || blocks_per_wave == 2 ||
                  blocks_per_wave == 4 || blocks_per_wave == 8 || blocks_per_wave == 16,
              "%s: blocks_per_wave (%d) must be %d (persistent), 2, 4, 8 or 16", fn,
              (int)blocks_per_wave, MSA_STREAM_PROBE_PERSISTENT);
    return launch_result(msa::launch_stream_read_probe(static_cast<const uint8_t*>(src),
                                                       bytes / msa::kProbeBlockBytes,
                                                       blocks_per_wave, sink, stream),
                         fn);
}

int64_t msa_prefill_plan_words(int64_t num_tokens, int32_t batch, int32_t cols)
{
    static const char* fn = "msa_prefill_plan_words";
    g_last_error[0] = '\0';
    MSA_CHECK(num_tokens >= 1 && num_tokens <= 0x7FFFFFFF,
              "%s: num_tokens (%lld) must be in [1, 2^31)", fn, (long long)num_tokens);
    MSA_CHECK(batch >= 1 && batch <= MSA_PREFILL_MAX_BATCH, "%s: batch (%d) must be in [1, %d]",
              fn, batch, MSA_PREFILL_MAX_BATCH);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SCORE_COLS, "%s: cols (%d) must be in (0, %d]", fn, cols,
              MSA_MAX_SCORE_COLS);
    // windows <= num_tokens / 64 + batch; items per window <= ceil(cols / item columns)
    const int64_t windows = num_tokens / MSA_PREFILL_WINDOW_TOKENS + batch;
    const int64_t per_window = (cols + msa::kPrefillItemCols - 1) / msa::kPrefillItemCols;
    return MSA_PREFILL_PLAN_HEADER_WORDS + MSA_PREFILL_ITEM_WORDS * windows * per_window;
}

int msa_prefill_window_plan(const int32_t* qo_indptr, const int32_t* seq_lens, int32_t batch,
                            int32_t num_tokens, int32_t cols, int32_t* plan, int64_t plan_words,
                            int32_t* errors, hipStream_t stream)
{
    static const char* fn = "msa_prefill_window_plan";
    g_last_error[0] = '\0';
    MSA_CHECK(qo_indptr && seq_lens && plan, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(qo_indptr, 4) && aligned(seq_lens, 4) && aligned(plan, 4) &&
                  aligned(errors, 4),
              "%s: int32 arrays must be 4-byte aligned", fn);
    MSA_CHECK(batch >= 1 && batch <= MSA_PREFILL_MAX_BATCH, "%s: batch (%d) must be in [1, %d]",
              fn, batch, MSA_PREFILL_MAX_BATCH);
    MSA_CHECK(num_tokens >= 1, "%s: num_tokens (%d) must be >= 1", fn, num_tokens);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SCORE_COLS && cols % 4 == 0,
              "%s: cols (%d) must satisfy 0 < cols <= %d and cols %% 4 == 0", fn, cols,
              MSA_MAX_SCORE_COLS);
    MSA_CHECK(plan_words >= MSA_PREFILL_PLAN_HEADER_WORDS + MSA_PREFILL_ITEM_WORDS,
              "%s: plan_words (%lld) must hold the header and one item", fn,
              (long long)plan_words);
    msa::PrefillPlanParams p;
    p.qo_indptr = qo_indptr;
    p.seq_lens = seq_lens;
    p.plan = plan;
    p.capacity = (plan_words - MSA_PREFILL_PLAN_HEADER_WORDS) / MSA_PREFILL_ITEM_WORDS;
    if (p.capacity > 0x7FFFFFF8)
        p.capacity = 0x7FFFFFF8;
    p.errors = errors;
    p.batch = batch;
    p.num_tokens = num_tokens;
    p.cols = cols;
    return launch_result(msa::launch_prefill_plan(p, stream), fn);
}

int msa_prefill_local(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                      const int32_t* block_table, int64_t block_table_stride, int32_t batch,
                      int32_t page_size,
                      const int32_t* plan, int64_t plan_words, float* score_scratch,
                      int32_t num_tokens, int32_t cols, const int32_t* num_valid_pages,
                      int32_t init_blocks, int32_t local_blocks, int32_t num_ranges,
                      msa_top16_row* carrier, int32_t* errors, hipStream_t stream)
{
    static const char* fn = "msa_prefill_local";
    g_last_error[0] = '\0';
    MSA_CHECK(index_q && index_k && block_table && plan && score_scratch && num_valid_pages &&
                  carrier,
              "%s: null pointer argument", fn);
    MSA_CHECK(aligned(index_q, 16) && aligned(index_k, 16) && aligned(score_scratch, 16),
              "%s: index_q, index_k and score_scratch must be 16-byte aligned", fn);
    MSA_CHECK(aligned(block_table, 4) && aligned(plan, 4) && aligned(num_valid_pages, 4) &&
                  aligned(carrier, 4) && aligned(errors, 4),
              "%s: int32 arrays must be 4-byte aligned", fn);
    MSA_CHECK(page_size == 128 || page_size == 256, "%s: page_size (%d) must be 128 or 256", fn,
              page_size);
    MSA_CHECK(num_pages >= 1, "%s: num_pages (%lld) must be >= 1", fn, (long long)num_pages);
    MSA_CHECK(block_table_stride >= 1, "%s: block_table_stride (%lld) must be >= 1", fn,
              (long long)block_table_stride);
    MSA_CHECK(batch >= 1, "%s: batch (%d) must be >= 1", fn, batch);
    MSA_CHECK(num_tokens >= 1 && (int64_t)num_tokens * MSA_NUM_HEADS * num_ranges <= 0x7FFFFFFF,
              "%s: num_tokens (%d) must be >= 1 and tokens*4*ranges < 2^31", fn, num_tokens);
    MSA_CHECK(cols > 0 && cols <= MSA_MAX_SCORE_COLS && cols % 4 == 0,
              "%s: cols (%d) must satisfy 0 < cols <= %d and cols %% 4 == 0", fn, cols,
              MSA_MAX_SCORE_COLS);
    MSA_CHECK(num_ranges >= 1 && num_ranges <= cols && num_ranges <= MSA_MAX_RANGES,
              "%s: num_ranges (%d) must be in [1, min(cols, %d)]", fn, num_ranges,
              MSA_MAX_RANGES);
    MSA_CHECK(plan_words >= MSA_PREFILL_PLAN_HEADER_WORDS + MSA_PREFILL_ITEM_WORDS,
              "%s: plan_words (%lld) must hold the header and one item", fn,
              (long long)plan_words);
    int rc = check_forced(fn, init_blocks, local_blocks);
    if (rc != MSA_OK)
        return rc;
    int64_t capacity = (plan_words - MSA_PREFILL_PLAN_HEADER_WORDS) / MSA_PREFILL_ITEM_WORDS;
    if (capacity > 0x7FFFFFF8)
        capacity = 0x7FFFFFF8;

    msa::PrefillScoreParams sp;
    sp.q = index_q;
    sp.k = index_k;
    sp.num_pages = num_pages;
    sp.bt = block_table;
    sp.bt_stride = block_table_stride;
    sp.bt_rows = batch;
    sp.plan = plan;
    sp.capacity = capacity;
    sp.out = score_scratch;
    sp.errors = errors;
    sp.page_size = page_size;
    sp.cols = cols;
    sp.num_tokens = num_tokens;
    rc = launch_result(msa::launch_prefill_score(sp, capacity, stream), fn);
    if (rc != MSA_OK)
        return rc;

    msa::SelectParams p;
    p.scores = score_scratch;
    p.nvp = num_valid_pages;
    p.out = carrier;
    p.errors = errors;
    p.num_tokens = num_tokens;
    p.cols = cols;
    p.init_blocks = init_blocks;
    p.local_blocks = local_blocks;
    p.num_ranges = num_ranges;
    p.width = (cols + num_ranges - 1) / num_ranges;
    p.index_scale = 1;
    p.index_offset = 0;
    return launch_result(msa::launch_top16_select(p, stream), fn);
}

int msa_prefill_merge(const msa_top16_row* received, int32_t num_tokens, int32_t num_ranges,
                      const int32_t* num_valid_pages, int32_t init_blocks, int32_t local_blocks,
                      msa_top16_row* output, int32_t* errors, hipStream_t stream)
{
    g_last_error[0] = '\0';
    msa::MergeParams p;
    const int rc = merge_impl("msa_prefill_merge", received, num_tokens, num_ranges,
                              MSA_MAX_RANGES, num_valid_pages, init_blocks, local_blocks, output,
                              errors, &p);
    if (rc != MSA_OK)
        return rc;
    return launch_result(msa::launch_top16_merge(p, stream), "msa_prefill_merge");
}

int msa_contraction_probe(const uint8_t* q, const uint8_t* k, int64_t tiles, int32_t form,
                          float* out, hipStream_t stream)
{
    static const char* fn = "msa_contraction_probe";
    g_last_error[0] = '\0';
    MSA_CHECK(q && k && out, "%s: null pointer argument", fn);
    MSA_CHECK(aligned(q, 16) && aligned(k, 16) && aligned(out, 4),
              "%s: q and k must be 16-byte aligned, out 4-byte aligned", fn);
    MSA_CHECK(tiles >= 1 && tiles <= 0x7FFFFFFF, "%s: tiles (%lld) must be in [1, 2^31)", fn,
              (long long)tiles);
    MSA_CHECK(form == MSA_PROBE_BF16 || form == MSA_PROBE_FP8_16X16X32 ||
                  form == MSA_PROBE_F8F6F4_16X16X128,
              "%s: unknown form %d", fn, form);
    return launch_result(msa::launch_contraction_probe(q, k, tiles, form, out, stream), fn);
}

int msa_warmup(void)
{
    g_last_error[0] = '\0';
    hipError_t e = msa::warmup_score_kernels();
    if (e == hipSuccess)
        e = msa::warmup_top16_kernels();
    if (e == hipSuccess)
        e = msa::warmup_prefill_kernels();
    return launch_result(e, "msa_warmup");
}

}  // extern "C"
