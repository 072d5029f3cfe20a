// Internal declarations shared by the library's translation units: launch
// parameter blocks and the launchers each kernel file provides. Host-side
// validation lives in msa_abi.hip; the launchers assume valid arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_indexer.h"

namespace msa {

constexpr int kHeads = MSA_NUM_HEADS;
constexpr int kDim = MSA_HEAD_DIM;
constexpr int kBlockTokens = MSA_BLOCK_TOKENS;
constexpr int kTop = MSA_TOPK;


struct ScoreParams {
    const uint8_t* q;        // [batch*dql, 4, 128] e4m3fn
    const uint8_t* k;        // [num_pages, page_size, 128] e4m3fn
    int64_t num_pages;
    const int32_t* bt;       // [batch, bt_stride]
    int64_t bt_stride;
    const int32_t* seq_lens; // [batch]
    float* out;              // [batch*dql, 4, cols]
    int32_t* errors;         // nullable
    int32_t batch;
    int32_t page_size;       // 128 or 256
    int32_t dql;             // 1..8
    int32_t cols;            // multiple of 4, <= 8192
    int32_t rank;            // row-sharded cache: this rank (0 when world_size == 1)
    int32_t world_size;      // 1: full page rows; 2 or 4: index_k holds rank's rows
};

struct SelectParams {
    const float* scores;     // [T, 4, cols]
    const int32_t* nvp;      // [T]
    msa_top16_row* out;      // [T, 4, R]
    int32_t* errors;         // nullable
    int32_t num_tokens;
    int32_t cols;
    int32_t init_blocks;
    int32_t local_blocks;
    int32_t num_ranges;
    int32_t width;           // ceil(cols / R)
    int32_t index_scale;     // column c stands for global id index_scale * c + index_offset
    int32_t index_offset;
};

struct MergeParams {
    const msa_top16_row* partial;  // [T, 4, R]
    const int32_t* nvp;            // [T]
    msa_top16_row* out;            // [T, 4]
    int32_t* errors;               // nullable
    int32_t num_tokens;
    int32_t num_ranges;
    int32_t init_blocks;
    int32_t local_blocks;
};

// Fused select + merge: at most this many ranges (one wave each) and at
// most 2048 columns per range.
constexpr int kMaxFusedRanges = 16;
// Duplicate-aware merge: one wave sorts at most this many rows' entries.
constexpr int kMaxDedupRanges = 64;
constexpr int kMaxFusedWidth = 2048;

struct SelectMergeParams {
    const float* scores;     // [T, 4, cols]
    const int32_t* nvp;      // [T]
    msa_top16_row* partial;  // [T, 4, R] or null
    msa_top16_row* out;      // [T, 4]
    int32_t* errors;         // nullable
    int32_t num_tokens;
    int32_t cols;
    int32_t init_blocks;
    int32_t local_blocks;
    int32_t num_ranges;
    int32_t width;           // ceil(cols / R)
};

// Scorer plus per-range select (and merge) in one launch (same ranges as
// SelectParams). Workspace: one 128-byte line per range (word 0: columns
// stored, word 1: select jobs done), then T * 4 merge tickets, then (pool
// mode) a 16-byte aligned plane of T * 4 * cols floats.
constexpr int kFusedLineWords = 32;
constexpr int kMaxFusedMergeRanges = 64;

// Words of the counters (range lines and tickets), and the word offset of the
// pool plane.
inline int64_t fused_counter_words(int64_t batch, int64_t dql, int64_t num_ranges)
{
    return batch * num_ranges * kFusedLineWords + batch * dql * 4;
}
inline int64_t fused_pool_offset(int64_t batch, int64_t dql, int64_t num_ranges)
{
    return (fused_counter_words(batch, dql, num_ranges) + 3) / 4 * 4;
}

struct ScoreSelectParams {
    ScoreParams score;       // score.out: the caller's plane, or the pool
    const int32_t* nvp;      // [batch*dql]
    msa_top16_row* out;      // [batch*dql, 4, R] range rows
    msa_top16_row* merged;   // [batch*dql, 4] or null
    int32_t* workspace;      // zero on entry and on exit
    int32_t init_blocks;
    int32_t local_blocks;
    int32_t num_ranges;
    int32_t width;           // ceil(cols / R) <= kMaxFusedWidth
    int32_t helpers;         // waves that run the select jobs (set by the launcher)
    int32_t pool;            // 1: score.out points into the workspace
};

// Prefill chain: columns per work item (an item's pages are held one per
// lane), and the most requests one plan takes (its LDS prefix array).
#ifndef MSA_PREFILL_ITEM_COLS
#define MSA_PREFILL_ITEM_COLS 32
#endif
constexpr int kPrefillItemCols = MSA_PREFILL_ITEM_COLS;
constexpr int kMaxPrefillBatch = 8192;

struct PrefillPlanParams {
    const int32_t* qo_indptr;  // [batch + 1]
    const int32_t* seq_lens;   // [batch]
    int32_t* plan;             // header + capacity items
    int64_t capacity;          // items the plan holds
    int32_t* errors;           // nullable
    int32_t batch;
    int32_t num_tokens;        // rows of index_q / of the plane
    int32_t cols;              // plane width
};

struct PrefillScoreParams {
    const uint8_t* q;        // [num_tokens, 4, 128] e4m3fn
    const uint8_t* k;        // [num_pages, page_size, 128] e4m3fn
    int64_t num_pages;
    const int32_t* bt;       // [bt_rows, bt_stride]
    int64_t bt_stride;
    int32_t bt_rows;
    const int32_t* plan;     // from the plan kernel
    int64_t capacity;        // items the plan holds
    float* out;              // [num_tokens, 4, cols]
    int32_t* errors;         // nullable
    int32_t page_size;
    int32_t cols;
    int32_t num_tokens;
};

hipError_t launch_score_decode(const ScoreParams& p, hipStream_t stream);
hipError_t launch_prefill_plan(const PrefillPlanParams& p, hipStream_t stream);
hipError_t launch_prefill_score(const PrefillScoreParams& p, int64_t capacity,
                                hipStream_t stream);
hipError_t launch_score_select(const ScoreSelectParams& q, hipStream_t stream);
hipError_t launch_top16_select_merge(const SelectMergeParams& p, hipStream_t stream);
hipError_t launch_top16_select(const SelectParams& p, hipStream_t stream);
hipError_t launch_top16_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_top16_merge_dedup(const MergeParams& p, hipStream_t stream);

// Loads the kernels of each file into the current device's context.
hipError_t warmup_score_kernels();
hipError_t warmup_top16_kernels();
hipError_t warmup_prefill_kernels();

}  // namespace msa
