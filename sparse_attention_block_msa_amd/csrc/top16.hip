// Top16 select and merge kernels for gfx950.
//
// Operation ("flashinfer.msa_ops.msa_icp_topk_select_publish", description;
// "flashinfer.msa_ops.prepare_msa_icp_indexer", init_blocks / local_blocks
// and the decode chain's merge): a row keeps its forced begin/end blocks
// ([0, init) and [n - local, n) within the valid ids [0, n)) and the best
// 16 - |forced| of its other valid blocks, ranked by score descending and
// then lower id, and lists them by ascending id; unused slots hold
// (-inf, -1). The merge applies the same rule to the union of a row's
// per-range lists.
//
// Design:
//  * A wave (64 lanes) owns a contiguous span of a row's elements; element i
//    of lane l is element span_lo + 64*i + l, so loads are coalesced and
//    "element order" == "id order".
//  * The wave-level selection itself is in top16_device.h.
//  * Spans longer than 1024 elements are split over 4 waves of one
//    workgroup; each wave selects its part, and wave 0 merges the four
//    partial rows from LDS with the same routine. Splitting is exact: a
//    block that belongs to the row's best K is also among the best of its
//    own part (fewer blocks beat it there than in the whole row).
#include <math.h>

#include "top16_device.h"

namespace msa {
namespace {

using namespace topk;

// One workgroup per (row, range): blockIdx.x = t * 4 + h, blockIdx.y = the
// range, so no integer division splits the job index. kMapped: column c
// stands for global id index_scale * c + index_offset
// (msa_top16_select_mapped); otherwise c is id c and the id arithmetic folds
// at compile time (with the scale read at run time, the interval bounds
// cost three integer divisions, dependent chains of about 30 instructions
// each, at the head of every select).
template <int V, int NW, bool kMapped>
__global__ __launch_bounds__(NW * 64) void top16_select_kernel(SelectParams p)
{
    __shared__ msa_top16_row part[NW];
    __shared__ CandBuf cand[NW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = (int)blockIdx.y;
    const int64_t th = blockIdx.x;
    const int64_t job = th * p.num_ranges + r;  // the output row ((t * 4) + h) * R + r
    const int t = (int)(th / kHeads);
    const int lo = r * p.width;
    const int span_lo = lo + wave * (V * 64);
    float sv[V];
    load_span<V>(p.scores + th * p.cols, p.cols, span_lo, lane, sv);

    const int scale = kMapped ? p.index_scale : 1;
    const int offset = kMapped ? p.index_offset : 0;
    // valid global ids: [0, n); the largest this plane can name is
    // index_scale * (cols - 1) + index_offset
    const int64_t n_max = (int64_t)scale * p.cols + offset;
    int n = p.nvp[t];
    if (n < 0 || n > n_max) {
        if (r == 0 && (th % kHeads) == 0 && threadIdx.x == 0 && p.errors)
            atomicAdd(p.errors, 1);
        n = n < 0 ? 0 : (int)n_max;
    }
    const int hi = min(lo + p.width, p.cols);
    const ColumnIds ci = column_ids(n, p.init_blocks, p.local_blocks, scale, offset);
    msa_top16_row* dst = NW == 1 ? p.out + job : &part[wave];
    select_loaded<V>(sv, span_lo, hi, ci, dst, lane, &cand[wave]);

    if (NW > 1) {
        __syncthreads();
        if (wave == 0)  // every forced id of the range is in exactly one partial row
            merge_lds_rows<NW>(part, n, p.init_blocks, p.local_blocks, -1, p.out + job, lane);
    }
}

// Rows per workgroup of the one-wave merge shapes when there are many rows:
// each wave merges its own row. On 32 768 one-range rows (a prefill merge)
// 2, 4 or 8 rows per workgroup took 7.2 us per launch against 9.9 us with
// one, the launch of 32 768 single-wave workgroups being what took the time.
constexpr int kMergeRowsPerGroup = 4;
constexpr int64_t kMergeManyRows = 16384;

template <int V, int NW>
__global__ __launch_bounds__(NW == 1 ? 64 * kMergeRowsPerGroup : NW * 64)
void top16_merge_kernel(MergeParams p)
{
    __shared__ msa_top16_row part[NW];
    __shared__ CandBuf cand[NW == 1 ? kMergeRowsPerGroup : NW];
    const int lane = threadIdx.x & 63;
    const int wave = NW == 1 ? 0 : threadIdx.x >> 6;
    // t * 4 + h; one-wave shapes may hold several rows, one per wave
    const int64_t th = NW == 1 ? (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)
                               : (int64_t)blockIdx.x;
    if (NW == 1 && th >= (int64_t)p.num_tokens * kHeads)
        return;
    const int t = (int)(th / kHeads);
    const int n = max(0, p.nvp[t]);
    const int total = p.num_ranges * kTop;  // entries in the concatenated rows
    const msa_top16_row* rows = p.partial + th * p.num_ranges;
    const int span_lo = wave * (V * 64);

    // Loads are unconditional (entry index clamped into the rows) so that
    // they overlap; entries past the end are masked afterwards.
    float sv[V];
    int iv[V];
    int pv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = min(span_lo + i * 64 + lane, total - 1);
        const int ep = max(e - 1, 0);
        sv[i] = rows[e / kTop].score[e % kTop];
        iv[i] = rows[e / kTop].id[e % kTop];
        pv[i] = rows[ep / kTop].id[ep % kTop];
    }
    uint32_t u[V];
    uint64_t fbits = 0;
    int n_forced = 0;
    bool disorder = false;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = span_lo + i * 64 + lane;
        const bool valid = e < total && iv[i] >= 0;
        const bool forced = valid && is_forced(iv[i], n, p.init_blocks, p.local_blocks);
        u[i] = valid && !forced ? order_key(sv[i]) : 0u;
        disorder |= valid && e > 0 && pv[i] >= iv[i];
        fbits |= (uint64_t)forced << i;
        n_forced += __popcll(__ballot(forced));
    }
    const uint64_t disorder_mask = __ballot(disorder);
    if (disorder_mask && lane == 0 && p.errors)
        atomicAdd(p.errors, 1);

    const int expected_forced = forced_count(n, p.init_blocks, p.local_blocks);
    if (V == 1 && p.num_ranges == 1) {
        // One row in (a prefill merge with R = 1): when it is already what the
        // merge would make of it (valid ids ascending in front, every forced
        // id present, canonical padding behind), the merge is the row itself
        // and is copied; any other row takes the selection below.
        const bool valid = lane < kTop && iv[0] >= 0;
        const uint64_t vmask = __ballot(valid);
        const int m = __popcll(vmask);
        // (a key of 0, a NaN score with every bit set, is no candidate: the
        // selection would drop it)
        const bool entry_ok = lane >= kTop ||
                              (valid ? order_key(sv[0]) != 0u
                                     : iv[0] == -1 && __float_as_uint(sv[0]) == 0xFF800000u);
        if (vmask == (1ull << m) - 1ull && __ballot(!entry_ok) == 0ull && !disorder_mask &&
            n_forced == expected_forced) {
            if (lane < kTop) {
                p.out[th].score[lane] = sv[0];
                p.out[th].id[lane] = iv[0];
            }
            return;
        }
    }
    msa_top16_row* dst = NW == 1 ? p.out + th : &part[wave];
    const int budget = NW == 1 ? kTop - expected_forced : kTop - n_forced;
    const int kept = select_row<V>(u, sv, fbits, budget, count_keys<V>(u), lane,
                                   &cand[threadIdx.x >> 6],
                                   [&](int i) { return iv[i]; },
                                   [&](float score, int id, int slot) {
                                       dst->score[slot] = score;
                                       dst->id[slot] = id;
                                   });
    pad_row(dst, kept, lane);
    // More than 16 kept entries: a forced id repeated in the input (rows
    // that are not disjoint ranges); the row holds the first 16.
    bool overflow = kept > kTop;

    int found_forced = n_forced;
    if (NW > 1) {
        if (overflow && lane == 0 && p.errors)
            atomicAdd(p.errors, 1);
        overflow = false;
        __syncthreads();
        if (wave == 0) {
            int kept_m = 0;
            found_forced = merge_lds_rows<NW>(part, n, p.init_blocks, p.local_blocks,
                                              kTop - expected_forced, p.out + th, lane, &kept_m);
            overflow = kept_m > kTop;
        }
    }
    if ((NW == 1 || wave == 0) && (found_forced < expected_forced || overflow) && lane == 0 &&
        p.errors)
        atomicAdd(p.errors, 1);
}

// Keeps the best K of the elements with key u != 0, ranked by key
// descending and then by lower id (ids are distinct among the candidates):
// take[i] is set for the kept ones. The K-th largest key thr comes from a
// bitwise descent; if more keys equal thr than are still needed, a second
// descent over their ids finds the lowest ones.
template <int V>
__device__ __forceinline__ void take_best(const uint32_t (&u)[V], const int (&id)[V], int K,
                                          bool (&take)[V])
{
#pragma unroll
    for (int i = 0; i < V; ++i)
        take[i] = false;
    if (K <= 0)
        return;
    uint32_t thr;
    if constexpr (V == 1) {
        thr = kth_largest_of_lanes(u[0], K, __lane_id());
    } else {
        uint32_t prefix = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t trial = prefix | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < V; ++i)
                cnt += __popcll(__ballot(u[i] >= trial));
            if (cnt >= K)
                prefix = trial;
        }
        thr = prefix;
    }
    int gt = 0, tied = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        gt += __popcll(__ballot(u[i] > thr));
        tied += __popcll(__ballot(u[i] == thr));
    }
    const int need = K - gt;  // >= 1 keys equal to thr are kept
    int cut = 0x7FFFFFFF;      // keep tied keys with id <= cut
    if (tied > need) {
        // the largest c with fewer than `need` tied ids below it: the
        // need-th smallest tied id is then c itself
        int c = 0;
        for (int bit = 30; bit >= 0; --bit) {
            const int trial = c | (1 << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < V; ++i)
                cnt += __popcll(__ballot(u[i] == thr && id[i] < trial));
            if (cnt < need)
                c = trial;
        }
        cut = c;
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
        take[i] = u[i] != 0u && (u[i] > thr || (u[i] == thr && id[i] <= cut));
}

template <int kSlots>
__device__ __forceinline__ int slot_of(int id)
{
    static_assert((kSlots & (kSlots - 1)) == 0, "power of two");
    constexpr int kBits = __builtin_ctz(kSlots);
    return (int)(((uint32_t)id * 2654435761u) >> (32 - kBits));  // Fibonacci hashing
}

// Merge of partial rows in any order, an id possibly in several of them
// (rows from ranks that each hold part of every page's rows): one wave per
// (token, head), 64V >= R * 16 entries, element i of lane l is entry 64i + l
// of the concatenated rows.
//  * Each id's best entry (highest score, the earliest of equal ones such as
//    -0 and +0) is found with an LDS hash table: a compare-and-swap claims
//    the id's slot, and a 64-bit atomic max keeps (rank key, -position).
//    The merge of row shards keeps an id's highest partial score: a block's
//    max over its rows is the max over the shards of their maxima.
//  * Forced ids are recomputed over [0, n) and kept; one missing from the
//    union is counted. The other best entries compete by (score descending,
//    id ascending) for 16 - |forced of [0, n)| slots: the keys at or above
//    the K-th largest lane maximum (at most 64, else all of them) go through
//    take_best.
//  * The kept entries (at most 16) are written by ascending id: each finds
//    its slot by counting the kept ids below its own.
template <int V>
__global__ __launch_bounds__(64) void top16_merge_dedup_kernel(MergeParams p)
{
    constexpr int kN = 64 * V;
    constexpr int kSlots = 2 * kN;
    __shared__ int slot_id[kSlots];
    __shared__ unsigned long long slot_best[kSlots];
    __shared__ Candidate cand[64];
    __shared__ float kept_score[kTop];
    __shared__ int kept_id[kTop];
    const int lane = threadIdx.x;
    const int64_t th = blockIdx.x;  // t * 4 + h
    const int t = (int)(th / kHeads);
    const int total = p.num_ranges * kTop;
    const msa_top16_row* rows = p.partial + th * p.num_ranges;

    for (int s = lane; s < kSlots; s += 64) {
        slot_id[s] = -1;
        slot_best[s] = 0ull;
    }
    float sv[V];
    int iv[V];
    unsigned long long pk[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = i * 64 + lane;
        const int ec = min(e, total - 1);
        iv[i] = e < total ? rows[ec / kTop].id[ec % kTop] : -1;
        sv[i] = rows[ec / kTop].score[ec % kTop];
        pk[i] = ((unsigned long long)order_key(sv[i]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
    }
    const int n = max(0, p.nvp[t]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    int hs[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        hs[i] = 0;
        if (iv[i] >= 0) {
            int h = slot_of<kSlots>(iv[i]);
            while (true) {  // at most kN ids in 2 * kN slots: a free slot exists
                int expected = -1;
                __hip_atomic_compare_exchange_strong(&slot_id[h], &expected, iv[i],
                                                     __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
                if (expected == -1 || expected == iv[i])
                    break;
                h = (h + 1) & (kSlots - 1);
            }
            hs[i] = h;
            __hip_atomic_fetch_max(&slot_best[h], pk[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    uint32_t u[V];
    bool forced[V];
    int n_forced = 0;
    uint32_t lane_max = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const bool best = iv[i] >= 0 && slot_best[hs[i]] == pk[i];
        forced[i] = best && is_forced(iv[i], n, p.init_blocks, p.local_blocks);
        u[i] = best && !forced[i] ? order_key(sv[i]) : 0u;
        n_forced += __popcll(__ballot(forced[i]));
        lane_max = max(lane_max, u[i]);
    }
    const int expected_forced = forced_count(n, p.init_blocks, p.local_blocks);
    if (n_forced < expected_forced && lane == 0 && p.errors)
        atomicAdd(p.errors, 1);
    const int K = min(kTop - expected_forced, count_keys<V>(u));

    // threshold filter: every key of the best K is >= theta
    uint32_t theta = 1u;
    if (K > 0)
        theta = max(kth_largest_of_lanes(lane_max, K, lane), 1u);
    int base = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const bool sel = K > 0 && u[i] >= theta;
        const uint64_t mask = __ballot(sel);
        const int slot = base + lanes_below(mask);
        if (sel && slot < 64) {
            Candidate c;
            c.key = u[i];
            c.score = sv[i];
            c.id = iv[i];
            cand[slot] = c;
        }
        base += __popcll(mask);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // the kept entries, compacted into kept_score / kept_id
    int m = 0;
    auto keep = [&](bool k, float score, int id) {
        const uint64_t mask = __ballot(k);
        if (k) {
            const int slot = m + lanes_below(mask);
            kept_score[slot] = score;
            kept_id[slot] = id;
        }
        m += __popcll(mask);
    };
#pragma unroll
    for (int i = 0; i < V; ++i)
        keep(forced[i], sv[i], iv[i]);
    if (base <= 64) {
        Candidate mine = {0u, -INFINITY, -1};
        if (lane < base)
            mine = cand[lane];
        const uint32_t u1[1] = {mine.key};
        const int id1[1] = {mine.id};
        bool take1[1];
        take_best<1>(u1, id1, K, take1);
        keep(take1[0], mine.score, mine.id);
    } else {  // heavy ties at theta: rank every value
        bool take[V];
        take_best<V>(u, iv, K, take);
#pragma unroll
        for (int i = 0; i < V; ++i)
            keep(take[i], sv[i], iv[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    msa_top16_row* dst = p.out + th;
    if (lane < m) {
        const int my_id = kept_id[lane];
        int rank = 0;
        for (int j = 0; j < m; ++j)
            rank += kept_id[j] < my_id ? 1 : 0;
        dst->score[rank] = kept_score[lane];
        dst->id[rank] = my_id;
    }
    pad_row(dst, m, lane);
}

// Select over R ranges and merge, one (token, head) row per workgroup: wave
// r selects range r exactly as top16_select_kernel does with one wave per
// range, writes its row to `partial` (when given) and to LDS, and wave 0 then
// merges the R rows exactly as top16_merge_kernel does (every forced id of
// the row is in one of them, so the budget is K = 16 - |forced of [0, n)|).
// The merge first prunes: wave r also reports theta_r, the key of its
// range's K-th best candidate (0 if it has fewer or the search did not
// rank them). The row's K-th best key is at least every theta_r (range r
// alone holds K keys >= theta_r), so the row's best K are among the entries
// with keys >= max theta_r, and with forced entries those usually fit one
// wave: they are ranked as the range selects rank their survivors.
// Otherwise the merge selects over all R rows.
template <int V, int VM>
__global__ __launch_bounds__(1024) void top16_select_merge_kernel(SelectMergeParams p)
{
    __shared__ msa_top16_row part[kMaxFusedRanges];
    __shared__ CandBuf cand[kMaxFusedRanges];
    __shared__ uint32_t range_kth[kMaxFusedRanges];
    const int lane = threadIdx.x & 63;
    const int r = threadIdx.x >> 6;
    const int64_t th = blockIdx.x;  // t * 4 + h
    const int t = (int)(th / kHeads);
    const int lo = r * p.width;
    float sv[V];
    load_span<V>(p.scores + th * p.cols, p.cols, lo, lane, sv);

    int n = p.nvp[t];
    if (n < 0 || n > p.cols) {
        if ((th % kHeads) == 0 && threadIdx.x == 0 && p.errors)
            atomicAdd(p.errors, 1);
        n = n < 0 ? 0 : p.cols;
    }
    const int budget = kTop - forced_count(n, p.init_blocks, p.local_blocks);
    msa_top16_row* mine = &part[r];
    uint32_t kth = 0u;
    select_loaded<V>(sv, lo, min(lo + p.width, p.cols), column_ids(n, p.init_blocks,
                                                                  p.local_blocks, 1, 0),
                     mine, lane, &cand[r], budget, &kth);
    if (lane == 0)
        range_kth[r] = kth;
    __syncthreads();
    if (p.partial && lane < 2 * kTop)
        reinterpret_cast<int*>(p.partial + th * p.num_ranges + r)[lane] =
            reinterpret_cast<const int*>(mine)[lane];
    if (r != 0)
        return;

    // wave 0: merge the R rows from LDS
    uint32_t theta = 1u;
    for (int w = 0; w < p.num_ranges; ++w)
        theta = max(theta, range_kth[w]);
    const int total = p.num_ranges * kTop;
    float mv[VM];
    int iv[VM];
#pragma unroll
    for (int i = 0; i < VM; ++i) {
        const int e = min(i * 64 + lane, total - 1);
        mv[i] = part[e / kTop].score[e % kTop];
        iv[i] = part[e / kTop].id[e % kTop];
    }
    uint32_t um[VM];
    uint64_t fm = 0;
#pragma unroll
    for (int i = 0; i < VM; ++i) {
        const bool valid = i * 64 + lane < total && iv[i] >= 0;
        const bool forced = valid && is_forced(iv[i], n, p.init_blocks, p.local_blocks);
        um[i] = valid && !forced ? order_key(mv[i]) : 0u;
        fm |= (uint64_t)forced << i;
    }
    msa_top16_row* dst = p.out + th;
    auto emit = [&](float score, int id, int slot) {
        dst->score[slot] = score;
        dst->id[slot] = id;
    };
    const int n_cand = count_keys<VM>(um);
    const int K = min(budget, n_cand);
    const int survivors = compact_selected<true>(um, mv, fm, K > 0 ? theta : ~0u, lane, &cand[0],
                                                 [&](int i) { return iv[i]; });
    const int kept_m = survivors <= 64
                           ? rank_select(&cand[0], survivors, K, lane, 0, nullptr, emit)
                           : select_row<VM>(um, mv, fm, budget, n_cand, lane, &cand[0],
                                            [&](int i) { return iv[i]; }, emit);
    pad_row(dst, kept_m, lane);
}

// Whole-row Top16 in one pass, for msa_top16_select_merge without per-range
// rows: the merge of a row's split lists equals the select of the whole row,
// so one selection over the row gives the same rows.
//  * Wave w loads span [64Vw, 64V(w+1)) of the row and takes theta_w, the
//    K-th largest of its 64 lane maxima (K = 16 - |forced ids of the row|).
//    A span with at least K candidates has at least K keys >= theta_w, so
//    theta = the largest such theta_w is at most the row's K-th largest key:
//    every key of the best K, ties at the K-th included, is >= theta.
//  * Each wave compacts its forced entries and its keys >= theta into its own
//    LDS segment (at most 64), in element (= id) order. When the segments hold
//    at most 128 entries together, wave 0 selects among them with one or two
//    values per lane, the segments read in wave order (ascending ids).
//    Otherwise (heavy ties, or spans too short to bound the row) every wave
//    selects its span as msa_top16_select does and wave 0 merges the NW rows
//    (exact by the same argument).
template <int V, int NW>
__global__ __launch_bounds__(NW * 64) void top16_row_select_kernel(SelectMergeParams p)
{
    constexpr int VM = NW * kTop / 64 > 0 ? NW * kTop / 64 : 1;  // merge values per lane
    __shared__ CandBuf seg[NW];
    __shared__ int seg_count[NW];
    __shared__ uint32_t theta_w[NW];
    __shared__ msa_top16_row part[NW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t th = blockIdx.x;  // t * 4 + h
    const int t = (int)(th / kHeads);
    const int span_lo = wave * 64 * V;
    float sv[V];
    load_span<V>(p.scores + th * p.cols, p.cols, span_lo, lane, sv);

    int n = p.nvp[t];
    if (n < 0 || n > p.cols) {
        if ((th % kHeads) == 0 && threadIdx.x == 0 && p.errors)
            atomicAdd(p.errors, 1);
        n = n < 0 ? 0 : p.cols;
    }
    const ColumnIds ci = column_ids(n, p.init_blocks, p.local_blocks, 1, 0);
    const int K = kTop - forced_count(n, p.init_blocks, p.local_blocks);

    // keys of the span, as select_loaded forms them
    const int valid_hi = min(min(p.cols, ci.valid_end), span_lo + V * 64);
    const int n_valid = max(0, valid_hi - span_lo);
    const int n_init = max(0, min(valid_hi, ci.init_end) - span_lo);
    const int n_local = max(0, valid_hi - max(span_lo, ci.local_begin));
    const int n_both = max(0, min(valid_hi, ci.init_end) - max(span_lo, ci.local_begin));
    const int n_cand = n_valid - (n_init + n_local - n_both);
    uint32_t u[V];
    uint64_t fbits = 0;
    uint32_t lane_max = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = span_lo + i * 64 + lane;
        const bool valid = c < valid_hi;
        const bool forced = valid && (c < ci.init_end || c >= ci.local_begin);
        u[i] = valid && !forced ? order_key(sv[i]) : 0u;
        fbits |= (uint64_t)forced << i;
        lane_max = max(lane_max, u[i]);
    }
    uint32_t tw = 0;  // 0: this span does not bound the row
    if (K > 0 && n_cand >= K)
        tw = max(kth_largest_of_lanes(lane_max, K, lane), 1u);
    if (lane == 0)
        theta_w[wave] = tw;
    __syncthreads();
    uint32_t theta = 1u;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        theta = max(theta, theta_w[w]);

    int base = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const bool forced = (fbits >> i) & 1ull;
        const bool sel = forced || (K > 0 && u[i] >= theta);
        const uint64_t mask = __ballot(sel);
        const int slot = base + lanes_below(mask);
        if (sel && slot < 64)  // candidates have keys >= theta >= 1
            cand_store(&seg[wave], slot, forced ? 0u : u[i], sv[i], span_lo + i * 64 + lane);
        base += __popcll(mask);
    }
    if (lane == 0)
        seg_count[wave] = base;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        total += min(seg_count[w], 129);  // a segment past 64 forces the fallback
    bool fits = total <= 128;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        fits = fits && seg_count[w] <= 64;
    msa_top16_row* dst = p.out + th;
    if (fits) {
        if (wave != 0)
            return;
        // element e of the concatenated segments (wave order: ascending ids)
        auto gather = [&](int e) {
            Candidate c = {0u, -INFINITY, -1};
            int before = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int cnt = seg_count[w];
                if (e >= before && e < before + cnt)
                    c = cand_load(&seg[w], e - before);
                before += cnt;
            }
            return c;
        };
        if (total <= 64) {
            const Candidate mine = gather(lane);
            const bool have = lane < total;
            const uint32_t u1[1] = {have ? mine.key : 0u};
            const uint64_t f1 = (have && mine.key == 0u) ? 1ull : 0ull;
            const int kept = wave_select<1>(u1, f1, K, count_keys<1>(u1), [&](int, int slot) {
                dst->score[slot] = mine.score;
                dst->id[slot] = mine.id;
            });
            pad_row(dst, kept, lane);
        } else {
            const Candidate mine[2] = {gather(lane), gather(64 + lane)};
            uint32_t u2[2];
            uint64_t f2 = 0;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bool have = 64 * i + lane < total;
                u2[i] = have ? mine[i].key : 0u;
                f2 |= (uint64_t)(have && mine[i].key == 0u) << i;
            }
            const int kept = wave_select<2>(u2, f2, K, count_keys<2>(u2), [&](int i, int slot) {
                dst->score[slot] = mine[i].score;
                dst->id[slot] = mine[i].id;
            });
            pad_row(dst, kept, lane);
        }
        return;
    }

    // fallback: select every span, then merge the NW rows
    select_loaded<V>(sv, span_lo, p.cols, ci, &part[wave], lane, &seg[wave]);
    __syncthreads();
    if (wave != 0)
        return;
    float mv[VM];
    int iv[VM];
#pragma unroll
    for (int i = 0; i < VM; ++i) {
        const int e = min(i * 64 + lane, NW * kTop - 1);
        mv[i] = part[e / kTop].score[e % kTop];
        iv[i] = part[e / kTop].id[e % kTop];
    }
    uint32_t um[VM];
    uint64_t fm = 0;
#pragma unroll
    for (int i = 0; i < VM; ++i) {
        const bool valid = i * 64 + lane < NW * kTop && iv[i] >= 0;
        const bool forced = valid && is_forced(iv[i], n, p.init_blocks, p.local_blocks);
        um[i] = valid && !forced ? order_key(mv[i]) : 0u;
        fm |= (uint64_t)forced << i;
    }
    const int kept_m = select_row<VM>(um, mv, fm, K, count_keys<VM>(um), lane, &seg[0],
                                      [&](int i) { return iv[i]; },
                                      [&](float score, int id, int slot) {
                                          dst->score[slot] = score;
                                          dst->id[slot] = id;
                                      });
    pad_row(dst, kept_m, lane);
}

// Launch shape: spans up to 1024 elements use one wave with V = the next
// power of two >= span/64; longer spans use 4 waves with V = 4 .. 48 (on
// 2048-element rows the 4-wave split measured 2 us faster per launch than
// one wave with V = 32).
struct Shape {
    int v;
    int nw;
};

#ifndef MSA_SELECT_ONE_WAVE_MAX_V
#define MSA_SELECT_ONE_WAVE_MAX_V 16
#endif

Shape pick_shape(int64_t span)
{
    const int64_t per_lane = (span + 63) / 64;
    if (per_lane <= MSA_SELECT_ONE_WAVE_MAX_V) {
        int v = 1;
        while (v < per_lane)
            v *= 2;
        return {v, 1};
    }
    const int64_t per_lane4 = (span + 255) / 256;
    return {per_lane4 <= 4 ? 4 : per_lane4 <= 8 ? 8 : per_lane4 <= 16 ? 16 : per_lane4 <= 32 ? 32 : 48, 4};
}

template <int V, int NW>
hipError_t launch_select_shape(const SelectParams& p, hipStream_t stream)
{
    const int64_t rows = (int64_t)p.num_tokens * kHeads;
    const bool mapped = p.index_scale != 1 || p.index_offset != 0;
    const void* fn = mapped ? reinterpret_cast<const void*>(&top16_select_kernel<V, NW, true>)
                            : reinterpret_cast<const void*>(&top16_select_kernel<V, NW, false>);
    void* args[] = {const_cast<SelectParams*>(&p)};
    return hipLaunchKernel(fn, dim3((unsigned)rows, (unsigned)p.num_ranges), dim3(NW * 64), args,
                           0, stream);
}

template <int V, int NW>
hipError_t launch_merge_shape(const MergeParams& p, hipStream_t stream)
{
    const int64_t jobs = (int64_t)p.num_tokens * kHeads;
    const int rows = NW == 1 && jobs >= kMergeManyRows ? kMergeRowsPerGroup : 1;
    void* args[] = {const_cast<MergeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&top16_merge_kernel<V, NW>),
                           dim3((unsigned)((jobs + rows - 1) / rows)), dim3(NW * 64 * rows), args,
                           0, stream);
}

#define MSA_FOR_EACH_SHAPE(X) \
    X(1, 1) X(2, 1) X(4, 1) X(8, 1) X(16, 1) X(32, 1) X(4, 4) X(8, 4) X(16, 4) X(32, 4) X(48, 4)

}  // namespace

hipError_t launch_top16_select(const SelectParams& p, hipStream_t stream)
{
    const Shape s = pick_shape(p.width);
#define X(V, NW)                                      \
    if (s.v == V && s.nw == NW)                       \
        return launch_select_shape<V, NW>(p, stream);
    MSA_FOR_EACH_SHAPE(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_top16_merge(const MergeParams& p, hipStream_t stream)
{
    const Shape s = pick_shape((int64_t)p.num_ranges * kTop);
#define X(V, NW)                                     \
    if (s.v == V && s.nw == NW)                      \
        return launch_merge_shape<V, NW>(p, stream);
    MSA_FOR_EACH_SHAPE(X)
#undef X
    return hipErrorInvalidValue;
}

#define MSA_FOR_EACH_DEDUP_SHAPE(X) X(1) X(2) X(4) X(8) X(16)

template <int V>
hipError_t launch_dedup_shape(const MergeParams& p, hipStream_t stream)
{
    void* args[] = {const_cast<MergeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&top16_merge_dedup_kernel<V>),
                           dim3((unsigned)((int64_t)p.num_tokens * kHeads)), dim3(64), args, 0,
                           stream);
}

template <int V, int VM>
hipError_t launch_fused_shape(const SelectMergeParams& p, hipStream_t stream)
{
    void* args[] = {const_cast<SelectMergeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&top16_select_merge_kernel<V, VM>),
                           dim3((unsigned)((int64_t)p.num_tokens * kHeads)),
                           dim3(p.num_ranges * 64), args, 0, stream);
}

#define MSA_FOR_EACH_FUSED_SHAPE(X) \
    X(1, 1) X(2, 1) X(4, 1) X(8, 1) X(16, 1) X(32, 1) \
    X(1, 2) X(2, 2) X(4, 2) X(8, 2) X(16, 2) X(32, 2) \
    X(1, 4) X(2, 4) X(4, 4) X(8, 4) X(16, 4) X(32, 4)

#define MSA_FOR_EACH_ROW_SHAPE(X) \
    X(1, 1) X(2, 1) X(4, 1) X(8, 1) X(16, 1) X(16, 2) X(16, 4) X(16, 8) X(32, 8)

template <int V, int NW>
hipError_t launch_row_shape(const SelectMergeParams& p, hipStream_t stream)
{
    void* args[] = {const_cast<SelectMergeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&top16_row_select_kernel<V, NW>),
                           dim3((unsigned)((int64_t)p.num_tokens * kHeads)), dim3(NW * 64), args,
                           0, stream);
}

hipError_t launch_top16_select_merge(const SelectMergeParams& p, hipStream_t stream)
{
    if (p.partial == nullptr) {
        // no per-range rows asked for: one selection over the whole row.
        // Spans of 1024 columns per wave (up to 8 waves): on N(0,1) rows of
        // 8192 columns and K = 8 the row bound then passes about 37 keys
        // (fewer than 64 in 99.5% of rows); spans of 512 pass about 65.
        const int nw = p.cols <= 1024 ? 1 : p.cols <= 2048 ? 2 : p.cols <= 4096 ? 4 : 8;
        const int v = p.cols <= 64 ? 1 : p.cols <= 128 ? 2 : p.cols <= 256 ? 4
                    : p.cols <= 512 ? 8 : p.cols <= 8192 ? 16 : 32;
#define X(V, NW)                                   \
        if (v == V && nw == NW)                    \
            return launch_row_shape<V, NW>(p, stream);
        MSA_FOR_EACH_ROW_SHAPE(X)
#undef X
        return hipErrorInvalidValue;
    }
    // one wave per range: V = the next power of two >= ceil(width / 64), <= 32
    int v = 1;
    while (v * 64 < p.width)
        v *= 2;
    const int vm = p.num_ranges <= 4 ? 1 : p.num_ranges <= 8 ? 2 : 4;
#define X(V, VM)                                   \
    if (v == V && vm == VM)                        \
        return launch_fused_shape<V, VM>(p, stream);
    MSA_FOR_EACH_FUSED_SHAPE(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_top16_merge_dedup(const MergeParams& p, hipStream_t stream)
{
    // one wave; 64 * V >= R * 16 entries (R <= 64)
    int v = 1;
    while (v * 64 < p.num_ranges * kTop)
        v *= 2;
#define X(V)        \
    if (v == V)     \
        return launch_dedup_shape<V>(p, stream);
    MSA_FOR_EACH_DEDUP_SHAPE(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t warmup_top16_kernels()
{
    hipFuncAttributes attr;
    hipError_t e = hipSuccess;
#define X(V, NW)                                                                                  \
    if (e == hipSuccess)                                                                          \
        e = hipFuncGetAttributes(&attr,                                                           \
                                 reinterpret_cast<const void*>(&top16_select_kernel<V, NW, false>)); \
    if (e == hipSuccess)                                                                          \
        e = hipFuncGetAttributes(&attr,                                                           \
                                 reinterpret_cast<const void*>(&top16_select_kernel<V, NW, true>)); \
    if (e == hipSuccess)                                                                          \
        e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&top16_merge_kernel<V, NW>));
    MSA_FOR_EACH_SHAPE(X)
#undef X
#define X(V, VM)                                                                               \
    if (e == hipSuccess)                                                                       \
        e = hipFuncGetAttributes(&attr,                                                        \
                                 reinterpret_cast<const void*>(&top16_select_merge_kernel<V, VM>));
    MSA_FOR_EACH_FUSED_SHAPE(X)
#undef X
#define X(V)                                                                                      \
    if (e == hipSuccess)                                                                          \
        e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&top16_merge_dedup_kernel<V>));
    MSA_FOR_EACH_DEDUP_SHAPE(X)
#undef X
#define X(V, NW)                                                                                 \
    if (e == hipSuccess)                                                                         \
        e = hipFuncGetAttributes(&attr,                                                          \
                                 reinterpret_cast<const void*>(&top16_row_select_kernel<V, NW>));
    MSA_FOR_EACH_ROW_SHAPE(X)
#undef X
    return e;
}

}  // namespace msa
