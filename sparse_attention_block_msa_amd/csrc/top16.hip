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

template <int V, int NW>
__global__ __launch_bounds__(NW * 64) void top16_select_kernel(SelectParams p)
{
    __shared__ msa_top16_row part[NW];
    __shared__ Candidate cand[NW][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t job = blockIdx.x;  // ((t * 4) + h) * R + r
    const int r = (int)(job % p.num_ranges);
    const int64_t th = job / p.num_ranges;
    const int t = (int)(th / kHeads);
    const int lo = r * p.width;
    const int span_lo = lo + wave * (V * 64);
    float sv[V];
    load_span<V>(p.scores + th * p.cols, p.cols, span_lo, lane, sv);

    // valid global ids: [0, n); the largest this plane can name is
    // index_scale * (cols - 1) + index_offset
    const int64_t n_max = (int64_t)p.index_scale * p.cols + p.index_offset;
    int n = p.nvp[t];
    if (n < 0 || n > n_max) {
        if (r == 0 && (th % kHeads) == 0 && threadIdx.x == 0 && p.errors)
            atomicAdd(p.errors, 1);
        n = n < 0 ? 0 : (int)n_max;
    }
    const int hi = min(lo + p.width, p.cols);
    const ColumnIds ci = column_ids(n, p.init_blocks, p.local_blocks, p.index_scale,
                                    p.index_offset);
    msa_top16_row* dst = NW == 1 ? p.out + job : &part[wave];
    select_loaded<V>(sv, span_lo, hi, ci, dst, lane, cand[wave]);

    if (NW > 1) {
        __syncthreads();
        if (wave == 0)  // every forced id of the range is in exactly one partial row
            merge_lds_rows<NW>(part, n, p.init_blocks, p.local_blocks, -1, p.out + job, lane);
    }
}

template <int V, int NW>
__global__ __launch_bounds__(NW * 64) void top16_merge_kernel(MergeParams p)
{
    __shared__ msa_top16_row part[NW];
    __shared__ Candidate cand[NW][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t th = blockIdx.x;  // t * 4 + h
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
    msa_top16_row* dst = NW == 1 ? p.out + th : &part[wave];
    const int budget = NW == 1 ? kTop - expected_forced : kTop - n_forced;
    const int kept = select_row<V>(u, sv, fbits, budget, count_keys<V>(u), lane, cand[wave],
                                   [&](int i) { return iv[i]; },
                                   [&](float score, int id, int slot) {
                                       dst->score[slot] = score;
                                       dst->id[slot] = id;
                                   });
    pad_row(dst, kept, lane);

    int found_forced = n_forced;
    if (NW > 1) {
        __syncthreads();
        if (wave == 0)
            found_forced = merge_lds_rows<NW>(part, n, p.init_blocks, p.local_blocks,
                                              kTop - expected_forced, p.out + th, lane);
    }
    if ((NW == 1 || wave == 0) && found_forced < expected_forced && lane == 0 && p.errors)
        atomicAdd(p.errors, 1);
}

// Inverse of order_key, up to the sign of zero (order_key maps -0 to +0).
__device__ __forceinline__ uint32_t key_to_bits(uint32_t k)
{
    return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}

// Sort element of the duplicate-aware merge: hi = id (0x7FFFFFFF for an
// empty slot), lo = ~order_key(score), tag = position in the concatenated
// rows (low 16 bits) | 0x80000000 if the score is -0. Ordered by
// (hi, lo, position): ascending id, then score descending, then earliest.
struct SortEl {
    uint32_t hi, lo, tag;
};

__device__ __forceinline__ bool sort_before(const SortEl& a, const SortEl& b)
{
    if (a.hi != b.hi)
        return a.hi < b.hi;
    if (a.lo != b.lo)
        return a.lo < b.lo;
    return (a.tag & 0xFFFFu) < (b.tag & 0xFFFFu);
}

// Sorts the wave's 64V elements by sort_before. Element e = V * lane + i sits
// in slot i of `lane` (lane-major), so stages whose partner is fewer than V
// elements away swap registers within a lane and only the stages with
// partners V or more apart read the partner lane (three shuffles per
// element). The network is fully unrolled, so every register index is a
// compile-time constant.
template <int V>
__device__ __forceinline__ void bitonic_sort_wave(SortEl (&el)[V], int lane)
{
    constexpr int kN = 64 * V;
#pragma unroll
    for (int k = 2; k <= kN; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j < V) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const int i2 = i ^ j;
                    if (i2 > i) {
                        const bool up = ((V * lane + i) & k) == 0;
                        if (sort_before(el[i2], el[i]) == up) {
                            const SortEl t = el[i];
                            el[i] = el[i2];
                            el[i2] = t;
                        }
                    }
                }
            } else {
                const int lj = j / V;  // partner lane distance
                const bool lower = (lane & lj) == 0;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const bool up = ((V * lane + i) & k) == 0;
                    SortEl o;
                    o.hi = (uint32_t)__shfl_xor((int)el[i].hi, lj);
                    o.lo = (uint32_t)__shfl_xor((int)el[i].lo, lj);
                    o.tag = (uint32_t)__shfl_xor((int)el[i].tag, lj);
                    // the lower element keeps the min when up, the max otherwise
                    const bool keep_min = lower == up;
                    if (sort_before(o, el[i]) == keep_min)
                        el[i] = o;
                }
            }
        }
    }
}

// Merge of partial rows in any order, an id possibly in several of them
// (rows from ranks that each hold part of every page's rows): one wave per
// (token, head). The row's R * 16 entries are sorted by (id ascending, score
// descending, position) with a wave-wide bitonic network in registers, so
// each id's entries are adjacent with its highest score first (the earliest
// of equal ones, e.g. -0 and +0). The first entry of each id is kept (the
// merge of row shards keeps an id's highest partial score: a block's max over
// its rows is the max over the shards of their maxima). The kept entries go
// through LDS into the select's element order (element i of lane l is sorted
// position 64i + l, so element order is id order) and the usual selection
// runs. Forced ids are recomputed over [0, n); one missing from the union is
// counted.
template <int V>
__global__ __launch_bounds__(64) void top16_merge_dedup_kernel(MergeParams p)
{
    __shared__ uint32_t sid[64 * V];
    __shared__ uint32_t sraw[64 * V];
    __shared__ Candidate cand[64];
    const int lane = threadIdx.x;
    const int64_t th = blockIdx.x;  // t * 4 + h
    const int t = (int)(th / kHeads);
    const int total = p.num_ranges * kTop;
    const msa_top16_row* rows = p.partial + th * p.num_ranges;
    SortEl el[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = V * lane + i;
        const int ec = min(e, total - 1);
        int id = rows[ec / kTop].id[ec % kTop];
        float sc = rows[ec / kTop].score[ec % kTop];
        if (e >= total || id < 0) {
            id = 0x7FFFFFFF;  // sorts after every real id; dropped below
            sc = -INFINITY;
        }
        el[i].hi = (uint32_t)id;
        el[i].lo = ~order_key(sc);
        el[i].tag = (uint32_t)e | (__float_as_uint(sc) == 0x80000000u ? 0x80000000u : 0u);
    }
    const int n = max(0, p.nvp[t]);
    bitonic_sort_wave<V>(el, lane);

    // drop repeated ids (the previous element is slot i - 1, or the previous
    // lane's last slot) and hand the survivors to the select's layout
    const uint32_t prev_lane_last = (uint32_t)__shfl_up((int)el[V - 1].hi, 1);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const uint32_t prev = i > 0 ? el[i - 1].hi : (lane > 0 ? prev_lane_last : 0xFFFFFFFFu);
        const bool kept = el[i].hi != 0x7FFFFFFFu && el[i].hi != prev;
        const uint32_t bits = (el[i].tag & 0x80000000u) ? 0x80000000u : key_to_bits(~el[i].lo);
        sid[V * lane + i] = kept ? el[i].hi : 0xFFFFFFFFu;
        sraw[V * lane + i] = bits;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float sv[V];
    int iv[V];
    uint32_t u[V];
    uint64_t fbits = 0;
    int n_forced = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const uint32_t id = sid[i * 64 + lane];
        const bool kept = id != 0xFFFFFFFFu;
        sv[i] = __uint_as_float(sraw[i * 64 + lane]);
        iv[i] = (int)id;
        const bool forced = kept && is_forced((int)id, n, p.init_blocks, p.local_blocks);
        u[i] = kept && !forced ? order_key(sv[i]) : 0u;
        fbits |= (uint64_t)forced << i;
        n_forced += __popcll(__ballot(forced));
    }
    const int expected_forced = forced_count(n, p.init_blocks, p.local_blocks);
    if (n_forced < expected_forced && lane == 0 && p.errors)
        atomicAdd(p.errors, 1);
    msa_top16_row* dst = p.out + th;
    const int kept = select_row<V>(u, sv, fbits, kTop - expected_forced, count_keys<V>(u), lane,
                                   cand, [&](int i) { return iv[i]; },
                                   [&](float score, int id, int slot) {
                                       dst->score[slot] = score;
                                       dst->id[slot] = id;
                                   });
    pad_row(dst, kept, lane);
}

// Select over R ranges and merge, one (token, head) row per workgroup: wave
// r selects range r exactly as top16_select_kernel does with one wave per
// range, writes its row to `partial` (when given) and to LDS, and wave 0 then
// merges the R rows exactly as top16_merge_kernel does (every forced id of
// the row is in one of them, so the budget is 16 - |forced of [0, n)|).
template <int V, int VM>
__global__ __launch_bounds__(1024) void top16_select_merge_kernel(SelectMergeParams p)
{
    __shared__ msa_top16_row part[kMaxFusedRanges];
    __shared__ Candidate cand[kMaxFusedRanges][64];
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
    msa_top16_row* mine = &part[r];
    select_loaded<V>(sv, lo, min(lo + p.width, p.cols), column_ids(n, p.init_blocks,
                                                                  p.local_blocks, 1, 0),
                     mine, lane, cand[r]);
    __syncthreads();
    if (p.partial && lane < 2 * kTop)
        reinterpret_cast<int*>(p.partial + th * p.num_ranges + r)[lane] =
            reinterpret_cast<const int*>(mine)[lane];
    if (r != 0)
        return;

    // wave 0: merge the R rows from LDS
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
    const int kept_m = select_row<VM>(um, mv, fm, kTop - forced_count(n, p.init_blocks, p.local_blocks),
                                      count_keys<VM>(um), lane, cand[0], [&](int i) { return iv[i]; },
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
    const int64_t jobs = (int64_t)p.num_tokens * kHeads * p.num_ranges;
    void* args[] = {const_cast<SelectParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&top16_select_kernel<V, NW>),
                           dim3((unsigned)jobs), dim3(NW * 64), args, 0, stream);
}

template <int V, int NW>
hipError_t launch_merge_shape(const MergeParams& p, hipStream_t stream)
{
    const int64_t jobs = (int64_t)p.num_tokens * kHeads;
    void* args[] = {const_cast<MergeParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&top16_merge_kernel<V, NW>),
                           dim3((unsigned)jobs), dim3(NW * 64), args, 0, stream);
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

hipError_t launch_top16_select_merge(const SelectMergeParams& p, hipStream_t stream)
{
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
        e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&top16_select_kernel<V, NW>)); \
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
    return e;
}

}  // namespace msa
