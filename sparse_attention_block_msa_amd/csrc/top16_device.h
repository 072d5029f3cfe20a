// Wave-level Top16 selection shared by the select/merge kernels and the
// fused scorer. Every routine here runs on one 64-lane wave.
//
// Rule ("flashinfer.msa_ops.msa_icp_topk_select_publish", description;
// "flashinfer.msa_ops.prepare_msa_icp_indexer", init_blocks / local_blocks):
// a row keeps its forced begin/end blocks ([0, init) and [n - local, n)
// within the valid ids [0, n)) and the best 16 - |forced| of its other valid
// blocks, ranked by score descending and then lower id, and lists them by
// ascending id; unused slots hold (-inf, -1).
//
//  * Ranking key: the fp32 score mapped to an order-preserving uint32 (with -0
//    mapped to +0, so -0 and +0 tie); non-candidates get key 0, below every
//    real score. The K-th largest key is found by a 32-step bitwise descent in
//    which each step counts keys >= a trial value with one ballot + popcount
//    per register (no cross-lane reduction needed). Ties at that key are
//    broken by element order using the same ballots and mbcnt.
//  * Kept elements are compacted to their ascending-id slot with mbcnt.
#pragma once

#include <math.h>

#include "msa_internal.h"

namespace msa {
namespace topk {

__device__ __forceinline__ uint32_t order_key(float s)
{
    uint32_t b = __float_as_uint(s);
    if (b == 0x80000000u)
        b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int is_forced(int id, int n, int init_blocks, int local_blocks)
{
    return id >= 0 && id < n && (id < init_blocks || id >= n - local_blocks);
}

// Value of lane (this lane ^ j), j a power of two below 64, on the VALU
// alone (no LDS round trip): DPP quad permutes for 1 and 2; DPP row rotates
// within 16-lane rows for 4 (rotate by 12 reads lane +4, by 4 reads lane -4;
// the lane's bit 2 picks) and 8 (rotate by 8); the permlane16 and permlane32
// swaps for 16 and 32. (Lane layouts checked on the device. The LDS swizzle
// these replace for 4, 8 and 16 waited an LDS round trip per exchange.)
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int lane)
{
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    } else if constexpr (J == 4) {
        const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0xF, true);
        const uint32_t down = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, true);
        return (lane & 4) ? down : up;
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
    } else if constexpr (J == 16) {
        const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? sw[0] : sw[1];
    } else {
        static_assert(J == 32, "lane_xor: J must be a power of two below 64");
        const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return lane < 32 ? sw[1] : sw[0];
    }
}

template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t x, int lane)
{
    const uint32_t o = lane_xor<J>(x, lane);
    const bool keep_min = ((lane & J) == 0) == ((lane & K) == 0);
    return keep_min ? min(x, o) : max(x, o);
}

__device__ __forceinline__ uint32_t lane_xor_any(uint32_t v, int j, int lane)
{
    switch (j) {  // j is a compile-time constant wherever this is unrolled
    case 1:
        return lane_xor<1>(v, lane);
    case 2:
        return lane_xor<2>(v, lane);
    case 4:
        return lane_xor<4>(v, lane);
    case 8:
        return lane_xor<8>(v, lane);
    case 16:
        return lane_xor<16>(v, lane);
    default:
        return lane_xor<32>(v, lane);
    }
}

// K-th largest of the wave's 64V keys (element i of lane l is 64i + l),
// 1 <= K <= 64V, in every lane: a bitonic network sorts them ascending,
// partners 64 or more apart within a lane, nearer ones across lanes.
template <int V>
__device__ __forceinline__ uint32_t kth_largest_of_wave(const uint32_t (&u)[V], int K, int lane)
{
    constexpr int kN = 64 * V;
    uint32_t x[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        x[i] = u[i];
#pragma unroll
    for (int k = 2; k <= kN; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 64) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const int i2 = i ^ (j >> 6);
                    if (i2 > i) {
                        const bool up = ((i * 64) & k) == 0;
                        const uint32_t lo = min(x[i], x[i2]), hi = max(x[i], x[i2]);
                        x[i] = up ? lo : hi;
                        x[i2] = up ? hi : lo;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const uint32_t o = lane_xor_any(x[i], j, lane);
                    const int e = i * 64 + lane;
                    const bool keep_min = ((e & j) == 0) == ((e & k) == 0);
                    x[i] = keep_min ? min(x[i], o) : max(x[i], o);
                }
            }
        }
    }
    const int e = kN - K;
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < V; ++i)
        if (e / 64 == i)
            r = (uint32_t)__builtin_amdgcn_readlane((int)x[i], e % 64);
    return r;
}

// Sorts one value per lane ascending across the wave (a 64-element bitonic
// network of 21 exchange steps) and returns the K-th largest (lane 64 - K),
// 1 <= K <= 64, in every lane.
__device__ __forceinline__ uint32_t kth_largest_of_lanes(uint32_t x, int K, int lane)
{
    x = bitonic_step<2, 1>(x, lane);
    x = bitonic_step<4, 2>(x, lane);
    x = bitonic_step<4, 1>(x, lane);
    x = bitonic_step<8, 4>(x, lane);
    x = bitonic_step<8, 2>(x, lane);
    x = bitonic_step<8, 1>(x, lane);
    x = bitonic_step<16, 8>(x, lane);
    x = bitonic_step<16, 4>(x, lane);
    x = bitonic_step<16, 2>(x, lane);
    x = bitonic_step<16, 1>(x, lane);
    x = bitonic_step<32, 16>(x, lane);
    x = bitonic_step<32, 8>(x, lane);
    x = bitonic_step<32, 4>(x, lane);
    x = bitonic_step<32, 2>(x, lane);
    x = bitonic_step<32, 1>(x, lane);
    x = bitonic_step<64, 32>(x, lane);
    x = bitonic_step<64, 16>(x, lane);
    x = bitonic_step<64, 8>(x, lane);
    x = bitonic_step<64, 4>(x, lane);
    x = bitonic_step<64, 2>(x, lane);
    x = bitonic_step<64, 1>(x, lane);
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 64 - K);
}

// Number of candidate keys (u != 0) in the wave.
template <int V>
__device__ __forceinline__ int count_keys(const uint32_t (&u)[V])
{
    int n = 0;
#pragma unroll
    for (int i = 0; i < V; ++i)
        n += __popcll(__ballot(u[i] != 0u));
    return n;
}

// Wave-level select. Element i of this lane has key u[i] (0 = not a
// candidate) and is forced if bit i of fbits is set; n_cand is the number of
// candidates (count_keys). Keeps all forced elements and the best
// min(budget, n_cand) candidates, and calls emit(i, slot) for each kept
// element, slots ascending in element order. Returns the number of kept
// elements (uniform). Only slots below kTop are emitted: more than kTop kept
// elements (forced entries repeated in malformed merge input) return a count
// above kTop, which callers report, and never write past a row.
template <int V, class Emit>
__device__ __forceinline__ int wave_select(const uint32_t (&u)[V], uint64_t fbits, int budget,
                                           int n_cand, Emit&& emit)
{
    const int K = min(budget, n_cand);

    uint32_t thr = 0xFFFFFFFFu;
    int need = 0;
    if (K > 0) {
        if constexpr (V == 1) {
            thr = kth_largest_of_lanes(u[0], K, __lane_id());  // the K-th largest key
        } else if constexpr (V == 2) {
            thr = kth_largest_of_wave<2>(u, K, __lane_id());
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
            thr = prefix;  // the K-th largest key
        }
        int gt = 0;
#pragma unroll
        for (int i = 0; i < V; ++i)
            gt += __popcll(__ballot(u[i] > thr));
        need = K - gt;  // how many keys equal to thr are kept (lowest ids first)
    }

    int base = 0, tie_base = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const bool tie = K > 0 && u[i] == thr;
        const uint64_t tie_mask = __ballot(tie);
        const bool take = ((fbits >> i) & 1ull) ||
                          (K > 0 && (u[i] > thr || (tie && tie_base + lanes_below(tie_mask) < need)));
        const uint64_t take_mask = __ballot(take);
        const int slot = base + lanes_below(take_mask);
        if (take && slot < kTop)
            emit(i, slot);
        base += __popcll(take_mask);
        tie_base += __popcll(tie_mask);
    }
    return base;
}

// One entry (key, raw score, id); the duplicate-aware merge's buffer.
struct Candidate {
    uint32_t key;
    float score;
    int id;
};

// Compaction buffer of one wave (wave_select_filtered / select_row /
// select_loaded): 64 compacted entries, then one spill entry per lane, which
// the compaction's unselected lanes write to (so that its stores need no
// branch). Forced entries carry key 0, the others keys >= 1, so ids keep all
// 31 bits. Stored as two arrays of 8-byte words, so that a wave's stores
// and reads of one word per lane touch consecutive banks:
//  * pair[s] = key << 32 | order, order = ~s: the pairs order entries by key,
//    then by lower slot, and are unique within a buffer;
//  * payload[s] = id << 32 | score bits.
constexpr int kCandSlots = 128;
struct CandBuf {
    uint64_t pair[kCandSlots];
    uint64_t payload[kCandSlots];
};

// Two ds_write2_b32, whose data operands are any registers: with 8-byte
// stores (or one 16-byte store) the compiler forms register pairs (tuples)
// for every element of a fully unrolled compaction, which pushed the
// 32-values-per-lane select past its register budget. A wave's LDS
// operations complete in order, so these untracked stores need no wait
// before its own later reads.
__device__ __forceinline__ void cand_store(CandBuf* b, int slot, uint32_t key, float score,
                                           int id)
{
    typedef __attribute__((address_space(3))) uint64_t lds_u64;
    const uint32_t a = (uint32_t)(uintptr_t)(lds_u64*)&b->pair[slot];
    const uint32_t c = (uint32_t)(uintptr_t)(lds_u64*)&b->payload[slot];
    asm volatile("ds_write2_b32 %0, %2, %3 offset1:1\n\t"
                 "ds_write2_b32 %1, %4, %5 offset1:1"
                 :
                 : "v"(a), "v"(c), "v"(~(uint32_t)slot), "v"(key), "v"(score), "v"(id)
                 : "memory");
}

__device__ __forceinline__ Candidate cand_load(const CandBuf* b, int slot)
{
    const uint64_t w = b->payload[slot];
    return {(uint32_t)(b->pair[slot] >> 32), __uint_as_float((uint32_t)w), (int)(w >> 32)};
}

// Compacts the selected elements (keys >= theta, and with kForced also the
// elements whose bit of fbits is set) in element order into buf[0 .. 64);
// returns how many were selected (uniform). Only the first 64 are stored;
// callers take another path when more are selected. Keys are stored as they
// are: forced elements carry key 0. Every element is stored, an unselected
// one (or one past 64) to its lane's spill entry 64 + lane, so the loop has
// no branch; each register costs one ballot, its count on the scalar unit
// and one LDS store.
template <bool kForced, int V, class IdOf>
__device__ __forceinline__ int compact_selected(const uint32_t (&u)[V], const float (&sv)[V],
                                                uint64_t fbits, uint32_t theta, int lane,
                                                CandBuf* buf, IdOf&& id_of)
{
    const int spill = 64 + lane;
    int base = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bool sel = u[i] >= theta;
        if constexpr (kForced)
            sel = sel || ((fbits >> i) & 1ull);
        const uint64_t mask = __ballot(sel);
        const int at = base + lanes_below(mask);  // every lane: no exec-masked region
        const int slot = min(sel ? at : spill, spill);
        cand_store(buf, slot, u[i], sv[i], id_of(i));
        base += __popcll(mask);
    }
    return base;
}

// Ranks the n <= 64 entries buf[0, n) that compact_selected stored (element
// order; forced entries carry key 0, the others keys >= 1) and keeps the
// forced ones and the K best others by key descending, then lower slot (=
// lower element): each lane counts the entries whose (key, order) pair
// exceeds its own, reading every pair from LDS at one address for all lanes
// (a broadcast), two per instruction. The pairs are unique, so the ranks
// are; no tie pass is needed. Kept entries are emitted in slot order with
// emit(score, id, slot) for slots below kTop. With q > 0, *qkey receives the
// key of the non-forced entry of rank q - 1 (0 if there are fewer than q).
// Returns the number kept (uniform).
template <class Emit>
__device__ __forceinline__ int rank_select(CandBuf* buf, int n, int K, int lane, int q,
                                           uint32_t* qkey, Emit&& emit)
{
    if (n < 64 && lane == 0)  // a zero pair past the last entry: pairs are read two at a time
        buf->pair[n] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool have = lane < n;
    uint64_t me = 0ull, payload = 0ull;
    if (have) {
        me = buf->pair[lane];
        payload = buf->payload[lane];
    }
    int rank = 0;
    for (int j = 0; j < n; j += 2)
        rank += (int)(buf->pair[j] > me) + (int)(buf->pair[j + 1] > me);
    const uint32_t key = (uint32_t)(me >> 32);
    const bool forced = have && key == 0u;
    const bool keep = forced || (have && rank < K);
    const uint64_t kept = __ballot(keep);
    const int slot = lanes_below(kept);
    if (keep && slot < kTop)
        emit(__uint_as_float((uint32_t)payload), (int)(payload >> 32), slot);
    if (q > 0) {
        const uint64_t at = __ballot(have && !forced && rank == q - 1);
        *qkey = at ? (uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(at)) : 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return __popcll(kept);
}

// Wave-level select, same contract as wave_select, for V > 1 values per lane.
// Elements are (u[i], sv[i], id_of(i)); forced elements carry key 0. Every
// key of the best K is >= theta, the K-th largest of the 64 per-lane maxima
// (at least K keys are >= it), so when the keys >= theta plus the forced
// elements number at most 64 they are compacted in element order into `buf`
// (kCandSlots entries; one per lane) and ranked there with one value per
// lane (rank_select, whose q / qkey this passes on); otherwise the full
// V-value search runs (and *qkey, if asked for, is 0).
template <int V, class IdOf, class Emit>
__device__ __forceinline__ int wave_select_filtered(const uint32_t (&u)[V], const float (&sv)[V],
                                                    uint64_t fbits, int budget, int n_cand,
                                                    int lane, CandBuf* buf, IdOf&& id_of,
                                                    Emit&& emit, int q = 0,
                                                    uint32_t* qkey = nullptr)
{
    uint32_t lane_max = 0;
#pragma unroll
    for (int i = 0; i < V; ++i)
        lane_max = max(lane_max, u[i]);
    const int K = min(budget, n_cand);
    uint32_t theta = 1u;
    if (K > 0)
        theta = max(kth_largest_of_lanes(lane_max, K, lane), 1u);
    // with no candidate to keep, theta admits no key (a key of ~0u, a NaN
    // score, may pass it but is then never kept: the budget is 0)
    if (K == 0)
        theta = ~0u;
    const int base = __ballot(fbits != 0ull) != 0ull
                         ? compact_selected<true>(u, sv, fbits, theta, lane, buf, id_of)
                         : compact_selected<false>(u, sv, fbits, theta, lane, buf, id_of);
    if (base > 64) {  // heavy ties at theta: rank all V values per lane instead
        if (q > 0)
            *qkey = 0u;
        return wave_select<V>(u, fbits, budget, n_cand,
                              [&](int i, int slot) { emit(sv[i], id_of(i), slot); });
    }
    return rank_select(buf, base, K, lane, q, qkey, emit);
}

#ifndef MSA_SELECT_DIRECT_MAX_V
#define MSA_SELECT_DIRECT_MAX_V 2
#endif

// Picks the search for V values per lane: direct for small V, filtered above.
// n_cand is the number of candidate keys (u != 0).
// With q > 0, *qkey receives the key of the candidate of rank q - 1 when the
// filtered search finds it (0 otherwise, and always on the direct path).
template <int V, class IdOf, class Emit>
__device__ __forceinline__ int select_row(const uint32_t (&u)[V], const float (&sv)[V],
                                          uint64_t fbits, int budget, int n_cand, int lane,
                                          CandBuf* buf, IdOf&& id_of, Emit&& emit, int q = 0,
                                          uint32_t* qkey = nullptr)
{
    if (V <= MSA_SELECT_DIRECT_MAX_V) {
        if (q > 0)
            *qkey = 0u;
        return wave_select<V>(u, fbits, budget, n_cand,
                              [&](int i, int slot) { emit(sv[i], id_of(i), slot); });
    }
    return wave_select_filtered<V>(u, sv, fbits, budget, n_cand, lane, buf, id_of, emit, q, qkey);
}

__device__ __forceinline__ void pad_row(msa_top16_row* row, int kept, int lane)
{
    if (lane >= kept && lane < kTop) {
        row->score[lane] = -INFINITY;
        row->id[lane] = -1;
    }
}

// Second level of a split row: the NW partial rows in LDS are merged by wave
// 0 into `out`. Forced ids are recomputed from (n, init, local). The
// candidate budget is `budget`, or 16 - (forced entries found) if budget < 0.
// Returns the number of forced entries found (uniform in wave 0); *kept_out
// receives the number of entries kept (above kTop only for repeated forced
// ids in malformed input; then only the first kTop are written).
template <int NW>
__device__ __forceinline__ int merge_lds_rows(const msa_top16_row* part, int n, int init_blocks,
                                              int local_blocks, int budget, msa_top16_row* out,
                                              int lane, int* kept_out = nullptr)
{
    static_assert(NW * kTop <= 64, "partial rows must fit one wave");
    uint32_t u[1] = {0u};
    uint64_t fbits = 0;
    float s = -INFINITY;
    int id = -1;
    if (lane < NW * kTop) {
        s = part[lane / kTop].score[lane % kTop];
        id = part[lane / kTop].id[lane % kTop];
    }
    const bool forced = is_forced(id, n, init_blocks, local_blocks);
    if (forced)
        fbits = 1;
    else if (id >= 0)
        u[0] = order_key(s);
    const int n_forced = __popcll(__ballot(forced));
    if (budget < 0)
        budget = kTop - n_forced;
    const int kept = wave_select<1>(u, fbits, budget, count_keys<1>(u), [&](int, int slot) {
        out->score[slot] = s;
        out->id[slot] = id;
    });
    pad_row(out, kept, lane);
    if (kept_out)
        *kept_out = kept;
    return n_forced;
}

// |[0, min(init, n)) U [max(0, n - local), n)|
__device__ __forceinline__ int forced_count(int n, int init_blocks, int local_blocks)
{
    if (n <= 0)
        return 0;
    const int a = min(init_blocks, n);
    const int s = max(0, n - local_blocks);
    return a + (n - s) - max(0, a - s);
}

// Loads the span [span_lo, span_lo + 64V) of a row of `cols` scores at srow
// into sv (element i of lane l is span_lo + 64i + l). All V loads are issued
// unconditionally (index clamped into the row) so that they overlap; callers
// issue them before anything else that waits on memory, and invalid elements
// are masked by select_loaded. With kDeviceScope the loads are agent-scope
// atomic loads, which read values other waves stored at agent scope without a
// cache invalidation.
template <int V, bool kDeviceScope = false>
__device__ __forceinline__ void load_span(const float* srow, int cols, int span_lo, int lane,
                                          float (&sv)[V])
{
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const float* src = srow + min(span_lo + i * 64 + lane, cols - 1);
        if (kDeviceScope)
            sv[i] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            sv[i] = *src;
    }
}

// Column c of a select row stands for global block id scale * c + offset
// (scale 1, offset 0 when the plane's columns are the global blocks). With n
// valid global ids, the valid, init-forced and local-forced ids are then the
// columns [0, valid_end), [0, init_end) and [local_begin, valid_end).
struct ColumnIds {
    int scale;
    int offset;
    int valid_end;
    int init_end;
    int local_begin;
};

// Smallest column whose id is >= id (0 if every column's is).
__device__ __forceinline__ int first_column_at_least(int id, int scale, int offset)
{
    return id <= offset ? 0 : (id - offset + scale - 1) / scale;
}

__device__ __forceinline__ ColumnIds column_ids(int n, int init_blocks, int local_blocks,
                                                int scale, int offset)
{
    ColumnIds ci;
    ci.scale = scale;
    ci.offset = offset;
    ci.valid_end = first_column_at_least(n, scale, offset);
    ci.init_end = first_column_at_least(min(init_blocks, n), scale, offset);
    ci.local_begin = first_column_at_least(max(0, n - local_blocks), scale, offset);
    return ci;
}

// Bits i (0 <= i < V) of the elements of this lane that fall in columns
// [a, b): element i of the lane is column col0 + 64 i (col0 = span_lo + lane),
// so they are the i in [ceil((a - col0) / 64), ceil((b - col0) / 64)).
template <int V>
__device__ __forceinline__ uint64_t column_interval_bits(int a, int b, int col0)
{
    const int lo = max(0, (a - col0 + 63) >> 6);
    const int hi = min(V, max(0, (b - col0 + 63) >> 6));
    return hi > lo ? (1ull << hi) - (1ull << lo) : 0ull;
}

// Selects over a span loaded by load_span, within the column range ending at
// hi. The candidate budget is 16 minus the forced ids found in the span.
// Writes the kept entries (global ids) and the padding to dst and returns the
// number kept. q / qkey: as select_row.
template <int V>
__device__ __forceinline__ int select_loaded(const float (&sv)[V], int span_lo, int hi,
                                             const ColumnIds& ci, msa_top16_row* dst, int lane,
                                             CandBuf* buf, int q = 0, uint32_t* qkey = nullptr)
{
    // Valid columns of the span: [span_lo, valid_hi). Forced columns are
    // [0, init_end) and [local_begin, valid_end), so the candidates (valid,
    // not forced) are the one interval [cand_lo, cand_hi). Counts and masks
    // are interval arithmetic: no per-element test but one compare.
    const int valid_hi = min(min(hi, ci.valid_end), span_lo + V * 64);
    const int n_valid = max(0, valid_hi - span_lo);
    const int n_init = max(0, min(valid_hi, ci.init_end) - span_lo);
    const int n_local = max(0, valid_hi - max(span_lo, ci.local_begin));
    const int n_both = max(0, min(valid_hi, ci.init_end) - max(span_lo, ci.local_begin));
    const int n_forced = n_init + n_local - n_both;
    const int cand_lo = max(span_lo, ci.init_end);
    const uint32_t cand_len = (uint32_t)max(0, min(valid_hi, ci.local_begin) - cand_lo);
    const int rel = span_lo + lane - cand_lo;  // element i: column - cand_lo = rel + 64 i
    uint32_t u[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        u[i] = (uint32_t)(rel + 64 * i) < cand_len ? order_key(sv[i]) : 0u;
    uint64_t fbits = 0;
    if (n_forced > 0)  // only near a row's ends
        fbits = column_interval_bits<V>(span_lo, min(valid_hi, ci.init_end), span_lo + lane) |
                column_interval_bits<V>(max(span_lo, ci.local_begin), valid_hi, span_lo + lane);
    const int kept = select_row<V>(u, sv, fbits, kTop - n_forced, n_valid - n_forced, lane, buf,
                                   [&](int i) { return ci.scale * (span_lo + i * 64 + lane) + ci.offset; },
                                   [&](float score, int id, int slot) {
                                       dst->score[slot] = score;
                                       dst->id[slot] = id;
                                   },
                                   q, qkey);
    pad_row(dst, kept, lane);
    return kept;
}

}  // namespace topk
}  // namespace msa
