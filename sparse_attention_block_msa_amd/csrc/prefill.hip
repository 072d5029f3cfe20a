// Prefill chain kernels for gfx950: the window plan and the chunk scorer.
//
// Operation ("flashinfer.msa_ops.prepare_msa_icp_indexer", the prefill chain
// prefill_window_plan -> prefill_local -> exchange -> prefill_merge, with the
// plane element of "flashinfer.msa_ops.msa_icp_decode_index_score_sharded"):
// request b scores a chunk of q_len_b query tokens, rows [qo_indptr[b],
// qo_indptr[b + 1]) of index_q, token j at position seq_len_b - q_len_b + j.
// For each token t, head h and column c < W_b = min(roundup4(ceil(seq_len_b /
// 128)), cols):
//   plane[t, h, c] = max over keys p of B128 block c with p <= pos_t of
//                    q[t, h, :] . k[p, :]   (-inf if the block has none).
// Top16 select and merge of the plane's rows are the decode kernels.
//
// Design:
//  * Window plan (one workgroup). Each request's chunk is cut into windows
//    of 64 consecutive query tokens. A window needs the columns up to the
//    block of its last token, [0, needed), cut into work items of at most
//    kItemCols columns; the last item of a window also writes -inf to the
//    columns [needed, W_b) that no token of the window can see. Items are
//    listed by (request, window, column range) in a caller-owned plan:
//    a header (item count, and the batch, token count and plane width the
//    plan was made for) followed by 8-word items.
//  * Chunk scorer, one 2-wave workgroup per item. The window's 256 query rows
//    (64 tokens x 4 heads, contiguous in index_q) are split 128 per wave and
//    converted once to bf16 MFMA B operands held in registers. For every
//    column of the item the two waves stage the block's 16 KiB of keys in
//    LDS (global_load_lds, 64 rows per wave, XOR-swizzled as in the decode
//    scorer; the next column's DMA is in flight while a column is
//    contracted), then each wave contracts them with its 128 rows (8 key
//    tiles x 8 query tiles x 4 chained v_mfma_f32_16x16x32_bf16), masks keys
//    past a token's position in the blocks that reach past the wave's first
//    token and takes the block max. The maxima wait in LDS and go out as
//    32-byte runs per row every 8 columns. A key meets up to 256 query rows
//    here, 2*128*256 flops per 128-byte key: the kernel is MFMA-bound, and
//    several workgroups per CU hide each other's DMA waits.
//    Keys are loaded with the default cache policy, since every window of a
//    request re-reads the same blocks.
//  * Workgroups take items in an XCD-aware order (workgroup i runs on XCD
//    i % 8): each XCD takes one contiguous share of the item list, so the
//    windows that share a request's key blocks meet in one L2.
#include <math.h>

#include "msa_internal.h"
#include "score_tile.h"

namespace msa {
namespace {

using namespace keytile;

#ifndef MSA_PREFILL_WAVES_PER_EU
#define MSA_PREFILL_WAVES_PER_EU 2  // register cap: 128 query rows of operands per wave
#endif

constexpr int kWindow = MSA_PREFILL_WINDOW_TOKENS;
constexpr int kItemWords = MSA_PREFILL_ITEM_WORDS;
constexpr int kHeaderWords = MSA_PREFILL_PLAN_HEADER_WORDS;
constexpr int kItemCols = kPrefillItemCols;
constexpr int kPlanThreads = 256;
constexpr int kXcds = 8;
static_assert(kItemCols % 4 == 0 && kItemCols <= 64, "an item's pages are held one per lane");
static_assert(kWindow == 64, "the scorer holds 16 tokens x 4 heads per wave");

// Exclusive prefix sum of one int per thread over the workgroup (tmp holds
// kPlanThreads ints); *total receives the sum of all.
__device__ int block_exclusive_scan(int v, int* tmp, int* total)
{
    const int tid = threadIdx.x;
    tmp[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int x = tid >= off ? tmp[tid - off] : 0;
        __syncthreads();
        tmp[tid] += x;
        __syncthreads();
    }
    *total = tmp[kPlanThreads - 1];
    const int excl = tmp[tid] - v;
    __syncthreads();
    return excl;
}

// Written plane columns of a request: roundup4(ceil(seq / 128)), at most cols.
__device__ __forceinline__ int prefill_written_cols(int seq, int cols)
{
    if (seq <= 0)
        return 0;
    const int64_t w = (((int64_t)seq + kBlockTokens - 1) / kBlockTokens + 3) / 4 * 4;
    return w > cols ? cols : (int)w;
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillPlanParams p)
{
    __shared__ int win_base[kMaxPrefillBatch + 1];  // windows before request b
    __shared__ int tmp[kPlanThreads];
    __shared__ int bad;
    const int tid = threadIdx.x;
    if (tid == 0)
        bad = 0;
    __syncthreads();

    // windows per request and their prefix sum
    int windows = 0;
    for (int b0 = 0; b0 < p.batch; b0 += kPlanThreads) {
        const int b = b0 + tid;
        int nw = 0;
        if (b < p.batch) {
            const int lo = p.qo_indptr[b], hi = p.qo_indptr[b + 1], seq = p.seq_lens[b];
            if (lo < 0 || hi < lo || hi > p.num_tokens) {
                atomicAdd(&bad, 1);  // a malformed chunk is skipped
            } else if (seq > 0 && hi > lo) {
                nw = (hi - lo + kWindow - 1) / kWindow;
                const int64_t w = (((int64_t)seq + kBlockTokens - 1) / kBlockTokens + 3) / 4 * 4;
                if (w > p.cols)
                    atomicAdd(&bad, 1);  // the plane cuts the request's columns short
            }
        }
        int total;
        const int excl = block_exclusive_scan(nw, tmp, &total);
        if (b < p.batch)
            win_base[b] = windows + excl;
        windows += total;
    }
    if (tid == 0)
        win_base[p.batch] = windows;
    __syncthreads();

    // items of every window, listed by (request, window, column range)
    int64_t items = 0;
    for (int w0 = 0; w0 < windows; w0 += kPlanThreads) {
        const int gw = w0 + tid;
        int cnt = 0, b = 0, token0 = 0, ntok = 0, pos0 = 0, needed = 0, wb = 0, seq = 0;
        if (gw < windows) {
            // the request holding window gw: the last b with win_base[b] <= gw
            int lo = 0, hi = p.batch;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (win_base[mid] <= gw)
                    lo = mid;
                else
                    hi = mid;
            }
            b = lo;
            const int q0 = p.qo_indptr[b];
            const int qlen = p.qo_indptr[b + 1] - q0;
            const int w = gw - win_base[b];
            seq = p.seq_lens[b];
            token0 = q0 + kWindow * w;
            ntok = min(kWindow, qlen - kWindow * w);
            pos0 = seq - qlen + kWindow * w;
            const int64_t pos_last = (int64_t)pos0 + ntok - 1;
            wb = prefill_written_cols(seq, p.cols);
            needed = pos_last < 0 ? 0 : (int)min((int64_t)wb, pos_last / kBlockTokens + 1);
            cnt = needed > 0 ? (needed + kItemCols - 1) / kItemCols : 1;
        }
        int total;
        const int excl = block_exclusive_scan(cnt, tmp, &total);
        for (int r = 0; r < cnt; ++r) {
            const int64_t idx = items + excl + r;
            if (idx >= p.capacity)
                break;
            int32_t* dst = p.plan + kHeaderWords + idx * kItemWords;
            const int col0 = r * kItemCols;
            dst[0] = b;
            dst[1] = token0;
            dst[2] = ntok;
            dst[3] = pos0;
            dst[4] = col0;
            dst[5] = needed > 0 ? min(kItemCols, needed - col0) : 0;
            dst[6] = r == cnt - 1 ? wb : 0;
            dst[7] = seq;
        }
        items += total;
    }
    if (tid == 0) {
        p.plan[0] = (int)min(items, p.capacity);
        p.plan[1] = p.batch;
        p.plan[2] = p.num_tokens;
        p.plan[3] = p.cols;
        const int over = items > p.capacity ? 1 : 0;  // items past the capacity are dropped
        if ((bad + over) != 0 && p.errors)
            atomicAdd(p.errors, bad + over);
    }
}

// Launch shape of the chunk scorer: kWaves waves of kWaveTiles 16-row query
// tiles each cover the window's 64 tokens x 4 heads. With 8 tiles (128 rows)
// per wave every converted key operand feeds 8 MFMAs, and two waves per
// SIMD hold the 128 query operand registers each.
#ifndef MSA_PREFILL_WAVE_TILES
#define MSA_PREFILL_WAVE_TILES 8
#endif
constexpr int kWaveTiles = MSA_PREFILL_WAVE_TILES;
constexpr int kWaveRows = 16 * kWaveTiles;
constexpr int kWaves = kWindow * kHeads / kWaveRows;
constexpr int kWaveKeyRows = kBlockTokens / kWaves;  // key rows each wave stages per block
static_assert(kWaves * kWaveRows == kWindow * kHeads && kWaveKeyRows % 8 == 0, "bad shape");
// Plane columns a lane holds before storing them (a 32-byte run per row).
constexpr int kStoreCols = 8;
static_assert(kItemCols % kStoreCols == 0 && kStoreCols % 4 == 0, "runs must stay aligned");
// a lane stores kWaveTiles / 4 rows: wave rows lane, lane + 64, ...
static_assert(kWaveTiles % 4 == 0, "whole 16-lane groups per row slot");
constexpr int kLaneRows = kWaveTiles / 4;

// One column of one item for one wave: the block in `tile` against the
// wave's kWaveRows query rows. On return mx[n] holds, in every lane, the
// block max of wave row 16n + lane % 16. kMask: key k of the block is
// visible to wave row 16n + r only if k <= lim0 + (16n + r) / 4 (the row's
// token offset from the wave's first token).
template <bool kMask>
__device__ __forceinline__ void prefill_block(const uint8_t* tile,
                                              const Bf16Slice (&qb)[kWaveTiles], int r16, int g,
                                              int lim0, float (&mx)[kWaveTiles])
{
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < kWaveTiles; ++n)
        mx[n] = -INFINITY;
    for (int kt = 0; kt < 8; ++kt) {
        const Bf16Slice kb = to_bf16(read_row_slice(tile, kt * 16 + r16, g));
        // step-major over the query tiles: consecutive MFMAs never depend on
        // each other, and a tile's result is read kWaveTiles MFMAs after its
        // last step was issued
        v4f a[kWaveTiles];
        // The wave issues its MFMA burst at raised priority, so that on its
        // SIMD the burst goes first and the other wave's conversions and
        // maxima fill the cycles the matrix core is busy. Measured (chains
        // back to back, outputs bit-identical): 460-463 -> 437-449 us on the
        // 8192-token window, 275 -> 256-270 us on four 2048-token chunks.
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int n = 0; n < kWaveTiles; ++n)
            a[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb.op[0], qb[n].op[0], zero, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < 4; ++s) {
#pragma unroll
            for (int n = 0; n < kWaveTiles; ++n)
                a[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb.op[s], qb[n].op[s], a[n], 0, 0,
                                                               0);
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int n = 0; n < kWaveTiles; ++n) {
            v4f x = a[n];
            if (kMask) {
                // lane: keys kt*16 + 4g .. +3 for query row 16n + r16
                const int lim = lim0 + 4 * n + (r16 >> 2) - (kt * 16 + 4 * g);
                x.x = 0 <= lim ? x.x : -INFINITY;
                x.y = 1 <= lim ? x.y : -INFINITY;
                x.z = 2 <= lim ? x.z : -INFINITY;
                x.w = 3 <= lim ? x.w : -INFINITY;
            }
            mx[n] = fmaxf(fmaxf(fmaxf(fmaxf(mx[n], x.x), x.y), x.z), x.w);
        }
    }
#pragma unroll
    for (int n = 0; n < kWaveTiles; ++n) {
        mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 16));
        mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 32));
    }
}

// s_waitcnt immediates (gfx9 encoding): at most n vector-memory operations
// of the wave outstanding (expcnt and lgkmcnt at their maxima), and every LDS
// access of the wave returned (vmcnt and expcnt at their maxima).
constexpr int wait_vmcnt(int n)
{
    return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}
constexpr int kWaitLgkmcnt0 = 0xC07F;
constexpr int kStageLoads = kWaveKeyRows / 8;  // DMA instructions per wave per block

// This wave's kWaveKeyRows rows of a block, from `src_rows` into LDS at
// `dst_rows` with the swizzle of stage_piece. Issued as inline assembly, so
// the compiler, which cannot tell the two tiles apart, adds no DMA waits of
// its own before LDS reads; the caller waits with explicit vmcnt counts.
// Default cache policy: the windows of a request re-read the same blocks.
__device__ __forceinline__ void stage_rows_async(const uint8_t* src_rows, uint8_t* dst_rows,
                                                 int lane)
{
#pragma unroll
    for (int t = 0; t < kStageLoads; ++t) {
        const int row = 8 * t + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr)(dst_rows + t * 1024);
        const uint8_t* src = src_rows + row * kDim + chunk * 16;
        asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
    }
}

__global__ __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(MSA_PREFILL_WAVES_PER_EU)))
void prefill_score_kernel(PrefillScoreParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kBlockTokens * kDim];
    // each lane's block maxima of kStoreCols columns for its rows, laid
    // out [column][row slot][thread] so that a lane's accesses never share a
    // bank with another lane's
    __shared__ float held[kStoreCols][kLaneRows][kWaves * 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int g = lane >> 4;

    // The plan must be the one made for this plane; otherwise nothing runs.
    const int count = p.plan[0];
    if (p.plan[2] != p.num_tokens || p.plan[3] != p.cols || count < 0 || count > p.capacity) {
        if (blockIdx.x == 0 && tid == 0 && p.errors)
            atomicAdd(p.errors, 1);
        return;
    }
    const int plan_batch = min(p.plan[1], p.bt_rows);  // requests the block table holds
    const int per_xcd = (count + kXcds - 1) / kXcds;
    const int i = blockIdx.x;
    const int slot = (i % kXcds) * per_xcd + i / kXcds;
    if (i / kXcds >= per_xcd || slot >= count)
        return;
    const int32_t* iw = p.plan + kHeaderWords + (int64_t)slot * kItemWords;
    const int b = iw[0], token0 = iw[1], ntok = iw[2], pos0 = iw[3];
    const int col0 = iw[4], ncols = iw[5], fill_end = iw[6];
    if (b < 0 || b >= plan_batch || token0 < 0 || ntok < 1 || ntok > kWindow ||
        (int64_t)token0 + ntok > p.num_tokens || col0 < 0 || ncols < 0 || ncols > kItemCols ||
        col0 + ncols > p.cols || fill_end > p.cols) {
        if (tid == 0 && p.errors)
            atomicAdd(p.errors, 1);
        return;
    }

    const int col_shift = p.page_size == 256 ? 1 : 0;
    constexpr int kWaveTokens = kWaveRows / kHeads;
    const int64_t row_base = (int64_t)token0 * kHeads + wave * kWaveRows;  // wave's first row
    const int wave_tokens = ntok - kWaveTokens * wave;                      // may be <= 0

    // the wave's query rows as bf16 B operands (rows of tokens past the
    // window's end are zero and never stored)
    Bf16Slice qb[kWaveTiles];
#pragma unroll
    for (int n = 0; n < kWaveTiles; ++n) {
        v8i raw = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        if (4 * n + (r16 >> 2) < wave_tokens)
            raw = load_row_slice(p.q + (row_base + 16 * n + r16) * kDim, g);
        qb[n] = to_bf16(raw);
    }

    // block-table entries of the item's pages, one per lane (every wave
    // holds the same copy)
    const int pg0 = col0 >> col_shift;
    const int npg = ncols > 0 ? ((col0 + ncols - 1) >> col_shift) - pg0 + 1 : 0;
    int entry = 0;
    bool bad = false;
    if (lane < npg) {
        const int64_t idx = (int64_t)pg0 + lane;
        if (idx >= p.bt_stride) {
            bad = true;
        } else {
            const int v = p.bt[(int64_t)b * p.bt_stride + idx];
            if (v < 0 || (int64_t)v >= p.num_pages)
                bad = true;
            else
                entry = v;
        }
    }
    const uint64_t bad_mask = __ballot(bad);
    if (bad_mask != 0 && tid == 0 && p.errors)
        atomicAdd(p.errors, (int)__popcll(bad_mask));

    // Lane l stores wave rows 16n + l % 16 for the tiles n with n % 4 == l / 16.
    float* out_rows = p.out + (row_base + lane) * p.cols;
    const int wave_pos0 = pos0 + kWaveTokens * wave;  // position of the wave's first token

    // Two tiles: column i + 1's DMA is in flight while column i is
    // contracted. A column with a bad entry stages page 0 (never read), so
    // every column issues the same DMA instructions.
    auto rows_of = [&](int c) -> const uint8_t* {
        const int pi = (c >> col_shift) - pg0;
        const int page = ((bad_mask >> pi) & 1ull) ? 0 : __builtin_amdgcn_readlane(entry, pi);
        return p.k + ((int64_t)page * p.page_size + (c & ((1 << col_shift) - 1)) * kBlockTokens +
                      wave * kWaveKeyRows) * kDim;
    };
    if (ncols > 0)
        stage_rows_async(rows_of(col0), tiles[0] + wave * kWaveKeyRows * kDim, lane);
    for (int i = 0; i < ncols; ++i) {
        const int c = col0 + i;
        const uint8_t* cur = tiles[i & 1];
        if (i + 1 < ncols) {
            stage_rows_async(rows_of(c + 1), tiles[(i + 1) & 1] + wave * kWaveKeyRows * kDim,
                             lane);
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(kStageLoads));  // column i of this wave landed
        } else {
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
        }
        __builtin_amdgcn_s_barrier();  // and every other wave's
        const int pi = (c >> col_shift) - pg0;
        if (wave_tokens > 0) {
            float mx[kWaveTiles];
            if ((bad_mask >> pi) & 1ull) {
#pragma unroll
                for (int n = 0; n < kWaveTiles; ++n)
                    mx[n] = -INFINITY;
            } else {
                const int key0 = c * kBlockTokens;
                if (key0 + (kBlockTokens - 1) > wave_pos0)
                    prefill_block<true>(cur, qb, r16, g, wave_pos0 - key0, mx);
                else
                    prefill_block<false>(cur, qb, r16, g, 0, mx);
            }
#pragma unroll
            for (int n = 0; n < kWaveTiles; n += 4) {
                const float v = g == 0 ? mx[n] : g == 1 ? mx[n + 1] : g == 2 ? mx[n + 2] : mx[n + 3];
                held[i % kStoreCols][n / 4][tid] = v;
            }
            // Every kStoreCols columns (and after the item's last), each
            // lane stores its rows' held run of columns: plane stores share
            // the vector-memory counter with the key DMA, so fewer, wider
            // stores stall the next column's wait less, and whole 16-byte
            // runs leave no partly written lines behind.
            if (i % kStoreCols == kStoreCols - 1 || i == ncols - 1) {
                const int i0 = i - i % kStoreCols;  // col0 + i0 is a multiple of kStoreCols
                const int nb = i - i0 + 1;
#pragma unroll
                for (int n = 0; n < kWaveTiles; n += 4) {
                    // wave row 16n + lane: token offset (16n + lane) / 4
                    if (4 * n + (lane >> 2) >= wave_tokens)
                        continue;
                    float* dst = out_rows + (int64_t)16 * n * p.cols + col0 + i0;
                    int j = 0;
                    for (; j + 4 <= nb; j += 4) {
                        const v4f v = {held[j][n / 4][tid], held[j + 1][n / 4][tid],
                                       held[j + 2][n / 4][tid], held[j + 3][n / 4][tid]};
                        *reinterpret_cast<v4f*>(dst + j) = v;
                    }
                    for (; j < nb; ++j)
                        dst[j] = held[j][n / 4][tid];
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);  // this wave's reads of `cur` returned
        __builtin_amdgcn_s_barrier();               // every wave's: `cur` may be refilled
    }

    // columns no token of the window can see
    const int f0 = col0 + ncols;
    if (fill_end > f0) {
        const int nf = fill_end - f0;
        const int total = ntok * kHeads * nf;  // <= 256 rows x 8192 columns
        float* base = p.out + (int64_t)token0 * kHeads * p.cols;
        for (int e = tid; e < total; e += kWaves * 64) {
            const int row = e / nf;
            base[(int64_t)row * p.cols + f0 + (e - row * nf)] = -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill_plan(const PrefillPlanParams& p, hipStream_t stream)
{
    void* args[] = {const_cast<PrefillPlanParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_plan_kernel), dim3(1),
                           dim3(kPlanThreads), args, 0, stream);
}

hipError_t launch_prefill_score(const PrefillScoreParams& p, int64_t capacity,
                                hipStream_t stream)
{
    // a whole number of workgroups per XCD covers every slot of the plan
    const int64_t grid = (capacity + kXcds - 1) / kXcds * kXcds;
    void* args[] = {const_cast<PrefillScoreParams*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_score_kernel),
                           dim3((unsigned)grid), dim3(kWaves * 64), args, 0, stream);
}

hipError_t warmup_prefill_kernels()
{
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_plan_kernel));
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&prefill_score_kernel));
    return e;
}

}  // namespace msa
