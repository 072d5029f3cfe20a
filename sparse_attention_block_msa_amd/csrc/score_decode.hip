// Score-plane kernels for gfx950.
//
// Operation ("flashinfer.msa_ops.msa_icp_decode_index_score_sharded",
// description and parameters): for each request b, decode token j and index
// head h, and each B128 block c of the request,
//   plane[(b*dql + j), h, c] = max over keys p of block c with p < seq_len and
//                              p <= seq_len - dql + j of  q[b*dql + j, h, :] . k[p, :]
// (-inf if the block has no such key). Columns are written up to the request's
// block count rounded up to a multiple of four and no further. On a cache
// whose pages are split by rows over ranks, a rank's column is a page of its
// row shard instead (ColumnGeometry below).
//
// Design (one wave = 64 lanes per workgroup):
//  * Work split: a fixed grid of waves (a whole number per SIMD) cuts all
//    requests' written columns, laid end to end, into equal contiguous ranges
//    of 4-column groups (score_wave_range). A wave converts the Q tile of the
//    request it is in (4*dql <= 32 rows of 128 fp8 bytes) to bf16 once and
//    keeps it in registers as the B operand of the MFMA. Small batches use
//    single columns as the unit instead (latency mode). Waves take their
//    ranges in an XCD-aware order (split_slot), so each of the device's XCDs
//    works on one contiguous eighth of the groups.
//  * A B128 block is 128 keys x 128 bytes = 16 KiB, contiguous inside one
//    page. It is staged through a per-wave 4 KiB LDS tile in four pieces of
//    32 keys with global_load_lds_dwordx4 (latency mode: one 16 KiB piece;
//    row-sharded columns of 64 or 128 rows: 64-row pieces):
//    each DMA instruction moves 1 KiB of whole 128-byte rows (a fully
//    contiguous, non-temporal read), and the per-lane source addresses are
//    chosen so the tile lands XOR-swizzled, letting the MFMA-layout
//    ds_read_b128s hit every LDS bank once. Loads never occupy VGPRs.
//    (Loading the MFMA layout straight into registers needs half-row 64-byte
//    accesses per instruction; measured on MI355X, that pattern streams at
//    about 5.2 TB/s against 6.5 TB/s for whole-row DMA.)
//  * Contraction: every e4m3fn value is exactly a bf16 value, so each key
//    tile is converted with v_cvt_scalef32_pk_bf16_fp8 (scale 1.0, two values
//    per instruction) and contracted with v_mfma_f32_16x16x32_bf16, four
//    instructions chained through the fp32 accumulator per 128-dim dot
//    product. The fp8 MFMA forms (16x16x128 f8f6f4, 16x16x32 fp8) were
//    measured on gfx950 (msa_contraction_probe) to sum groups of fp8
//    products with up to about 2e-5 of sum|q_i k_i| error on N(0,1) data and
//    2e-4 on full-range codes, above the 1e-5 bound this kernel guarantees;
//    the bf16 form measured at most 3e-7. The path is HBM-bound either way
//    (8*dql flop per index-K byte), so the bf16 rate costs no throughput.
//  * Lane l of a 16x16 result holds keys 4*(l/16)..+3 of the tile for query
//    row l%16, so the block max is a per-lane max over 8 tiles x 4 values
//    followed by a max across the four 16-lane groups. The causal mask is
//    applied only in blocks that reach past the first token's position.
//  * A window's (<= 16 columns) block maxima collect in a small per-wave LDS
//    array and are stored to the plane only when the window is done, so no
//    DMA wait ever waits on a plane store.
//  * score_select_kernel runs the same scoring and then the per-range Top16
//    select in the same launch (see its comment).
//
// Byte order inside a lane's operands: the 32 bytes a lane supplies per row
// are bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte row
// (g = lane/16); byte b of that slice becomes element b%8 of the operand of
// instruction b/8, for the key rows (A) and the query rows (B) alike. The dot
// product is a sum over all 128 dims, so any byte-to-k assignment that A and
// B share gives the same sum.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "msa_internal.h"
#include "score_tile.h"
#include "top16_device.h"

namespace msa {
namespace {

// Launch shape: one 64-lane wave per workgroup, a block staged in kParts
// pieces (LDS use: 4 KiB tile + 2 KiB results per wave), a grid of 3
// (<= 16 query rows) or 2 (32 rows) waves per SIMD, measured best on the
// five workloads.
#ifndef MSA_SCORE_LOAD_AUX
#define MSA_SCORE_LOAD_AUX 2  // cache-policy bits of the index-K DMA: nt (non-temporal)
#endif
#ifndef MSA_SCORE_PARTS
#define MSA_SCORE_PARTS 4
#endif

#ifndef MSA_SCORE_CHUNK
#define MSA_SCORE_CHUNK 16  // columns per window (LDS result buffer)
#endif
#ifndef MSA_SCORE_WAVES_PER_SIMD_16
#define MSA_SCORE_WAVES_PER_SIMD_16 3  // grid: waves per SIMD for up to 16 query rows
#endif
#ifndef MSA_SCORE_WAVES_PER_SIMD_32
#define MSA_SCORE_WAVES_PER_SIMD_32 2  // grid: waves per SIMD for 17..32 query rows
#endif
#ifndef MSA_SCORE_LATENCY_WAVES_PER_SIMD
#define MSA_SCORE_LATENCY_WAVES_PER_SIMD 2  // small batches: batch*cols <= CUs*4*this
#endif
#ifndef MSA_SCORE_REG_WAVES_16
#define MSA_SCORE_REG_WAVES_16 MSA_SCORE_WAVES_PER_SIMD_16  // register cap: waves per SIMD
#endif
#ifndef MSA_SCORE_REG_WAVES_32
#define MSA_SCORE_REG_WAVES_32 MSA_SCORE_WAVES_PER_SIMD_32
#endif

constexpr int kChunk = MSA_SCORE_CHUNK;
// a window's block-table entries are held one per lane
static_assert(kChunk % 4 == 0 && kChunk <= 64, "bad window width");

using namespace keytile;

// Scores one B128 block against the NT query tiles. The block is staged
// through the wave's LDS tile in kParts pieces of 8 / kParts key tiles (16
// keys each): DMA, wait, then convert and contract each tile. Other waves on
// the SIMD keep HBM busy meanwhile. On return mx[n] holds, in every lane,
// the block max of query row 16n + lane%16. kMask: keys whose in-block index
// exceeds lim[n] are excluded.
template <int NT, int kParts, bool kMask>
__device__ __forceinline__ void score_block(const uint8_t* block, uint8_t* tile,
                                            const Bf16Slice (&qb)[NT], int lane, int r16, int g,
                                            const int (&lim)[NT], float (&mx)[NT],
                                            int parts = kParts)
{
    constexpr int kTiles = 8 / kParts;
    constexpr int kPieceRows = kTiles * 16;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NT; ++n)
        mx[n] = -INFINITY;
#pragma unroll
    for (int part = 0; part < kParts; ++part) {
        if (part >= parts)  // a row-sharded column holds fewer keys
            break;
        stage_piece<kPieceRows, MSA_SCORE_LOAD_AUX>(block + part * kPieceRows * kDim, tile, lane);
        __builtin_amdgcn_s_waitcnt(0);  // the piece's DMA has landed in LDS
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            const int mt = part * kTiles + t;
            const Bf16Slice kt = to_bf16(read_row_slice(tile, t * 16 + r16, g));
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                v4f a = zero;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt.op[s], qb[n].op[s], a, 0, 0, 0);
                if (kMask) {
                    const int k0 = mt * 16 + g * 4;
                    a.x = (k0 + 0 <= lim[n]) ? a.x : -INFINITY;
                    a.y = (k0 + 1 <= lim[n]) ? a.y : -INFINITY;
                    a.z = (k0 + 2 <= lim[n]) ? a.z : -INFINITY;
                    a.w = (k0 + 3 <= lim[n]) ? a.w : -INFINITY;
                }
                mx[n] = fmaxf(mx[n], max4(a));
            }
        }
        __syncthreads();  // the tile's reads are done before the next DMA reuses it
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 16));
        mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 32));
    }
}

// Written plane columns of a request: roundup4(ceil(seq / col_stride))
// clamped to the plane width (*clamped says whether the width cut it short).
// col_stride is 128 (a column per B128 block), or page_size on a row-sharded
// cache (a column per page).
__device__ __forceinline__ int written_cols(int seq, int cols, bool& clamped,
                                            int col_stride = kBlockTokens)
{
    clamped = false;
    if (seq <= 0)
        return 0;
    const int64_t nblk = ((int64_t)seq + col_stride - 1) / col_stride;
    const int64_t w = (nblk + 3) / 4 * 4;
    clamped = w > cols;
    return clamped ? cols : (int)w;
}

// The wave's place in the work split. Workgroups are dispatched to the
// device's XCDs round-robin (workgroup i to XCD i % kXcds), and each XCD has
// its own L2 and its own share of the fabric to HBM. With a grid that is a
// whole number of waves per XCD, slot = (i % kXcds) * (grid / kXcds) + i /
// kXcds gives every XCD one contiguous eighth of the units, so the XCDs'
// loads differ by at most one unit however uneven the per-wave shares are.
#ifndef MSA_SCORE_XCD_SPLIT
#define MSA_SCORE_XCD_SPLIT 1
#endif
constexpr int kXcds = 8;

__device__ __forceinline__ int split_slot()
{
    const int i = blockIdx.x, grid = gridDim.x;
    if (!MSA_SCORE_XCD_SPLIT || grid % kXcds != 0)
        return i;
    return (i % kXcds) * (grid / kXcds) + i / kXcds;
}

// Wave-wide sum and inclusive prefix sum on the VALU alone (the lane
// exchanges of topk::lane_xor: DPP and permlane swaps, no LDS round trip).
// They sit on every wave's path to its first index-K load, where a shuffle
// through ds_bpermute cost an LDS round trip and a wait per step.
__device__ __forceinline__ int wave_sum(int v, int lane)
{
    v += (int)topk::lane_xor<1>((uint32_t)v, lane);
    v += (int)topk::lane_xor<2>((uint32_t)v, lane);
    v += (int)topk::lane_xor<4>((uint32_t)v, lane);
    v += (int)topk::lane_xor<8>((uint32_t)v, lane);
    v += (int)topk::lane_xor<16>((uint32_t)v, lane);
    v += (int)topk::lane_xor<32>((uint32_t)v, lane);
    return v;
}

// Butterfly prefix sum: before the step with partner distance j, `total` is
// the sum over the aligned block of j lanes holding this lane and `prefix`
// the sum over that block's lanes up to this one; the partner block (lanes
// ^ j) holds the other half of the aligned 2j-lane block, and it precedes
// this lane's half when bit j of the lane is set.
template <int J>
__device__ __forceinline__ void scan_step(int& prefix, int& total, int lane)
{
    const int o = (int)topk::lane_xor<J>((uint32_t)total, lane);
    if (lane & J)
        prefix += o;
    total += o;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane)
{
    int prefix = v, total = v;
    scan_step<1>(prefix, total, lane);
    scan_step<2>(prefix, total, lane);
    scan_step<4>(prefix, total, lane);
    scan_step<8>(prefix, total, lane);
    scan_step<16>(prefix, total, lane);
    scan_step<32>(prefix, total, lane);
    return prefix;
}

// Where a plane column's keys are.
//  * Full page rows ("flashinfer.msa_ops.msa_icp_decode_index_score_sharded",
//    with every page's rows on this device): column c is global B128 block
//    c, keys [128c, 128c + 128), rows [(c % cpp) * 128, +128) of page
//    c / cpp (cpp = page_size / 128 columns per page).
//  * Row-sharded cache (same page, index_k shard [pages, page_size /
//    world_size, 128] and the description's columns): the rank holds rows
//    [rank * R, rank * R + R) of every page, R = page_size / world_size;
//    column c is the request's page c, its keys are the positions
//    c * page_size + rank * R + i (i < R), rows [0, R) of the shard page.
struct ColumnGeometry {
    int col_shift;   // log2(columns per block-table entry)
    int col_stride;  // key positions per column step
    int pos_off;     // position of a column's first key minus c * col_stride
    int page_rows;   // key rows per stored page
    int col_rows;    // keys per column
    int parts;       // DMA pieces (128 / kParts keys each) per column
};

// kParts: pieces per B128 block of the instance; a column of col_rows keys
// takes col_rows / (128 / kParts) of them (the host picks an instance whose
// piece divides the column).
template <bool kSharded, int kParts>
__device__ __forceinline__ ColumnGeometry column_geometry(const ScoreParams& p)
{
    ColumnGeometry gm;
    if constexpr (kSharded) {
        const int r = p.page_size / p.world_size;
        gm.col_shift = 0;
        gm.col_stride = p.page_size;
        gm.pos_off = p.rank * r;
        gm.page_rows = r;
        gm.col_rows = r;
        gm.parts = r / (kBlockTokens / kParts);
    } else {
        gm.col_shift = p.page_size == 256 ? 1 : 0;
        gm.col_stride = kBlockTokens;
        gm.pos_off = 0;
        gm.page_rows = p.page_size;
        gm.col_rows = kBlockTokens;
        gm.parts = kParts;
    }
    return gm;
}

// Columns of a request with at least one key below seq (the rest of its
// written columns are padding, -inf).
__device__ __forceinline__ int key_columns(int seq, const ColumnGeometry& gm)
{
    if (seq <= gm.pos_off)
        return 0;
    return (int)(((int64_t)seq - gm.pos_off + gm.col_stride - 1) / gm.col_stride);
}

// Block-table entries of a window, one per lane.
struct WindowPages {
    int page;           // this lane's page (0 for an entry that is out of range)
    uint64_t bad_mask;  // lanes whose entry was out of range
};

// Issues the loads of the block-table entries of columns [c_begin, c_last]
// of request b (at most kChunk pages), one per lane.
__device__ __forceinline__ WindowPages load_window_pages(const ScoreParams& p, int b, int c_begin,
                                                         int c_last, int lane, int ps_shift)
{
    const int pg_begin = c_begin >> ps_shift;
    const int pg_count = (c_last >> ps_shift) - pg_begin + 1;
    WindowPages w;
    w.page = 0;
    bool bad = false;
    if (lane < pg_count) {
        const int64_t idx = (int64_t)pg_begin + lane;
        if (idx >= p.bt_stride) {
            bad = true;
        } else {
            const int v = p.bt[(int64_t)b * p.bt_stride + idx];
            if (v < 0 || (int64_t)v >= p.num_pages)
                bad = true;
            else
                w.page = v;
        }
    }
    w.bad_mask = __ballot(bad);
    return w;
}

// Scores one window: columns [c_begin, c_end) of request b (at most kChunk;
// multiples of kUnit = 4, or any columns for kUnit = 1), whose block-table
// entries are in wp. Columns at or past nblk are padding (-inf). The
// block maxima collect in res and are stored once, after the window's last
// block: on this ISA stores share the vector-memory counter with the DMA, so
// a store issued mid-window would make every later DMA wait also wait for it.
template <int NT, int kParts, bool kDeviceScope, int kUnit>
__device__ __forceinline__ void score_window(const ScoreParams& p, const ColumnGeometry& gm,
                                             int b, int seq, int nblk, int c_begin, int c_end,
                                             const WindowPages& wp, const Bf16Slice (&qb)[NT],
                                             const int (&pos)[NT], uint8_t* tile,
                                             float (*res)[kChunk], int lane, int r16, int g)
{
    const int rows = p.dql * kHeads;
    const int64_t row_base = (int64_t)b * rows;
    const int ps_shift = gm.col_shift;  // log2(columns per page)
    const int c_last = min(c_end, nblk) - 1;  // < c_begin if the window is all padding
    const int pg_begin = c_begin >> ps_shift;
    const int my_page = wp.page;
    const uint64_t bad_mask = wp.bad_mask;
    if (bad_mask != 0 && lane == 0 && p.errors)
        atomicAdd(p.errors, (int)__popcll(bad_mask));

    auto block_ptr = [&](int c) -> const uint8_t* {
        const int page = __builtin_amdgcn_readlane(my_page, (c >> ps_shift) - pg_begin);
        const int half = c & ((1 << ps_shift) - 1);
        return p.k + ((int64_t)page * gm.page_rows + half * kBlockTokens) * kDim;
    };

    const int first_masked = seq - p.dql;  // columns reaching past this key need the mask
    for (int c = c_begin; c < c_end; ++c) {
        float mx[NT];
        int lim[NT];
        const int key0 = c * gm.col_stride + gm.pos_off;  // position of the column's first key
#pragma unroll
        for (int n = 0; n < NT; ++n)
            lim[n] = pos[n] - key0;
        const bool has_keys =
            c <= c_last && !((bad_mask >> ((min(c, c_last) >> ps_shift) - pg_begin)) & 1ull);
        if (!has_keys) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                mx[n] = -INFINITY;
        } else if (key0 + (gm.col_rows - 1) > first_masked) {
            score_block<NT, kParts, true>(block_ptr(c), tile, qb, lane, r16, g, lim, mx,
                                          gm.parts);
        } else {
            score_block<NT, kParts, false>(block_ptr(c), tile, qb, lane, r16, g, lim, mx,
                                           gm.parts);
        }
        // lanes of group g == n keep query row 16n + lane%16
#pragma unroll
        for (int n = 0; n < NT; ++n)
            if (g == n)
                res[n * 16 + r16][c - c_begin] = mx[n];
    }

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    static_assert(kUnit == 4 || kUnit == 1, "unsupported store mode");
    if constexpr (kUnit == 1) {  // single-column stores: windows need not be 4-aligned
        const int ncol = c_end - c_begin;
        for (int i = lane; i < rows * ncol; i += 64) {
            const int rho = i / ncol;
            const int c = i - rho * ncol;
            float* dst = p.out + (row_base + rho) * p.cols + c_begin + c;
            if (kDeviceScope)  // written through to the device's coherence point
                __hip_atomic_store(dst, res[rho][c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                *dst = res[rho][c];
        }
    }
    if constexpr (kUnit == 4) {
        const int quads = (c_end - c_begin) / 4;  // float4 groups per row
        for (int i = lane; i < rows * quads; i += 64) {
            const int rho = i / quads;
            const int q4 = i - rho * quads;
            const v4f v = *reinterpret_cast<const v4f*>(&res[rho][q4 * 4]);
            float* dst = p.out + (row_base + rho) * p.cols + c_begin + q4 * 4;
            if (kDeviceScope) {
                // Written through to the device's coherence point: the sc1
                // policy, which an agent-scope atomic store of one dword
                // also carries, on one 16-byte store (the four dwords need
                // no atomicity together; readers wait for the producing
                // wave's counter release first). Its completion is awaited
                // with an explicit vmcnt(0) before that release.
                asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(dst), "v"(v)
                             : "memory");
            } else {
                *reinterpret_cast<v4f*>(dst) = v;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work split: the plane columns every request writes (a multiple of 4 each)
// are laid end to end and cut into gridDim.x equal, contiguous ranges of
// kUnit-column units (4, or 1 for small batches), one per wave; a range may
// run across request boundaries.
// Ragged batches therefore load every wave alike, and a wave pays its setup
// (sequence lengths, Q tile) once rather than per request chunk.
// segment_done(b, c_begin, c_end) runs after the wave has issued the plane
// stores of columns [c_begin, c_end) of request b, once per request it
// touches. With kDeviceScope the plane stores are agent-scope atomic stores.
template <int NT, int kParts, bool kDeviceScope, int kUnit, bool kSharded, class SegmentDone>
__device__ __forceinline__ void score_wave_range(const ScoreParams& p, uint8_t* tile,
                                                 float (*res)[kChunk], SegmentDone&& segment_done)
{
    const ColumnGeometry gm = column_geometry<kSharded, kParts>(p);
    const int slot = split_slot();
    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int rows = p.dql * kHeads;

    // Latency mode with one wave per (request, column) of the plane: the wave
    // knows its column without the prefix pass over seq_lens, so its
    // sequence length, Q tile and block-table entry load together.
    if constexpr (kUnit == 1 && !kSharded) {
        if ((int64_t)gridDim.x == (int64_t)p.batch * p.cols) {
            const int b = (int)(blockIdx.x / p.cols);
            const int c = (int)(blockIdx.x % p.cols);
            const int64_t row_base = (int64_t)b * rows;
            const int pidx = c >> gm.col_shift;
            int entry = -1;
            if (pidx < p.bt_stride)  // inside the table's row: safe to read early
                entry = p.bt[(int64_t)b * p.bt_stride + pidx];
            v8i qraw[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int rho = n * 16 + r16;
                qraw[n] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                if (rho < rows)
                    qraw[n] = load_row_slice(p.q + (row_base + rho) * kDim, g);
            }
            const int seq = p.seq_lens[b];
            bool clamped;
            const int wcols = written_cols(seq, p.cols, clamped, gm.col_stride);
            if (c >= wcols)
                return;
            if (clamped && c == 0 && lane == 0 && p.errors)
                atomicAdd(p.errors, 1);
            const int nblk = key_columns(seq, gm);
            // the entry counts only for a column with keys, as the window
            // loads would have read it
            const bool bad = c < nblk && (pidx >= p.bt_stride || entry < 0 ||
                                          (int64_t)entry >= p.num_pages);
            WindowPages wp;
            wp.page = bad ? 0 : entry;
            wp.bad_mask = __ballot(bad && lane == 0);
            Bf16Slice qb[NT];
            int pos[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                pos[n] = seq - p.dql + ((n * 16 + r16) >> 2);
                qb[n] = to_bf16(qraw[n]);
            }
            score_window<NT, kParts, kDeviceScope, kUnit>(p, gm, b, seq, nblk, c, c + 1, wp, qb,
                                                          pos, tile, res, lane, r16, g);
            segment_done(b, c, c + 1);
            return;
        }
    }

    // Groups of all requests, this wave's range [g_lo, g_hi), the request b
    // holding g_lo and the groups before it (base). One pass over seq_lens
    // when the batch fits one wave, two otherwise.
    int64_t g_lo, g_hi;
    int b = 0;
    int64_t base = 0;
    // batch <= 64: lane b holds seq_lens[b], and each request's length is
    // taken from it (seq_next; -1: load it)
    const int seq_lane = p.batch <= 64 && lane < p.batch ? p.seq_lens[lane] : 0;
    int seq_next = -1;
    if (p.batch <= 64) {
        bool clamped;
        const int gb = lane < p.batch ? written_cols(seq_lane, p.cols, clamped, gm.col_stride) / kUnit
                                      : 0;
        const int incl = wave_inclusive_scan(gb, lane);
        const int64_t total = __builtin_amdgcn_readlane(incl, 63);
        g_lo = total * (int64_t)slot / gridDim.x;
        g_hi = total * ((int64_t)slot + 1) / gridDim.x;
        if (g_lo >= g_hi)
            return;
        const int l = __ffsll((unsigned long long)__ballot(incl > g_lo)) - 1;
        b = l;
        base = __builtin_amdgcn_readlane(incl - gb, l);
        seq_next = __builtin_amdgcn_readlane(seq_lane, l);
    } else {
        int64_t total = 0;
        for (int b0 = 0; b0 < p.batch; b0 += 64) {
            bool clamped;
            const int bb = b0 + lane;
            const int gb = bb < p.batch
                               ? written_cols(p.seq_lens[bb], p.cols, clamped, gm.col_stride) / kUnit
                               : 0;
            total += wave_sum(gb, lane);
        }
        g_lo = total * (int64_t)slot / gridDim.x;
        g_hi = total * ((int64_t)slot + 1) / gridDim.x;
        if (g_lo >= g_hi)
            return;
        for (int b0 = 0; b0 < p.batch; b0 += 64) {
            bool clamped;
            const int bb = b0 + lane;
            const int gb = bb < p.batch
                               ? written_cols(p.seq_lens[bb], p.cols, clamped, gm.col_stride) / kUnit
                               : 0;
            const int incl = wave_inclusive_scan(gb, lane);
            const int chunk_total = __builtin_amdgcn_readlane(incl, 63);
            if (base + chunk_total > g_lo) {
                const int l = __ffsll((unsigned long long)__ballot(base + incl > g_lo)) - 1;
                b = b0 + l;
                base += __builtin_amdgcn_readlane(incl - gb, l);
                break;
            }
            base += chunk_total;
        }
    }

    int64_t gcur = g_lo;
    while (gcur < g_hi) {
        const int seq = seq_next >= 0 ? seq_next : p.seq_lens[b];
        seq_next = -1;
        bool clamped;
        const int wcols = written_cols(seq, p.cols, clamped, gm.col_stride);
        if (wcols == 0) {  // requests with no columns own no groups
            ++b;
            if (p.batch <= 64 && b < p.batch)
                seq_next = __builtin_amdgcn_readlane(seq_lane, b);
            continue;
        }
        if (clamped && gcur == base && lane == 0 && p.errors)
            atomicAdd(p.errors, 1);
        const int nblk = key_columns(seq, gm);
        const int64_t row_base = (int64_t)b * rows;
        const int64_t g_end_b = base + wcols / kUnit;
        const int c_stop = (int)((min(g_hi, g_end_b) - base) * kUnit);
        const int c_first = (int)((gcur - base) * kUnit);
        int c = c_first;

        // Q tile loads and the first window's block-table loads go out
        // together; the tile is converted once both have landed.
        v8i qraw[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int rho = n * 16 + r16;
            qraw[n] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            if (rho < rows)
                qraw[n] = load_row_slice(p.q + (row_base + rho) * kDim, g);
        }
        int c_end = min(c + kChunk, c_stop);
        WindowPages wp = load_window_pages(p, b, c, min(c_end, nblk) - 1, lane, gm.col_shift);
        Bf16Slice qb[NT];
        int pos[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            pos[n] = seq - p.dql + ((n * 16 + r16) >> 2);
            qb[n] = to_bf16(qraw[n]);
        }
        while (true) {
            score_window<NT, kParts, kDeviceScope, kUnit>(p, gm, b, seq, nblk, c, c_end, wp, qb,
                                                          pos, tile, res, lane, r16, g);
            c = c_end;
            if (c >= c_stop)
                break;
            c_end = min(c + kChunk, c_stop);
            wp = load_window_pages(p, b, c, min(c_end, nblk) - 1, lane, gm.col_shift);
        }
        segment_done(b, c_first, c_stop);
        gcur = min(g_hi, g_end_b);
        base = g_end_b;
        ++b;
        if (p.batch <= 64 && b < p.batch)
            seq_next = __builtin_amdgcn_readlane(seq_lane, b);
    }
}

template <int NT, int kParts, int kWavesPerEU, int kUnit, bool kSharded>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void score_decode_kernel(ScoreParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[(8 / kParts) * 16 * kDim];
    __shared__ __attribute__((aligned(16))) float res[32][kChunk];  // block maxima of a window
    score_wave_range<NT, kParts, false, kUnit, kSharded>(p, tile, res, [](int, int, int) {});
}

// s_waitcnt immediate (gfx9 encoding) that waits for every outstanding
// vector-memory operation of the wave, stores included: vmcnt(0), with
// expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// Polls of a helper's wait in score_select_kernel before it gives up and
// counts an error. Every wait there ends by the launch's protocol (below);
// this bound only keeps a defect from hanging the device.
constexpr uint32_t kMaxPolls = 1u << 20;

// Counters of range rr (its own 128-byte line: adds to different ranges do not
// queue behind each other): columns stored, and select jobs done.
__device__ __forceinline__ int32_t* range_line(const ScoreSelectParams& q, int64_t rr)
{
    return q.workspace + rr * kFusedLineWords;
}

__device__ __forceinline__ int32_t* merge_tickets(const ScoreSelectParams& q)
{
    return q.workspace + (int64_t)q.score.batch * q.num_ranges * kFusedLineWords;
}

// Wave-uniform agent-scope atomics, issued by lane 0.
__device__ __forceinline__ int lane0_load(const int32_t* a)
{
    int v = 0;
    if (__lane_id() == 0)
        v = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int lane0_add(int32_t* a, int n)
{
    int v = 0;
    if (__lane_id() == 0)
        v = __hip_atomic_fetch_add(a, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(v);
}

// An add whose old value is not needed (the wave does not wait for it).
__device__ __forceinline__ void lane0_add_posted(int32_t* a, int n)
{
    if (__lane_id() == 0)
        __hip_atomic_fetch_add(a, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void lane0_store(int32_t* a, int v)
{
    if (__lane_id() == 0)
        __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Columns of range r that a request writing wb columns writes (the range
// counter's final value).
__device__ __forceinline__ int range_columns(const ScoreSelectParams& q, int wb, int r)
{
    const int lo = r * q.width;
    return max(0, min(min(lo + q.width, q.score.cols), wb) - lo);
}

// Merge of row th's R range rows (written through by other waves, read with
// agent-scope loads) into merged[th], exactly as msa_top16_merge does with
// n = max(0, num_valid_pages) (a forced id missing from the rows, possible
// only for num_valid_pages past the plane, is counted); VM values per lane
// cover R * 16 <= 64 * VM entries.
template <int VM>
__device__ __forceinline__ void fused_merge(const ScoreSelectParams& q, int64_t th, int n,
                                            int lane, topk::CandBuf* buf)
{
    using namespace topk;
    const int total = q.num_ranges * kTop;
    const int32_t* rows = reinterpret_cast<const int32_t*>(q.out + th * q.num_ranges);
    float mv[VM];
    int iv[VM];
#pragma unroll
    for (int i = 0; i < VM; ++i) {
        const int e = min(i * 64 + lane, total - 1);
        const int32_t* row = rows + (e / kTop) * 2 * kTop;
        mv[i] = __int_as_float(
            __hip_atomic_load(row + e % kTop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        iv[i] = __hip_atomic_load(row + kTop + e % kTop, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t um[VM];
    uint64_t fm = 0;
    int n_forced = 0;
#pragma unroll
    for (int i = 0; i < VM; ++i) {
        const bool valid = i * 64 + lane < total && iv[i] >= 0;
        const bool forced = valid && is_forced(iv[i], n, q.init_blocks, q.local_blocks);
        um[i] = valid && !forced ? order_key(mv[i]) : 0u;
        fm |= (uint64_t)forced << i;
        n_forced += __popcll(__ballot(forced));
    }
    const int expected_forced = forced_count(n, q.init_blocks, q.local_blocks);
    msa_top16_row* dst = q.merged + th;
    const int kept = select_row<VM>(um, mv, fm, kTop - expected_forced, count_keys<VM>(um), lane,
                                    buf, [&](int i) { return iv[i]; },
                                    [&](float score, int id, int slot) {
                                        dst->score[slot] = score;
                                        dst->id[slot] = id;
                                    });
    pad_row(dst, kept, lane);
    if ((n_forced < expected_forced || kept > kTop) && lane == 0 && q.score.errors)
        atomicAdd(q.score.errors, 1);
}

// Score plane (or pool) and per-range Top16 rows, and optionally their merge,
// in one launch ("flashinfer.msa_ops.prepare_msa_icp_indexer", decode: a fused
// scorer can replace the score and select steps, with caller-owned pool
// storage). Protocol:
//  1. Every wave scores its columns as score_decode_kernel does, storing them
//     written through to the device's coherence point (sc1). After each
//     request segment it waits for those stores, then adds the segment's
//     columns to each range's counter (a posted add: nothing waits on it).
//     A range is complete when its counter reaches the columns it writes.
//  2. Select jobs ((range, row of the range) pairs, range-major) belong to
//     q.helpers waves spread evenly over the grid's slots, each with a
//     contiguous block of jobs. For each it waits until the job's range is
//     complete, selects its row of the range exactly as top16_select_kernel
//     does (agent-scope loads of the plane), writes the range row written
//     through, and adds 1 to the range's done count; the helper that
//     completes that count (every other job of the range has then seen the
//     range complete) clears both of the range's counters. Only helpers
//     wait, the launcher keeps them to at most half the waves the device
//     holds at once, and scoring never waits, so every wave of the grid gets
//     a slot and every range completes.
//  3. With a merged output, a job then adds 1 to its (token, head) ticket; the
//     job that brings it to R merges the R rows as msa_top16_merge does and
//     clears the ticket.
// The workspace thus holds zeros again when the launch ends (unless a wait
// gives up, which counts an error).
template <int NT, int kParts, int kWavesPerEU, int V, int kUnit>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void score_select_kernel(ScoreSelectParams q)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[(8 / kParts) * 16 * kDim];
    __shared__ __attribute__((aligned(16))) float res[32][kChunk];
    __shared__ topk::CandBuf cand;
    __shared__ msa_top16_row row_buf;
    const ScoreParams& p = q.score;
    const int lane = threadIdx.x;
    const int R = q.num_ranges;
    const int w = q.width;
    const int rows_per_range = p.dql * kHeads;
    const int64_t total_jobs = (int64_t)p.batch * R * rows_per_range;

    // 1. scoring
    score_wave_range<NT, kParts, true, kUnit, false>(p, tile, res, [&](int b, int c_begin, int c_end) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the segment's stores are complete
        for (int r = c_begin / w; r * w < c_end; ++r) {
            const int n = min(c_end, (r + 1) * w) - max(c_begin, r * w);
            lane0_add_posted(range_line(q, (int64_t)b * R + r), n);
        }
    });

    // 2. and 3. select jobs, then merges. Helper k sits at slot
    // floor(k * grid / helpers) and runs the range-major jobs
    // [k * total / helpers, (k + 1) * total / helpers): for even ranges those
    // are rows of ranges this wave's neighbours scored (on its own XCD), which
    // complete about when the helper's own scoring does.
    const int64_t helpers = q.helpers;
    const int64_t grid = gridDim.x;
    const int64_t slot = kUnit == 1 ? (int64_t)blockIdx.x : (int64_t)split_slot();
    const int64_t k = (slot * helpers + grid - 1) / grid;
    if (k >= helpers || k * grid / helpers != slot)
        return;
    int32_t* tickets = merge_tickets(q);
    const int64_t job_end = (k + 1) * total_jobs / helpers;
    for (int64_t c = k * total_jobs / helpers; c < job_end; ++c) {
        const int64_t rr = c / rows_per_range;
        const int row = (int)(c - rr * rows_per_range);
        const int b = (int)(rr / R);
        const int r = (int)(rr - (int64_t)b * R);
        const int t = b * p.dql + row / kHeads;
        const int64_t th = (int64_t)t * kHeads + row % kHeads;
        // valid ids [0, n): num_valid_pages, clamped to the plane (and, for
        // the pool, to the columns this launch writes)
        bool clamped;
        const int wb = written_cols(p.seq_lens[b], p.cols, clamped);
        const int limit = q.pool ? wb : p.cols;
        const int nvp = q.nvp[t];
        int32_t* line = range_line(q, rr);
        const int want = range_columns(q, wb, r);
        uint32_t polls = 0;
        while (lane0_load(line) != want) {
            if (++polls > kMaxPolls) {
                if (lane == 0 && p.errors)
                    atomicAdd(p.errors, 1);
                return;
            }
            __builtin_amdgcn_s_sleep(4);
        }

        int n = nvp;
        if (n < 0 || n > limit) {
            if (r == 0 && (row % kHeads) == 0 && lane == 0 && p.errors)
                atomicAdd(p.errors, 1);
            n = n < 0 ? 0 : limit;
        }
        const int lo = r * w;
        const int hi = min(lo + w, p.cols);
        float sv[V];
        topk::load_span<V, true>(p.out + th * p.cols, p.cols, lo, lane, sv);
        topk::select_loaded<V>(sv, lo, hi, topk::column_ids(n, q.init_blocks, q.local_blocks, 1, 0),
                               &row_buf, lane, &cand);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the range row, written through (a merging wave reads it)
        int32_t* dst = reinterpret_cast<int32_t*>(q.out + th * R + r);
        if (lane < 2 * kTop)
            __hip_atomic_store(dst + lane, reinterpret_cast<const int32_t*>(&row_buf)[lane],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (q.merged != nullptr) {
            if (R == 1) {
                if (lane < 2 * kTop)
                    reinterpret_cast<int32_t*>(q.merged + th)[lane] =
                        reinterpret_cast<const int32_t*>(&row_buf)[lane];
            } else {
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the row is stored
                if (lane0_add(tickets + th, 1) == R - 1) {
                    const int nm = max(0, nvp);  // as msa_top16_merge reads it
                    if (R <= 4)
                        fused_merge<1>(q, th, nm, lane, &cand);
                    else if (R <= 8)
                        fused_merge<2>(q, th, nm, lane, &cand);
                    else if (R <= 16)
                        fused_merge<4>(q, th, nm, lane, &cand);
                    else
                        fused_merge<16>(q, th, nm, lane, &cand);
                    lane0_store(tickets + th, 0);
                }
            }
        }
        if (lane0_add(line + 1, 1) == rows_per_range - 1) {
            lane0_store(line, 0);
            lane0_store(line + 1, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

constexpr int kParts = MSA_SCORE_PARTS;

// Grid size: a whole number of waves per SIMD of the device (every wave
// gets an equal share of the work, so an uneven count would leave some SIMDs
// with one wave more than others and set the tail). Registers are capped for
// that many waves per SIMD.
template <int NT>
constexpr int waves_per_simd()
{
    return NT == 1 ? MSA_SCORE_WAVES_PER_SIMD_16 : MSA_SCORE_WAVES_PER_SIMD_32;
}

template <int NT>
const void* score_kernel_fn()
{
    constexpr int kRegWaves = NT == 1 ? MSA_SCORE_REG_WAVES_16 : MSA_SCORE_REG_WAVES_32;
    return reinterpret_cast<const void*>(&score_decode_kernel<NT, kParts, kRegWaves, 4, false>);
}

// Row-sharded cache: one rank's share, streaming grid, its shard columns
// (32, 64 or 128 rows) staged in the same 32-row pieces as whole blocks.
// Measured over rotating shard copies of the 4 x 1 Mi-key cache, 64-row
// pieces took 44.5 / 25.1 us at world sizes 2 / 4 against 43.8 / 24.8 us.
template <int NT>
const void* score_sharded_kernel_fn()
{
    constexpr int kRegWaves = NT == 1 ? MSA_SCORE_REG_WAVES_16 : MSA_SCORE_REG_WAVES_32;
    return reinterpret_cast<const void*>(&score_decode_kernel<NT, kParts, kRegWaves, 4, true>);
}

// Small batches: one column per work unit and a whole block per DMA round
// trip (16 KiB LDS tile), so that every block gets its own wave and pays one
// memory latency instead of four.
template <int NT>
const void* score_latency_kernel_fn()
{
    return reinterpret_cast<const void*>(
        &score_decode_kernel<NT, 1, MSA_SCORE_LATENCY_WAVES_PER_SIMD, 1, false>);
}

// Waves per SIMD a streaming instance of the fused kernel is built for (its
// register budget). 32 values per lane do not fit the 3-waves-per-SIMD budget
// of the 16-row scorer (spills), so that instance takes the 2-wave budget;
// its grid is sized the same way, so that every wave of it is resident at
// once (a grid sized for 3 waves per SIMD ran its last third as a second
// round: 92 us against 77 us per step at the 2048-column workload).
constexpr int score_select_waves_per_simd(int nt, int v)
{
    return nt == 1 ? (v >= 32 ? 2 : MSA_SCORE_REG_WAVES_16) : MSA_SCORE_REG_WAVES_32;
}

template <int NT, int V, bool kLatency>
const void* score_select_kernel_fn()
{
    constexpr int kRegWaves = score_select_waves_per_simd(NT, V);
    if constexpr (kLatency)  // one column per wave, a block per DMA round trip
        return reinterpret_cast<const void*>(
            &score_select_kernel<NT, 1, MSA_SCORE_LATENCY_WAVES_PER_SIMD, V, 1>);
    else
        return reinterpret_cast<const void*>(&score_select_kernel<NT, kParts, kRegWaves, V, 4>);
}

// Compute units of the current device (host query, cached per device; the
// cache is safe to fill from several host threads at once).
int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Scorer grid: one wave per workgroup, a whole number of waves per SIMD, no
// more waves than 4-column groups can exist.
int64_t score_grid(const ScoreParams& p)
{
    const bool small_q = p.dql * kHeads <= 16;
    const int64_t waves =
        (int64_t)device_cus() * 4 * (small_q ? waves_per_simd<1>() : waves_per_simd<2>());
    const int64_t max_groups = (int64_t)p.batch * (p.cols / 4);
    return max_groups < waves ? max_groups : waves;
}

hipError_t launch_score_decode(const ScoreParams& p, hipStream_t stream)
{
    void* args[] = {const_cast<ScoreParams*>(&p)};
    const bool small_q = p.dql * kHeads <= 16;
    if (p.world_size > 1) {
        const void* fn = small_q ? score_sharded_kernel_fn<1>() : score_sharded_kernel_fn<2>();
        return hipLaunchKernel(fn, dim3((unsigned)score_grid(p)), dim3(64), args, 0, stream);
    }
    const int64_t max_cols = (int64_t)p.batch * p.cols;
    const int64_t latency_waves = (int64_t)device_cus() * 4 * MSA_SCORE_LATENCY_WAVES_PER_SIMD;
    if (max_cols <= latency_waves) {
        const void* fn = small_q ? score_latency_kernel_fn<1>() : score_latency_kernel_fn<2>();
        return hipLaunchKernel(fn, dim3((unsigned)max_cols), dim3(64), args, 0, stream);
    }
    const void* fn = small_q ? score_kernel_fn<1>() : score_kernel_fn<2>();
    return hipLaunchKernel(fn, dim3((unsigned)score_grid(p)), dim3(64), args, 0, stream);
}

// Values per lane of the fused kernel's select (spans up to 256, 1024 and
// 2048 columns), streaming or latency mode.
#define MSA_FOR_EACH_SCORE_SELECT(X)                                                  \
    X(1, 4, false) X(1, 16, false) X(1, 32, false) X(2, 4, false) X(2, 16, false)     \
    X(2, 32, false) X(1, 4, true) X(1, 16, true) X(1, 32, true) X(2, 4, true)         \
    X(2, 16, true) X(2, 32, true)

hipError_t launch_score_select(const ScoreSelectParams& q, hipStream_t stream)
{
    const int nt = q.score.dql * kHeads <= 16 ? 1 : 2;
    const int v = q.width <= 256 ? 4 : q.width <= 1024 ? 16 : q.width <= kMaxFusedWidth ? 32 : 0;
    // the scorer's rule: small batches score one column per wave
    const int64_t max_cols = (int64_t)q.score.batch * q.score.cols;
    const bool latency =
        max_cols <= (int64_t)device_cus() * 4 * MSA_SCORE_LATENCY_WAVES_PER_SIMD;
    const void* fn = nullptr;
#define X(NT, V, L)                                  \
    if (nt == NT && v == V && latency == L)          \
        fn = score_select_kernel_fn<NT, V, L>();
    MSA_FOR_EACH_SCORE_SELECT(X)
#undef X
    if (fn == nullptr)
        return hipErrorInvalidValue;
    const int64_t groups = (int64_t)q.score.batch * (q.score.cols / 4);
    const int64_t grid =
        latency ? max_cols
                : std::min(groups, (int64_t)device_cus() * 4 * score_select_waves_per_simd(nt, v));
    // Helpers wait for ranges; at most half of the waves the device holds at
    // once may, so that the rest of the grid always finds slots.
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0);
    if (e != hipSuccess)
        return e;
    const int64_t resident = (int64_t)per_cu * device_cus();
    const int64_t jobs = (int64_t)q.score.batch * q.num_ranges * q.score.dql * kHeads;
    if (resident < 2)
        return hipErrorInvalidConfiguration;
    ScoreSelectParams qh = q;
    qh.helpers = (int)std::min(std::min(jobs, resident / 2), grid);
    void* args[] = {&qh};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64), args, 0, stream);
}

hipError_t warmup_score_kernels()
{
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, score_kernel_fn<1>());
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&attr, score_kernel_fn<2>());
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&attr, score_sharded_kernel_fn<1>());
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&attr, score_sharded_kernel_fn<2>());
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&attr, score_latency_kernel_fn<1>());
    if (e == hipSuccess)
        e = hipFuncGetAttributes(&attr, score_latency_kernel_fn<2>());
#define X(NT, V, L)       \
    if (e == hipSuccess)  \
        e = hipFuncGetAttributes(&attr, score_select_kernel_fn<NT, V, L>());
    MSA_FOR_EACH_SCORE_SELECT(X)
#undef X
    return e;
}

}  // namespace msa
