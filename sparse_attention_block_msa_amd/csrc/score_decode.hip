// Score-plane kernel for gfx950.
//
// Operation ("flashinfer.msa_ops.msa_icp_decode_index_score_sharded",
// description and parameters): for each request b, decode token j and index
// head h, and each B128 block c of the request,
//   plane[(b*dql + j), h, c] = max over keys p of block c with p < seq_len and
//                              p <= seq_len - dql + j of  q[b*dql + j, h, :] . k[p, :]
// (-inf if the block has no such key). Columns are written up to the request's
// block count rounded up to a multiple of four and no further.
//
// Design (one wave = 64 lanes per workgroup):
//  * A wave owns a chunk of consecutive columns of one request. Its Q tile
//    (4*dql <= 32 rows of 128 fp8 bytes) is converted once to bf16 and stays
//    in registers for the whole chunk as the B operand of the MFMA.
//  * A B128 block is 128 keys x 128 bytes = 16 KiB, contiguous inside one
//    page. It is staged through a per-wave 4 KiB LDS tile in four pieces of
//    32 keys with global_load_lds_dwordx4: each DMA instruction moves 1 KiB
//    of whole 128-byte rows (a fully contiguous, non-temporal read), and the
//    per-lane source addresses are chosen so the tile lands XOR-swizzled,
//    letting the MFMA-layout ds_read_b128s hit every LDS bank once. Loads
//    never occupy VGPRs, so the kernel runs 4-6 waves per SIMD and the
//    occupancy hides HBM latency. (Loading the MFMA layout straight into
//    registers needs half-row 64-byte accesses per instruction; measured on
//    MI355X, that pattern streams at about 5.2 TB/s against 6.5 TB/s for
//    whole-row DMA.)
//  * Contraction: every e4m3fn value is exactly a bf16 value, so each key
//    tile is converted with v_cvt_scalef32_pk_bf16_fp8 (scale 1.0, two values
//    per instruction) and contracted with v_mfma_f32_16x16x32_bf16, four
//    instructions chained through the fp32 accumulator per 128-dim dot
//    product. The fp8 MFMA forms (16x16x128 f8f6f4, 16x16x32 fp8) were
//    measured on gfx950 to sum groups of fp8 products with up to about
//    2e-5 of sum|q_i k_i| error on N(0,1) data and 2.4e-4 on full-range
//    codes, above the 1e-5 bound this kernel guarantees; the bf16 form
//    measured at most 3e-7. The path is HBM-bound either way (8*dql flop per
//    index-K byte), so the bf16 rate costs no throughput.
//  * Lane l of a 16x16 result holds keys 4*(l/16)..+3 of the tile for query
//    row l%16, so the block max is a per-lane max over 8 tiles x 4 values
//    followed by a max across the four 16-lane groups. The causal mask is
//    applied only in blocks that reach past the first token's position.
//  * The chunk's block maxima collect in a small per-wave LDS array and are
//    stored to the plane (64 contiguous bytes per query row) only when the
//    chunk is done, so no DMA wait ever waits on a plane store.
//
// Byte order inside a lane's operands: the 32 bytes a lane supplies per row
// are bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte row
// (g = lane/16); byte b of that slice becomes element b%8 of the operand of
// instruction b/8, for the key rows (A) and the query rows (B) alike. The dot
// product is a sum over all 128 dims, so any byte-to-k assignment that A and
// B share gives the same sum.
#include <math.h>

#include "msa_internal.h"

namespace msa {
namespace {

// Launch shape: one 64-lane wave per workgroup, a block staged in kParts
// pieces, and registers capped for 6 (<= 16 query rows) or 4 (32 rows)
// waves per SIMD (LDS use: 4 KiB per wave).
#ifndef MSA_SCORE_LOAD_AUX
#define MSA_SCORE_LOAD_AUX 2  // cache-policy bits of the index-K DMA: nt (non-temporal)
#endif
#ifndef MSA_SCORE_PARTS
#define MSA_SCORE_PARTS 4
#endif
#ifndef MSA_SCORE_WAVES_PER_EU_16
#define MSA_SCORE_WAVES_PER_EU_16 6  // up to 16 query rows (decode_query_len <= 4)
#endif
#ifndef MSA_SCORE_WAVES_PER_EU_32
#define MSA_SCORE_WAVES_PER_EU_32 4  // 17..32 query rows (more registers for the Q tile)
#endif
#ifndef MSA_SCORE_CHUNK
#define MSA_SCORE_CHUNK 16
#endif

constexpr int kChunk = MSA_SCORE_CHUNK;
static_assert(kChunk % 4 == 0 && kChunk <= kMaxScoreChunk, "bad chunk");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i load_row_slice(const uint8_t* row, int g)
{
    const v4i lo = *reinterpret_cast<const v4i*>(row + 16 * g);
    const v4i hi = *reinterpret_cast<const v4i*>(row + 64 + 16 * g);
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) void* global_ptr;

// One piece of a B128 block (kPieceRows consecutive key rows, 128 bytes each)
// is staged in a per-wave LDS tile. Row `row`, 16-byte chunk c of the piece
// sits at LDS chunk position (row, c ^ swz(row)): the 16 lanes that read
// chunk g of 16 consecutive rows then touch 16 distinct (row parity,
// position) pairs, i.e. all 64 banks once.
__device__ __forceinline__ int swz(int row)
{
    return (row >> 1) & 7;
}

// Copies kPieceRows rows (contiguous in HBM) into the LDS tile with the
// swizzle above. Each instruction moves 1 KiB = 8 whole rows: lane l fetches
// row 8t + l/8, chunk (l%8) ^ swz(row), and the DMA engine writes it to LDS
// byte 16*l of the instruction's 1 KiB slot. The loads are non-temporal:
// every key is read exactly once per call.
template <int kPieceRows>
__device__ __forceinline__ void stage_piece(const uint8_t* piece, uint8_t* tile, int lane)
{
#pragma unroll
    for (int t = 0; t < kPieceRows / 8; ++t) {
        const int row = 8 * t + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        __builtin_amdgcn_global_load_lds((global_ptr)(piece + row * kDim + chunk * 16),
                                         (lds_ptr)(tile + t * 1024), 16, 0, MSA_SCORE_LOAD_AUX);
    }
}

// The lane's 32-byte slice of tile row `row` (chunks g and 4 + g).
__device__ __forceinline__ v8i read_row_slice(const uint8_t* tile, int row, int g)
{
    const v4i lo = *reinterpret_cast<const v4i*>(tile + row * kDim + 16 * (g ^ swz(row)));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + row * kDim + 16 * ((4 + g) ^ swz(row)));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// 8 fp8 bytes (two dwords) -> 8 bf16 values, byte order kept. Exact.
__device__ __forceinline__ v8bf fp8x8_to_bf16(int w0, int w1)
{
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w0, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w0, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w1, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w1, 1.0f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

struct Bf16Slice {
    v8bf op[4];  // operand of instruction s = bytes [8s, 8s+8) of the lane's 32-byte slice
};

__device__ __forceinline__ Bf16Slice to_bf16(const v8i& raw)
{
    Bf16Slice t;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        t.op[s] = fp8x8_to_bf16(raw[2 * s], raw[2 * s + 1]);
    return t;
}

__device__ __forceinline__ float max4(v4f a)
{
    return fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
}

// Scores one B128 block against the NT query tiles. The block is staged
// through the wave's LDS tile in kParts pieces of 8 / kParts key tiles (16
// keys each): DMA, wait, then convert and contract each tile. Other waves on
// the SIMD keep HBM busy meanwhile. On return mx[n] holds, in every lane,
// the block max of query row 16n + lane%16. kMask: keys whose in-block index
// exceeds lim[n] are excluded.
template <int NT, int kParts, bool kMask>
__device__ __forceinline__ void score_block(const uint8_t* block, uint8_t* tile,
                                            const Bf16Slice (&qb)[NT], int lane, int r16, int g,
                                            const int (&lim)[NT], float (&mx)[NT])
{
    constexpr int kTiles = 8 / kParts;
    constexpr int kPieceRows = kTiles * 16;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NT; ++n)
        mx[n] = -INFINITY;
#pragma unroll
    for (int part = 0; part < kParts; ++part) {
        stage_piece<kPieceRows>(block + part * kPieceRows * kDim, tile, lane);
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

template <int NT, int kParts, int kWavesPerEU>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void score_decode_kernel(ScoreParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[(8 / kParts) * 16 * kDim];
    __shared__ __attribute__((aligned(16))) float res[32][kChunk];  // block maxima of the chunk
    const int lane = threadIdx.x;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int b = blockIdx.x / p.chunks_per_req;
    const int chunk = blockIdx.x - b * p.chunks_per_req;

    const int seq = p.seq_lens[b];
    if (seq <= 0)
        return;
    const int nblk = (int)(((int64_t)seq + kBlockTokens - 1) / kBlockTokens);
    int wcols = (int)(((int64_t)nblk + 3) / 4 * 4);
    if (wcols > p.cols) {
        if (chunk == 0 && lane == 0 && p.errors)
            atomicAdd(p.errors, 1);
        wcols = p.cols;
    }
    const int c_begin = chunk * kChunk;
    if (c_begin >= wcols)
        return;
    // c_begin is a multiple of 4 below roundup4(nblk), hence below nblk: the
    // chunk holds at least one block with keys.
    const int c_end = min(c_begin + kChunk, wcols);
    const int c_last = min(c_end, nblk) - 1;

    const int rows = p.dql * kHeads;
    const int64_t row_base = (int64_t)b * rows;
    const int ps_shift = p.page_size == 256 ? 1 : 0;  // log2(B128 blocks per page)

    // Block-table entries of this chunk, one per lane (at most kMaxScoreChunk).
    const int pg_begin = c_begin >> ps_shift;
    const int pg_count = (c_last >> ps_shift) - pg_begin + 1;
    int my_page = 0;
    bool my_bad = false;
    if (lane < pg_count) {
        const int64_t idx = (int64_t)pg_begin + lane;
        if (idx >= p.bt_stride) {
            my_bad = true;
        } else {
            const int v = p.bt[(int64_t)b * p.bt_stride + idx];
            if (v < 0 || (int64_t)v >= p.num_pages)
                my_bad = true;
            else
                my_page = v;
        }
    }
    const uint64_t bad_mask = __ballot(my_bad);
    if (bad_mask != 0 && lane == 0 && p.errors)
        atomicAdd(p.errors, (int)__popcll(bad_mask));

    auto block_ptr = [&](int c) -> const uint8_t* {
        const int page = __builtin_amdgcn_readlane(my_page, (c >> ps_shift) - pg_begin);
        const int half = c & ((1 << ps_shift) - 1);
        return p.k + ((int64_t)page * p.page_size + half * kBlockTokens) * kDim;
    };

    // Query tiles and token positions of the rows this lane's columns map to.
    Bf16Slice qb[NT];
    int pos[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int rho = n * 16 + r16;
        pos[n] = seq - p.dql + (rho >> 2);
        v8i raw = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        if (rho < rows)
            raw = load_row_slice(p.q + (row_base + rho) * kDim, g);
        qb[n] = to_bf16(raw);
    }

    const int first_masked = seq - p.dql;  // blocks reaching past this key need the mask
    for (int c = c_begin; c < c_end; ++c) {
        float mx[NT];
        int lim[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n)
            lim[n] = pos[n] - c * kBlockTokens;
        const bool has_keys =
            c <= c_last && !((bad_mask >> ((min(c, c_last) >> ps_shift) - pg_begin)) & 1ull);
        if (!has_keys) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                mx[n] = -INFINITY;
        } else if (c * kBlockTokens + (kBlockTokens - 1) > first_masked) {
            score_block<NT, kParts, true>(block_ptr(c), tile, qb, lane, r16, g, lim, mx);
        } else {
            score_block<NT, kParts, false>(block_ptr(c), tile, qb, lane, r16, g, lim, mx);
        }
        // lanes of group g == n keep query row 16n + lane%16
#pragma unroll
        for (int n = 0; n < NT; ++n)
            if (g == n)
                res[n * 16 + r16][c - c_begin] = mx[n];
    }

    // All plane stores are issued at the very end: on this ISA stores share
    // the vector-memory counter with the DMA, so a store issued mid-chunk
    // would make every later DMA wait also wait for it.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int quads = (c_end - c_begin) / 4;  // float4 groups per row
    for (int i = lane; i < rows * quads; i += 64) {
        const int rho = i / quads;
        const int q4 = i - rho * quads;
        const v4f v = *reinterpret_cast<const v4f*>(&res[rho][q4 * 4]);
        *reinterpret_cast<v4f*>(p.out + (row_base + rho) * p.cols + c_begin + q4 * 4) = v;
    }
}

}  // namespace

constexpr int kParts = MSA_SCORE_PARTS;

template <int NT>
const void* score_kernel_fn()
{
    constexpr int kWavesPerEU = NT == 1 ? MSA_SCORE_WAVES_PER_EU_16 : MSA_SCORE_WAVES_PER_EU_32;
    return reinterpret_cast<const void*>(&score_decode_kernel<NT, kParts, kWavesPerEU>);
}

int score_chunk_for(int batch, int cols)
{
    (void)batch;
    (void)cols;
    return MSA_SCORE_CHUNK;
}

hipError_t launch_score_decode(const ScoreParams& p, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)p.batch * p.chunks_per_req));
    const dim3 block(64);
    void* args[] = {const_cast<ScoreParams*>(&p)};
    const void* fn = p.dql * kHeads <= 16 ? score_kernel_fn<1>() : score_kernel_fn<2>();
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t warmup_score_kernels()
{
    hipFuncAttributes attr;
    hipError_t e = hipFuncGetAttributes(&attr, score_kernel_fn<1>());
    if (e != hipSuccess)
        return e;
    return hipFuncGetAttributes(&attr, score_kernel_fn<2>());
}

}  // namespace msa
