// Key-tile helpers shared by the decode and prefill scorers (gfx950): a
// B128 block of index-K rows (128 keys x 128 fp8 bytes) staged through LDS
// with an XOR swizzle by the DMA form of global loads, read back in the
// operand layout of v_mfma_f32_16x16x32_bf16, and converted exactly from
// e4m3fn to bf16.
//
// Operand layout: for a 16-row tile, lane l supplies row l % 16 and the
// 32-byte slice of it made of bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g +
// 16) (g = l / 16); byte b of the slice becomes element b % 8 of the operand
// of instruction b / 8 of four chained MFMAs. Key rows (A) and query rows (B)
// use the same assignment, so the four instructions sum all 128 products of
// a dot product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_internal.h"

namespace msa {
namespace keytile {

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
// byte 16*l of the instruction's 1 KiB slot. kAux holds the loads'
// cache-policy bits (the decode scorer reads every key once and streams it
// non-temporally; the prefill scorer re-reads keys and keeps them cached).
template <int kPieceRows, int kAux>
__device__ __forceinline__ void stage_piece(const uint8_t* piece, uint8_t* tile, int lane)
{
#pragma unroll
    for (int t = 0; t < kPieceRows / 8; ++t) {
        const int row = 8 * t + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        __builtin_amdgcn_global_load_lds((global_ptr)(piece + row * kDim + chunk * 16),
                                         (lds_ptr)(tile + t * 1024), 16, 0, kAux);
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

}  // namespace keytile
}  // namespace msa
