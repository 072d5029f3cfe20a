// Measurement aid (no page defines it): 128-dim e4m3fn dot products through
// three gfx950 MFMA forms, so that their fp32 accumulation error can be
// measured against exact products.
//
// Every finite e4m3fn value is exactly a bf16 value, so the bf16 form is the
// scorer's own contraction: each lane's fp8 slice is converted with
// v_cvt_scalef32_pk_bf16_fp8 (scale 1) and four v_mfma_f32_16x16x32_bf16 are
// chained through the accumulator. The two fp8 forms consume the codes
// directly: four chained v_mfma_f32_16x16x32_fp8_fp8, or one
// v_mfma_f32_16x16x128_f8f6f4 (both operands e4m3, no block scale).
//
// A tile is 16 query rows x 16 key rows (128 bytes each); one wave computes
// the tile's 256 dot products. For a dot product the assignment of the 128
// dims to (lane group, operand byte) only has to be the same for both
// operands, which it is in every form below.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "contraction_probe.h"

namespace msa {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of a 128-byte row.
__device__ __forceinline__ v8i row_slice(const uint8_t* row, int g)
{
    const v4i lo = *reinterpret_cast<const v4i*>(row + 16 * g);
    const v4i hi = *reinterpret_cast<const v4i*>(row + 64 + 16 * g);
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__device__ __forceinline__ v8bf to_bf16x8(int w0, int w1)
{
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w0, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w0, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w1, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w1, 1.0f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__global__ __launch_bounds__(64) void contraction_probe_kernel(const uint8_t* q, const uint8_t* k,
                                                               int form, float* out)
{
    const int64_t tile = blockIdx.x;
    const int lane = threadIdx.x;
    const int r = lane & 15;
    const int g = lane >> 4;
    const uint8_t* qrow = q + (tile * 16 + r) * 128;
    const uint8_t* krow = k + (tile * 16 + r) * 128;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (form == MSA_PROBE_BF16) {
        const v8i qs = row_slice(qrow, g), ks = row_slice(krow, g);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(ks[2 * s], ks[2 * s + 1]),
                                                          to_bf16x8(qs[2 * s], qs[2 * s + 1]),
                                                          acc, 0, 0, 0);
    } else if (form == MSA_PROBE_FP8_16X16X32) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const long a = *reinterpret_cast<const long*>(krow + 32 * s + 8 * g);
            const long b = *reinterpret_cast<const long*>(qrow + 32 * s + 8 * g);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, acc, 0, 0, 0);
        }
    } else {
        // zero format and scale operands: the unscaled e4m3 x e4m3 instruction
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(row_slice(krow, g),
                                                               row_slice(qrow, g), acc, 0, 0, 0,
                                                               0, 0, 0);
    }
    // lane l holds key rows 4*(l/16) .. +3 for query row l % 16
    float* o = out + tile * 256;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        o[r * 16 + 4 * g + v] = acc[v];
}

}  // namespace

hipError_t launch_contraction_probe(const uint8_t* q, const uint8_t* k, int64_t tiles, int form,
                                    float* out, hipStream_t stream)
{
    void* args[] = {const_cast<uint8_t**>(&q), const_cast<uint8_t**>(&k), &form, &out};
    return hipLaunchKernel(reinterpret_cast<const void*>(&contraction_probe_kernel),
                           dim3((unsigned)tiles), dim3(64), args, 0, stream);
}

}  // namespace msa
