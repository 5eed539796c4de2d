// mfma_common.h - pieces shared by the two places that compute delta on the matrix cores:
// the standalone delta projection (project_kernels.h) and the prefill that computes delta on
// its load path (prefill_rows_kernel.h).  Both must produce bit-identical delta, so both use
// these operand types, fragment loads, the MFMA itself and the softplus epilogue.
//
// MFMA 16x16x32 bf16 register layout (lane l of a wave):
//     A operand: A[row = l % 16][k = 8 * (l / 16) + j], j = 0..7
//     B operand: B[k = 8 * (l / 16) + j][col = l % 16]
//     result:    D[row = 4 * (l / 16) + i][col = l % 16], i = 0..3
// Both operands are 16-byte loads when their k index is contiguous in memory.
#pragma once

#include "scan_update.h"

namespace jscan {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));   // 16 raw bytes in registers

// 8 consecutive bf16 (16 bytes) as an MFMA operand.
__device__ __forceinline__ bf16x8_t load_frag(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(p));
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(e^-|z|), with t = e^-|z| in (0, 1].
// log1p(t) is the hardware log2 of 1 + t, except below t = 2^-10, where 1 + t would lose t's
// low bits and log1p(t) = t (1 - t/2 + ...) is t to within t/2 <= 2^-11 relative, below the
// bf16 precision (2^-8) the result is stored with.
__device__ __forceinline__ float softplus_f32(float z) {
    const float t = __builtin_amdgcn_exp2f(-fabsf(z) * kLog2e);
    const float l = t < 0x1.0p-10f ? t : __builtin_amdgcn_logf(1.0f + t) * 0.69314718055994530942f;
    return fmaxf(z, 0.0f) + l;
}

}  // namespace jscan
