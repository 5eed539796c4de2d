// project_kernels.h - the producer side of the scan: delta, B and C computed from x.
//
// The notes page ("Jamba: A Hybrid Transformer-Mamba Language Model", section "Mamba layer")
// has the scan's parameters depend on the input, B_t, C_t, delta_t = f(x_t), and applies
// RMSNorm inside the Jamba Mamba layer.  f is taken as the selective projection of Mamba-1:
//     [d_low | B | C] = W_x x_t                       (W_x: (R + 2N) x D, R the rank of delta)
//     d_low, B, C each RMS-normalised over its own width and scaled by a learned gain
//     delta_t = softplus(W_dt d_low + b_dt)          (W_dt: D x R, b_dt: D)
// Both products are dense contractions, so they run on the matrix cores: bf16 operands,
// fp32 accumulation (v_mfma_f32_16x16x32_bf16), with the normalisation and the softplus
// applied to the fp32 accumulators before the single rounding to bf16.
//
// MFMA 16x16x32 bf16 register layout (lane l of a wave):
//     A operand: A[row = l % 16][k = 8 * (l / 16) + j], j = 0..7
//     B operand: B[k = 8 * (l / 16) + j][col = l % 16]
//     result:    D[row = 4 * (l / 16) + i][col = l % 16], i = 0..3
// Both operands are 16-byte loads when their k index is contiguous in memory, so every matrix
// here is stored with k fastest: x is [M][D], W_x is [R + 2N][D], d_low is [M][R] and W_dt is
// [D][R] (the [out][in] layout of a linear layer).
#pragma once

#include "scan_update.h"

namespace jscan {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace proj {
constexpr int kRowsX = 128;   // x-projection rows (tokens) per work-group: 4 waves x 32
constexpr int kTileDt = 128;  // delta-projection tile: 128 channels x 128 tokens, 4 waves of 64 x 64
}

// 8 consecutive bf16 (16 bytes) as an MFMA operand.
__device__ __forceinline__ bf16x8_t load_frag(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum over the 16 lanes of a DPP row (lanes 16q .. 16q+15); every lane gets the total.
// The butterfly adds in a fixed order, so the result is the same in every lane.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x101F));   // xor 4
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x201F));   // xor 8
    return v;
}

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(e^-|z|), with e^-|z| in (0, 1].
__device__ __forceinline__ float softplus_f32(float z) {
    const float t = __builtin_amdgcn_exp2f(-fabsf(z) * kLog2e);
    // log1p(t): the series where 1 + t would lose t's low bits, the hardware log2 elsewhere
    const float l = t < 0x1.0p-10f ? t * (1.0f - t * (0.5f - t * (1.0f / 3.0f)))
                                   : __builtin_amdgcn_logf(1.0f + t) * 0.69314718055994530942f;
    return fmaxf(z, 0.0f) + l;
}

// x projection: one work-group = 128 rows (tokens) x all R + 2N output columns; wave w owns
// rows 32w .. 32w+31 as two 16-row tiles.  RT = R / 16 column tiles of d_low, then one tile
// each of B and C (N = 16).  The K loop walks D in steps of 32 with the next step's operands
// loaded while the current step's MFMAs run.
template <int RT>
__global__ __launch_bounds__(256) void xproj_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                    const float *__restrict__ g_d, const float *__restrict__ g_b,
                                                    const float *__restrict__ g_c, uint16_t *__restrict__ d_low,
                                                    uint16_t *__restrict__ Bo, uint16_t *__restrict__ Co, int64_t M,
                                                    int D, float eps) {
    constexpr int CT = RT + 2;   // column tiles
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t row0 = (int64_t)blockIdx.x * proj::kRowsX + wave * 32;
    const int r16 = l & 15, kq = 8 * (l >> 4);
    // A rows of this lane (clamped: rows past M compute garbage that is never stored)
    const uint16_t *xa[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) xa[t] = x + min(row0 + 16 * t + r16, M - 1) * D + kq;
    const uint16_t *wb = w + (int64_t)r16 * D + kq;   // column tile c adds 16 * c * D

    f32x4_t acc[2][CT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    bf16x8_t a[2][2], b[2][CT];
    auto load = [&](int s, int k0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) a[s][t] = load_frag(xa[t] + k0);
#pragma unroll
        for (int c = 0; c < CT; ++c) b[s][c] = load_frag(wb + (int64_t)16 * c * D + k0);
    };
    auto step = [&](int s) {
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[t][c] = mfma16(a[s][t], b[s][c], acc[t][c]);
    };
    load(0, 0);
    for (int k0 = 0; k0 < D; k0 += 64) {   // D % 64 == 0
        load(1, k0 + 32);
        step(0);
        if (k0 + 64 < D) load(0, k0 + 64);
        step(1);
    }

    // Epilogue.  Lane l holds rows 4 * (l / 16) + i of each 16-row tile, column 16 c + l % 16.
    // The sums of squares over a row are per-lane partial sums over the lane's columns, then
    // a sum over the 16 lanes of the DPP row.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = row0 + 16 * t + 4 * (l >> 4) + i;
            float sd = 0.f;
#pragma unroll
            for (int c = 0; c < RT; ++c) sd = __builtin_fmaf(acc[t][c][i], acc[t][c][i], sd);
            const float vb = acc[t][RT][i], vc = acc[t][RT + 1][i];
            sd = row16_sum(sd);
            const float sb = row16_sum(vb * vb), sc = row16_sum(vc * vc);
            const float nd = __builtin_amdgcn_rsqf(sd * (1.0f / (16 * RT)) + eps);
            const float nb = __builtin_amdgcn_rsqf(sb * (1.0f / 16) + eps);
            const float nc = __builtin_amdgcn_rsqf(sc * (1.0f / 16) + eps);
            if (row < M) {
#pragma unroll
                for (int c = 0; c < RT; ++c)
                    d_low[row * (16 * RT) + 16 * c + r16] = f32_to_bf16_bits(acc[t][c][i] * nd * g_d[16 * c + r16]);
                Bo[row * kDState + r16] = f32_to_bf16_bits(vb * nb * g_b[r16]);
                Co[row * kDState + r16] = f32_to_bf16_bits(vc * nc * g_c[r16]);
            }
        }
    }
}

// Delta projection: one work-group = 128 channels x 128 tokens of delta; wave w owns
// channels 64 (w & 1) .. +63 and tokens 64 (w >> 1) .. +63 as 4 x 4 MFMA tiles.  A = W_dt
// (rows = channels), B = d_low^T (columns = tokens), so each lane's result is 4 consecutive
// channels of one token: the epilogue adds the bias, applies softplus and writes 8 bytes.
template <int R>
__global__ __launch_bounds__(256) void dtproj_kernel(const uint16_t *__restrict__ d_low, const uint16_t *__restrict__ w,
                                                     const float *__restrict__ bias, uint16_t *__restrict__ delta,
                                                     int64_t M, int D, int ch_tiles) {
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t tok_tile = blockIdx.x / ch_tiles;
    const int ch0 = (blockIdx.x - (int)(tok_tile * ch_tiles)) * proj::kTileDt + 64 * (wave & 1);
    const int64_t tok0 = tok_tile * proj::kTileDt + 64 * (wave >> 1);
    const int r16 = l & 15, kq = 8 * (l >> 4);
    const uint16_t *wa = w + (int64_t)(ch0 + r16) * R + kq;                // channel tile u adds 16 u R
    const uint16_t *db[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) db[v] = d_low + min(tok0 + 16 * v + r16, M - 1) * R + kq;

    f32x4_t acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < R; k0 += 32) {
        bf16x8_t a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = load_frag(wa + 16 * u * R + k0);
#pragma unroll
        for (int v = 0; v < 4; ++v) b[v] = load_frag(db[v] + k0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = mfma16(a[u], b[v], acc[u][v]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = ch0 + 16 * u + 4 * (l >> 4);
        const float4 bs = *reinterpret_cast<const float4 *>(bias + c);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t tok = tok0 + 16 * v + r16;
            if (tok < M) {
                uint2 pk;
                pk.x = pack_bf16x2(softplus_f32(acc[u][v][0] + bs.x), softplus_f32(acc[u][v][1] + bs.y));
                pk.y = pack_bf16x2(softplus_f32(acc[u][v][2] + bs.z), softplus_f32(acc[u][v][3] + bs.w));
                *reinterpret_cast<uint2 *>(delta + tok * D + c) = pk;
            }
        }
    }
}

}  // namespace jscan
