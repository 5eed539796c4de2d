// project_kernels.h - the producer side of the scan: delta, B and C computed from x.
//
// The notes page ("Jamba: A Hybrid Transformer-Mamba Language Model", section "Mamba layer")
// has the scan's parameters depend on the input, B_t, C_t, delta_t = f(x_t), and applies
// RMSNorm inside the Jamba Mamba layer.  f is taken as the selective projection of Mamba-1:
//     [d_low | B | C] = W_x x_t                       (W_x: (R + 2N) x D, R the rank of delta)
//     d_low, B, C each RMS-normalised over its own width and scaled by a learned gain
//     delta_t = softplus(W_dt d_low + b_dt)          (W_dt: D x R, b_dt: D)
// Both products are dense contractions, so they run on the matrix cores: bf16 operands,
// fp32 accumulation (v_mfma_f32_16x16x32_bf16, layout in mfma_common.h), with the
// normalisation and the softplus applied to the fp32 accumulators before the single rounding
// to bf16.  Every matrix is stored with k fastest, so both operands are 16-byte loads: x is
// [M][D], W_x is [R + 2N][D], d_low is [M][R] and W_dt is [D][R] (the [out][in] layout of a
// linear layer).
#pragma once

#include "mfma_common.h"

namespace jscan {

namespace proj {
constexpr int kRowsX = 128;   // x-projection rows (tokens) per work-group: 4 waves x 32
constexpr int kTileDt = 128;  // delta-projection tile: 128 channels x 128 tokens, 4 waves of 64 x 64
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

// x projection: one work-group = 128 rows (tokens) x all R + 2N output columns, eight waves in
// a 4 x 2 grid: wave (wr, wc) owns rows 32 wr .. 32 wr + 31 (two 16-row tiles) and the half
// wc of the CT = R / 16 + 2 column tiles (d_low's R / 16 tiles, then one each of B and C).
// K (= D) goes in stages of 64: each stage's x tile [128][64] and W_x tile [16 CT][64] are
// loaded by all 512 threads into registers two stages ahead, then written to LDS (double-
// buffered) for the waves' MFMA operand reads.  LDS rows are padded to 72 bf16 (144 bytes),
// so the 16 rows one operand read touches fall on distinct banks.  Two waves per SIMD, and a
// register budget that keeps the accumulators in place, let one wave's operand reads and
// MFMAs overlap the other's.
namespace proj {
constexpr int kStageK = 64;          // K per stage
constexpr int kLdsRow = 72;          // bf16 per LDS row (64 + 8 padding)
constexpr int kXThreads = 512;       // threads of an x-projection work-group
}

// (ext_vector_type, not HIP's uint4 struct: copies of the struct type become memcpys that
// keep the whole set in scratch memory)
template <int CT> struct XprojRegs {
    static constexpr int kW = (16 * CT * 8 + proj::kXThreads - 1) / proj::kXThreads;
    u32x4_t xr[2];          // x: 128 rows x 8 chunks of 16 bytes = 1024 chunks, 2 per thread
    u32x4_t wr[kW];         // W_x: 16 CT rows x 8 chunks; the last one only in some waves
};

// Whether W_x chunk tid + 512 j exists.  16 CT * 8 chunks is a multiple of 64, so the answer is
// the same for a whole wave; it is taken from the wave's first lane to make that visible.
template <int CT>
__device__ __forceinline__ bool xproj_w_chunk(int j, int tid) {
    return __builtin_amdgcn_readfirstlane(tid) + proj::kXThreads * j < 16 * CT * 8;
}

template <int CT>
__device__ __forceinline__ void xproj_load(XprojRegs<CT> &g, const uint16_t *x, const uint16_t *w, int64_t row_base,
                                           int64_t M, int D, int k0, int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = tid + proj::kXThreads * j, r = i >> 3, part = i & 7;
        g.xr[j] = *reinterpret_cast<const u32x4_t *>(x + min(row_base + r, M - 1) * D + k0 + 8 * part);
    }
    // every lane loads (a missing chunk re-reads the last one): a load under a branch would be
    // waited for where the branch ends
#pragma unroll
    for (int j = 0; j < XprojRegs<CT>::kW; ++j) {
        const int i = min(tid + proj::kXThreads * j, 16 * CT * 8 - 1), r = i >> 3, part = i & 7;
        g.wr[j] = *reinterpret_cast<const u32x4_t *>(w + (int64_t)r * D + k0 + 8 * part);
    }
}

template <int CT>
__device__ __forceinline__ void xproj_store(const XprojRegs<CT> &g, uint16_t *xs, uint16_t *ws, int tid) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int i = tid + proj::kXThreads * j, r = i >> 3, part = i & 7;
        *reinterpret_cast<u32x4_t *>(xs + r * proj::kLdsRow + 8 * part) = g.xr[j];
    }
#pragma unroll
    for (int j = 0; j < XprojRegs<CT>::kW; ++j) {
        if (!xproj_w_chunk<CT>(j, tid)) continue;
        const int i = tid + proj::kXThreads * j, r = i >> 3, part = i & 7;
        *reinterpret_cast<u32x4_t *>(ws + r * proj::kLdsRow + 8 * part) = g.wr[j];
    }
}

// One stage's MFMAs of one wave: its 32 rows (two 16-row tiles) against its CH column tiles
// (from tile c0), two 32-wide k steps, operands read from LDS.  All of the stage's operands
// are requested before the first MFMA, so their LDS latency overlaps the matrix work.
template <int CH>
__device__ __forceinline__ void xproj_mfma(f32x4_t (&acc)[2][CH], const uint16_t *xs, const uint16_t *ws, int wr,
                                           int c0, int r16, int kq) {
    const uint16_t *xw = xs + (wr * 32 + r16) * proj::kLdsRow + kq;
    const uint16_t *wb = ws + (16 * c0 + r16) * proj::kLdsRow + kq;
    bf16x8_t a[2][2], b[2][CH];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        a[k][0] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(xw + 32 * k));
        a[k][1] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(xw + 16 * proj::kLdsRow + 32 * k));
#pragma unroll
        for (int c = 0; c < CH; ++c)
            b[k][c] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(wb + 16 * c * proj::kLdsRow + 32 * k));
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            acc[0][c] = mfma16(a[k][0], b[k][c], acc[0][c]);
            acc[1][c] = mfma16(a[k][1], b[k][c], acc[1][c]);
        }
}

template <int RT>
__global__ __launch_bounds__(proj::kXThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void xproj_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ g_d,
    const float *__restrict__ g_b, const float *__restrict__ g_c, uint16_t *__restrict__ d_low,
    uint16_t *__restrict__ Bo, uint16_t *__restrict__ Co, int64_t M, int D, float eps) {
    constexpr int CT = RT + 2;   // column tiles
    constexpr int CH = CT / 2;   // column tiles per wave
    static_assert(CT % 2 == 0 && CH <= RT, "each wave half must hold d_low tiles only or d_low then B and C");
    constexpr int kXs = proj::kRowsX * proj::kLdsRow, kWs = 16 * CT * proj::kLdsRow;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kXs];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][kWs];
    __shared__ float ssq[2][proj::kRowsX];   // d_low sums of squares of each column half, per row
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int wr = wave & 3, wc = wave >> 2, c0 = CH * wc;
    const int64_t row_base = (int64_t)blockIdx.x * proj::kRowsX;
    const int r16 = l & 15, kq = 8 * (l >> 4);
    const int stages = D / proj::kStageK;

    f32x4_t acc[2][CH];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Two named register sets (not an array) so that nothing is indexed at run time.
    XprojRegs<CT> Ga, Gb;
    xproj_load<CT>(Ga, x, w, row_base, M, D, 0, tid);
    if (stages > 1) xproj_load<CT>(Gb, x, w, row_base, M, D, proj::kStageK, tid);
    xproj_store<CT>(Ga, xs[0], ws[0], tid);
    if (stages > 2) xproj_load<CT>(Ga, x, w, row_base, M, D, 2 * proj::kStageK, tid);
    __syncthreads();

    // Stage s: MFMAs from LDS buffer s & 1; stage s+1 (in registers since stage s-2) goes to the
    // other buffer, and stage s+3 is requested into the registers it leaves.
    for (int s = 0; s < stages; s += 2) {
        xproj_mfma<CH>(acc, xs[0], ws[0], wr, c0, r16, kq);
        if (s + 1 < stages) {
            xproj_store<CT>(Gb, xs[1], ws[1], tid);
            if (s + 3 < stages) xproj_load<CT>(Gb, x, w, row_base, M, D, (s + 3) * proj::kStageK, tid);
        }
        __syncthreads();
        if (s + 1 < stages) {
            xproj_mfma<CH>(acc, xs[1], ws[1], wr, c0, r16, kq);
            if (s + 2 < stages) {
                xproj_store<CT>(Ga, xs[0], ws[0], tid);
                if (s + 4 < stages) xproj_load<CT>(Ga, x, w, row_base, M, D, (s + 4) * proj::kStageK, tid);
            }
            __syncthreads();
        }
    }

    // Epilogue.  Lane l holds rows 4 * (l / 16) + i of each 16-row tile, column 16 c + l % 16.
    // A row's sum of squares over d_low is a per-lane sum over the lane's d_low columns, then a
    // sum over the 16 lanes of the DPP row, then the two column halves' sums added through LDS
    // (half 0 + half 1, the same order in both waves).  B and C lie in half 1.
    constexpr int kDl1 = RT - CH;   // d_low tiles in half 1
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sd = 0.f;
            if (wc == 0) {
#pragma unroll
                for (int c = 0; c < CH; ++c) sd = __builtin_fmaf(acc[t][c][i], acc[t][c][i], sd);
            } else {
#pragma unroll
                for (int c = 0; c < kDl1; ++c) sd = __builtin_fmaf(acc[t][c][i], acc[t][c][i], sd);
            }
            sd = row16_sum(sd);
            if (r16 == 0) ssq[wc][wr * 32 + 16 * t + 4 * (l >> 4) + i] = sd;
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = wr * 32 + 16 * t + 4 * (l >> 4) + i;
            const int64_t row = row_base + rr;
            const float sd = ssq[0][rr] + ssq[1][rr];
            const float nd = __builtin_amdgcn_rsqf(sd * (1.0f / (16 * RT)) + eps);
            if (wc == 0) {
                if (row < M) {
#pragma unroll
                    for (int c = 0; c < CH; ++c)
                        d_low[row * (16 * RT) + 16 * c + r16] = f32_to_bf16_bits(acc[t][c][i] * nd * g_d[16 * c + r16]);
                }
            } else {
                const float vb = acc[t][kDl1][i], vc = acc[t][kDl1 + 1][i];
                const float sb = row16_sum(vb * vb), sc = row16_sum(vc * vc);
                const float nb = __builtin_amdgcn_rsqf(sb * (1.0f / 16) + eps);
                const float nc = __builtin_amdgcn_rsqf(sc * (1.0f / 16) + eps);
                if (row < M) {
#pragma unroll
                    for (int c = 0; c < kDl1; ++c)
                        d_low[row * (16 * RT) + 16 * (CH + c) + r16] =
                            f32_to_bf16_bits(acc[t][c][i] * nd * g_d[16 * (CH + c) + r16]);
                    Bo[row * kDState + r16] = f32_to_bf16_bits(vb * nb * g_b[r16]);
                    Co[row * kDState + r16] = f32_to_bf16_bits(vc * nc * g_c[r16]);
                }
            }
        }
    }
}

// Delta projection.  A work-group owns one 128-channel slice of W_dt and walks the token
// tiles t = g, g + G, g + 2G, ... (G groups per channel slice).  Each wave keeps its 64
// channels of W_dt as MFMA A operands in registers for the whole kernel; each 128-token tile
// of d_low is loaded by all 512 threads into registers one tile ahead and stored to LDS
// (double-buffered, rows padded to R + 8 bf16), from where the waves read their B operands
// (wave w of 8: channels 64 (w & 1) .. +63, tokens 32 (w >> 1) .. +31 of the tile).  Two waves
// per SIMD let one wave's softplus epilogue overlap the other's matrix work.  A = W_dt and
// B = d_low^T, so each lane's result is 4 consecutive channels of one token: the epilogue adds
// the bias, applies softplus and writes 8 bytes.
template <int R>
__global__ __launch_bounds__(512) void dtproj_kernel(const uint16_t *__restrict__ d_low, const uint16_t *__restrict__ w,
                                                     const float *__restrict__ bias, uint16_t *__restrict__ delta,
                                                     int64_t M, int D, int ch_tiles, int groups) {
    constexpr int KS = R / 32;                 // MFMA k steps
    constexpr int kRow = R + 8;                // LDS row (bf16), padded
    constexpr int kChunks = proj::kTileDt * R / 8 / 512;   // 16-byte chunks of a d_low tile per thread
    __shared__ __attribute__((aligned(16))) uint16_t ds[2][proj::kTileDt * kRow];
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int ct = blockIdx.x % ch_tiles, grp = blockIdx.x / ch_tiles;
    const int ch0 = ct * proj::kTileDt + 64 * (wave & 1);
    const int tw = 32 * (wave >> 1);           // this wave's token offset inside a tile
    const int r16 = l & 15, kq = 8 * (l >> 4);
    const int64_t tok_tiles = (M + proj::kTileDt - 1) / proj::kTileDt;

    bf16x8_t a[4][KS];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[u][ks] = load_frag(w + (int64_t)(ch0 + 16 * u + r16) * R + 32 * ks + kq);
    float4 bs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) bs[u] = *reinterpret_cast<const float4 *>(bias + ch0 + 16 * u + 4 * (l >> 4));

    u32x4_t pre[kChunks];
    auto load_tile = [&](int64_t t) {
#pragma unroll
        for (int j = 0; j < kChunks; ++j) {
            const int i = tid + 512 * j, r = i / (R / 8), part = i % (R / 8);
            pre[j] = *reinterpret_cast<const u32x4_t *>(d_low + min(t * proj::kTileDt + r, M - 1) * R + 8 * part);
        }
    };
    auto store_tile = [&](uint16_t *dst) {
#pragma unroll
        for (int j = 0; j < kChunks; ++j) {
            const int i = tid + 512 * j, r = i / (R / 8), part = i % (R / 8);
            *reinterpret_cast<u32x4_t *>(dst + r * kRow + 8 * part) = pre[j];
        }
    };

    int buf = 0;
    if (grp < tok_tiles) {
        load_tile(grp);
        store_tile(ds[0]);
    }
    __syncthreads();
    for (int64_t t = grp; t < tok_tiles; t += groups) {
        const int64_t tn = t + groups;
        if (tn < tok_tiles) load_tile(tn);      // in flight during this tile's MFMAs
        const uint16_t *bt = ds[buf] + (tw + r16) * kRow + kq;
        f32x4_t acc[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v) acc[u][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8_t b[2];
#pragma unroll
            for (int v = 0; v < 2; ++v)
                b[v] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(bt + 16 * v * kRow + 32 * ks));
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v) acc[u][v] = mfma16(a[u][ks], b[v], acc[u][v]);
        }
        // the next tile goes to LDS before this tile's stores are issued: waiting for its loads
        // then does not also wait for fresh stores (one counter covers both)
        if (tn < tok_tiles) store_tile(ds[buf ^ 1]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = ch0 + 16 * u + 4 * (l >> 4);
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int64_t tok = t * proj::kTileDt + tw + 16 * v + r16;
                if (tok < M) {
                    uint2 pk;
                    pk.x = pack_bf16x2(softplus_f32(acc[u][v][0] + bs[u].x), softplus_f32(acc[u][v][1] + bs[u].y));
                    pk.y = pack_bf16x2(softplus_f32(acc[u][v][2] + bs[u].z), softplus_f32(acc[u][v][3] + bs[u].w));
                    *reinterpret_cast<uint2 *>(delta + tok * D + c) = pk;
                }
            }
        }
        buf ^= 1;
        __syncthreads();
    }
}

}  // namespace jscan
