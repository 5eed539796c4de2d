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

// Two fp32 values rounded to bf16 and packed into one word, lo in the low half: one
// v_cvt_pk_bf16_f32, the same round-to-nearest-even as pack_bf16x2(), so the bits are equal.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

namespace proj {
constexpr int kRowsX = 256;   // x-projection rows (tokens) per work-group: 4 row groups x 64
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

// 16 bytes per lane from src straight into LDS at lds + 16 * lane (global_load_lds_dwordx4; lds
// is wave-uniform).  Written as a statement the compiler does not look into: given the
// builtin, it cannot tell which LDS array the load writes and waits for every such load in
// flight before later LDS writes, which undoes the prefetch.  Its caller orders the load with
// an explicit s_waitcnt and a barrier before any wave reads the data.  The address registers
// are read when the instruction issues; the instruction writes no register.  M0 (the LDS
// base of the load) is set here; nothing else in the library's kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// The same with the non-temporal hint, for data read once (it is not kept in the caches).
__device__ __forceinline__ void lds_dma16_nt(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt for an s_waitcnt that leaves `n` vector-memory operations outstanding (gfx9 encoding:
// low four bits and bits 14-15; expcnt and lgkmcnt at their maxima, so they do not wait).
template <int n> constexpr int vmcnt_only() { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// x projection: one work-group = 256 rows (tokens) x all R + 2N output columns.  Its waves form
// a (256 / 16 kRT) x 2 grid: wave (wr, wc) owns kRT 16-row tiles (rows 16 kRT wr ..) and the
// half wc of the CT = R / 16 + 2 column tiles (d_low's R / 16 tiles, then one each of B and
// C).  The launcher uses kRT = 4: eight waves, two per SIMD, each with 64 rows x 144 columns.
// Every work-group reads all of W_x, so the rows per work-group set how much W_x traffic the
// L2 serves per row of x: 256 rows halve it against 128 (with the loads below, 0.34 -> 0.25 ms
// on 64K x 8192, rank 256).
// K (= D) goes in stages of 64.  Each stage's x tile [256][64] and W_x tile [16 CT][64] go
// from memory straight into LDS (global_load_lds_dwordx4, 1 KB per wave instruction) and take
// no registers.  Two such stages fill the LDS, so a stage's loads are issued one stage before
// its MFMAs.  (Stages of 32 with three or four buffers, x still read in whole 128-byte lines,
// were slower, 0.31 ms: twice the barriers, each of which idles the matrix cores while a
// stage's first operands come from LDS.)  x is read once and loaded non-temporal.  A tile row
// (64 bf16, 128 bytes) holds its eight 16-byte chunks XOR-swizzled with (row / 2) % 8, so the
// 16 rows one operand read touches fall on distinct banks.
namespace proj {
constexpr int kStageK = 64;          // K per stage
constexpr int kXBufs = 2;            // stages in LDS: the one being read and the next in flight
constexpr int kXRowTiles = 4;        // 16-row tiles per wave (the launcher's layout)
constexpr int xproj_threads(int kRT) { return 2 * (kRowsX / (16 * kRT)) * 64; }
}

// LDS position (in 16-byte chunks) of chunk c of row r of a swizzled 64-wide tile.
__device__ __forceinline__ int swz64(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// One stage's MFMAs of one wave: its kRT row tiles (from row r0) against its CH column tiles
// (from tile c0), two 32-wide k steps, operands read from LDS.  Each k step's operands are
// requested before its first MFMA, so their LDS latency overlaps the matrix work (the other
// wave of the SIMD covers the rest); one k step at a time keeps the operands of 64 rows in
// the register budget of two waves per SIMD.
template <int kRT, int CH>
__device__ __forceinline__ void xproj_mfma(f32x4_t (&acc)[kRT][CH], const uint16_t *xs, const uint16_t *ws, int r0,
                                           int c0, int r16, int g4) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        bf16x8_t a[kRT], b[CH];
#pragma unroll
        for (int t = 0; t < kRT; ++t)
            a[t] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t *>(xs + 8 * swz64(r0 + 16 * t + r16, 4 * k + g4)));
#pragma unroll
        for (int c = 0; c < CH; ++c)
            b[c] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t *>(ws + 8 * swz64(16 * (c0 + c) + r16, 4 * k + g4)));
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int t = 0; t < kRT; ++t) acc[t][c] = mfma16(a[t], b[c], acc[t][c]);
    }
}

template <int RT, int kRT>
__global__ __launch_bounds__(proj::xproj_threads(kRT))
__attribute__((amdgpu_waves_per_eu(proj::xproj_threads(kRT) / 256, proj::xproj_threads(kRT) / 256))) void xproj_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, const float *__restrict__ g_d,
    const float *__restrict__ g_b, const float *__restrict__ g_c, uint16_t *__restrict__ d_low,
    uint16_t *__restrict__ Bo, uint16_t *__restrict__ Co, int64_t M, int D, float eps) {
    constexpr int CT = RT + 2;   // column tiles
    constexpr int CH = CT / 2;   // column tiles per wave
    static_assert(CT % 2 == 0 && CH <= RT, "each wave half must hold d_low tiles only or d_low then B and C");
    constexpr int kThreads = proj::xproj_threads(kRT), kWaves = kThreads / 64, kRowsW = 16 * kRT;
    constexpr int kXs = proj::kRowsX * proj::kStageK, kWs = 16 * CT * proj::kStageK;   // bf16 per stage
    constexpr int kXInst = kXs / 512 / kWaves;   // x DMA instructions per wave per stage
    constexpr int kWInstAll = kWs / 512;         // W DMA instructions per stage, dealt out to the
    constexpr int kWJ = (kWInstAll + kWaves - 1) / kWaves;   // waves in turn (at most kWJ each)
    static_assert(kXs % (512 * kWaves) == 0 && kWs % 512 == 0, "the tiles are whole wave instructions");
    __shared__ __attribute__((aligned(16))) uint16_t xs[proj::kXBufs][kXs];
    __shared__ __attribute__((aligned(16))) uint16_t ws[proj::kXBufs][kWs];
    __shared__ float ssq[2][proj::kRowsX];   // d_low sums of squares of each column half, per row
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    const int wr = wave >> 1, wc = wave & 1, c0 = CH * wc, r0 = kRowsW * wr;
    const int64_t row_base = (int64_t)blockIdx.x * proj::kRowsX;
    const int r16 = l & 15, g4 = l >> 4;
    const int stages = D / proj::kStageK;

    f32x4_t acc[kRT][CH];
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // This wave's loads of stage st into buffer b.  Wave instruction q of a tile fills its
    // chunk positions 64 q .. 64 q + 63; position P holds row P / 8's chunk (P % 8) ^ swizzle.
    // The x tile's instructions are split evenly over the waves; W instruction q goes to wave
    // q % kWaves.
    auto dma = [&](int st, int b) {
        const int k0 = st * proj::kStageK;
#pragma unroll
        for (int j = 0; j < kXInst; ++j) {
            const int q = wave * kXInst + j, P = q * 64 + l, r = P >> 3;
            const int c = (P & 7) ^ ((r >> 1) & 7);
            lds_dma16_nt(x + min(row_base + r, M - 1) * D + k0 + 8 * c,
                      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)(xs[b] + q * 512));
        }
#pragma unroll
        for (int j = 0; j < kWJ; ++j) {
            const int q = wave + kWaves * j;
            if (q < kWInstAll) {
                const int P = q * 64 + l, r = P >> 3;
                const int c = (P & 7) ^ ((r >> 1) & 7);
                lds_dma16(w + (int64_t)r * D + k0 + 8 * c,
                          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)(ws[b] + q * 512));
            }
        }
    };
    static_assert(proj::kXBufs == 2, "the loop below runs one stage ahead");
    dma(0, 0);
    for (int s = 0; s < stages; ++s) {
        __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());   // this wave's loads of stage s have landed
        __syncthreads();   // every wave's part of stage s is in; every wave is done with s - 1
        if (s + 1 < stages) dma(s + 1, (s + 1) & 1);
        xproj_mfma<kRT, CH>(acc, xs[s & 1], ws[s & 1], r0, c0, r16, g4);
    }

    // Epilogue.  Lane l holds rows 4 * (l / 16) + i of each 16-row tile, column 16 c + l % 16.
    // A row's sum of squares over d_low is a per-lane sum over the lane's d_low columns, then a
    // sum over the 16 lanes of the DPP row, then the two column halves' sums added through LDS
    // (half 0 + half 1, the same order in both waves).  B and C lie in half 1.
    constexpr int kDl1 = RT - CH;   // d_low tiles in half 1
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
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
            if (r16 == 0) ssq[wc][r0 + 16 * t + 4 * (l >> 4) + i] = sd;
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = r0 + 16 * t + 4 * (l >> 4) + i;
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

// Delta projection.  A work-group owns a 512-channel slice of W_dt: eight waves of 64 channels,
// each holding its channels of W_dt as MFMA A operands in registers for the whole kernel.  It
// walks the token tiles t = g, g + G, g + 2G, ... (G groups per channel slice, kDtTok tokens a
// tile), and every wave computes its 64 channels for all of a tile's tokens.  A = W_dt and
// B = d_low^T, so each lane's result is 4 consecutive channels of one token.  Every work-group
// reads the d_low tiles of its group from the L2, so the channels per work-group set that
// traffic (512 channels: 16 reads of d_low at D = 8192), and each token row of delta is written
// in runs of 1 KB.
//
// d_low tiles go from memory straight into LDS (global_load_lds_dwordx4: each wave
// instruction fills 1 KB of LDS, lane by lane), kDtBufs tiles deep, so a tile's loads are
// issued two tiles before it is used and take no registers.  (The three tile buffers are
// separate arrays so that each step of the loop, unrolled by three, names its own.)  Inside a
// tile row (one token's R values) the 16-byte chunks are stored XOR-swizzled with the row
// index, so the 16 rows one B-operand read touches fall on distinct banks.  Each wave's result
// (64 channels x 16 tokens) passes through a small LDS area of its own, which turns the MFMA
// layout (4 channels per lane) into whole 128-byte rows of delta: each lane then writes 16
// bytes.  Waves whose channels lie past D (D a multiple of 128, not of 512) load and wait like
// the others but compute and store nothing.
namespace proj {
constexpr int kDtCh = 512;    // channels per work-group: eight waves of 64
constexpr int kDtTok = 16;    // tokens per d_low tile
constexpr int kDtBufs = 3;    // d_low tiles in LDS: the one being read and two in flight
constexpr int kDtOutRow = 72; // bf16 per row of a wave's output area (64 channels + 8 padding)
}

template <int R>
__global__ __launch_bounds__(512) void dtproj_kernel(const uint16_t *__restrict__ d_low, const uint16_t *__restrict__ w,
                                                     const float *__restrict__ bias, uint16_t *__restrict__ delta,
                                                     int64_t M, int D, int ch_tiles, int groups) {
    constexpr int KS = R / 32;                                  // MFMA k steps
    constexpr int kRowChunks = R / 8;                           // 16-byte chunks per d_low row
    constexpr int kSwz = kRowChunks >= 16 ? 15 : kRowChunks - 1;
    constexpr int kDmaAll = proj::kDtTok * kRowChunks / 64;     // DMA wave instructions per tile
    constexpr int kSt = 2;                                      // global stores per wave per tile
    static_assert(proj::kDtTok * kRowChunks % 64 == 0 && kDmaAll >= 1 && kDmaAll <= 8,
                  "a tile is whole wave instructions, at most one per wave");
    __shared__ __attribute__((aligned(16))) uint16_t tiles0[proj::kDtTok * R];
    __shared__ __attribute__((aligned(16))) uint16_t tiles1[proj::kDtTok * R];
    __shared__ __attribute__((aligned(16))) uint16_t tiles2[proj::kDtTok * R];
    __shared__ __attribute__((aligned(16))) uint16_t outs[8][16 * proj::kDtOutRow];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
    // Work-groups go to the 8 XCDs in turn (work-group b to XCD b % 8).  The channel slices of a
    // token group are kept on one XCD, so each XCD's L2 fetches only its groups' d_low tiles
    // (when the group count is a multiple of 8; otherwise groups are spread over all XCDs).
    int ct = blockIdx.x % ch_tiles, grp = blockIdx.x / ch_tiles;
    if (groups % 8 == 0 && (int)gridDim.x == groups * ch_tiles) {
        const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
        grp = xcd * (groups / 8) + local / ch_tiles;
        ct = local % ch_tiles;
    }
    const int ch0 = ct * proj::kDtCh + 64 * wave;
    const bool active = ch0 < D;              // D is a multiple of 64: a wave is all in or all out
    const int chw = active ? ch0 : D - 64;    // an idle wave's (unused) operands: any valid rows
    const bool dma_wave = wave < kDmaAll;     // this wave issues one DMA instruction per tile
    const int r16 = l & 15, g4 = l >> 4, kq = 8 * g4;
    const int64_t tok_tiles = (M + proj::kDtTok - 1) / proj::kDtTok;
    const int count = grp < tok_tiles ? (int)((tok_tiles - grp + groups - 1) / groups) : 0;

    bf16x8_t a[4][KS];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[u][ks] = load_frag(w + (int64_t)(chw + 16 * u + r16) * R + 32 * ks + kq);
    float4 bs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) bs[u] = *reinterpret_cast<const float4 *>(bias + chw + 16 * u + 4 * g4);

    // This wave's share of tile i's loads into buf (instruction `wave` of the tile): LDS chunk
    // position P of the tile holds row P / kRowChunks, chunk (P % kRowChunks) ^ (row & kSwz).
    auto dma = [&](int i, uint16_t *buf) {
        if (dma_wave) {
            const int64_t t = grp + (int64_t)i * groups;
            const int P = wave * 64 + l;
            const int row = P / kRowChunks, c = (P % kRowChunks) ^ (row & kSwz);
            const int64_t tok = min(t * proj::kDtTok + row, M - 1);
            lds_dma16(d_low + tok * R + 8 * c,
                      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)(buf + wave * 64 * 8));
        }
    };
    // Wait for this wave's loads of tile j.  In issue order this wave's vector-memory operations
    // are tiles 0, 1 and 2's loads, then per step i: tile i + 3's loads and tile i's stores.
    // Tile j's loads (j >= 3) are issued in step j - 3, so before step j - 1 waits for them,
    // tile j - 3's stores, tile j + 1's loads and tile j - 2's stores come after them; tiles 1
    // and 2 have fewer operations behind them.  The last tile waits for everything (which also
    // covers groups of fewer than four tiles, and a partial tile's shorter store list, which is
    // only ever the last tile's).  Waves without loads wait for nothing: the loading waves wait
    // before the barrier that follows.
    auto wait_tile = [&](int j) {
        if (!dma_wave) return;
        if (j + 1 >= count) __builtin_amdgcn_s_waitcnt(vmcnt_only<0>());
        else if (j == 0 && count == 2) __builtin_amdgcn_s_waitcnt(vmcnt_only<1>());
        else if (j == 0) __builtin_amdgcn_s_waitcnt(vmcnt_only<2>());
        else if (!active) __builtin_amdgcn_s_waitcnt(vmcnt_only<1>());   // no stores
        else if (j == 1) __builtin_amdgcn_s_waitcnt(vmcnt_only<1>());
        else if (j == 2) __builtin_amdgcn_s_waitcnt(vmcnt_only<1 + kSt>());
        else __builtin_amdgcn_s_waitcnt(vmcnt_only<1 + 2 * kSt>());
    };
    // Tile i's products from rbuf: token r16 of the tile, channels 16 u + 4 g4 .. + 3.
    auto products = [&](const uint16_t *rbuf, f32x4_t (&acc)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = (4 * ks + g4) ^ (r16 & kSwz);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(rbuf + r16 * R + 8 * c));
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] = mfma16(a[u][ks], b, acc[u]);
        }
    };
    uint16_t *ow = outs[wave];
    // Tile i's rows out of this wave's output area: lane l writes 16 bytes (8 channels) of token
    // row l / 8 + 8 k, with the non-temporal hint (delta is not read again here).
    auto store = [&](int i) {
        const int64_t t = grp + (int64_t)i * groups;
#pragma unroll
        for (int k = 0; k < kSt; ++k) {
            const int orow = (l >> 3) + 8 * k, oc = l & 7;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ow + orow * proj::kDtOutRow + 8 * oc);
            const int64_t tok = t * proj::kDtTok + orow;
            if (tok < M) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(delta + tok * D + ch0 + 8 * oc));
        }
    };
    // Tile i + 1's products (from nbuf, into nxt) beside tile i's bias, softplus and bf16
    // rounding (from cur, into the output area), in KS slices: each slice issues one k step's
    // four MFMAs, then the vector work on 16 / KS of tile i's values while they run; the
    // scheduling barrier keeps the compiler from gathering the MFMAs back together.  The next k
    // step's operand read is issued a slice ahead.
    auto overlap = [&](const uint16_t *nbuf, f32x4_t (&nxt)[4], const f32x4_t (&cur)[4]) {
        constexpr int kPer = 16 / KS;   // values of tile i per slice (2, 4 or 8)
        uint32_t pw[8];                 // tile i's values packed in pairs, pair j = values 2j, 2j+1
        bf16x8_t b[2];
        auto read_b = [&](int ks) {
            const int c = (4 * ks + g4) ^ (r16 & kSwz);
            return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(nbuf + r16 * R + 8 * c));
        };
        auto value = [&](int j) {
            const int u = j >> 2, e = j & 3;
            const float bias = e == 0 ? bs[u].x : e == 1 ? bs[u].y : e == 2 ? bs[u].z : bs[u].w;
            return softplus_f32(cur[u][e] + bias);
        };
#pragma unroll
        for (int u = 0; u < 4; ++u) nxt[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        b[0] = read_b(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) b[(ks + 1) & 1] = read_b(ks + 1);
#pragma unroll
            for (int u = 0; u < 4; ++u) nxt[u] = mfma16(a[u][ks], b[ks & 1], nxt[u]);
#pragma unroll
            for (int j = kPer * ks; j < kPer * (ks + 1); j += 2) {
                const float v0 = value(j), v1 = value(j + 1);
                pw[j >> 1] = pack2_bf16(v0, v1);
                if ((j & 3) == 2)   // channel group u = j / 4 complete: 4 channels of token r16
                    *reinterpret_cast<uint2 *>(ow + r16 * proj::kDtOutRow + 16 * (j >> 2) + 4 * g4) =
                        make_uint2(pw[(j >> 1) - 1], pw[j >> 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Step i: tile i + 1's products beside tile i's epilogue; tile i + 3's loads go into dbuf
    // (tile i's buffer, whose products every wave finished in the step before the barrier).  The
    // last step's products read a buffer no load writes any more, and are not used.
    f32x4_t acc[2][4];
    auto step = [&](int i, const uint16_t *nbuf, uint16_t *dbuf, f32x4_t (&cur)[4], f32x4_t (&nxt)[4]) {
        if (i + 1 < count) {
            wait_tile(i + 1);
            __syncthreads();   // every wave's part of tile i + 1 is in; every wave is done with tile i's buffer
            if (i + 3 < count) dma(i + 3, dbuf);
        }
        if (!active) return;
        overlap(nbuf, nxt, cur);
        store(i);
    };
    if (count > 0) dma(0, tiles0);
    if (count > 1) dma(1, tiles1);
    if (count > 2) dma(2, tiles2);
    if (count > 0) {
        wait_tile(0);
        __syncthreads();
        if (active) products(tiles0, acc[0]);
    }
    for (int i = 0; i < count; i += 2 * proj::kDtBufs) {
        step(i, tiles1, tiles0, acc[0], acc[1]);
        if (i + 1 < count) step(i + 1, tiles2, tiles1, acc[1], acc[0]);
        if (i + 2 < count) step(i + 2, tiles0, tiles2, acc[0], acc[1]);
        if (i + 3 < count) step(i + 3, tiles1, tiles0, acc[1], acc[0]);
        if (i + 4 < count) step(i + 4, tiles2, tiles1, acc[0], acc[1]);
        if (i + 5 < count) step(i + 5, tiles0, tiles2, acc[1], acc[0]);
    }
}

}  // namespace jscan
