// prefill_rows_kernel.h - prefill for long sequences at small batch (the Jamba prefill
// shape: batch 1, D = 8192, N = 16, 4K-256K tokens).
//
// Why this mapping.  Each (channel, state) pair is a chain of L dependent updates.  Keeping
// the final state bit-identical to the decode step means every chain must be walked token
// by token in one lane, so all parallelism comes from batch * D * 16 chains: 131072 at
// batch 1.  That is 64 chains per SIMD on a 256-CU chip, so a lane carries G = 2 states and
// every SIMD runs exactly one wave.
//
// Lane layout.  A wave is 4 rows of 16 lanes.  Lane c of a row owns channel c of a 16-channel
// group; row r owns the state pair n = 8*sh + 2*r + {0,1}, where sh picks one half of the
// states.  Two waves (sh = 0, 1) cover all 16 states of one 16-channel group, and a
// 256-thread workgroup covers 32 channels (two groups).
//   * B_t[n] and C_t[n] are the same for all 16 lanes of a row.  A register holds 16
//     consecutive tokens' values of one state (lane c = token c), and the DPP row broadcast
//     (row_newbcast:k) hands token k's value to the whole row inside the multiply.  No extra
//     instruction is issued.
//   * delta_t[d] and delta_t[d] * x_t[d] are per lane (per channel).  The workgroup converts
//     each tile once into fp32 pairs in LDS, and every row reads them as a broadcast.
//   * y_t[d] = sum over 16 states = 2 states in-lane, 4 rows in-wave (two permlane swap
//     stages), then 2 waves through LDS.  The last stage is fused with the bf16 conversion
//     and a coalesced row store.
//
// Pipeline.  Tokens go in tiles of 64.  While tile k is computed, tile k+1 sits in LDS
// (converted) and tile k+2 is in flight from HBM into registers.  One workgroup barrier per
// tile orders the double-buffered LDS tiles and the double-buffered y exchange buffer.
// A ragged last tile is padded with identity tokens (delta = 0, x = -0, B = C = 0): they
// leave every state bit-identical (decay 2^0 = 1, input term -0) and their y is not stored.
#pragma once

#include "scan_update.h"

namespace jscan {

namespace rows {
constexpr int kT = 64;          // tokens per tile
constexpr int kCh = 32;         // channels per workgroup
constexpr int kThreads = 256;   // 4 waves
constexpr int kBcStride = kT + 8;   // LDS row length of the [n][token] B/C tiles (bank spread)
constexpr int kYStride = kCh + 8;   // LDS row length of the [token][channel] y exchange
// LDS (floats): delta*x/delta pairs [kT/2][kCh][4], B and C [16][kBcStride], y [2][kT][kYStride]
constexpr int kDxSize = kT / 2 * kCh * 4;
constexpr int kBcSize = kDState * kBcStride;
constexpr int kYSize = 2 * kT * kYStride;
}  // namespace rows

// Four consecutive elements from global memory as fp32 (bf16: one 8-byte load).
template <typename E> struct Vec4;
template <> struct Vec4<BF16> {
    using raw = uint2;
    static __device__ __forceinline__ raw load(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
    static __device__ __forceinline__ raw neg_zero() { return make_uint2(0x80008000u, 0x80008000u); }
    static __device__ __forceinline__ raw zero() { return make_uint2(0u, 0u); }
    static __device__ __forceinline__ void widen(raw r, float *f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    }
};
template <> struct Vec4<F32> {
    using raw = float4;
    static __device__ __forceinline__ raw load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
    static __device__ __forceinline__ raw neg_zero() { return make_float4(-0.0f, -0.0f, -0.0f, -0.0f); }
    static __device__ __forceinline__ raw zero() { return make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
    static __device__ __forceinline__ void widen(raw r, float *f) { f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w; }
};

// Registers holding one tile's share of raw inputs for one thread.
template <typename E> struct TileRegs {
    typename Vec4<E>::raw x[2], dl[2];   // tokens 2p and 2p+1, channels 4q..4q+3
    typename Vec4<E>::raw bc[2];         // B (threads 0-127) or C (128-255): one token, 8 states
};

// DPP row broadcast of lane k of each 16-lane row (row_newbcast:k).
template <int k> __device__ __forceinline__ float row_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + k, 0xF, 0xF, true));
}

typedef unsigned jscan_u2v __attribute__((vector_size(8)));
// (v, w) -> v = [v.lanes 0-31, w.lanes 0-31], w = [v.lanes 32-63, w.lanes 32-63]
__device__ __forceinline__ void swap32(float &v, float &w) {
    jscan_u2v r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, w),
                                                   false, false);
    const unsigned long long q = __builtin_bit_cast(unsigned long long, r);
    v = __builtin_bit_cast(float, (unsigned)q);
    w = __builtin_bit_cast(float, (unsigned)(q >> 32));
}
// (v, w) -> v = [v.row0, w.row0, v.row2, w.row2], w = [v.row1, w.row1, v.row3, w.row3]
__device__ __forceinline__ void swap16(float &v, float &w) {
    jscan_u2v r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), __builtin_bit_cast(unsigned, w),
                                                   false, false);
    const unsigned long long q = __builtin_bit_cast(unsigned long long, r);
    v = __builtin_bit_cast(float, (unsigned)q);
    w = __builtin_bit_cast(float, (unsigned)(q >> 32));
}

// Sum of four tokens' partials over the 4 rows: returns a register whose row r holds the
// row-sum of token kRowToken[r] = {0, 2, 1, 3}[r], added as (row0 + row2) + (row1 + row3).
__device__ __forceinline__ float reduce_rows4(float p0, float p1, float p2, float p3) {
    swap32(p0, p1);
    swap32(p2, p3);
    float u01 = p0 + p1, u23 = p2 + p3;
    swap16(u01, u23);
    return u01 + u23;
}

template <typename E>
__device__ __forceinline__ void load_tile(TileRegs<E> &R, const typename E::store_t *xb,
                                          const typename E::store_t *db, const typename E::store_t *bcb,
                                          int64_t t0, int64_t L, int D, int tid) {
    const int p = tid >> 3, q = tid & 7;  // token pair p, channel quad q
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t t = t0 + 2 * p + j;
        if (t < L) {
            R.x[j] = Vec4<E>::load(xb + t * D + 4 * q);
            R.dl[j] = Vec4<E>::load(db + t * D + 4 * q);
        } else {
            R.x[j] = Vec4<E>::neg_zero();
            R.dl[j] = Vec4<E>::zero();
        }
    }
    const int tb = (tid & 127) >> 1, nb = (tid & 1) * 8;  // B/C: one token, 8 states
    const int64_t t = t0 + tb;
#pragma unroll
    for (int j = 0; j < 2; ++j)
        R.bc[j] = t < L ? Vec4<E>::load(bcb + t * kDState + nb + 4 * j) : Vec4<E>::zero();
}

template <typename E>
__device__ __forceinline__ void stage_tile(const TileRegs<E> &R, float *dx_s, float *bc_s, int tid) {
    const int p = tid >> 3, q = tid & 7;
    float xv[2][4], dv[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        Vec4<E>::widen(R.x[j], xv[j]);
        Vec4<E>::widen(R.dl[j], dv[j]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float4 v;
        v.x = delta_x(dv[0][c], xv[0][c]);
        v.y = dv[0][c];
        v.z = delta_x(dv[1][c], xv[1][c]);
        v.w = dv[1][c];
        *reinterpret_cast<float4 *>(dx_s + (p * rows::kCh + 4 * q + c) * 4) = v;
    }
    const int tb = (tid & 127) >> 1, nb = (tid & 1) * 8;
    float* dst = bc_s + (tid >= 128 ? rows::kBcSize : 0);
    float f[8];
    Vec4<E>::widen(R.bc[0], f);
    Vec4<E>::widen(R.bc[1], f + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[(nb + j) * rows::kBcStride + tb] = f[j];
}

template <typename E>
__global__ __launch_bounds__(rows::kThreads, 1) void prefill_rows_kernel(
    const typename E::store_t *__restrict__ x, const typename E::store_t *__restrict__ dl,
    const float *__restrict__ A, const typename E::store_t *__restrict__ B,
    const typename E::store_t *__restrict__ C, const float *__restrict__ h0,
    typename E::store_t *__restrict__ y, float *__restrict__ h_final, int64_t L, int D, int blocks_per_row,
    int xcd_stride) {
    __shared__ __attribute__((aligned(16))) float dx_s[2][rows::kDxSize];
    __shared__ __attribute__((aligned(16))) float bc_s[2][2 * rows::kBcSize];
    __shared__ __attribute__((aligned(16))) float y_s[2][rows::kYSize];

    // Consecutive channel blocks go to the same XCD (work-groups are dealt round-robin over
    // the 8 XCDs), so the two blocks sharing a 128-byte row segment share one L2.
    int wg = blockIdx.x;
    if (xcd_stride > 0) wg = (wg & 7) * xcd_stride + (wg >> 3);
    const int b = wg / blocks_per_row;
    const int d0 = (wg - b * blocks_per_row) * rows::kCh;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;
    const int cg = wave >> 1, sh = wave & 1;
    const int ch = 16 * cg + c;             // channel inside the block
    const int d = d0 + ch;
    const int n0 = 8 * sh + 2 * r;          // this lane's states n0, n0 + 1

    const float a2_0 = scaled_A(A[(int64_t)d * kDState + n0]);
    const float a2_1 = scaled_A(A[(int64_t)d * kDState + n0 + 1]);
    float h_0 = 0.0f, h_1 = 0.0f;
    if (h0) {
        const float2 hv = *reinterpret_cast<const float2 *>(h0 + ((int64_t)b * D + d) * kDState + n0);
        h_0 = hv.x;
        h_1 = hv.y;
    }

    const int64_t row = (int64_t)b * L;
    const typename E::store_t *xb = x + row * D + d0;
    const typename E::store_t *db = dl + row * D + d0;
    const typename E::store_t *bcb = (tid < 128 ? B : C) + row * kDState;
    typename E::store_t *yb = y + row * D + d0;

    const int ntiles = (int)((L + rows::kT - 1) / rows::kT);
    TileRegs<E> R;
    load_tile<E>(R, xb, db, bcb, 0, L, D, tid);
    stage_tile<E>(R, dx_s[0], bc_s[0], tid);
    if (ntiles > 1) load_tile<E>(R, xb, db, bcb, rows::kT, L, D, tid);
    __syncthreads();

    for (int k = 0; k < ntiles; ++k) {
        const int cur = k & 1, nxt = cur ^ 1;
        // (a) tile k+1: registers -> LDS;  (b) tile k+2: HBM -> registers
        if (k + 1 < ntiles) {
            stage_tile<E>(R, dx_s[nxt], bc_s[nxt], tid);
            if (k + 2 < ntiles) load_tile<E>(R, xb, db, bcb, (int64_t)(k + 2) * rows::kT, L, D, tid);
        }
        // (c) the scan over tile k
        const float *dxs = dx_s[cur];
        const float *Bs = bc_s[cur];
        const float *Cs = bc_s[cur] + rows::kBcSize;
        float *ys = y_s[cur] + sh * rows::kT * rows::kYStride;
#pragma unroll 1
        for (int grp = 0; grp < rows::kT / 16; ++grp) {
            const int tg = grp * 16;
            // token tg + c of this row's two states; broadcast per token below
            const float Bt0 = Bs[n0 * rows::kBcStride + tg + c];
            const float Bt1 = Bs[(n0 + 1) * rows::kBcStride + tg + c];
            const float Ct0 = Cs[n0 * rows::kBcStride + tg + c];
            const float Ct1 = Cs[(n0 + 1) * rows::kBcStride + tg + c];
            float P[16];
#define JSCAN_TOKEN(TAU)                                                                         \
    {                                                                                            \
        const float4 v = *reinterpret_cast<const float4 *>(dxs + (((tg + TAU) >> 1) * rows::kCh + ch) * 4); \
        const float dxv = ((TAU) & 1) ? v.z : v.x;                                               \
        const float dv = ((TAU) & 1) ? v.w : v.y;                                                \
        h_0 = advance(h_0, dv, a2_0, dxv, row_bcast<TAU>(Bt0));                                  \
        h_1 = advance(h_1, dv, a2_1, dxv, row_bcast<TAU>(Bt1));                                  \
        P[TAU] = __builtin_fmaf(row_bcast<TAU>(Ct1), h_1, row_bcast<TAU>(Ct0) * h_0);           \
    }
            JSCAN_TOKEN(0) JSCAN_TOKEN(1) JSCAN_TOKEN(2) JSCAN_TOKEN(3)
            JSCAN_TOKEN(4) JSCAN_TOKEN(5) JSCAN_TOKEN(6) JSCAN_TOKEN(7)
            JSCAN_TOKEN(8) JSCAN_TOKEN(9) JSCAN_TOKEN(10) JSCAN_TOKEN(11)
            JSCAN_TOKEN(12) JSCAN_TOKEN(13) JSCAN_TOKEN(14) JSCAN_TOKEN(15)
#undef JSCAN_TOKEN
            // rows -> one register per 4 tokens; row r holds token 4j + {0,2,1,3}[r]
            const int rt = (r == 1) ? 2 : (r == 2) ? 1 : r;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float s = reduce_rows4(P[4 * j], P[4 * j + 1], P[4 * j + 2], P[4 * j + 3]);
                ys[(tg + 4 * j + rt) * rows::kYStride + ch] = s;
            }
        }
        __syncthreads();
        // (d) add the two state halves, round to the output dtype, store coalesced rows
        {
            const int t = tid >> 2, c8 = (tid & 3) * 8;
            const float *y0 = y_s[cur] + t * rows::kYStride + c8;
            const float *y1 = y0 + rows::kT * rows::kYStride;
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; j += 4) {
                const float4 u = *reinterpret_cast<const float4 *>(y0 + j);
                const float4 w = *reinterpret_cast<const float4 *>(y1 + j);
                o[j] = u.x + w.x; o[j + 1] = u.y + w.y; o[j + 2] = u.z + w.z; o[j + 3] = u.w + w.w;
            }
            const int64_t tt = (int64_t)k * rows::kT + t;
            if (tt < L) {
                typename E::store_t *dst = yb + tt * D + c8;
                if constexpr (sizeof(typename E::store_t) == 2) {
                    uint4 pk;
                    pk.x = pack_bf16x2(o[0], o[1]); pk.y = pack_bf16x2(o[2], o[3]);
                    pk.z = pack_bf16x2(o[4], o[5]); pk.w = pack_bf16x2(o[6], o[7]);
                    *reinterpret_cast<uint4 *>(dst) = pk;
                } else {
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                    *reinterpret_cast<float4 *>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
                }
            }
        }
    }
    *reinterpret_cast<float2 *>(h_final + ((int64_t)b * D + d) * kDState + n0) = make_float2(h_0, h_1);
}

// The row-mapped kernel needs whole 32-channel blocks; it is the better choice while
// batch * D is too small for one lane per channel to fill the chip.
inline bool rows_kernel_applies(int64_t batch, int64_t D) { return D % rows::kCh == 0 && batch * D <= 65536; }

template <typename E>
bool launch_prefill_rows(const typename E::store_t *x, const typename E::store_t *dl, const float *A,
                         const typename E::store_t *B, const typename E::store_t *C, const float *h0,
                         typename E::store_t *y, float *h_final, int64_t batch, int64_t L, int D,
                         hipStream_t stream) {
    const int blocks_per_row = D / rows::kCh;
    const int64_t blocks = batch * blocks_per_row;
    const int xcd_stride = (blocks % 8 == 0) ? (int)(blocks / 8) : 0;
    hipLaunchKernelGGL(prefill_rows_kernel<E>, dim3((unsigned)blocks), dim3(rows::kThreads), 0, stream, x, dl, A, B,
                       C, h0, y, h_final, L, D, blocks_per_row, xcd_stride);
    return true;
}

}  // namespace jscan
