// mimo_kernels.h - the multi-input, multi-output (MIMO) scan: each channel takes R inputs and
// gives R outputs, and B_t, C_t are N x R matrices shared by the channels (lesson page "Jamba -
// Hybrid SSM-Transformer", section "Mamba-3", item 3: matrix-valued projections in place of the
// per-feature scalar ones):
//     h_t[d][n] = Abar_t[d][n] h_{t-1}[d][n] + sum_r (delta_t[d] x_t[d][r]) B_t[n][r]
//     y_t[d][r] = sum_n C_t[n][r] h_t[d][n]
// Layouts: x, y [rows][D][R]; delta [rows][D]; B, C [rows][16][R].  The state is the
// single-input scan's [batch][D][16], so a decode step moves the same state bytes and does R
// times the arithmetic on them.  Every state element advances through mimo_input() and
// advance_input() (or advance_complex_input()), shared by the prefill and the step, so the
// prefill's final state is bit-identical to the step chain's; with R = 1 it is the
// single-input scan's bit for bit.
#pragma once

#include "scan_update.h"
#include "step_kernel.h"

namespace jscan {

// K consecutive elements as fp32 (K = 1, 2 or a multiple of 4; the address is aligned to the
// access: K elements of 2 or 4 bytes, at most 16 bytes per load).
template <typename E, int K> struct RowLoad;
template <int K> struct RowLoad<BF16, K> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&f)[K]) {
        if constexpr (K == 1) {
            f[0] = bf16_bits_to_f32(*p);
        } else if constexpr (K == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
            f[0] = bf16_lo(w);
            f[1] = bf16_hi(w);
        } else if constexpr (K % 8 == 0) {
#pragma unroll
            for (int i = 0; i < K / 8; ++i) {
                const uint4 w = reinterpret_cast<const uint4 *>(p)[i];
                f[8 * i + 0] = bf16_lo(w.x); f[8 * i + 1] = bf16_hi(w.x);
                f[8 * i + 2] = bf16_lo(w.y); f[8 * i + 3] = bf16_hi(w.y);
                f[8 * i + 4] = bf16_lo(w.z); f[8 * i + 5] = bf16_hi(w.z);
                f[8 * i + 6] = bf16_lo(w.w); f[8 * i + 7] = bf16_hi(w.w);
            }
        } else {
            static_assert(K == 4, "K must be 1, 2, 4 or a multiple of 8");
            const uint2 w = *reinterpret_cast<const uint2 *>(p);
            f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
        }
    }
};
template <int K> struct RowLoad<F32, K> {
    static __device__ __forceinline__ void load(const float *p, float (&f)[K]) {
        if constexpr (K == 1) {
            f[0] = *p;
        } else if constexpr (K == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(p);
            f[0] = v.x;
            f[1] = v.y;
        } else {
            static_assert(K % 4 == 0, "K must be 1, 2 or a multiple of 4");
#pragma unroll
            for (int i = 0; i < K / 4; ++i) {
                const float4 v = reinterpret_cast<const float4 *>(p)[i];
                f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
            }
        }
    }
};

// K consecutive fp32 values stored in the output dtype (same access sizes as RowLoad).
template <typename E, int K> struct RowStore;
template <int K> struct RowStore<BF16, K> {
    static __device__ __forceinline__ void store(uint16_t *p, const float (&f)[K]) {
        if constexpr (K == 1) {
            *p = f32_to_bf16_bits(f[0]);
        } else if constexpr (K == 2) {
            *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(f[0], f[1]);
        } else if constexpr (K % 8 == 0) {
#pragma unroll
            for (int i = 0; i < K / 8; ++i)
                reinterpret_cast<uint4 *>(p)[i] =
                    make_uint4(pack_bf16x2(f[8 * i], f[8 * i + 1]), pack_bf16x2(f[8 * i + 2], f[8 * i + 3]),
                               pack_bf16x2(f[8 * i + 4], f[8 * i + 5]), pack_bf16x2(f[8 * i + 6], f[8 * i + 7]));
        } else {
            static_assert(K == 4, "K must be 1, 2, 4 or a multiple of 8");
            *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
        }
    }
};
template <int K> struct RowStore<F32, K> {
    static __device__ __forceinline__ void store(float *p, const float (&f)[K]) {
        if constexpr (K == 1) {
            *p = f[0];
        } else if constexpr (K == 2) {
            *reinterpret_cast<float2 *>(p) = make_float2(f[0], f[1]);
        } else {
            static_assert(K % 4 == 0, "K must be 1, 2 or a multiple of 4");
#pragma unroll
            for (int i = 0; i < K / 4; ++i)
                reinterpret_cast<float4 *>(p)[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
        }
    }
};

// K consecutive elements at a wave-uniform address as fp32, read as 32-bit words so that the
// compiler can fetch them through the scalar cache (K even, the address 4-byte aligned).
template <typename E, int K> struct UniformRow;
template <int K> struct UniformRow<BF16, K> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&f)[K]) {
        static_assert(K % 2 == 0, "K must be even");
        const uint32_t *w = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
        for (int i = 0; i < K / 2; ++i) {
            f[2 * i] = bf16_lo(w[i]);
            f[2 * i + 1] = bf16_hi(w[i]);
        }
    }
};
template <int K> struct UniformRow<F32, K> {
    static __device__ __forceinline__ void load(const float *p, float (&f)[K]) {
#pragma unroll
        for (int i = 0; i < K; ++i) f[i] = p[i];
    }
};

// ---- prefill: one lane per (row, channel), all 16 states in registers ----------------------
// A work-group is one wave of 64 consecutive channels of one batch row, so B_t and C_t (N x R)
// are the same for the whole wave and are read through the scalar cache; the channel's R
// inputs and R outputs are one vector access each.  One lane carries a channel's whole state,
// so the R outputs need no exchange between lanes.  With the exponential-trapezoidal rule (kTrap;
// tr.lam like delta, tr.x_prev [rows][D][R], tr.B_prev [rows][16][R]) the previous token's input
// enters each step first (mimo_left_in); the lane keeps the previous token's x, and reads its B
// row again through the scalar cache.
template <typename E, AForm AF, int R, bool kTrap = false>
__global__ __launch_bounds__(64) void prefill_mimo_lane_kernel(
    const typename E::store_t *__restrict__ x, const typename E::store_t *__restrict__ dl,
    const float *__restrict__ A, const typename E::store_t *__restrict__ B, const typename E::store_t *__restrict__ C,
    const float *__restrict__ h0, typename E::store_t *__restrict__ y, float *__restrict__ h_final, int64_t L, int D,
    int blocks_per_row, Trap tr) {
    const int b = blockIdx.x / blocks_per_row;
    const int d = (blockIdx.x - b * blocks_per_row) * 64 + threadIdx.x;
    if (d >= D) return;   // no cross-lane work, so idle lanes may leave

    constexpr bool kScalarA = AF == AForm::ScaledIdentity, kComplexA = AF == AForm::ComplexPairs;
    float a2[kDState], h[kDState];
#pragma unroll
    for (int n = 0; n < kDState; ++n) {
        if constexpr (kComplexA) {   // (A2, turns) of complex entry n / 2
            const ComplexA ca = complex_A(A[(int64_t)d * kDState + (n & ~1)], A[(int64_t)d * kDState + (n | 1)]);
            a2[n] = (n & 1) ? ca.turns : ca.a2;
        } else {
            a2[n] = scaled_A(kScalarA ? A[d] : A[(int64_t)d * kDState + n]);
        }
        h[n] = h0 ? h0[((int64_t)b * D + d) * kDState + n] : 0.0f;
    }
    using S = typename E::store_t;
    const S *xr = x + ((int64_t)b * L * D + d) * R;
    const S *dr = dl + (int64_t)b * L * D + d;
    S *yr = y + ((int64_t)b * L * D + d) * R;
    const S *Br = B + (int64_t)b * L * kDState * R;
    const S *Cr = C + (int64_t)b * L * kDState * R;
    const S *lr = kTrap ? static_cast<const S *>(tr.lam) + (int64_t)b * L * D + d : nullptr;
    const S *Bp0 = (kTrap && tr.B_prev) ? static_cast<const S *>(tr.B_prev) + (int64_t)b * kDState * R : nullptr;
    float xprev[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xprev[r] = 0.0f;
    if (kTrap && tr.x_prev) RowLoad<E, R>::load(static_cast<const S *>(tr.x_prev) + ((int64_t)b * D + d) * R, xprev);

    for (int64_t t = 0; t < L; ++t) {
        float xv[R], dx[R];
        RowLoad<E, R>::load(xr + t * D * R, xv);
        const float dv = E::load(dr + t * D);
#pragma unroll
        for (int r = 0; r < R; ++r) dx[r] = delta_x(dv, xv[r]);
        // B_t and C_t in pairs of states (2R values), so that at most 4R of them are live at once
        const S *Bt = Br + t * kDState * R;
        const S *Ct = Cr + t * kDState * R;
        if constexpr (kTrap) {   // the left end point in first; q replaces delta * x below
            const float lv = E::load(lr + t * D);
            float pl[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                pl[r] = trap_left(dv, lv, xprev[r]);
                dx[r] = trap_right(dv, lv, xv[r]);
                xprev[r] = xv[r];
            }
            const S *Bp = t > 0 ? Bt - kDState * R : Bp0;   // the previous token's B row, or none
#pragma unroll
            for (int k = 0; k < kDState / 2; ++k) {
                float bp[2 * R];
                if (Bp) {
                    UniformRow<E, 2 * R>::load(Bp + 2 * k * R, bp);
                } else {
#pragma unroll
                    for (int i = 0; i < 2 * R; ++i) bp[i] = 0.0f;
                }
                h[2 * k] = mimo_left_in<R>(h[2 * k], pl, bp);
                h[2 * k + 1] = mimo_left_in<R>(h[2 * k + 1], pl, bp + R);
            }
        }
        const float abar = kScalarA ? decay(dv, a2[0]) : 0.0f;
#pragma unroll
        for (int k = 0; k < kDState / 2; ++k) {
            float bp[2 * R];
            UniformRow<E, 2 * R>::load(Bt + 2 * k * R, bp);
            if constexpr (kComplexA) {
                advance_complex_input(h[2 * k], h[2 * k + 1], dv, ComplexA{a2[2 * k], a2[2 * k + 1]},
                                      mimo_input<R>(dx, bp), mimo_input<R>(dx, bp + R));
            } else {
                h[2 * k] = advance_input(h[2 * k], kScalarA ? abar : decay(dv, a2[2 * k]), mimo_input<R>(dx, bp));
                h[2 * k + 1] =
                    advance_input(h[2 * k + 1], kScalarA ? abar : decay(dv, a2[2 * k + 1]), mimo_input<R>(dx, bp + R));
            }
        }
        float yo[R];
#pragma unroll
        for (int k = 0; k < kDState / 2; ++k) {
            float cp[2 * R];
            UniformRow<E, 2 * R>::load(Ct + 2 * k * R, cp);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                yo[r] = k == 0 ? cp[r] * h[0] : __builtin_fmaf(cp[r], h[2 * k], yo[r]);
                yo[r] = __builtin_fmaf(cp[R + r], h[2 * k + 1], yo[r]);
            }
        }
        RowStore<E, R>::store(yr + t * D * R, yo);
    }
#pragma unroll
    for (int n = 0; n < kDState; ++n) h_final[((int64_t)b * D + d) * kDState + n] = h[n];
}

// ---- decode step: one lane per (channel, quad of states) and two batch rows ----------------
// The mapping of the single-input step (step_kernel.h): the quad's four lanes hold states
// 4q..4q+3 of a channel, so the state is read and written once with 16-byte accesses.  A
// work-group's lanes all serve the same two batch rows, so their B and C rows (N x R each) are
// converted to fp32 once per work-group into LDS, one value per thread, and each lane reads its
// quad's R columns from there.  A lane forms its four input terms and its four C h products per
// output; two DPP quad exchanges sum each output over the quad, and lane q stores outputs q and
// q + 4, so the quad writes its R outputs as one contiguous run.  With the exponential-trapezoidal
// rule (kTrap) the previous token's x (xp, rows like x) and B (bp, rows like B, staged with B and
// C) enter first as the left end point (mimo_left_in), weighted by 1 - lam (rows like delta).
namespace mimo_step {
constexpr int kRows = 2;   // batch rows per lane
}
template <typename E, AForm AF, int R, bool kTrap = false>
__global__ __launch_bounds__(256) void step_mimo_kernel(float *__restrict__ h, const typename E::store_t *__restrict__ x,
                                                        const typename E::store_t *__restrict__ dl,
                                                        const float *__restrict__ A,
                                                        const typename E::store_t *__restrict__ Bt,
                                                        const typename E::store_t *__restrict__ Ct,
                                                        typename E::store_t *__restrict__ y, int batch, int D,
                                                        int blocks_per_rows, int64_t ld_x, int64_t ld_d,
                                                        int64_t ld_bc, int64_t ld_y,
                                                        const typename E::store_t *__restrict__ lam,
                                                        const typename E::store_t *__restrict__ xp,
                                                        const typename E::store_t *__restrict__ bp) {
    constexpr int NR = mimo_step::kRows;
    constexpr int kBC = kDState * R;                 // values of one B or C row
    constexpr int kW = kTrap ? 3 : 2;                // B, C (and the previous token's B)
    __shared__ __attribute__((aligned(16))) float bc_s[NR][kW][kBC];
    const int rg = blockIdx.x / blocks_per_rows;
    const int lane_in_row = (blockIdx.x - rg * blocks_per_rows) * 256 + threadIdx.x;
    const bool active = lane_in_row < D * 4;         // whole quads are active or not
    const int d = active ? lane_in_row >> 2 : 0, q = lane_in_row & 3;
    using S = typename E::store_t;

    // every row's state, x and delta requested first (the state with non-temporal accesses, as in
    // the single-input step), so that they are in flight while B and C are staged
    float4 h4[NR];
    float xv[NR][R], dv[NR], xpv[NR][R], lv[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        // a missing last row re-reads the row before it and stores nothing
        const int b = min(rg * NR + j, batch - 1);
        if (active) {
            h4[j] = load_state(h + ((int64_t)b * D + d) * kDState + q * 4);
            RowLoad<E, R>::load(x + (int64_t)b * ld_x + (int64_t)d * R, xv[j]);
            dv[j] = E::load(dl + (int64_t)b * ld_d + d);
            if constexpr (kTrap) {
                RowLoad<E, R>::load(xp + (int64_t)b * ld_x + (int64_t)d * R, xpv[j]);
                lv[j] = E::load(lam + (int64_t)b * ld_d + d);
            }
        }
    }
    for (int i = threadIdx.x; i < NR * kW * kBC; i += 256) {
        const int j = i / (kW * kBC), w = (i / kBC) % kW, k = i % kBC;
        const int b = min(rg * NR + j, batch - 1);
        bc_s[j][w][k] = E::load((w == 0 ? Bt : w == 1 ? Ct : bp) + (int64_t)b * ld_bc + k);
    }
    __syncthreads();
    if (!active) return;

    constexpr bool kScalarA = AF == AForm::ScaledIdentity, kComplexA = AF == AForm::ComplexPairs;
    const float4 av = kScalarA ? make_float4(A[d], A[d], A[d], A[d])
                               : *reinterpret_cast<const float4 *>(A + (int64_t)d * kDState + q * 4);
    const float a2v[4] = {scaled_A(av.x), scaled_A(av.y), scaled_A(av.z), scaled_A(av.w)};
    const ComplexA ca0 = complex_A(av.x, av.y), ca1 = complex_A(av.z, av.w);
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int b = rg * NR + j;
        float bq[4 * R], cq[4 * R], pq[4 * R];
#pragma unroll
        for (int i = 0; i < R; ++i) {   // the quad's rows 4q..4q+3 of B and C: 4R consecutive values
            const float4 vb = reinterpret_cast<const float4 *>(&bc_s[j][0][q * 4 * R])[i];
            const float4 vc = reinterpret_cast<const float4 *>(&bc_s[j][1][q * 4 * R])[i];
            bq[4 * i] = vb.x; bq[4 * i + 1] = vb.y; bq[4 * i + 2] = vb.z; bq[4 * i + 3] = vb.w;
            cq[4 * i] = vc.x; cq[4 * i + 1] = vc.y; cq[4 * i + 2] = vc.z; cq[4 * i + 3] = vc.w;
            if constexpr (kTrap) {
                const float4 vp = reinterpret_cast<const float4 *>(&bc_s[j][kW - 1][q * 4 * R])[i];
                pq[4 * i] = vp.x; pq[4 * i + 1] = vp.y; pq[4 * i + 2] = vp.z; pq[4 * i + 3] = vp.w;
            }
        }
        float hv[4] = {h4[j].x, h4[j].y, h4[j].z, h4[j].w};
        float dx[R];
#pragma unroll
        for (int r = 0; r < R; ++r) dx[r] = delta_x(dv[j], xv[j][r]);
        if constexpr (kTrap) {   // the left end point in first; q replaces delta * x below
            float pl[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                pl[r] = trap_left(dv[j], lv[j], xpv[j][r]);
                dx[r] = trap_right(dv[j], lv[j], xv[j][r]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = mimo_left_in<R>(hv[i], pl, pq + i * R);
        }
        if constexpr (kComplexA) {
            advance_complex_input(hv[0], hv[1], dv[j], ca0, mimo_input<R>(dx, bq), mimo_input<R>(dx, bq + R));
            advance_complex_input(hv[2], hv[3], dv[j], ca1, mimo_input<R>(dx, bq + 2 * R), mimo_input<R>(dx, bq + 3 * R));
        } else {
            const float abar = decay(dv[j], a2v[0]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hv[i] = advance_input(hv[i], kScalarA ? abar : decay(dv[j], a2v[i]), mimo_input<R>(dx, bq + i * R));
        }
        float p[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float s = cq[r] * hv[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) s = __builtin_fmaf(cq[i * R + r], hv[i], s);
            // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of the quad ends with the quad's sum
            s = s + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
            s = s + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
            p[r] = s;
        }
        if (b < batch) {
            store_state(h + ((int64_t)b * D + d) * kDState + q * 4, make_float4(hv[0], hv[1], hv[2], hv[3]));
            S *yp = y + (int64_t)b * ld_y + (int64_t)d * R;
#pragma unroll
            for (int r0 = 0; r0 < R; r0 += 4) {   // lane q stores output r0 + q
                if (r0 + q < R) {
                    float v = p[r0];
#pragma unroll
                    for (int k = 1; k < 4 && r0 + k < R; ++k) v = (q == k) ? p[r0 + k] : v;
                    E::store(yp + r0 + q, v);
                }
            }
        }
    }
}

}  // namespace jscan
