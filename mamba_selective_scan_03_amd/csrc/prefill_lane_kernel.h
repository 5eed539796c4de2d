// prefill_lane_kernel.h - the general prefill: one lane per (batch row, channel), all 16
// states of the channel in registers, tokens walked one after the other.
//
// It handles every shape the ABI accepts and serves those the row-mapped kernel does not
// (D not a multiple of 32).  A workgroup is one wave of 64 consecutive channels of one batch
// row, so the token's B_t and C_t rows are the same for the whole wave and are fetched once
// per wave through the scalar cache; x and delta are read as one coalesced row segment per
// token.
#pragma once

#include "scan_update.h"

namespace jscan {

// One lane scans one channel of one row (see Segments) from the row's initial state (zero
// when h0 is null), writing y and the row's final state.  With a scaled-identity
// A (AF), A is a[D] and the channel's one decay per token serves all 16 states; with a complex
// state, states 2k and 2k+1 form one complex state advanced by advance_complex().  With the
// exponential-trapezoidal rule (Trap, see trap_left_in) each token also takes in the previous
// token's input; the token before the row's first is (xp[row][D], bp[row][16]), or none.
template <typename E, AForm AF = AForm::Diagonal, bool kTrap = false>
__global__ __launch_bounds__(64) void prefill_lane_kernel(
    const typename E::store_t *__restrict__ x, const typename E::store_t *__restrict__ dl,
    const float *__restrict__ A, const typename E::store_t *__restrict__ B,
    const typename E::store_t *__restrict__ C, const float *__restrict__ h0,
    typename E::store_t *__restrict__ y, float *__restrict__ h_final, Segments sg, int D, int blocks_per_row,
    Trap tr) {
    const int vrow = blockIdx.x / blocks_per_row;
    const int d = (blockIdx.x - vrow * blocks_per_row) * 64 + threadIdx.x;
    if (d >= D) return;  // no cross-lane work below, so idle lanes may leave
    const RowSpan span = row_span(sg, vrow);

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
        h[n] = h0 ? h0[((int64_t)vrow * D + d) * kDState + n] : 0.0f;
    }
    const int64_t row = span.tok0;
    const typename E::store_t *xr = x + row * D + d;
    const typename E::store_t *dr = dl + row * D + d;
    typename E::store_t *yr = y + row * D + d;
    const typename E::store_t *Br = B + row * kDState;
    const typename E::store_t *Cr = C + row * kDState;

    using S = typename E::store_t;
    const S *lr = kTrap ? static_cast<const S *>(tr.lam) + row * D + d : nullptr;
    float xprev = 0.0f, bprev[kDState];
#pragma unroll
    for (int n = 0; n < kDState; ++n) bprev[n] = 0.0f;
    if (kTrap && tr.x_prev) {
        xprev = E::load(static_cast<const S *>(tr.x_prev) + (int64_t)vrow * D + d);
#pragma unroll
        for (int n = 0; n < kDState; ++n) bprev[n] = E::load(static_cast<const S *>(tr.B_prev) + vrow * kDState + n);
    }

    for (int64_t t = 0; t < span.len; ++t) {
        const float xv = E::load(xr + t * D), dv = E::load(dr + t * D);
        float dx = delta_x(dv, xv);
        if constexpr (kTrap) {   // left end point in; q replaces delta * x below
            const float lv = E::load(lr + t * D);
            const float pl = trap_left(dv, lv, xprev);
            dx = trap_right(dv, lv, xv);
            xprev = xv;
#pragma unroll
            for (int n = 0; n < kDState; ++n) {
                const float b = E::load(Br + t * kDState + n);
                h[n] = trap_left_in(h[n], pl, bprev[n]);
                bprev[n] = b;
            }
        }
        const float abar = kScalarA ? decay(dv, a2[0]) : 0.0f;
        float acc = 0.0f;
        if constexpr (kComplexA) {
#pragma unroll
            for (int k = 0; k < kDState / 2; ++k)
                advance_complex(h[2 * k], h[2 * k + 1], dv, ComplexA{a2[2 * k], a2[2 * k + 1]}, dx,
                                E::load(Br + t * kDState + 2 * k), E::load(Br + t * kDState + 2 * k + 1));
#pragma unroll
            for (int n = 0; n < kDState; ++n) acc = __builtin_fmaf(E::load(Cr + t * kDState + n), h[n], acc);
        } else {
#pragma unroll
            for (int n = 0; n < kDState; ++n) {
                const float b = E::load(Br + t * kDState + n);
                h[n] = kScalarA ? advance_decayed(h[n], abar, dx, b) : advance(h[n], dv, a2[n], dx, b);
                acc = __builtin_fmaf(E::load(Cr + t * kDState + n), h[n], acc);
            }
        }
        E::store(yr + t * D, acc);
    }
    if (span.state >= 0) {
#pragma unroll
        for (int n = 0; n < kDState; ++n) h_final[((int64_t)span.state * D + d) * kDState + n] = h[n];
    }
}

// Fills the final state when there are no tokens: copies h0, or writes zeros.
__global__ __launch_bounds__(256) void copy_state_kernel(const float *__restrict__ h0,
                                                         float *__restrict__ h_final, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) h_final[i] = h0 ? h0[i] : 0.0f;
}

}  // namespace jscan
