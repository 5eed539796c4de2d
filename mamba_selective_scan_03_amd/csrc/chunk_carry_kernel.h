// chunk_carry_kernel.h - the middle pass of the time-parallel prefill: the starting state of
// every segment of a sequence, from the segments' zero-start end states and delta sums.
//
// Over a run of tokens the S6 update h -> exp(delta A) h + delta B x (notes page "Jamba: A
// Hybrid Transformer-Mamba Language Model", section "Mamba layer") is affine in h, and the
// composition of the run's maps is h -> exp(A * sum(delta)) h + h_loc, where h_loc is the
// run's end state when it starts from zero.  Walking the segments in order therefore gives
//     h_in[0] = h0,   h_in[s+1] = exp(A * S[s]) * h_in[s] + h_loc[s].
// The decay uses the same exp2(delta * A2) form as a token update, with the segment's
// delta sum S[s] in place of one token's delta.
#pragma once

#include "scan_update.h"

namespace jscan {

// One thread per (sequence b, channel d, state n).  hbuf[row][D][N] holds h_loc on entry and
// h_in on exit (row = b * n_seg + s); dsum[row][D] holds the segments' delta sums.
__global__ __launch_bounds__(256) void chunk_carry_kernel(float *__restrict__ hbuf, const float *__restrict__ dsum,
                                                          const float *__restrict__ A, const float *__restrict__ h0,
                                                          int64_t count, int D, int n_seg) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (b * D + d) * N + n
    if (i >= count) return;
    const int n = (int)(i & (kDState - 1));
    const int64_t bd = i / kDState;
    const int d = (int)(bd % D);
    const int64_t b = bd / D;
    const float a2 = scaled_A(A[(int64_t)d * kDState + n]);
    float h = h0 ? h0[i] : 0.0f;
    for (int s = 0; s < n_seg; ++s) {
        const int64_t row = b * n_seg + s;
        const int64_t k = (row * D + d) * kDState + n;
        const float h_loc = hbuf[k];
        hbuf[k] = h;
        h = __builtin_fmaf(decay(dsum[row * D + d], a2), h, h_loc);
    }
}

}  // namespace jscan
