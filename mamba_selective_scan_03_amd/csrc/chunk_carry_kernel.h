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
//
// The walk is itself split in two levels, so that no thread runs a long serial chain of
// memory reads: the segments form kGroups consecutive groups; each group's maps compose into
// one affine map h -> P h + H (P the product of its decays); a group's starting state is
// h0 carried through the maps of the groups before it; and each group then walks its own
// segments from that state.
#pragma once

#include "scan_update.h"

namespace jscan {

namespace carry {
constexpr int kGroups = 16;   // segment groups per sequence, one wave each
constexpr int kPairs = 64;    // (channel, state) pairs per work-group, one per lane
constexpr int kBlock = 16;    // segments whose inputs a thread holds in registers at once
constexpr int kThreads = kGroups * kPairs;
}  // namespace carry

// Work-group: kGroups waves x kPairs lanes; lane p of wave g handles pair i = blockIdx.x *
// kPairs + p, i = (b * D + d) * N + n, and segment group g of sequence b.  hbuf[row][D][N]
// holds h_loc on entry and h_in on exit (row = b * n_seg + s); dsum[row][D] holds the
// segments' delta sums.
__global__ __launch_bounds__(carry::kThreads) void chunk_carry_kernel(float *__restrict__ hbuf,
                                                                      const float *__restrict__ dsum,
                                                                      const float *__restrict__ A,
                                                                      const float *__restrict__ h0, int64_t count,
                                                                      int D, int n_seg) {
    using namespace carry;
    __shared__ float lds_p[kGroups][kPairs], lds_h[kGroups][kPairs];
    const int g = threadIdx.x / kPairs, p = threadIdx.x % kPairs;
    const int64_t i = (int64_t)blockIdx.x * kPairs + p;
    const bool live = i < count;   // every thread reaches the barrier
    const int64_t ic = live ? i : count - 1;
    const int n = (int)(ic & (kDState - 1));
    const int64_t bd = ic / kDState;
    const int d = (int)(bd % D);
    const int64_t b = bd / D;
    const float a2 = scaled_A(A[(int64_t)d * kDState + n]);
    const int per = (n_seg + kGroups - 1) / kGroups;
    const int s_begin = min(g * per, n_seg), s_end = min(s_begin + per, n_seg);

    // decays and h_loc of segments s0 .. s0 + kBlock - 1 of this group (clamped reads)
    float e[kBlock], hl[kBlock];
    auto load = [&](int s0) {
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            const int64_t row = b * n_seg + min(s0 + j, n_seg - 1);
            hl[j] = hbuf[(row * D + d) * kDState + n];
            e[j] = dsum[row * D + d];
        }
#pragma unroll
        for (int j = 0; j < kBlock; ++j) e[j] = decay(e[j], a2);
    };

    // 1. the group's composed map h -> P h + H
    float P = 1.0f, H = 0.0f;
    for (int s0 = s_begin; s0 < s_end; s0 += kBlock) {
        load(s0);
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            if (s0 + j < s_end) {
                P = e[j] * P;
                H = __builtin_fmaf(e[j], H, hl[j]);
            }
        }
    }
    lds_p[g][p] = P;
    lds_h[g][p] = H;
    __syncthreads();

    // 2. the group's starting state: h0 through the maps of the groups before it
    float h = (h0 && live) ? h0[i] : 0.0f;
    for (int g2 = 0; g2 < g; ++g2) h = __builtin_fmaf(lds_p[g2][p], h, lds_h[g2][p]);

    // 3. the group's own segments, from that state (inputs still in registers when the group
    // has at most kBlock segments)
    for (int s0 = s_begin; s0 < s_end; s0 += kBlock) {
        if (per > kBlock) load(s0);
#pragma unroll
        for (int j = 0; j < kBlock; ++j) {
            if (s0 + j < s_end) {
                if (live) hbuf[((b * n_seg + s0 + j) * D + d) * kDState + n] = h;
                h = __builtin_fmaf(e[j], h, hl[j]);
            }
        }
    }
}

inline void launch_chunk_carry(float *hbuf, const float *dsum, const float *A, const float *h0, int64_t count, int D,
                               int n_seg, hipStream_t stream) {
    const int64_t blocks = (count + carry::kPairs - 1) / carry::kPairs;
    hipLaunchKernelGGL(chunk_carry_kernel, dim3((unsigned)blocks), dim3(carry::kThreads), 0, stream, hbuf, dsum, A, h0,
                       count, D, n_seg);
}

}  // namespace jscan
