// step_kernel.h - one decode token for a batch of sequences (constant-memory decoding:
// only the previous state and the current token are read; lesson page "Jamba - Hybrid
// SSM-Transformer", section "SSM on one page").
//
// Mapping: one lane per (batch row b, channel d, quad q); the quad's four lanes hold
// states 4q..4q+3 of the channel, so a wave reads and writes 1 KiB of contiguous state with
// 16-byte accesses.  The state is read and written exactly once (in place), which makes
// the kernel HBM-bound: 128 of the ~134 bytes moved per (b, d) are state.
// y_t[d] is the sum over the quad: each lane adds its four C*h terms in increasing n, then
// two DPP quad exchanges add (q0+q1)+(q2+q3); every lane of the quad ends with the same sum.
#pragma once

#include "scan_update.h"

namespace jscan {

template <typename E>
__global__ __launch_bounds__(256) void step_kernel(float *__restrict__ h,
                                                   const typename E::store_t *__restrict__ x,
                                                   const typename E::store_t *__restrict__ dl,
                                                   const float *__restrict__ A,
                                                   const typename E::store_t *__restrict__ Bt,
                                                   const typename E::store_t *__restrict__ Ct,
                                                   typename E::store_t *__restrict__ y, int D,
                                                   int blocks_per_row, int64_t ld_xd, int64_t ld_bc) {
    const int b = blockIdx.x / blocks_per_row;
    const int lane_in_row = (blockIdx.x - b * blocks_per_row) * 256 + threadIdx.x;
    if (lane_in_row >= D * 4) return;  // whole quads leave together (D * 4 is a multiple of 4)
    const int d = lane_in_row >> 2, q = lane_in_row & 3;

    float *hp = h + ((int64_t)b * D + d) * kDState + q * 4;
    const float4 hv = *reinterpret_cast<const float4 *>(hp);
    const float4 av = *reinterpret_cast<const float4 *>(A + (int64_t)d * kDState + q * 4);
    const float xv = E::load(x + (int64_t)b * ld_xd + d);
    const float dv = E::load(dl + (int64_t)b * ld_xd + d);
    const typename E::store_t *bp = Bt + (int64_t)b * ld_bc + q * 4;
    const typename E::store_t *cp = Ct + (int64_t)b * ld_bc + q * 4;

    const float dx = delta_x(dv, xv);
    float4 hn;
    hn.x = advance(hv.x, dv, scaled_A(av.x), dx, E::load(bp + 0));
    hn.y = advance(hv.y, dv, scaled_A(av.y), dx, E::load(bp + 1));
    hn.z = advance(hv.z, dv, scaled_A(av.z), dx, E::load(bp + 2));
    hn.w = advance(hv.w, dv, scaled_A(av.w), dx, E::load(bp + 3));
    *reinterpret_cast<float4 *>(hp) = hn;

    float p = E::load(cp + 0) * hn.x;
    p = __builtin_fmaf(E::load(cp + 1), hn.y, p);
    p = __builtin_fmaf(E::load(cp + 2), hn.z, p);
    p = __builtin_fmaf(E::load(cp + 3), hn.w, p);
    // quad_perm [1,0,3,2] then [2,3,0,1]
    p = p + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, p), 0xB1, 0xF, 0xF, true));
    p = p + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, p), 0x4E, 0xF, 0xF, true));
    if (q == 0) E::store(y + (int64_t)b * ld_xd + d, p);
}

}  // namespace jscan
