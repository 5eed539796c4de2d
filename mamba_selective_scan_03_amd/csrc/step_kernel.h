// step_kernel.h - one decode token for a batch of sequences (constant-memory decoding:
// only the previous state and the current token are read; lesson page "Jamba - Hybrid
// SSM-Transformer", section "SSM on one page").
//
// Mapping: one lane per (channel d, quad q) and kRows batch rows; the quad's four lanes hold
// states 4q..4q+3 of the channel, so a wave reads and writes 1 KiB of contiguous state per
// row with 16-byte accesses.  A lane loads its A quad once for all its rows and has all its
// rows' state in flight at once.  The state is read and written exactly once (in place), which
// makes the kernel HBM-bound: 128 of the ~134 bytes moved per (b, d) are state.  On MI355X it
// moves the state faster than the runtime's device-to-device copy does.
// y_t[d] is the sum over the quad: each lane adds its four C*h terms in increasing n, then
// two DPP quad exchanges add (q0+q1)+(q2+q3); every lane of the quad ends with the same sum.
#pragma once

#include "scan_update.h"

namespace jscan {

namespace step {
constexpr int kRows = 2;   // batch rows per lane
}

// The state is streamed: every element is read once and written once per token, and a
// 28-layer token step moves 7 GiB, far beyond the caches.  Non-temporal accesses keep it from
// evicting anything on its way through (about 9% faster than ordinary accesses here).
typedef float step_f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_state(const float *p) {
    const step_f4 v = __builtin_nontemporal_load(reinterpret_cast<const step_f4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_state(float *p, float4 v) {
    __builtin_nontemporal_store(step_f4{v.x, v.y, v.z, v.w}, reinterpret_cast<step_f4 *>(p));
}

// Four consecutive B or C values of one row as fp32.
template <typename E> struct Quad;
template <> struct Quad<BF16> {
    static __device__ __forceinline__ float4 load(const uint16_t *p) {
        const uint2 w = *reinterpret_cast<const uint2 *>(p);
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    }
};
template <> struct Quad<F32> {
    static __device__ __forceinline__ float4 load(const float *p) { return *reinterpret_cast<const float4 *>(p); }
};

// With a scaled-identity A (AF), A is a[D]: one decay per (row, channel) serves the quad.  With
// a complex state the quad is two complex states, (4q, 4q+1) and (4q+2, 4q+3).  With the
// exponential-trapezoidal rule (kTrap) the previous token's x (xp, rows like x) and B (bp, rows
// like B) enter as the step's left end point, weighted by 1 - lam (lam, rows like x).
template <typename E, AForm AF = AForm::Diagonal, bool kTrap = false>
__global__ __launch_bounds__(256) void step_kernel(float *__restrict__ h,
                                                   const typename E::store_t *__restrict__ x,
                                                   const typename E::store_t *__restrict__ dl,
                                                   const float *__restrict__ A,
                                                   const typename E::store_t *__restrict__ Bt,
                                                   const typename E::store_t *__restrict__ Ct,
                                                   typename E::store_t *__restrict__ y, int batch, int D,
                                                   int blocks_per_rows, int64_t ld_xd, int64_t ld_bc, int64_t ld_y,
                                                   const typename E::store_t *__restrict__ lam,
                                                   const typename E::store_t *__restrict__ xp,
                                                   const typename E::store_t *__restrict__ bp) {
    constexpr int NR = step::kRows;
    const int rg = blockIdx.x / blocks_per_rows;   // group of NR batch rows
    const int lane_in_row = (blockIdx.x - rg * blocks_per_rows) * 256 + threadIdx.x;
    if (lane_in_row >= D * 4) return;  // whole quads leave together (D * 4 is a multiple of 4)
    const int d = lane_in_row >> 2, q = lane_in_row & 3;

    constexpr bool kScalarA = AF == AForm::ScaledIdentity, kComplexA = AF == AForm::ComplexPairs;
    const float4 av = kScalarA ? make_float4(A[d], A[d], A[d], A[d])
                               : *reinterpret_cast<const float4 *>(A + (int64_t)d * kDState + q * 4);
    const float a0 = scaled_A(av.x), a1 = scaled_A(av.y), a2 = scaled_A(av.z), a3 = scaled_A(av.w);
    const ComplexA ca0 = complex_A(av.x, av.y), ca1 = complex_A(av.z, av.w);
    float4 hv[NR], bv[NR], cv[NR], bpv[NR];
    float xv[NR], dv[NR], lv[NR], xpv[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        // a missing last row re-reads the row before it and stores nothing
        const int b = min(rg * NR + j, batch - 1);
        hv[j] = load_state(h + ((int64_t)b * D + d) * kDState + q * 4);
        xv[j] = E::load(x + (int64_t)b * ld_xd + d);
        dv[j] = E::load(dl + (int64_t)b * ld_xd + d);
        bv[j] = Quad<E>::load(Bt + (int64_t)b * ld_bc + q * 4);
        cv[j] = Quad<E>::load(Ct + (int64_t)b * ld_bc + q * 4);
        if constexpr (kTrap) {
            lv[j] = E::load(lam + (int64_t)b * ld_xd + d);
            xpv[j] = E::load(xp + (int64_t)b * ld_xd + d);
            bpv[j] = Quad<E>::load(bp + (int64_t)b * ld_bc + q * 4);
        }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        const int b = rg * NR + j;
        float dx = delta_x(dv[j], xv[j]);
        if constexpr (kTrap) {   // left end point in, then the update with q in place of delta * x
            const float pl = trap_left(dv[j], lv[j], xpv[j]);
            dx = trap_right(dv[j], lv[j], xv[j]);
            hv[j].x = trap_left_in(hv[j].x, pl, bpv[j].x);
            hv[j].y = trap_left_in(hv[j].y, pl, bpv[j].y);
            hv[j].z = trap_left_in(hv[j].z, pl, bpv[j].z);
            hv[j].w = trap_left_in(hv[j].w, pl, bpv[j].w);
        }
        float4 hn;
        if constexpr (kComplexA) {
            hn = hv[j];
            advance_complex(hn.x, hn.y, dv[j], ca0, dx, bv[j].x, bv[j].y);
            advance_complex(hn.z, hn.w, dv[j], ca1, dx, bv[j].z, bv[j].w);
        } else if constexpr (kScalarA) {
            const float abar = decay(dv[j], a0);
            hn.x = advance_decayed(hv[j].x, abar, dx, bv[j].x);
            hn.y = advance_decayed(hv[j].y, abar, dx, bv[j].y);
            hn.z = advance_decayed(hv[j].z, abar, dx, bv[j].z);
            hn.w = advance_decayed(hv[j].w, abar, dx, bv[j].w);
        } else {
            hn.x = advance(hv[j].x, dv[j], a0, dx, bv[j].x);
            hn.y = advance(hv[j].y, dv[j], a1, dx, bv[j].y);
            hn.z = advance(hv[j].z, dv[j], a2, dx, bv[j].z);
            hn.w = advance(hv[j].w, dv[j], a3, dx, bv[j].w);
        }
        float p = cv[j].x * hn.x;
        p = __builtin_fmaf(cv[j].y, hn.y, p);
        p = __builtin_fmaf(cv[j].z, hn.z, p);
        p = __builtin_fmaf(cv[j].w, hn.w, p);
        // quad_perm [1,0,3,2] then [2,3,0,1]
        p = p + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, p), 0xB1, 0xF, 0xF, true));
        p = p + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, p), 0x4E, 0xF, 0xF, true));
        if (b < batch) {
            store_state(h + ((int64_t)b * D + d) * kDState + q * 4, hn);
            if (q == 0) E::store(y + (int64_t)b * ld_y + d, p);
        }
    }
}

}  // namespace jscan
