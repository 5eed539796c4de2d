// prefill_seg_lane_kernel.h - the two scan passes of the time-parallel prefill: one lane per
// (segment row, channel) with all 16 states of the channel in registers.
//
// Why this mapping.  The time-parallel prefill cuts each sequence into segments, so it can
// create as many independent rows as it needs.  With enough of them (several waves per SIMD) a
// lane can own a whole channel: B_t and C_t are then the same for every lane of the wave
// (one segment row, one token at a time) and reach the arithmetic as scalar (SGPR)
// operands, and the output's sum over the 16 states stays in the lane.  Measured on the
// MI355X, that removes the costliest parts of the row-mapped kernel's work per state
// element: the DPP broadcasts of B and C (1.5 FMA slots each) and the cross-lane sum over
// states (permlane swaps, about 3.6 slots each), and several waves per SIMD issue at several
// times the rate of one.  A state element then costs its arithmetic alone: the exponent
// product, the exponential, the input product and the state FMA (plus the output's share).
//
// Memory access.  x and delta are read per token as one coalesced row piece of the wave's 64
// channels, through buffer loads whose per-token offset is a scalar register, in two sets of
// eight tokens: one set is in flight while the other is consumed.  The token's B row (16
// values) is a scalar load issued one token ahead, right after the wait for the current
// token's row: scalar loads complete out of order, so a wait for one of them waits for all,
// and issuing the next token's load before that wait would expose its latency.  The C row is
// loaded at the same point for the current token; its 16 state updates cover the latency.
// y is written with buffer stores in the same addressing.
//
// The update of each state is advance(), the one definition every kernel uses.  In a
// sequence's first segment, which starts from the caller's state, the output sums the states
// in the order of the kernel the sequential prefill uses for the same D (kRowsOrder: the
// row-mapped kernel's pairs and halves when D is a multiple of 32), so that segment
// reproduces the sequential prefill bit for bit.  Other segments, and every segment when D is
// not a multiple of 32, sum with one fma per state in state order (7 fewer instructions a
// token than the pairs and halves).
#pragma once

#include <type_traits>

#include "scan_update.h"

namespace jscan {

namespace seglane {
constexpr int kSet = 8;                 // tokens of x and delta per register set
constexpr int kBlock = 2 * kSet;        // tokens per main-loop trip (both sets)
constexpr int kWavesPerSimd = 4;        // the register budget the kernel is compiled for
constexpr int kThreads = 256;           // work-group: four waves of 64 channels of one row
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer resource, gfx9 family
constexpr bool kTouch = true;           // bring B and C lines into the L2 a set ahead

// A raw buffer resource at `base` with no range limit: every offset the kernel forms stays
// inside its row (token indexes are clamped to the row before they become offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, kRsrcWord3);
}
}  // namespace seglane

// Buffer access of one element: the raw bits travel in a 32-bit register.
template <typename E> struct SegIO;
template <> struct SegIO<BF16> {
    static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, (int)so, 0);
    }
    static __device__ __forceinline__ float value(uint32_t bits) { return bf16_bits_to_f32(bits); }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, float v, uint32_t vo, uint32_t so) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, (int)vo, (int)so, 0);
    }
};
template <> struct SegIO<F32> {
    static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, (int)so, 0);
    }
    static __device__ __forceinline__ float value(uint32_t bits) { return __uint_as_float(bits); }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, float v, uint32_t vo, uint32_t so) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)vo, (int)so, 0);
    }
};

// One token's B (or C) row: raw words read through wave-uniform addresses (scalar loads), and
// their 16 values as fp32 (the bf16 halves are split by scalar shifts and masks at use).
template <typename E> struct BcRow;
template <> struct BcRow<BF16> {
    uint32_t w[kDState / 2];
    __device__ __forceinline__ void load(const uint16_t *p) {
        const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
        for (int k = 0; k < kDState / 2; ++k) w[k] = q[k];
    }
    __device__ __forceinline__ float operator[](int n) const {
        return (n & 1) ? bf16_hi(w[n >> 1]) : bf16_lo(w[n >> 1]);
    }
};
template <> struct BcRow<F32> {
    float w[kDState];
    __device__ __forceinline__ void load(const float *p) {
#pragma unroll
        for (int n = 0; n < kDState; ++n) w[n] = p[n];
    }
    __device__ __forceinline__ float operator[](int n) const { return w[n]; }
};

// Holds the wave until the scalar load into `w` (and with it every scalar load issued
// earlier) has arrived: the empty statement reads the register, so the compiler puts the
// wait for it here.
__device__ __forceinline__ void wait_scalar(uint32_t w) { asm volatile("" ::"s"(w)); }
__device__ __forceinline__ void wait_scalar(float w) { asm volatile("" ::"s"(w)); }

// y of one channel from its 16 states and the token's C row, in the row-mapped kernel's order:
// pairs (n0, n0 + 1) as fma(C[n0+1], h[n0+1], C[n0] h[n0]), within each half of the states
// (r0 + r2) + (r1 + r3), then the two halves.
template <typename E> __device__ __forceinline__ float contract_row(const float (&h)[kDState], const BcRow<E> &c) {
    float u[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n0 = 8 * sh + 2 * r;
            p[r] = __builtin_fmaf(c[n0 + 1], h[n0 + 1], c[n0] * h[n0]);
        }
        u[sh] = (p[0] + p[2]) + (p[1] + p[3]);
    }
    return u[0] + u[1];
}

// y of one channel in the per-lane kernel's order: one fma per state, states in order.
template <typename E> __device__ __forceinline__ float contract_seq(const float (&h)[kDState], const BcRow<E> &c) {
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < kDState; ++n) acc = __builtin_fmaf(c[n], h[n], acc);
    return acc;
}

// One lane scans one channel of one row (see Segments) from the row's initial state (zero
// when h0 is null).  A segment-summary launch (kSummary) writes no y; it writes the row's
// final state and the sum of the row's delta values to dsum[row][D].  A work-group is
// kThreads consecutive channels of one row; its waves share no data but the scalar cache.
// kRowsOrder picks the first segment's summation order (see the file comment).  Offsets are 32-bit:
// a token row is D * 4 <= 2^26 bytes and no offset spans more than 16 token rows.
template <typename E, bool kSummary, bool kRowsOrder>
__global__ __launch_bounds__(seglane::kThreads) __attribute__((amdgpu_waves_per_eu(seglane::kWavesPerSimd))) void
prefill_seg_lane_kernel(const typename E::store_t *__restrict__ x, const typename E::store_t *__restrict__ dl,
                        const float *__restrict__ A, const typename E::store_t *__restrict__ B,
                        const typename E::store_t *__restrict__ C, const float *__restrict__ h0,
                        typename E::store_t *__restrict__ y, float *__restrict__ h_final, float *__restrict__ dsum,
                        Segments sg, int D, int blocks_per_row) {
    using S = typename E::store_t;
    using IO = SegIO<E>;
    using seglane::kBlock;
    using seglane::kSet;
    const int vrow = blockIdx.x / blocks_per_row;
    const int d = (blockIdx.x - vrow * blocks_per_row) * seglane::kThreads + threadIdx.x;
    if (d >= D) return;   // no cross-lane work below, so idle lanes may leave
    const RowSpan span = row_span(sg, vrow);
    const int len = (int)span.len;   // a segment is shorter than 2^31 tokens (checked on the host)

    float a2[kDState], h[kDState];
#pragma unroll
    for (int n = 0; n < kDState; ++n) {
        a2[n] = scaled_A(A[(int64_t)d * kDState + n]);
        h[n] = h0 ? h0[((int64_t)vrow * D + d) * kDState + n] : 0.0f;
    }
    // row bases are wave-uniform; a lane's element is vo bytes on, a token rowb bytes on
    const S *xb = x + span.tok0 * D, *db = dl + span.tok0 * D;
    S *yb = y + span.tok0 * D;
    const S *Bb = B + span.tok0 * kDState, *Cb = C + span.tok0 * kDState;
    const uint32_t rowb = (uint32_t)D * (uint32_t)sizeof(S), vo = (uint32_t)d * (uint32_t)sizeof(S);

    // The scan of the row, with the output summed in the rows kernel's order (kRo) or in state
    // order.  One token: the state update and (unless kSummary) the output.
    float dacc = 0.0f;
    auto scan = [&](auto rows_order) {
        constexpr bool kRo = decltype(rows_order)::value;
        auto token = [&](float xv, float dv, const BcRow<E> &bc, const BcRow<E> &cc, __amdgpu_buffer_rsrc_t ry,
                         uint32_t so) {
            const float dx = delta_x(dv, xv);
#pragma unroll
            for (int n = 0; n < kDState; ++n) h[n] = advance(h[n], dv, a2[n], dx, bc[n]);
            if constexpr (kSummary)
                dacc += dv;
            else
                IO::store(ry, kRo ? contract_row<E>(h, cc) : contract_seq<E>(h, cc), vo, so);
        };

        // x and delta of kSet tokens from t0 (indexes past the row end re-read its last token,
        // and those values are never used), addressed from the clamped first token.  Before
        // them, one word of each 128-byte line of those tokens' B and C rows is read (the same
        // address in every lane), so that the scalar loads of the rows, kSet tokens later, hit
        // the L2.
        constexpr int kRowBytes = kDState * (int)sizeof(S);
        constexpr int kLines = kSet * kRowBytes / 128;
        constexpr int kTouches = seglane::kTouch ? (kSummary ? 1 : 2) * kLines : 0;
        uint32_t xr[2][kSet], dr[2][kSet], tq[2][kTouches > 0 ? kTouches : 1];
        auto fetch = [&](uint32_t(&xs)[kSet], uint32_t(&ds)[kSet], uint32_t(&tch)[kTouches > 0 ? kTouches : 1],
                         int t0) {
            const int tb = t0 < len ? t0 : len - 1;
            if constexpr (kTouches > 0) {
                const __amdgpu_buffer_rsrc_t rb = seglane::rsrc(Bb + (int64_t)tb * kDState);
                const __amdgpu_buffer_rsrc_t rc = seglane::rsrc(Cb + (int64_t)tb * kDState);
#pragma unroll
                for (int k = 0; k < kLines; ++k) {
                    const int t = t0 + k * (128 / kRowBytes) < len ? t0 + k * (128 / kRowBytes) : len - 1;
                    const uint32_t so = (uint32_t)(t - tb) * (uint32_t)kRowBytes;
                    tch[k] = __builtin_amdgcn_raw_buffer_load_b32(rb, 0, (int)so, 0);
                    if constexpr (!kSummary)
                        tch[kLines + k] = __builtin_amdgcn_raw_buffer_load_b32(rc, 0, (int)so, 0);
                }
            }
            const __amdgpu_buffer_rsrc_t rx = seglane::rsrc(xb + (int64_t)tb * D);
            const __amdgpu_buffer_rsrc_t rd = seglane::rsrc(db + (int64_t)tb * D);
#pragma unroll
            for (int j = 0; j < kSet; ++j) {
                const int t = t0 + j < len ? t0 + j : len - 1;
                const uint32_t so = (uint32_t)(t - tb) * rowb;
                xs[j] = IO::load(rx, vo, so);
                ds[j] = IO::load(rd, vo, so);
            }
        };
        // B rows: token t's in set t & 1 (t0 is even), the next token's loaded right after the
        // wait for this token's.  The C row of a token is loaded at the same point and is first
        // used after the token's 16 state updates.
        BcRow<E> bc[2], cc;
        bc[0].load(Bb);
        auto run = [&](const uint32_t(&xs)[kSet], const uint32_t(&ds)[kSet],
                       const uint32_t(&tch)[kTouches > 0 ? kTouches : 1], int t0) {
            const __amdgpu_buffer_rsrc_t ry = seglane::rsrc(yb + (int64_t)t0 * D);
#pragma unroll
            for (int j = 0; j < kSet; ++j) {
                const int cur = j & 1;
                const int tn = t0 + j + 1 < len ? t0 + j + 1 : len - 1;
                __builtin_amdgcn_sched_barrier(0);
                wait_scalar(bc[cur].w[0]);
                __builtin_amdgcn_sched_barrier(0);
                bc[cur ^ 1].load(Bb + (int64_t)tn * kDState);
                if constexpr (!kSummary) cc.load(Cb + (int64_t)(t0 + j) * kDState);
                __builtin_amdgcn_sched_barrier(0);
                token(IO::value(xs[j]), IO::value(ds[j]), bc[cur], cc, ry, (uint32_t)j * rowb);
                if (j == 0) {
                    // the touches are older than this token's x, so they have arrived: retire them
#pragma unroll
                    for (int k = 0; k < kTouches; ++k) asm volatile("" ::"v"(tch[k]));
                }
            }
        };
        const int whole = len - len % kBlock;
        fetch(xr[0], dr[0], tq[0], 0);
        for (int t0 = 0; t0 < whole; t0 += kBlock) {
            // The SIMD issues from its oldest wave first, so without this the first of its
            // waves would run far ahead and the last would finish alone, at the slow one-wave
            // issue rate.  A wave lowers its priority as it advances, which keeps them level.
            const int quarter = (t0 * 4) / len;
            if (quarter == 0)
                __builtin_amdgcn_s_setprio(3);
            else if (quarter == 1)
                __builtin_amdgcn_s_setprio(2);
            else if (quarter == 2)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
            fetch(xr[1], dr[1], tq[1], t0 + kSet);
            __builtin_amdgcn_sched_barrier(0);
            run(xr[0], dr[0], tq[0], t0);
            fetch(xr[0], dr[0], tq[0], t0 + kBlock);
            __builtin_amdgcn_sched_barrier(0);
            run(xr[1], dr[1], tq[1], t0 + kSet);
        }
        // the last len % 16 tokens, one at a time
        for (int t = whole; t < len; ++t) {
            BcRow<E> b1, c1;
            b1.load(Bb + (int64_t)t * kDState);
            if constexpr (!kSummary) c1.load(Cb + (int64_t)t * kDState);
            const int64_t at = (int64_t)t * D;
            const __amdgpu_buffer_rsrc_t rx = seglane::rsrc(xb + at), rd = seglane::rsrc(db + at);
            token(IO::value(IO::load(rx, vo, 0)), IO::value(IO::load(rd, vo, 0)), b1, c1, seglane::rsrc(yb + at),
                  0);
        }
    };
    // only a first segment needs the rows kernel's order (see the file comment)
    if constexpr (kSummary || !kRowsOrder)
        scan(std::false_type{});
    else if (vrow % sg.n_seg == 0)
        scan(std::true_type{});
    else
        scan(std::false_type{});
    if (span.state >= 0) {
#pragma unroll
        for (int n = 0; n < kDState; ++n) h_final[((int64_t)span.state * D + d) * kDState + n] = h[n];
    }
    if constexpr (kSummary) dsum[(int64_t)vrow * D + d] = dacc;
}

template <typename E, bool kSummary, bool kRowsOrder>
void launch_prefill_seg_lane(const typename E::store_t *x, const typename E::store_t *dl, const float *A,
                             const typename E::store_t *B, const typename E::store_t *C, const float *h0,
                             typename E::store_t *y, float *h_final, float *dsum, const Segments &sg, int64_t nrows,
                             int D, hipStream_t stream) {
    const int blocks_per_row = (D + seglane::kThreads - 1) / seglane::kThreads;
    hipLaunchKernelGGL((prefill_seg_lane_kernel<E, kSummary, kRowsOrder>), dim3((unsigned)(nrows * blocks_per_row)),
                       dim3(seglane::kThreads), 0, stream, x, dl, A, B, C, h0, y, h_final, dsum, sg, D, blocks_per_row);
}

}  // namespace jscan
