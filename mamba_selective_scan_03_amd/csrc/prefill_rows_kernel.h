// prefill_rows_kernel.h - prefill for long sequences at small batch (the Jamba prefill
// shape: batch 1, D = 8192, N = 16, 4K-256K tokens).
//
// Why this mapping.  Each (channel, state) pair is a chain of L dependent updates.  Keeping
// the final state bit-identical to the decode step means every chain must be walked token
// by token in one lane, so all parallelism comes from batch * D * 16 chains: 131072 at
// batch 1.  That is 128 chains per SIMD on a 256-CU chip, so a lane carries G = 2 states and
// every SIMD runs exactly one scan wave.
//
// Lane layout.  A wave is 4 rows of 16 lanes.  Lane c of a row owns channel c of a 16-channel
// group; row r owns the state pair n = 8*sh + 2*r + {0,1}, where sh picks one half of the
// states.  Two waves (sh = 0, 1) cover all 16 states of one 16-channel group, and a
// 256-thread workgroup covers 32 channels (two groups).
//   * B_t[n] (and, with fp32 output, C_t[n]) is the same for all 16 lanes of a row.  A
//     register holds 16 consecutive tokens' values of one state (lane c = token c), and the
//     DPP row broadcast (row_newbcast:k) hands token k's value to the whole row inside the
//     multiply.  No extra instruction is issued.
//   * delta_t[d] and delta_t[d] * x_t[d] are per lane (per channel).  The workgroup converts
//     each tile once into fp32 pairs in LDS, and every row reads them as a broadcast.  With a
//     scaled-identity A (AForm::ScaledIdentity: one a[d] for all states of a channel) the pair
//     carries the channel's decay 2^(delta * a2[d]) in place of delta, computed once per
//     (token, channel) while staging, and the scan waves run no exponential at all.
//   * y_t[d] = sum over 16 states: each wave's 8 states, then its 2 waves through LDS (the
//     last stage fused with the bf16 conversion and a coalesced row store).  With bf16 output
//     a wave's share is a small product on the matrix cores, its states (rounded to bf16)
//     against C as an MFMA operand (c_operand_bases()); with delta computed on the load path
//     the lanes' 2-state partials are summed over the 4 rows there instead (row_sum_operands());
//     with fp32 output the 2-state partials are summed over the rows by permlane swaps.
//
// Pipeline.  Tokens go in tiles of 64.  While tile k is scanned, tile k+1 is converted from
// registers into LDS and tiles k+2 and k+3 are in flight from HBM into two register sets,
// so every HBM load has two tiles of work to arrive.  One workgroup barrier per tile orders
// the double-buffered LDS tiles and the double-buffered y exchange buffer; the staging, the
// HBM requests and the previous tile's y stores are spread into the scan of the first group.
// A ragged last tile is padded with identity tokens (delta = 0, x = -0, B = C = 0): they
// leave every state bit-identical (decay 2^0 = 1, input term -0) and their y is not stored.
//
// Modes (template parameters): delta computed on the load path from the low-rank projection
// (kFused), the form of A (AF: diagonal, scaled identity, complex pairs) and the
// exponential-trapezoidal rule
// (kTrap: the helper waves also stage the left-end weights and the previous token's B, and the
// scan lane takes the left end point in first, one more DPP-fused FMA per state element).
#pragma once

#include "mfma_common.h"
#include "scan_update.h"

namespace jscan {

namespace rows {
constexpr int kT = 64;          // tokens per tile
constexpr int kCh = 32;         // channels per workgroup
constexpr int kThreads = 512;   // 4 scan waves + 4 helper waves
constexpr int kHalf = 256;      // threads per role
// LDS row lengths, padded so that the accesses of a wave spread over all banks:
constexpr int kDxStride = (kCh + 1) * 4;   // [token pair][channel][4]: +1 float4 per pair row
constexpr int kBcStride = kT + 8;          // [state][token] B and C tiles
constexpr int kYStride = kCh + 16;         // [token][channel] y exchange (kCh + 8, which puts
                                           // the 4 rows of a wave in distinct banks, measured slower)
// The same with the contraction on the matrix cores with C as an operand, whose 16-byte stores
// put token t of a group at t * kYStrideC: an odd number of 16-byte units, so the 16 tokens'
// stores fall on distinct banks (the 64K scan 1.83 -> 1.77 ms; the fused scan, which keeps the
// row sums of partials, was slower with it and keeps kYStride)
constexpr int kYStrideC = kCh + 12;
// LDS (floats): delta*x/delta pairs [kT/2][kDxStride], B and C [16][kBcStride], y [2][kT][kYStride]
constexpr int kDxSize = kT / 2 * kDxStride;
constexpr int kBcSize = kDState * kBcStride;
constexpr int kYSize = 2 * kT * kYStride;
// Trapezoidal rule: the left-end weights p [kT/4][kPStride] (4 tokens of a channel per float4)
constexpr int kPStride = kCh * 4 + 4;
constexpr int kPSize = kT / 4 * kPStride;
// bf16 output: the C operands of the output MFMAs, [group][state half][table, zeros][lane][4 dwords]
// per tile buffer (see c_operands())
constexpr int kSelLane = 4;                    // dwords per lane entry
constexpr int kSelHalf = 2 * 64 * kSelLane;    // table and zero block of one state half
constexpr int kSelGroup = 2 * kSelHalf;        // both state halves of a 16-token group
constexpr int kSelSize = (kT / 16) * kSelGroup;
}  // namespace rows

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
    // trapezoidal rule only: lam of tokens 2p, 2p+1; x of token 2p-1; B (or C) of token tb-1
    typename Vec4<E>::raw lam[2], xp, bcp[2];
};

// Where a trapezoidal prefill's helper thread finds the token before its row's first: the
// caller's x_prev and B_prev rows (B_prev is also read, unused, by the C threads), or, with
// none given, any valid address whose value staging then replaces by zero.
template <typename E> struct PrevRow {
    const typename E::store_t *lam;   // lam of the work-group's channels, token 0 of the row
    const typename E::store_t *x;     // x_prev + 4q of this thread's channels, or a stand-in
    const typename E::store_t *bc;    // B_prev + nb, or a stand-in
    bool given;
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

// acc + (lane k's c_tile, broadcast over the row) * h in one v_fmac_f32_dpp: the DPP
// operand folds into the multiply-add, so the broadcast issues no instruction of its own.
// The compiler does not fold DPP into v_fmac by itself.  `c_tile` is only ever written by
// LDS reads, never by a VALU op in the two preceding instructions, so no DPP wait state is
// needed; the leading s_nop on k == 0 keeps that true even if register allocation moves it.
template <int k> __device__ __forceinline__ float fmac_bcast(float acc, float c_tile, float h) {
    if constexpr (k == 0)
        asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(acc) : "v"(c_tile), "v"(h));
    else
        asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(acc) : "v"(c_tile), "v"(h), "i"(k));
    return acc;
}

// fmac_bcast() for the lane's two states in one asm statement, so that the compiler, which
// cannot see into it, waits once for both results rather than once for each.
template <int k> __device__ __forceinline__ void fmac2_bcast(float &a0, float &a1, float t0, float t1, float v) {
    if constexpr (k == 0)
        asm("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %3, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(a0), "+v"(a1) : "v"(t0), "v"(t1), "v"(v));
    else
        asm("v_fmac_f32_dpp %0, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(a0), "+v"(a1) : "v"(t0), "v"(t1), "v"(v), "i"(k));
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
// Two reduce_rows4() interleaved, so that no swap reads an add of the instruction before it.
__device__ __forceinline__ void reduce_rows4x2(const float (&P)[8], float &ra, float &rb) {
    float a0 = P[0], a1 = P[1], a2 = P[2], a3 = P[3], b0 = P[4], b1 = P[5], b2 = P[6], b3 = P[7];
    swap32(a0, a1);
    swap32(b0, b1);
    swap32(a2, a3);
    swap32(b2, b3);
    float a01 = a0 + a1, b01 = b0 + b1, a23 = a2 + a3, b23 = b2 + b3;
    swap16(a01, a23);
    swap16(b01, b23);
    ra = a01 + a23;
    rb = b01 + b23;
}

// Requests one tile's raw inputs.  The loads are unconditional per lane: a load inside a
// divergent branch makes the compiler wait for it where the branch merges, which would expose
// the full HBM latency.  Whole tiles take 32-bit lane offsets from a tile base; the last,
// partial tile re-reads token L-1 for tokens past the end, which staging then replaces by
// identity tokens.
template <typename E, bool kLoadDelta = true, bool kTrap = false>
__device__ __forceinline__ void load_tile(TileRegs<E> &R, const typename E::store_t *xb,
                                          const typename E::store_t *db, const typename E::store_t *bcb,
                                          int64_t t0, int64_t L, int D, int tid,
                                          const PrevRow<E> &pr = PrevRow<E>{nullptr, nullptr, nullptr, false}) {
    const int p = tid >> 3, q = tid & 7;                   // token pair p, channel quad q
    const int tb = (tid & 127) >> 1, nb = (tid & 1) * 8;  // B/C: one token, 8 states
    if (t0 + rows::kT <= L) {
        const typename E::store_t *xt = xb + t0 * D, *dt = db + t0 * D, *bt = bcb + t0 * kDState;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int off = (2 * p + j) * D + 4 * q;
            R.x[j] = Vec4<E>::load(xt + off);
            if constexpr (kLoadDelta) R.dl[j] = Vec4<E>::load(dt + off);
            if constexpr (kTrap) R.lam[j] = Vec4<E>::load(pr.lam + t0 * D + off);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) R.bc[j] = Vec4<E>::load(bt + tb * kDState + nb + 4 * j);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t t = min(t0 + 2 * p + j, L - 1);
            R.x[j] = Vec4<E>::load(xb + t * D + 4 * q);
            if constexpr (kLoadDelta) R.dl[j] = Vec4<E>::load(db + t * D + 4 * q);
            if constexpr (kTrap) R.lam[j] = Vec4<E>::load(pr.lam + t * D + 4 * q);
        }
        const int64_t t = min(t0 + tb, L - 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) R.bc[j] = Vec4<E>::load(bcb + t * kDState + nb + 4 * j);
    }
    if constexpr (kTrap) {
        // the previous token of pair p and of B/C token tb (clamped like the tokens themselves;
        // token -1 is the caller's previous token)
        const int64_t tp = min(t0 + 2 * p - 1, L - 1), tq = min(t0 + tb - 1, L - 1);
        R.xp = Vec4<E>::load(tp >= 0 ? xb + tp * D + 4 * q : pr.x);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            R.bcp[j] = Vec4<E>::load(tq >= 0 ? bcb + tq * kDState + nb + 4 * j : pr.bc + 4 * j);
    }
}

// ---- delta computed on the load path ---------------------------------------------------
// With the producer's second projection folded in, the helper waves compute each tile's delta
// themselves: delta = softplus(W_dt d_low + b_dt) for the tile's 64 tokens and the work-group's
// 32 channels, on the matrix cores, with the same MFMA sequence, bias add, softplus and bf16
// rounding as the separate delta projection (project_kernels.h), so the scan sees bit-identical
// delta values.  Helper wave hw computes the 16 tokens 16 hw .. 16 hw + 15 that its own lanes
// stage, so the result only has to move between lanes of one wave (through a small per-wave
// LDS area, which needs no barrier).
struct DeltaProj {
    const uint16_t *d_low;   // [tokens][kRank] bf16, tokens in the order of x's rows
    const uint16_t *w_dt;    // [D][kRank] bf16
    const float *b_dt;       // [D] fp32
};
namespace fused {
constexpr int kRank = 256;               // rank of the low-rank delta input
constexpr int kKS = kRank / 32;          // MFMA k steps
constexpr int kXchRow = 36;              // bf16 per row of the per-wave exchange (32 + 4)
constexpr int kXchWave = 16 * kXchRow;   // one wave's exchange area: 16 tokens
}

// This lane's MFMA B operands (its token's d_low row, all k) for the tile starting at t0.
__device__ __forceinline__ void load_dlow(u32x4_t (&f)[fused::kKS], const uint16_t *d_low, int64_t row, int64_t t0,
                                          int64_t L, int hw, int l) {
    const int64_t t = row + min(t0 + 16 * hw + (l & 15), L - 1);
#pragma unroll
    for (int ks = 0; ks < fused::kKS; ++ks)
        f[ks] = *reinterpret_cast<const u32x4_t *>(d_low + t * fused::kRank + 32 * ks + 8 * (l >> 4));
}

// delta for this wave's 16 tokens x 32 channels, rounded to bf16, into the staging registers
// R.dl of the lanes that stage those tokens.
__device__ __forceinline__ void fused_delta(const u32x4_t (&f)[fused::kKS], const bf16x8_t (&wf)[2][fused::kKS],
                                            const float4 (&bias)[2], uint16_t *xch, TileRegs<BF16> &R, int l) {
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < fused::kKS; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[u] = mfma16(wf[u][ks], __builtin_bit_cast(bf16x8_t, f[ks]), acc[u]);
    // lane l holds channels 16u + 4 (l / 16) + i of token l % 16
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        uint2 pk;
        pk.x = pack_bf16x2(softplus_f32(acc[u][0] + bias[u].x), softplus_f32(acc[u][1] + bias[u].y));
        pk.y = pack_bf16x2(softplus_f32(acc[u][2] + bias[u].z), softplus_f32(acc[u][3] + bias[u].w));
        *reinterpret_cast<uint2 *>(xch + (l & 15) * fused::kXchRow + 16 * u + 4 * (l >> 4)) = pk;
    }
    // the staging lane (token pair l / 8, channel quad l % 8) reads its two tokens' 4 channels
#pragma unroll
    for (int j = 0; j < 2; ++j)
        R.dl[j] = *reinterpret_cast<const uint2 *>(xch + (2 * (l >> 3) + j) * fused::kXchRow + 4 * (l & 7));
}

// Converts one quarter of a tile from registers into LDS: channel 4q + part of this thread's
// (delta*x, delta) fp32 pairs, and states nb + 2*part, nb + 2*part + 1 of its B or C token.
// With a scaled-identity A the second member is the channel's decay 2^(delta * a2), a2 taken
// from a2q (this thread's four channels).  Tokens at or past L become identity tokens
// (delta = 0, x = -0, B = C = 0; their decay is exactly 1).  A tile is staged a quarter per
// 16-token group so that the LDS writes never pile up behind each other.
//
// With the trapezoidal rule (kTrap) the pair's first member is q = (lam delta) x, the left-end
// weight p = ((1 - lam) delta) x_prev of each token goes to p_s, and the B threads also stage
// B of the previous token into the third B/C tile (zero for tokens at or past L, and for token
// 0 of a row without a previous token).  A token at or past L gets p = -0, so with its zero
// previous B the left-end term is -0 and the state stays bit-identical.
template <typename E, int part, AForm AF, bool kTrap, bool kCOps>
__device__ __forceinline__ void stage_part(const TileRegs<E> &R, float *dx_s, float *bc_s, float *p_s, uint32_t *cs_s,
                                           int64_t t0, int64_t L, int tid, const float4 &a2q, bool prev_given) {
    constexpr bool kScalarA = AF == AForm::ScaledIdentity;
    const float a2 = part == 0 ? a2q.x : part == 1 ? a2q.y : part == 2 ? a2q.z : a2q.w;
    const int p = tid >> 3, q = tid & 7;
    float4 v;
    {
        float xv[4], dv[4], lv[4], xpv[4];
        const bool live0 = t0 + 2 * p < L, live1 = t0 + 2 * p + 1 < L;
        Vec4<E>::widen(live0 ? R.x[0] : Vec4<E>::neg_zero(), xv);
        Vec4<E>::widen(live0 ? R.dl[0] : Vec4<E>::zero(), dv);
        float p0 = 0.0f, p1 = 0.0f;
        if constexpr (kTrap) {
            Vec4<E>::widen(live0 ? R.lam[0] : Vec4<E>::zero(), lv);
            Vec4<E>::widen((t0 + 2 * p > 0 || prev_given) ? R.xp : Vec4<E>::zero(), xpv);
            v.x = trap_right(dv[part], lv[part], xv[part]);
            p0 = live0 ? trap_left(dv[part], lv[part], xpv[part]) : -0.0f;
            xpv[part] = xv[part];   // token 2p is token 2p+1's previous one
        } else {
            v.x = delta_x(dv[part], xv[part]);
        }
        v.y = kScalarA ? decay(dv[part], a2) : dv[part];
        Vec4<E>::widen(live1 ? R.x[1] : Vec4<E>::neg_zero(), xv);
        Vec4<E>::widen(live1 ? R.dl[1] : Vec4<E>::zero(), dv);
        if constexpr (kTrap) {
            Vec4<E>::widen(live1 ? R.lam[1] : Vec4<E>::zero(), lv);
            v.z = trap_right(dv[part], lv[part], xv[part]);
            p1 = live1 ? trap_left(dv[part], lv[part], xpv[part]) : -0.0f;
            *reinterpret_cast<float2 *>(p_s + (p >> 1) * rows::kPStride + (4 * q + part) * 4 + 2 * (p & 1)) =
                make_float2(p0, p1);
        } else {
            v.z = delta_x(dv[part], xv[part]);
        }
        v.w = kScalarA ? decay(dv[part], a2) : dv[part];
    }
    *reinterpret_cast<float4 *>(dx_s + p * rows::kDxStride + (4 * q + part) * 4) = v;
    const int tb = (tid & 127) >> 1, nb = (tid & 1) * 8;
    const bool live = t0 + tb < L;
    if constexpr (kCOps) {
        if (tid >= 128) {   // whole waves: the C threads write their pair of states nb + 2 part, + 1 as
                            // the raw bf16 pair, into the table entry of lane (row part, column tb % 16)
            const typename Vec4<E>::raw r = live ? R.bc[part >> 1] : Vec4<E>::zero();
            const uint32_t pair = (part & 1) ? r.y : r.x;
            cs_s[(tb >> 4) * rows::kSelGroup + (nb >> 3) * rows::kSelHalf + (16 * part + (tb & 15)) * rows::kSelLane +
                 (tb & 3)] = pair;
        } else {
            float f[4];
            Vec4<E>::widen(live ? R.bc[part >> 1] : Vec4<E>::zero(), f);
            bc_s[(nb + 2 * part) * rows::kBcStride + tb] = f[(2 * part) & 3];
            bc_s[(nb + 2 * part + 1) * rows::kBcStride + tb] = f[(2 * part + 1) & 3];
        }
    } else {
        float *dst = bc_s + (tid >= 128 ? rows::kBcSize : 0);
        float f[4];
        Vec4<E>::widen(live ? R.bc[part >> 1] : Vec4<E>::zero(), f);
        dst[(nb + 2 * part) * rows::kBcStride + tb] = f[(2 * part) & 3];
        dst[(nb + 2 * part + 1) * rows::kBcStride + tb] = f[(2 * part + 1) & 3];
    }
    if constexpr (kTrap) {
        if (tid < 128) {   // whole waves: the B threads
            const bool prev_live = live && (t0 + tb > 0 || prev_given);
            float f[4];
            Vec4<E>::widen(prev_live ? R.bcp[part >> 1] : Vec4<E>::zero(), f);
            float *bp = bc_s + 2 * rows::kBcSize;
            bp[(nb + 2 * part) * rows::kBcStride + tb] = f[(2 * part) & 3];
            bp[(nb + 2 * part + 1) * rows::kBcStride + tb] = f[(2 * part + 1) & 3];
        }
    }
}
template <typename E, AForm AF, bool kTrap = false, bool kCOps = false>
__device__ __forceinline__ void stage_tile(const TileRegs<E> &R, float *dx_s, float *bc_s, float *p_s, uint32_t *cs_s,
                                           int64_t t0, int64_t L, int tid, const float4 &a2q, bool prev_given = false) {
    stage_part<E, 0, AF, kTrap, kCOps>(R, dx_s, bc_s, p_s, cs_s, t0, L, tid, a2q, prev_given);
    stage_part<E, 1, AF, kTrap, kCOps>(R, dx_s, bc_s, p_s, cs_s, t0, L, tid, a2q, prev_given);
    stage_part<E, 2, AF, kTrap, kCOps>(R, dx_s, bc_s, p_s, cs_s, t0, L, tid, a2q, prev_given);
    stage_part<E, 3, AF, kTrap, kCOps>(R, dx_s, bc_s, p_s, cs_s, t0, L, tid, a2q, prev_given);
}

// One 16-token group's LDS operands for one lane: (delta*x, delta) of its channel for the 16
// tokens, and token (tg + c)'s B and C of the lane's two states (broadcast per token later).
// They are read in two halves (tokens 0-7 with B and C, then tokens 8-15), each issued half a
// group ahead of its use: a wave may have at most 15 LDS operations in flight, and larger
// bursts stall issue until the oldest complete.
// A trapezoidal scan also reads the 16 tokens' left-end weights p (pv) and the previous token's
// B of its two states (bp0, bp1; broadcast per token like B).
// With bf16 output the lane reads, instead of C, the B operands of the group's four output
// MFMAs (cs; see c_operands()).
struct GroupRegs {
    float4 v[8];
    float b0, b1, c0, c1;
    float4 pv[4];
    float bp0, bp1;
    u32x4_t cs[4];
};
template <int H, bool kTrap = false, bool kCOps = false>
__device__ __forceinline__ void load_half(GroupRegs &g, const float *dxs, const float *bcs, const float *ps, int tg,
                                          int ch, int n0, int c, const uint32_t *const *selp = nullptr, int selo = 0) {
#pragma unroll
    for (int i = 4 * H; i < 4 * H + 4; ++i)
        g.v[i] = *reinterpret_cast<const float4 *>(dxs + ((tg >> 1) + i) * rows::kDxStride + ch * 4);
    if constexpr (kTrap) {
#pragma unroll
        for (int i = 2 * H; i < 2 * H + 2; ++i)
            g.pv[i] = *reinterpret_cast<const float4 *>(ps + ((tg >> 2) + i) * rows::kPStride + ch * 4);
    }
    if constexpr (H == 0) {
        g.b0 = bcs[n0 * rows::kBcStride + tg + c];
        g.b1 = bcs[(n0 + 1) * rows::kBcStride + tg + c];
        if constexpr (kCOps) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                g.cs[m] = *reinterpret_cast<const u32x4_t *>(selp[m] + selo + (tg >> 4) * rows::kSelGroup);
        } else {
            g.c0 = bcs[rows::kBcSize + n0 * rows::kBcStride + tg + c];
            g.c1 = bcs[rows::kBcSize + (n0 + 1) * rows::kBcStride + tg + c];
        }
        if constexpr (kTrap) {
            g.bp0 = bcs[2 * rows::kBcSize + n0 * rows::kBcStride + tg + c];
            g.bp1 = bcs[2 * rows::kBcSize + (n0 + 1) * rows::kBcStride + tg + c];
        }
    }
}

template <int i> __device__ __forceinline__ float component(const float4 &v) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One token: advance this lane's two states and return C*h summed over them.  With a
// scaled-identity A the pair's second member is already the decay; with a complex state the
// lane's two states are one complex state and (a2_0, a2_1) its prepared ComplexA.
template <int TAU, AForm AF, bool kTrap = false, bool kNoPartial = false>
__device__ __forceinline__ float token_step(const GroupRegs &g, float &h_0, float &h_1, float a2_0, float a2_1) {
    if constexpr (kTrap) {   // the left end point: h + p * B_prev, the DPP broadcast folded in
        const float pl = component<TAU & 3>(g.pv[TAU >> 2]);
        fmac2_bcast<TAU>(h_0, h_1, g.bp0, g.bp1, pl);
    }
    const float4 v = g.v[TAU >> 1];
    const float dxv = (TAU & 1) ? v.z : v.x;
    const float dv = (TAU & 1) ? v.w : v.y;
    if constexpr (AF == AForm::ComplexPairs) {
        advance_complex(h_0, h_1, dv, ComplexA{a2_0, a2_1}, dxv, row_bcast<TAU>(g.b0), row_bcast<TAU>(g.b1));
    } else if constexpr (AF == AForm::ScaledIdentity) {
        h_0 = advance_decayed(h_0, dv, dxv, row_bcast<TAU>(g.b0));
        h_1 = advance_decayed(h_1, dv, dxv, row_bcast<TAU>(g.b1));
    } else {
        h_0 = advance(h_0, dv, a2_0, dxv, row_bcast<TAU>(g.b0));
        h_1 = advance(h_1, dv, a2_1, dxv, row_bcast<TAU>(g.b1));
    }
    if constexpr (kNoPartial) return 0.0f;
    else return fmac_bcast<TAU>(row_bcast<TAU>(g.c0) * h_0, g.c1, h_1);
}

// How a wave sums y over its 8 states (OutSum):
//   Permlane: in-lane over the lane's two states, then over the 4 rows by permlane swaps (fp32);
//   RowMma:   in-lane, then the 4-row sum on the matrix cores (row_sum_operands());
//   CMma:     the whole contraction with C on the matrix cores (c_operand_bases()).
enum class OutSum : int { Permlane, RowMma, CMma };

// Advance this lane's two states over tokens 8H..8H+7 of a 16-token group and leave their y
// partials (summed over the wave's 4 rows) in the y exchange rows `ys` (row = token in group).
// With RowMma or CMma (bf16 output) the sum runs on the matrix cores instead: two MFMAs per half
// accumulate into d (zeroed by the first half), which the caller stores.
template <int H, AForm AF, bool kTrap = false, OutSum OS = OutSum::Permlane>
__device__ __forceinline__ void scan_half(const GroupRegs &g, float &h_0, float &h_1, float a2_0, float a2_1, float *ys,
                                          int rt, int ch, f32x4_t &d, const bf16x8_t *sel) {
    if constexpr (OS == OutSum::CMma) {
        uint32_t hp[8];
#define JSCAN_STEP(i)                                                           \
    token_step<8 * H + (i), AF, kTrap, true>(g, h_0, h_1, a2_0, a2_1);           \
    hp[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{h_0, h_1}), bf16x2_t));
        JSCAN_STEP(0) JSCAN_STEP(1) JSCAN_STEP(2) JSCAN_STEP(3)
        JSCAN_STEP(4) JSCAN_STEP(5) JSCAN_STEP(6) JSCAN_STEP(7)
#undef JSCAN_STEP
        const f32x4_t d0 = H == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : d;
        d = mfma16(__builtin_bit_cast(bf16x8_t, (u32x4_t{hp[0], hp[1], hp[2], hp[3]})),
                   __builtin_bit_cast(bf16x8_t, g.cs[2 * H]), d0);
        d = mfma16(__builtin_bit_cast(bf16x8_t, (u32x4_t{hp[4], hp[5], hp[6], hp[7]})),
                   __builtin_bit_cast(bf16x8_t, g.cs[2 * H + 1]), d);
    } else {
        float P[8];
#define JSCAN_STEP(i) P[i] = token_step<8 * H + (i), AF, kTrap>(g, h_0, h_1, a2_0, a2_1);
        JSCAN_STEP(0) JSCAN_STEP(1) JSCAN_STEP(2) JSCAN_STEP(3)
        JSCAN_STEP(4) JSCAN_STEP(5) JSCAN_STEP(6) JSCAN_STEP(7)
#undef JSCAN_STEP
        if constexpr (OS == OutSum::RowMma) {
            const bf16x8_t pa = __builtin_convertvector((f32x8_t{P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7]}), bf16x8_t);
            d = mfma16(pa, sel[H], H == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : d);
        } else {
            // rows -> one register per 4 tokens; row r holds token 4j + {0,2,1,3}[r]
            float ra, rb;
            reduce_rows4x2(P, ra, rb);
            ys[(8 * H + rt) * rows::kYStride + ch] = ra;
            ys[(8 * H + 4 + rt) * rows::kYStride + ch] = rb;
        }
    }
}

// The 4-row sum of a 16-token group on the matrix cores, from the lanes' partials.  Lane (r, c)
// holds its partials of tokens 0-7 (first half) and 8-15 (second half) of the group as bf16, so
// a half's partials are the A operand A[c][8r + j] = partial of row r, token j; the constant B
// operand sel[0] is the one-hot B[8r + j][col] = (j == col) for col < 8, and sel[1] the same for
// col = 8 + j.  The two MFMAs give D[c][tok] = sum over r of the token's partials, in the layout
// of the contraction below.  The partials are rounded to bf16 once (2^-9 relative).
__device__ __forceinline__ void row_sum_operands(bf16x8_t (&sel)[2], int lane) {
    const int col = lane & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel[0][j] = (__bf16)(col == j ? 1.0f : 0.0f);
        sel[1][j] = (__bf16)(col == 8 + j ? 1.0f : 0.0f);
    }
}

// The output contraction of bf16 output on the matrix cores.  For a 16-token group, a wave's
// share of y is y[c][t] = sum over its 8 states n of C_t[n] h_t[c][n], for its 16 channels c.
// MFMA m (m = 0..3) covers tokens 4m .. 4m + 3 with k = 8 r + 2 t' + s (row r, token 4m + t',
// state n0(r) + s):
//   A[c][k] = h of lane (r, c) after token 4m + t', state s, rounded to bf16: the lane's own
//             states, four tokens in four registers;
//   B[k][col] = C_col[n0(r) + s] where col = 4m + t', else 0: lane (r, col) holds, for the m
//             with col / 4 = m, the bf16 pair C_col[n0], C_col[n0 + 1] in register col % 4 and
//             zeros elsewhere, and zeros for the other three m.
// The four MFMAs accumulate D[c][col] = y share of channel c, token col, four channels of one
// token per lane, written to the exchange rows with one 16-byte write.  The helper waves stage
// the B operands: a table per (group, state half) in which each lane's entry holds the raw bf16
// pair in its register col % 4 (the other registers are zeroed once), and a zero block; lane
// (r, col) reads the table for its m and the zero block for the other three, at the same
// offsets, so the reads need no per-lane selection.  Products of bf16 values are exact and the
// MFMA sums in fp32, so y differs from the fp32 contraction by the rounding of h to bf16
// (2^-9 relative per term), below y's own rounding to bf16.
__device__ __forceinline__ void c_operand_bases(const uint32_t *(&selp)[4], const uint32_t *cs_s, int sh, int lane) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int z = (m == ((lane & 15) >> 2)) ? 0 : 1;
        selp[m] = cs_s + sh * rows::kSelHalf + (z * 64 + lane) * rows::kSelLane;
    }
}
__device__ __forceinline__ void row_sum_store(const f32x4_t &d, float *ys, int cg, int lane, int yst) {
    *reinterpret_cast<f32x4_t *>(ys + (lane & 15) * yst + 16 * cg + 4 * (lane >> 4)) = d;
}

// The same half split in two: the tokens' partials (computed in one scheduling region) and their
// reduction over rows and store (done in the next region, beside the next half's tokens).  The
// scaled-identity form, whose tokens are short, runs its halves this way: 2% faster there, 2%
// slower for the diagonal A.
template <int H, AForm AF, bool kTrap = false>
__device__ __forceinline__ void half_partials(const GroupRegs &g, float &h_0, float &h_1, float a2_0, float a2_1,
                                              float (&P)[8]) {
#define JSCAN_STEP(i) P[i] = token_step<8 * H + (i), AF, kTrap>(g, h_0, h_1, a2_0, a2_1);
    JSCAN_STEP(0) JSCAN_STEP(1) JSCAN_STEP(2) JSCAN_STEP(3)
    JSCAN_STEP(4) JSCAN_STEP(5) JSCAN_STEP(6) JSCAN_STEP(7)
#undef JSCAN_STEP
}
template <int H>
__device__ __forceinline__ void half_store(const float (&P)[8], float *ys, int rt, int ch) {
    float ra, rb;
    reduce_rows4x2(P, ra, rb);
    ys[(8 * H + rt) * rows::kYStride + ch] = ra;
    ys[(8 * H + 4 + rt) * rows::kYStride + ch] = rb;
}

// The last step of y for one tile: this thread's token row t = tid / 4 and 8 channels, as the
// two state halves' sums read from the exchange buffer.
struct FinalRegs {
    float4 u[2], w[2];
};
__device__ __forceinline__ void read_final(FinalRegs &F, const float *y_tile, int tid, int yst) {
    const int t = tid >> 2, c8 = (tid & 3) * 8;
    const float *y0 = y_tile + t * yst + c8;
    const float *y1 = y0 + rows::kT * yst;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        F.u[j] = *reinterpret_cast<const float4 *>(y0 + 4 * j);
        F.w[j] = *reinterpret_cast<const float4 *>(y1 + 4 * j);
    }
}
template <typename E>
__device__ __forceinline__ void write_final(const FinalRegs &F, typename E::store_t *yb, int64_t t0, int64_t L, int D,
                                            int tid) {
    const int t = tid >> 2, c8 = (tid & 3) * 8;
    float o[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        o[4 * j] = F.u[j].x + F.w[j].x;
        o[4 * j + 1] = F.u[j].y + F.w[j].y;
        o[4 * j + 2] = F.u[j].z + F.w[j].z;
        o[4 * j + 3] = F.u[j].w + F.w[j].w;
    }
    const int64_t tt = t0 + t;
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

// One work-group scans 32 channels of one row (see Segments) from the row's initial state
// (zero when h0 is null).  With kFused, delta is not read: the helper waves compute it from dp (bf16 only).  With
// a scaled-identity A (AF), A is a[D] (one value per channel) instead of A[D][16]; with a
// complex state, A[D][16] holds 8 complex entries per channel as (real, imaginary) pairs.  With
// kTrap the exponential-trapezoidal rule replaces the Euler rule (extra inputs in tr).
template <typename E, bool kFused = false, AForm AF = AForm::Diagonal, bool kTrap = false>
__global__ __launch_bounds__(rows::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_rows_kernel(
    const typename E::store_t *__restrict__ x, const typename E::store_t *__restrict__ dl,
    const float *__restrict__ A, const typename E::store_t *__restrict__ B,
    const typename E::store_t *__restrict__ C, const float *__restrict__ h0,
    typename E::store_t *__restrict__ y, float *__restrict__ h_final, Segments sg, int D, int blocks_per_row,
    int xcd_stride, DeltaProj dp, Trap tr) {
    static_assert(!kFused || sizeof(typename E::store_t) == 2, "the fused delta path is bf16 only");
    static_assert((AF == AForm::Diagonal && !kTrap) || !kFused,
                  "the other forms of A and the trapezoidal rule run the plain prefill");
    constexpr bool kScalarA = AF == AForm::ScaledIdentity;
    using S = typename E::store_t;
    // bf16 output: the output contraction on the matrix cores, with C as an MFMA operand
    // (c_operand_bases()), or, with delta computed here, whose helper waves keep the matrix cores
    // busy with delta's MFMAs, only the 4-row sum of the lanes' partials (row_sum_operands(): half
    // the MFMAs).  fp32 output keeps the fp32 contraction, in-lane and by permlane swaps.
    constexpr OutSum OS = sizeof(S) != 2 ? OutSum::Permlane : kFused ? OutSum::RowMma : OutSum::CMma;
    constexpr bool kRowMma = OS != OutSum::Permlane;   // the row sums on the matrix cores
    constexpr bool kCOps = OS == OutSum::CMma;         // C operand tables in LDS
    __shared__ __attribute__((aligned(16))) float dx_s[2][rows::kDxSize];
    __shared__ __attribute__((aligned(16))) float bc_s[2][(kTrap ? 3 : 2) * rows::kBcSize];
    __shared__ __attribute__((aligned(16))) float p_s[2][kTrap ? rows::kPSize : 4];
    constexpr int kYS = kCOps ? rows::kYStrideC : rows::kYStride;   // y exchange row stride
    __shared__ __attribute__((aligned(16))) float y_s[2][2 * rows::kT * kYS];
    __shared__ __attribute__((aligned(16))) uint16_t xch_s[kFused ? 4 * fused::kXchWave : 8];
    __shared__ __attribute__((aligned(16))) uint32_t cs_s[2][kCOps ? rows::kSelSize : 4];

    // Consecutive channel blocks go to the same XCD (work-groups are dealt round-robin over
    // the 8 XCDs), so the two blocks sharing a 128-byte row segment share one L2.
    int wg = blockIdx.x;
    if (xcd_stride > 0) wg = (wg & 7) * xcd_stride + (wg >> 3);
    const int vrow = wg / blocks_per_row;
    const int d0 = (wg - vrow * blocks_per_row) * rows::kCh;

    const RowSpan span = row_span(sg, vrow);
    const int64_t row = span.tok0, L = span.len;
    const int ntiles = (int)((L + rows::kT - 1) / rows::kT);

    if (threadIdx.x >= rows::kHalf) {
        // ---------------- helper waves: HBM <-> LDS, never touch the states ----------------
        // Tile k+1 is converted into LDS while the scan waves work on tile k, and the y halves
        // of tile k-1 are summed, rounded and stored.  Each tile's raw inputs are requested
        // two tiles before they are staged.
        const int tid = threadIdx.x - rows::kHalf;
        const typename E::store_t *xb = x + row * D + d0;
        const typename E::store_t *db = dl + row * D + d0;
        const typename E::store_t *bcb = (tid < 128 ? B : C) + row * kDState;
        typename E::store_t *yb = y + row * D + d0;
        TileRegs<E> R[2];
        // fused delta: W_dt operands and biases of this wave's 32 channels, d_low operand ring
        const int hw = tid >> 6, l = tid & 63;
        bf16x8_t wf[2][fused::kKS];
        float4 bias[2];
        u32x4_t dfr[2][fused::kKS];
        uint16_t *xch = xch_s + (kFused ? hw * fused::kXchWave : 0);
        // scaled-identity A: A2 of this thread's staging channels 4q .. 4q + 3
        float4 a2q = make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (kScalarA) {
            const float4 av = *reinterpret_cast<const float4 *>(A + d0 + 4 * (tid & 7));
            a2q = make_float4(scaled_A(av.x), scaled_A(av.y), scaled_A(av.z), scaled_A(av.w));
        }
        // trapezoidal rule: lam, and the caller's previous token (or stand-ins staged as zero)
        const bool prev_given = kTrap && tr.x_prev != nullptr;
        PrevRow<E> pr{nullptr, nullptr, nullptr, prev_given};
        if constexpr (kTrap) {
            pr.lam = static_cast<const S *>(tr.lam) + row * D + d0;
            pr.x = prev_given ? static_cast<const S *>(tr.x_prev) + (int64_t)vrow * D + d0 + 4 * (tid & 7)
                              : xb + 4 * (tid & 7);
            pr.bc = prev_given ? static_cast<const S *>(tr.B_prev) + (int64_t)vrow * kDState + (tid & 1) * 8
                               : bcb + (tid & 1) * 8;
        }
        if constexpr (kFused) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int ks = 0; ks < fused::kKS; ++ks)
                    wf[u][ks] = load_frag(dp.w_dt + (int64_t)(d0 + 16 * u + (l & 15)) * fused::kRank + 32 * ks +
                                          8 * (l >> 4));
                bias[u] = *reinterpret_cast<const float4 *>(dp.b_dt + d0 + 16 * u + 4 * (l >> 4));
            }
        }
        load_tile<E, !kFused, kTrap>(R[0], xb, db, bcb, 0, L, D, tid, pr);
        if constexpr (kCOps) {
            // the C operand tables start as zeros; staging only ever writes each entry's live register
            u32x4_t *z = reinterpret_cast<u32x4_t *>(&cs_s[0][0]);
#pragma unroll
            for (int i = 0; i < 2 * rows::kSelSize / 4 / rows::kHalf; ++i) z[tid + rows::kHalf * i] = u32x4_t{0, 0, 0, 0};
            __syncthreads();
        }
        if constexpr (kFused) {
            load_dlow(dfr[0], dp.d_low, row, 0, L, hw, l);
            fused_delta(dfr[0], wf, bias, xch, R[0], l);
        }
        stage_tile<E, AF, kTrap, kCOps>(R[0], dx_s[0], bc_s[0], p_s[0], cs_s[0], 0, L, tid, a2q, prev_given);
        // tiles 1 and 2, in the order the loop issues its loads
        load_tile<E, !kFused, kTrap>(R[1], xb, db, bcb, rows::kT, L, D, tid, pr);
        if constexpr (kFused) load_dlow(dfr[1], dp.d_low, row, rows::kT, L, hw, l);
        load_tile<E, !kFused, kTrap>(R[0], xb, db, bcb, 2 * rows::kT, L, D, tid, pr);
        if constexpr (kFused) load_dlow(dfr[0], dp.d_low, row, 2 * rows::kT, L, hw, l);
        __syncthreads();
        FinalRegs F;
        // With delta computed here the helper waves' path through a tile is as long as the scan
        // waves', so their waits matter.  The compiler waits for a load's registers by counting
        // the loads issued after it; where a path may skip some of them it counts the fewest, so
        // a load skipped on the last tiles made it wait, on every tile, for the loads issued one
        // tile earlier.  In the fused mode every tile therefore issues tile k + 3's loads (past the
        // last tile they reload clamped rows, unused) and the loop runs whole pairs of tiles, so
        // that every wait leaves the next tile's loads in flight (fused prefill 2.42 -> 2.16 ms on
        // 64K x 8192).  The other modes, bound by their scan waves, keep the plain loop.
        auto tile = [&](auto cur_c, int k) {
            constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
            if (k + 1 < ntiles) {
                if constexpr (kFused) fused_delta(dfr[nxt], wf, bias, xch, R[nxt], l);
                stage_tile<E, AF, kTrap, kCOps>(R[nxt], dx_s[nxt], bc_s[nxt], p_s[nxt], cs_s[nxt],
                                                  (int64_t)(k + 1) * rows::kT, L, tid, a2q, prev_given);
                if (!kFused && k + 3 < ntiles)
                    load_tile<E, !kFused, kTrap>(R[nxt], xb, db, bcb, (int64_t)(k + 3) * rows::kT, L, D, tid, pr);
            }
            if constexpr (kFused) {
                load_tile<E, !kFused, kTrap>(R[nxt], xb, db, bcb, (int64_t)(k + 3) * rows::kT, L, D, tid, pr);
                load_dlow(dfr[nxt], dp.d_low, row, (int64_t)(k + 3) * rows::kT, L, hw, l);
            }
            if (k > 0) {
                read_final(F, y_s[nxt], tid, kYS);
                write_final<E>(F, yb, (int64_t)(k - 1) * rows::kT, L, D, tid);
            }
            __syncthreads();
        };
        if constexpr (kFused) {
            int k = 0;
            for (; k + 1 < ntiles; k += 2) {
                tile(IntConst<0>{}, k);
                tile(IntConst<1>{}, k + 1);
            }
            if (k < ntiles) tile(IntConst<0>{}, k);
        } else {
            for (int k = 0; k < ntiles; k += 2) {
                tile(IntConst<0>{}, k);
                if (k + 1 < ntiles) tile(IntConst<1>{}, k + 1);
            }
        }
        read_final(F, y_s[(ntiles - 1) & 1], tid, kYS);
        write_final<E>(F, yb, (int64_t)(ntiles - 1) * rows::kT, L, D, tid);
        return;
    }

    // ---------------- scan waves: the states, token by token ----------------
    // The scan wave outranks the helper wave sharing its SIMD, so the helper only issues in the
    // cycles the scan wave leaves idle.
    __builtin_amdgcn_s_setprio(3);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;
    const int cg = wave >> 1, sh = wave & 1;
    const int ch = 16 * cg + c;             // channel inside the block
    const int d = d0 + ch;
    const int n0 = 8 * sh + 2 * r;          // this lane's states n0, n0 + 1

    // diagonal: the lane's two A2 values; complex: the prepared entry of its complex state
    float a2_0 = 0.0f, a2_1 = 0.0f;
    if constexpr (AF == AForm::Diagonal) {
        a2_0 = scaled_A(A[(int64_t)d * kDState + n0]);
        a2_1 = scaled_A(A[(int64_t)d * kDState + n0 + 1]);
    } else if constexpr (AF == AForm::ComplexPairs) {
        const ComplexA ca = complex_A(A[(int64_t)d * kDState + n0], A[(int64_t)d * kDState + n0 + 1]);
        a2_0 = ca.a2;
        a2_1 = ca.turns;
    }
    float h_0 = 0.0f, h_1 = 0.0f;
    if (h0) {
        const float2 hv = *reinterpret_cast<const float2 *>(h0 + ((int64_t)vrow * D + d) * kDState + n0);
        h_0 = hv.x;
        h_1 = hv.y;
    }
    const int rt = (r == 1) ? 2 : (r == 2) ? 1 : r;   // token slot of this row after reduce_rows4
    const uint32_t *selp[4] = {nullptr, nullptr, nullptr, nullptr};
    bf16x8_t sel[2];
    if constexpr (kCOps) {
        c_operand_bases(selp, &cs_s[0][0], sh, lane);
        __syncthreads();   // the C operand tables zeroed by the helper waves
    } else if constexpr (kRowMma) {
        row_sum_operands(sel, lane);
    }
    __syncthreads();   // tile 0 staged by the helper waves
    GroupRegs G[2];
    load_half<0, kTrap, kCOps>(G[0], dx_s[0], bc_s[0], p_s[0], 0, ch, n0, c, selp, 0);
    load_half<1, kTrap, kCOps>(G[0], dx_s[0], bc_s[0], p_s[0], 0, ch, n0, c, selp, 0);

    // Per tile: four 16-token groups, each group's LDS operands read (in two halves) while the
    // previous group is scanned.  One barrier per tile, shared with the helper waves, orders
    // the double-buffered LDS tiles and the double-buffered y exchange.  The loop runs two
    // tiles per trip so that every buffer index is a compile-time constant.
#define JSCAN_SB __builtin_amdgcn_sched_barrier(0)
    auto tile = [&](auto cur_c, int k) {
        constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
        float *ys = y_s[cur] + sh * rows::kT * kYS;
        const float *dxc = dx_s[cur], *bcc = bc_s[cur], *psc = p_s[cur];
        if constexpr (AF != AForm::ScaledIdentity || kRowMma) {
            // With the row sums on the matrix cores, a group's sums are stored in the next
            // scheduling region, when its MFMAs have had a half group's tokens to finish.
            f32x4_t dn, dsum;
#define JSCAN_H0(GR, off)                                                                              \
    scan_half<0, AF, kTrap, OS>(GR, h_0, h_1, a2_0, a2_1, ys + (off) * kYS, rt, ch, dn, sel); \
    if constexpr (kRowMma && (off) > 0) row_sum_store(dsum, ys + ((off) - 16) * kYS, cg, lane, kYS);
#define JSCAN_H1(GR, off)                                                                              \
    scan_half<1, AF, kTrap, OS>(GR, h_0, h_1, a2_0, a2_1, ys + (off) * kYS, rt, ch, dn, sel); \
    if constexpr (kRowMma) dsum = dn;
            constexpr int so = cur * rows::kSelSize;
            load_half<0, kTrap, kCOps>(G[1], dxc, bcc, psc, 16, ch, n0, c, selp, so);
            JSCAN_SB;
            JSCAN_H0(G[0], 0)
            JSCAN_SB;
            load_half<1, kTrap, kCOps>(G[1], dxc, bcc, psc, 16, ch, n0, c, selp, so);
            JSCAN_SB;
            JSCAN_H1(G[0], 0)
            JSCAN_SB;
            load_half<0, kTrap, kCOps>(G[0], dxc, bcc, psc, 32, ch, n0, c, selp, so);
            JSCAN_SB;
            JSCAN_H0(G[1], 16)
            JSCAN_SB;
            load_half<1, kTrap, kCOps>(G[0], dxc, bcc, psc, 32, ch, n0, c, selp, so);
            JSCAN_SB;
            JSCAN_H1(G[1], 16)
            JSCAN_SB;
            load_half<0, kTrap, kCOps>(G[1], dxc, bcc, psc, 48, ch, n0, c, selp, so);
            JSCAN_SB;
            JSCAN_H0(G[0], 32)
            JSCAN_SB;
            load_half<1, kTrap, kCOps>(G[1], dxc, bcc, psc, 48, ch, n0, c, selp, so);
            JSCAN_SB;
            JSCAN_H1(G[0], 32)
            JSCAN_SB;
            JSCAN_H0(G[1], 48)
            JSCAN_SB;
            JSCAN_H1(G[1], 48)
            if constexpr (kRowMma) row_sum_store(dsum, ys + 48 * kYS, cg, lane, kYS);
#undef JSCAN_H0
#undef JSCAN_H1
        } else {
            float Pa[8], Pb[8];
            load_half<0, kTrap>(G[1], dxc, bcc, psc, 16, ch, n0, c);
            JSCAN_SB;
            half_partials<0, AF, kTrap>(G[0], h_0, h_1, a2_0, a2_1, Pa);
            JSCAN_SB;
            load_half<1, kTrap>(G[1], dxc, bcc, psc, 16, ch, n0, c);
            JSCAN_SB;
            half_partials<1, AF, kTrap>(G[0], h_0, h_1, a2_0, a2_1, Pb);
            half_store<0>(Pa, ys, rt, ch);
            JSCAN_SB;
            load_half<0, kTrap>(G[0], dxc, bcc, psc, 32, ch, n0, c);
            JSCAN_SB;
            half_partials<0, AF, kTrap>(G[1], h_0, h_1, a2_0, a2_1, Pa);
            half_store<1>(Pb, ys, rt, ch);
            JSCAN_SB;
            load_half<1, kTrap>(G[0], dxc, bcc, psc, 32, ch, n0, c);
            JSCAN_SB;
            half_partials<1, AF, kTrap>(G[1], h_0, h_1, a2_0, a2_1, Pb);
            half_store<0>(Pa, ys + 16 * rows::kYStride, rt, ch);
            JSCAN_SB;
            load_half<0, kTrap>(G[1], dxc, bcc, psc, 48, ch, n0, c);
            JSCAN_SB;
            half_partials<0, AF, kTrap>(G[0], h_0, h_1, a2_0, a2_1, Pa);
            half_store<1>(Pb, ys + 16 * rows::kYStride, rt, ch);
            JSCAN_SB;
            load_half<1, kTrap>(G[1], dxc, bcc, psc, 48, ch, n0, c);
            JSCAN_SB;
            half_partials<1, AF, kTrap>(G[0], h_0, h_1, a2_0, a2_1, Pb);
            half_store<0>(Pa, ys + 32 * rows::kYStride, rt, ch);
            JSCAN_SB;
            half_partials<0, AF, kTrap>(G[1], h_0, h_1, a2_0, a2_1, Pa);
            half_store<1>(Pb, ys + 32 * rows::kYStride, rt, ch);
            JSCAN_SB;
            half_partials<1, AF, kTrap>(G[1], h_0, h_1, a2_0, a2_1, Pb);
            half_store<0>(Pa, ys + 48 * rows::kYStride, rt, ch);
            JSCAN_SB;
            half_store<1>(Pb, ys + 48 * rows::kYStride, rt, ch);
        }
        __syncthreads();
        if (k + 1 < ntiles) {
            load_half<0, kTrap, kCOps>(G[0], dx_s[nxt], bc_s[nxt], p_s[nxt], 0, ch, n0, c, selp, nxt * rows::kSelSize);
            load_half<1, kTrap, kCOps>(G[0], dx_s[nxt], bc_s[nxt], p_s[nxt], 0, ch, n0, c, selp, nxt * rows::kSelSize);
        }
    };
#undef JSCAN_SB
    for (int k = 0; k < ntiles; k += 2) {
        tile(IntConst<0>{}, k);
        if (k + 1 < ntiles) tile(IntConst<1>{}, k + 1);
    }
    if (span.state >= 0)
        *reinterpret_cast<float2 *>(h_final + ((int64_t)span.state * D + d) * kDState + n0) = make_float2(h_0, h_1);
}

// The row-mapped kernel needs whole 32-channel blocks.  It serves every batch: even where one
// lane per channel would fill the chip (batch * D above 65536), the lane kernel runs at a third
// of its rate per element (its loads of x and delta are single elements, not staged tiles).
inline bool rows_kernel_applies(int64_t /*batch*/, int64_t D) { return D % rows::kCh == 0; }

// Launches one work-group per 32 channels of each of the `nrows` rows described by sg.
template <typename E, bool kFused = false, AForm AF = AForm::Diagonal, bool kTrap = false>
void launch_prefill_rows(const typename E::store_t *x, const typename E::store_t *dl, const float *A,
                         const typename E::store_t *B, const typename E::store_t *C, const float *h0,
                         typename E::store_t *y, float *h_final, const Segments &sg, int64_t nrows,
                         int D, hipStream_t stream, DeltaProj dp = DeltaProj{nullptr, nullptr, nullptr},
                         Trap tr = Trap{nullptr, nullptr, nullptr}) {
    const int blocks_per_row = D / rows::kCh;
    const int64_t blocks = nrows * blocks_per_row;
    const int xcd_stride = (blocks % 8 == 0) ? (int)(blocks / 8) : 0;
    hipLaunchKernelGGL((prefill_rows_kernel<E, kFused, AF, kTrap>), dim3((unsigned)blocks),
                       dim3(rows::kThreads), 0, stream, x, dl, A, B, C, h0, y, h_final, sg, D, blocks_per_row,
                       xcd_stride, dp, tr);
}

}  // namespace jscan
