// prefill_mimo_rows_kernel.h - the MIMO prefill (R = 2, 4 or 8 inputs and outputs per channel)
// for long sequences at small batch, on the row-mapped design of prefill_rows_kernel.h.
//
// Mapping.  As in the single-input kernel, a lane carries two states (n0, n0 + 1) of one
// channel: a wave is 4 rows x 16 lanes, lane c of a row owns channel c of a 16-channel group,
// row r owns states 8 sh + 2 r + {0, 1}, and two waves (sh = 0, 1) cover a group's 16 states.
// A 512-thread work-group runs 4 such scan waves (32 channels) and 4 helper waves.
//   * B_t[n][r] and C_t[n][r] are the same for a whole row: a register holds 16 tokens' values
//     of one (state, rank) (lane c = token c) and the DPP row broadcast hands token k's value to
//     the row inside the multiply, as for the single-input B and C.
//   * delta_t * x_t[d][r] (R values) and delta_t (or, with a scaled-identity A, the decay) are
//     per channel; the helper waves stage them in LDS in fp32, and the rows read them as
//     broadcasts.
//   * The R outputs of a token are summed over the wave's 4 rows R at a time (reduce_rows4 on
//     four (token, rank) partials, so each row ends with one of them), then over the two waves
//     by the helper waves, which round to the output dtype and store.
// Tiles are kT = 32 tokens for R <= 4 and 16 for R = 8, so that the R-fold LDS areas stay
// within the work-group's share.  One barrier per tile; the helper waves stage tile k + 1,
// request tile k + 3 and store the outputs of tile k - 1 while the scan waves scan tile k.
// With the exponential-trapezoidal rule (kTrap) the helper waves also stage
// p_r = ((1 - lam) delta) x_{t-1}[r] like delta x, and the previous token's B as a third B/C
// tile; the scan lane takes the left end point in first (mimo_left_in, the DPP broadcast folded
// in).  Tiles are then 16 tokens at R = 4, and R = 8 runs the lane kernel.
// Tokens past L are identity tokens (delta = 0, x = -0, B = C = 0), which leave every state
// bit-identical.
#pragma once

#include "mimo_kernels.h"
#include "prefill_rows_kernel.h"

namespace jscan {

namespace mrows {
template <int R, bool kTrap = false> struct Cfg {
    static_assert(R == 2 || R == 4 || (R == 8 && !kTrap), "rank 2, 4 or 8 (8 without the trapezoidal rule)");
    static constexpr int kT = (R <= 4 && !(kTrap && R == 4)) ? 32 : 16;   // tokens per tile
    static constexpr int kCh = 32;                 // channels per work-group
    static constexpr int kThreads = 512;
    static constexpr int kHalf = 256;
    // helper threads: x and delta, one token and CPT channels per thread
    static constexpr int kTPT = kHalf / kT;         // threads per token
    static constexpr int kCPT = kCh / kTPT;         // channels per thread (4 or 2)
    static constexpr int kXV = kCPT * R;            // x values per thread
    // B (threads 0-127) and C (128-255): one token and SPT states per thread
    static constexpr int kTPB = 128 / kT;
    static constexpr int kSPT = kDState / kTPB;
    static constexpr int kBV = kSPT * R;
    // LDS (floats): dx [kT][kXS] (channel-major rows of kCh * R); delta [kT/4][kCh][4]; B and C
    // [kT][kTS] (token rows of [16 states][R ranks]); y partials [2 halves][kT][kYS].  At R = 4 and 8 without the trapezoidal rule
    // the dx and y token rows are padded by 4 floats, so that the helper threads' 16-byte
    // accesses (8 or 16 threads per token, 16 floats each) spread over all 32 LDS banks instead
    // of a quarter of them: 2-3% faster there.  The same padding measured 1-2% slower at R = 2 and
    // with the trapezoidal rule, which keep unpadded rows.
    static constexpr int kPad = (R == 2 || kTrap) ? 0 : 4;
    static constexpr int kXS = kCh * R + kPad;
    static constexpr int kDxSize = kT * kXS;
    static constexpr int kDlSize = kT * kCh;
    // A scan lane reads its two states' 2R values of one token as 16-byte reads, 16 lanes on 16
    // consecutive tokens; the token rows are padded by 4 floats so that those reads spread over
    // the banks.
    static constexpr int kTS = kDState * R + 4;
    static constexpr int kBcSize = kT * kTS;
    static constexpr int kBcTiles = kTrap ? 3 : 2;   // B, C (and the previous token's B)
    static constexpr int kYS = kCh * R + (R == 2 ? 32 : kPad);
    static constexpr int kYSize = 2 * kT * kYS;
};
}  // namespace mrows

// K raw elements of a row (bf16: 16-bit patterns, K = 2, 4 or a multiple of 8; f32: K = 2 or a
// multiple of 4), kept packed until they are staged.
template <typename E, int K> struct RawRow;
template <int K> struct RawRow<BF16, K> {
    static constexpr int kW = K == 2 ? 1 : K == 4 ? 2 : K / 2;   // 32-bit words
    uint32_t w[kW];
    __device__ __forceinline__ void load(const uint16_t *p) {
        if constexpr (K == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else if constexpr (K == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            w[0] = v.x;
            w[1] = v.y;
        } else {
#pragma unroll
            for (int i = 0; i < K / 8; ++i) {
                const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        }
    }
    __device__ __forceinline__ float get(int i) const { return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]); }
};
template <int K> struct RawRow<F32, K> {
    float v[K];
    __device__ __forceinline__ void load(const float *p) {
        if constexpr (K == 2) {
            const float2 a = *reinterpret_cast<const float2 *>(p);
            v[0] = a.x;
            v[1] = a.y;
        } else {
#pragma unroll
            for (int i = 0; i < K / 4; ++i) {
                const float4 a = reinterpret_cast<const float4 *>(p)[i];
                v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
            }
        }
    }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};

template <typename E, int R, bool kTrap = false> struct MimoTileRegs {
    using C = mrows::Cfg<R, kTrap>;
    RawRow<E, C::kXV> x;     // token tid / kTPT, channels kCPT (tid % kTPT) .. + kCPT, all ranks
    RawRow<E, C::kCPT> dl;   // the same token and channels
    RawRow<E, C::kBV> bc;    // B or C: the token and kSPT states of bc_thread(), all ranks
    // trapezoidal rule only: lam of the token and channels; x of the token before; B (or C) of
    // the token before
    RawRow<E, C::kCPT> lam;
    RawRow<E, C::kXV> xp;
    RawRow<E, C::kBV> bcp;
};

// Where a trapezoidal helper thread finds the token before its row's first: the caller's
// x_prev and B_prev (at this thread's channels and states), or stand-ins staged as zero.
template <typename E> struct MimoPrev {
    const typename E::store_t *lam, *x, *bc;
    bool given;
};

// The B or C thread's token (tb) and first state (s0) within a tile.  Consecutive threads take
// consecutive tokens, so a half-wave's 16-byte staging stores land on consecutive padded token
// rows and spread over the LDS banks.  Every use (loads, staging, the previous token's row) goes
// through here.
template <int R, bool kTrap>
__device__ __forceinline__ void bc_thread(int tid, int &tb, int &s0) {
    using C = mrows::Cfg<R, kTrap>;
    tb = (tid & 127) % C::kT;
    s0 = (tid & 127) / C::kT * C::kSPT;
}

// Requests one tile's raw inputs (tokens past L re-read token L - 1; staging replaces them).
template <typename E, int R, bool kTrap = false>
__device__ __forceinline__ void mimo_load_tile(MimoTileRegs<E, R, kTrap> &Rg, const typename E::store_t *xb,
                                               const typename E::store_t *db, const typename E::store_t *bcb,
                                               int64_t t0, int64_t L, int D, int tid,
                                               const MimoPrev<E> &pr = MimoPrev<E>{nullptr, nullptr, nullptr, false}) {
    using C = mrows::Cfg<R, kTrap>;
    const int t = tid / C::kTPT, c0 = (tid % C::kTPT) * C::kCPT;
    const int64_t tt = min(t0 + t, L - 1);
    Rg.x.load(xb + (tt * D + c0) * R);
    Rg.dl.load(db + tt * D + c0);
    int tb, s0;
    bc_thread<R, kTrap>(tid, tb, s0);
    const int64_t tq = min(t0 + tb, L - 1);
    Rg.bc.load(bcb + (tq * kDState + s0) * R);
    if constexpr (kTrap) {
        Rg.lam.load(pr.lam + tt * D + c0);
        const int64_t tp = min(t0 + t - 1, L - 1), tb1 = min(t0 + tb - 1, L - 1);
        Rg.xp.load(tp >= 0 ? xb + (tp * D + c0) * R : pr.x);
        Rg.bcp.load(tb1 >= 0 ? bcb + (tb1 * kDState + s0) * R : pr.bc);
    }
}

// Converts one tile into LDS: dx = delta * x per (token, channel, rank), delta (or the decay
// 2^(delta a2) with a scaled-identity A) per (token, channel), and the B and C tiles.
//
// With the trapezoidal rule dx holds q = (lam delta) x, p_s the left-end weights p = ((1 - lam)
// delta) x_{t-1}, and the B threads stage the previous token's B as the third tile (zero for
// tokens at or past L and, without a caller's previous token, for the row's token 0).  A token
// at or past L gets p = -0, so its left-end term (-0 times a zero B) leaves the state as it is.
template <typename E, int R, AForm AF, bool kTrap = false>
__device__ __forceinline__ void mimo_stage_tile(const MimoTileRegs<E, R, kTrap> &Rg, float *dx_s, float *dl_s,
                                                float *bc_s, float *p_s, int64_t t0, int64_t L, int tid,
                                                const float (&a2c)[mrows::Cfg<R, kTrap>::kCPT], bool prev_given) {
    using C = mrows::Cfg<R, kTrap>;
    const int t = tid / C::kTPT, c0 = (tid % C::kTPT) * C::kCPT;
    const bool live = t0 + t < L;
    const bool has_prev = t0 + t > 0 || prev_given;
    float dx[C::kXV], pv[C::kXV];
#pragma unroll
    for (int ci = 0; ci < C::kCPT; ++ci) {
        const float dv = live ? Rg.dl.get(ci) : 0.0f;
        if constexpr (kTrap) {
            const float lv = live ? Rg.lam.get(ci) : 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                dx[ci * R + r] = trap_right(dv, lv, live ? Rg.x.get(ci * R + r) : -0.0f);
                pv[ci * R + r] = live ? trap_left(dv, lv, has_prev ? Rg.xp.get(ci * R + r) : 0.0f) : -0.0f;
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) dx[ci * R + r] = delta_x(dv, live ? Rg.x.get(ci * R + r) : -0.0f);
        }
        dl_s[((t >> 2) * C::kCh + c0 + ci) * 4 + (t & 3)] = AF == AForm::ScaledIdentity ? decay(dv, a2c[ci]) : dv;
    }
    float *dst = dx_s + t * C::kXS + c0 * R;
#pragma unroll
    for (int i = 0; i < C::kXV / 4; ++i)
        reinterpret_cast<float4 *>(dst)[i] = make_float4(dx[4 * i], dx[4 * i + 1], dx[4 * i + 2], dx[4 * i + 3]);
    if constexpr (kTrap) {
        float *pd = p_s + t * C::kXS + c0 * R;
#pragma unroll
        for (int i = 0; i < C::kXV / 4; ++i)
            reinterpret_cast<float4 *>(pd)[i] = make_float4(pv[4 * i], pv[4 * i + 1], pv[4 * i + 2], pv[4 * i + 3]);
    }
    int tb, s0;
    bc_thread<R, kTrap>(tid, tb, s0);
    const bool live_bc = t0 + tb < L;
    // this thread's kBV values (i = (n - s0) * R + r) are one contiguous run of its token's row
    float4 *tile = reinterpret_cast<float4 *>(bc_s + (tid >= 128 ? C::kBcSize : 0) + tb * C::kTS + s0 * R);
#pragma unroll
    for (int i = 0; i < C::kBV / 4; ++i)
        tile[i] = live_bc ? make_float4(Rg.bc.get(4 * i), Rg.bc.get(4 * i + 1), Rg.bc.get(4 * i + 2), Rg.bc.get(4 * i + 3))
                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if constexpr (kTrap) {
        if (tid < 128) {   // whole waves: the B threads
            const bool prev_live = live_bc && (t0 + tb > 0 || prev_given);
            float4 *bp = reinterpret_cast<float4 *>(bc_s + 2 * C::kBcSize + tb * C::kTS + s0 * R);
#pragma unroll
            for (int i = 0; i < C::kBV / 4; ++i)
                bp[i] = prev_live ? make_float4(Rg.bcp.get(4 * i), Rg.bcp.get(4 * i + 1), Rg.bcp.get(4 * i + 2),
                                                Rg.bcp.get(4 * i + 3))
                                  : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
}

// The outputs of one tile: this thread's token and channels, the two state halves' partial sums
// added, rounded and stored as one contiguous run of kCPT * R values.
template <typename E, int R, bool kTrap = false>
__device__ __forceinline__ void mimo_write_final(const float *y_tile, typename E::store_t *yb, int64_t t0, int64_t L,
                                                 int D, int tid) {
    using C = mrows::Cfg<R, kTrap>;
    const int t = tid / C::kTPT, c0 = (tid % C::kTPT) * C::kCPT;
    if (t0 + t >= L) return;
    const float *p0 = y_tile + t * C::kYS + c0 * R;
    const float *p1 = p0 + C::kT * C::kYS;
    float o[C::kXV];
#pragma unroll
    for (int i = 0; i < C::kXV / 4; ++i) {
        const float4 u = reinterpret_cast<const float4 *>(p0)[i], w = reinterpret_cast<const float4 *>(p1)[i];
        o[4 * i] = u.x + w.x; o[4 * i + 1] = u.y + w.y; o[4 * i + 2] = u.z + w.z; o[4 * i + 3] = u.w + w.w;
    }
    if constexpr (C::kXV % 4 == 2) {
        const float2 u = *reinterpret_cast<const float2 *>(p0 + C::kXV - 2);
        const float2 w = *reinterpret_cast<const float2 *>(p1 + C::kXV - 2);
        o[C::kXV - 2] = u.x + w.x;
        o[C::kXV - 1] = u.y + w.y;
    }
    RowStore<E, C::kXV>::store(yb + ((t0 + t) * D + c0) * R, o);
}

// The scan lane's LDS operands for 4 tokens: dx (R per token) and delta of its channel (and the
// left-end weights p with the trapezoidal rule).
template <int R> struct QuarterRegs {
    float dx[4][R], p[4][R];
    float4 dl;
};
template <int R, int kXS>
__device__ __forceinline__ void mimo_load_ranks(float (&dst)[4][R], const float *src, int t4, int ch) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float *p = src + (t4 + k) * kXS + ch * R;
        if constexpr (R == 2) {
            const float2 v = *reinterpret_cast<const float2 *>(p);
            dst[k][0] = v.x;
            dst[k][1] = v.y;
        } else {
#pragma unroll
            for (int i = 0; i < R / 4; ++i) {
                const float4 v = reinterpret_cast<const float4 *>(p)[i];
                dst[k][4 * i] = v.x; dst[k][4 * i + 1] = v.y; dst[k][4 * i + 2] = v.z; dst[k][4 * i + 3] = v.w;
            }
        }
    }
}
template <int R, bool kTrap>
__device__ __forceinline__ void mimo_load_quarter(QuarterRegs<R> &q, const float *dx_s, const float *dl_s,
                                                  const float *p_s, int t4, int ch) {
    using C = mrows::Cfg<R, kTrap>;
    mimo_load_ranks<R, C::kXS>(q.dx, dx_s, t4, ch);
    if constexpr (kTrap) mimo_load_ranks<R, C::kXS>(q.p, p_s, t4, ch);
    q.dl = *reinterpret_cast<const float4 *>(dl_s + ((t4 >> 2) * C::kCh + ch) * 4);
}

// The lane's B and C registers for one 16-token group: (state n0 + i, rank r) at [i][r]; lane c
// holds token tg + c (and the previous token's B with the trapezoidal rule).
template <int R> struct BcRegs {
    float b[2][R], c[2][R], bp[2][R];
};
template <int R>
__device__ __forceinline__ void mimo_read_pair(float (&dst)[2][R], const float *src) {
    // states n0 and n0 + 1, all ranks: 2R contiguous floats
#pragma unroll
    for (int j = 0; j < 2 * R / 4; ++j) {
        const float4 v = reinterpret_cast<const float4 *>(src)[j];
        dst[(4 * j) / R][(4 * j) % R] = v.x;
        dst[(4 * j + 1) / R][(4 * j + 1) % R] = v.y;
        dst[(4 * j + 2) / R][(4 * j + 2) % R] = v.z;
        dst[(4 * j + 3) / R][(4 * j + 3) % R] = v.w;
    }
}
template <int R, bool kTrap>
__device__ __forceinline__ void mimo_load_bc(BcRegs<R> &g, const float *bc_s, int tg, int n0, int c) {
    using C = mrows::Cfg<R, kTrap>;
    const float *row = bc_s + (tg + c) * C::kTS + n0 * R;
    mimo_read_pair<R>(g.b, row);
    mimo_read_pair<R>(g.c, row + C::kBcSize);
    if constexpr (kTrap) mimo_read_pair<R>(g.bp, row + 2 * C::kBcSize);
}

// The token's DPP-fused FMAs as few asm statements.  The compiler cannot see into an asm
// statement, so it treats each one's results as possibly late (a transcendental's) and waits a
// cycle before the next instruction that reads them; one statement per group of independent
// chains (the lane's two states, or the R ranks) keeps those waits to one per statement.  The
// plain products before them are the compiler's own v_mul_f32_dpp (row_bcast() folded into the
// multiply).  Every B, C and B_prev operand broadcast here is only ever written by LDS reads;
// the leading s_nop on token 0 is the same margin as in fmac_bcast().
#define JSCAN_RB " row_newbcast:%[k] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define JSCAN_F(d, t, v) "v_fmac_f32_dpp %[" #d "], %[" #t "], %[" #v "]" JSCAN_RB
#define JSCAN_ASM_K(TAU)                                      \
    if constexpr ((TAU) == 0) asm("s_nop 1\n\t" BODY : OUTS : INS); \
    else asm(BODY : OUTS : INS);

// u_s += (B_s[r] of token TAU) * dx[r] for r = 1 .. R-1, for both states s, r increasing.
template <int TAU, int R>
__device__ __forceinline__ void mimo_input_tail(const BcRegs<R> &g, const float (&dx)[R], float &u0, float &u1) {
    if constexpr (R == 2) {
#define BODY JSCAN_F(u0, b01, x1) JSCAN_F(u1, b11, x1)
#define OUTS [u0] "+v"(u0), [u1] "+v"(u1)
#define INS [b01] "v"(g.b[0][1]), [b11] "v"(g.b[1][1]), [x1] "v"(dx[1]), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    } else if constexpr (R == 4) {
#define BODY JSCAN_F(u0, b01, x1) JSCAN_F(u1, b11, x1) JSCAN_F(u0, b02, x2) JSCAN_F(u1, b12, x2) \
             JSCAN_F(u0, b03, x3) JSCAN_F(u1, b13, x3)
#define OUTS [u0] "+v"(u0), [u1] "+v"(u1)
#define INS [b01] "v"(g.b[0][1]), [b11] "v"(g.b[1][1]), [x1] "v"(dx[1]), [b02] "v"(g.b[0][2]), \
            [b12] "v"(g.b[1][2]), [x2] "v"(dx[2]), [b03] "v"(g.b[0][3]), [b13] "v"(g.b[1][3]), [x3] "v"(dx[3]), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    } else {
        static_assert(R == 8, "rank 2, 4 or 8");
#define BODY JSCAN_F(u0, b01, x1) JSCAN_F(u1, b11, x1) JSCAN_F(u0, b02, x2) JSCAN_F(u1, b12, x2) \
             JSCAN_F(u0, b03, x3) JSCAN_F(u1, b13, x3) JSCAN_F(u0, b04, x4) JSCAN_F(u1, b14, x4) \
             JSCAN_F(u0, b05, x5) JSCAN_F(u1, b15, x5) JSCAN_F(u0, b06, x6) JSCAN_F(u1, b16, x6) \
             JSCAN_F(u0, b07, x7) JSCAN_F(u1, b17, x7)
#define OUTS [u0] "+v"(u0), [u1] "+v"(u1)
#define INS [b01] "v"(g.b[0][1]), [b11] "v"(g.b[1][1]), [x1] "v"(dx[1]), [b02] "v"(g.b[0][2]), \
            [b12] "v"(g.b[1][2]), [x2] "v"(dx[2]), [b03] "v"(g.b[0][3]), [b13] "v"(g.b[1][3]), [x3] "v"(dx[3]), \
            [b04] "v"(g.b[0][4]), [b14] "v"(g.b[1][4]), [x4] "v"(dx[4]), [b05] "v"(g.b[0][5]), \
            [b15] "v"(g.b[1][5]), [x5] "v"(dx[5]), [b06] "v"(g.b[0][6]), [b16] "v"(g.b[1][6]), [x6] "v"(dx[6]), \
            [b07] "v"(g.b[0][7]), [b17] "v"(g.b[1][7]), [x7] "v"(dx[7]), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    }
}

// P[r] += (C_1[r] of token TAU) * h_1 for every rank r (P[r] already holds C_0[r] * h_0).
template <int TAU, int R>
__device__ __forceinline__ void mimo_output_tail(const BcRegs<R> &g, float h_1, float (&P)[R]) {
    if constexpr (R == 2) {
#define BODY JSCAN_F(p0, c0, h) JSCAN_F(p1, c1, h)
#define OUTS [p0] "+v"(P[0]), [p1] "+v"(P[1])
#define INS [c0] "v"(g.c[1][0]), [c1] "v"(g.c[1][1]), [h] "v"(h_1), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    } else if constexpr (R == 4) {
#define BODY JSCAN_F(p0, c0, h) JSCAN_F(p1, c1, h) JSCAN_F(p2, c2, h) JSCAN_F(p3, c3, h)
#define OUTS [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [p3] "+v"(P[3])
#define INS [c0] "v"(g.c[1][0]), [c1] "v"(g.c[1][1]), [c2] "v"(g.c[1][2]), [c3] "v"(g.c[1][3]), [h] "v"(h_1), \
            [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    } else {
#define BODY JSCAN_F(p0, c0, h) JSCAN_F(p1, c1, h) JSCAN_F(p2, c2, h) JSCAN_F(p3, c3, h) \
             JSCAN_F(p4, c4, h) JSCAN_F(p5, c5, h) JSCAN_F(p6, c6, h) JSCAN_F(p7, c7, h)
#define OUTS [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [p3] "+v"(P[3]), [p4] "+v"(P[4]), \
             [p5] "+v"(P[5]), [p6] "+v"(P[6]), [p7] "+v"(P[7])
#define INS [c0] "v"(g.c[1][0]), [c1] "v"(g.c[1][1]), [c2] "v"(g.c[1][2]), [c3] "v"(g.c[1][3]), \
            [c4] "v"(g.c[1][4]), [c5] "v"(g.c[1][5]), [c6] "v"(g.c[1][6]), [c7] "v"(g.c[1][7]), [h] "v"(h_1), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    }
}

// The trapezoidal left end point: h_s += (B_prev_s[r] of token TAU) * p[r], r increasing, as
// mimo_left_in().
template <int TAU, int R>
__device__ __forceinline__ void mimo_left_tail(const BcRegs<R> &g, const float (&pl)[R], float &h_0, float &h_1) {
    if constexpr (R == 2) {
#define BODY JSCAN_F(h0, q00, p0) JSCAN_F(h1, q10, p0) JSCAN_F(h0, q01, p1) JSCAN_F(h1, q11, p1)
#define OUTS [h0] "+v"(h_0), [h1] "+v"(h_1)
#define INS [q00] "v"(g.bp[0][0]), [q10] "v"(g.bp[1][0]), [p0] "v"(pl[0]), [q01] "v"(g.bp[0][1]), \
            [q11] "v"(g.bp[1][1]), [p1] "v"(pl[1]), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    } else {
        static_assert(R == 4, "the trapezoidal rule runs rank 2 or 4 here");
#define BODY JSCAN_F(h0, q00, p0) JSCAN_F(h1, q10, p0) JSCAN_F(h0, q01, p1) JSCAN_F(h1, q11, p1) \
             JSCAN_F(h0, q02, p2) JSCAN_F(h1, q12, p2) JSCAN_F(h0, q03, p3) JSCAN_F(h1, q13, p3)
#define OUTS [h0] "+v"(h_0), [h1] "+v"(h_1)
#define INS [q00] "v"(g.bp[0][0]), [q10] "v"(g.bp[1][0]), [p0] "v"(pl[0]), [q01] "v"(g.bp[0][1]), \
            [q11] "v"(g.bp[1][1]), [p1] "v"(pl[1]), [q02] "v"(g.bp[0][2]), [q12] "v"(g.bp[1][2]), [p2] "v"(pl[2]), \
            [q03] "v"(g.bp[0][3]), [q13] "v"(g.bp[1][3]), [p3] "v"(pl[3]), [k] "i"(TAU)
        JSCAN_ASM_K(TAU)
#undef BODY
#undef OUTS
#undef INS
    }
}
#undef JSCAN_ASM_K
#undef JSCAN_F
#undef JSCAN_RB

// One token (TAU within its 16-token group): advance the lane's two states and leave the R
// partial outputs (C h summed over the two states) in P.  The rank-R input of state n is
// dx_0 B[n][0] then + dx_r B[n][r] in increasing r, with B broadcast from lane TAU; this is
// mimo_input(), bit for bit.
template <int TAU, int R, AForm AF, bool kTrap>
__device__ __forceinline__ void mimo_token(const BcRegs<R> &g, const float (&dx)[R], const float (&pl)[R], float dv,
                                           float &h_0, float &h_1, float a2_0, float a2_1, float (&P)[R]) {
    if constexpr (kTrap) mimo_left_tail<TAU, R>(g, pl, h_0, h_1);   // h + sum_r p_r B_prev[r]
    float u0 = row_bcast<TAU>(g.b[0][0]) * dx[0];
    float u1 = row_bcast<TAU>(g.b[1][0]) * dx[0];
    mimo_input_tail<TAU, R>(g, dx, u0, u1);
    if constexpr (AF == AForm::ComplexPairs) {
        advance_complex_input(h_0, h_1, dv, ComplexA{a2_0, a2_1}, u0, u1);
    } else if constexpr (AF == AForm::ScaledIdentity) {
        h_0 = advance_input(h_0, dv, u0);
        h_1 = advance_input(h_1, dv, u1);
    } else {
        h_0 = advance_input(h_0, decay(dv, a2_0), u0);
        h_1 = advance_input(h_1, decay(dv, a2_1), u1);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) P[r] = row_bcast<TAU>(g.c[0][r]) * h_0;
    mimo_output_tail<TAU, R>(g, h_1, P);
}

// Four tokens TQ .. TQ + 3 of a group, then their 4R partials summed over the wave's rows, two
// reductions of four partials interleaved.  Without the trapezoidal rule and with a real state,
// a pair takes ranks 2p and 2p + 1 of the four tokens, so that row j ends with both ranks of
// token {0,2,1,3}[j] and stores them as one 8-byte write (1-3% faster there, 2% slower in the
// other two modes); otherwise a group is four consecutive partials i0 .. i0 + 3 (i = token * R +
// rank) and row j holds i0 + {0,2,1,3}[j].  The sums are the same either way.
// and written to this wave's half of the y exchange.
template <int TQ, int R, AForm AF, bool kTrap>
__device__ __forceinline__ void mimo_quarter(const BcRegs<R> &g, const QuarterRegs<R> &q, float &h_0, float &h_1,
                                             float a2_0, float a2_1, float *ys, int tq0, int rt, int ch) {
    using C = mrows::Cfg<R, kTrap>;
    float P[4][R];
    mimo_token<TQ + 0, R, AF, kTrap>(g, q.dx[0], q.p[0], q.dl.x, h_0, h_1, a2_0, a2_1, P[0]);
    mimo_token<TQ + 1, R, AF, kTrap>(g, q.dx[1], q.p[1], q.dl.y, h_0, h_1, a2_0, a2_1, P[1]);
    mimo_token<TQ + 2, R, AF, kTrap>(g, q.dx[2], q.p[2], q.dl.z, h_0, h_1, a2_0, a2_1, P[2]);
    mimo_token<TQ + 3, R, AF, kTrap>(g, q.dx[3], q.p[3], q.dl.w, h_0, h_1, a2_0, a2_1, P[3]);
    if constexpr (!kTrap && AF != AForm::ComplexPairs) {
#pragma unroll
        for (int p = 0; p < R / 2; ++p) {   // ranks 2p and 2p + 1 of the four tokens, interleaved
            const float Q[8] = {P[0][2 * p], P[1][2 * p], P[2][2 * p], P[3][2 * p],
                                P[0][2 * p + 1], P[1][2 * p + 1], P[2][2 * p + 1], P[3][2 * p + 1]};
            float sa, sb;
            reduce_rows4x2(Q, sa, sb);
            *reinterpret_cast<float2 *>(ys + (tq0 + rt) * C::kYS + ch * R + 2 * p) = make_float2(sa, sb);
        }
    } else {
#pragma unroll
        for (int m = 0; m < R; m += 2) {   // two groups of four partials at a time, interleaved
            const int i0 = 4 * m;
            float Q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) Q[j] = P[(i0 + j) / R][(i0 + j) % R];
            float sa, sb;
            reduce_rows4x2(Q, sa, sb);
            const int ia = i0 + rt, ib = i0 + 4 + rt;
            ys[(tq0 + ia / R) * C::kYS + ch * R + (ia % R)] = sa;
            ys[(tq0 + ib / R) * C::kYS + ch * R + (ib % R)] = sb;
        }
    }
}

template <typename E, AForm AF, int R, bool kTrap = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mimo_rows_kernel(
    const typename E::store_t *__restrict__ x, const typename E::store_t *__restrict__ dl,
    const float *__restrict__ A, const typename E::store_t *__restrict__ B, const typename E::store_t *__restrict__ C,
    const float *__restrict__ h0, typename E::store_t *__restrict__ y, float *__restrict__ h_final, int64_t L, int D,
    int blocks_per_row, int xcd_stride, Trap tr) {
    using Cf = mrows::Cfg<R, kTrap>;
    constexpr int kT = Cf::kT;
    __shared__ __attribute__((aligned(16))) float dx_s[2][Cf::kDxSize];
    __shared__ __attribute__((aligned(16))) float dl_s[2][Cf::kDlSize];
    __shared__ __attribute__((aligned(16))) float bc_s[2][Cf::kBcTiles * Cf::kBcSize];
    __shared__ __attribute__((aligned(16))) float y_s[2][Cf::kYSize];
    __shared__ __attribute__((aligned(16))) float p_s[2][kTrap ? Cf::kDxSize : 4];

    int wg = blockIdx.x;
    if (xcd_stride > 0) wg = (wg & 7) * xcd_stride + (wg >> 3);
    const int b = wg / blocks_per_row;
    const int d0 = (wg - b * blocks_per_row) * Cf::kCh;
    const int ntiles = (int)((L + kT - 1) / kT);
    using S = typename E::store_t;

    if (threadIdx.x >= Cf::kHalf) {
        // ---------------- helper waves ----------------
        const int tid = threadIdx.x - Cf::kHalf;
        const S *xb = x + (int64_t)b * L * D * R + (int64_t)d0 * R;
        const S *db = dl + (int64_t)b * L * D + d0;
        const S *bcb = (tid < 128 ? B : C) + (int64_t)b * L * kDState * R;
        S *yb = y + (int64_t)b * L * D * R + (int64_t)d0 * R;
        float a2c[Cf::kCPT];
#pragma unroll
        for (int ci = 0; ci < Cf::kCPT; ++ci)
            a2c[ci] = AF == AForm::ScaledIdentity ? scaled_A(A[d0 + (tid % Cf::kTPT) * Cf::kCPT + ci]) : 0.0f;
        // trapezoidal rule: lam, and the caller's previous token (or stand-ins staged as zero)
        const bool prev_given = kTrap && tr.x_prev != nullptr;
        MimoPrev<E> pr{nullptr, nullptr, nullptr, prev_given};
        if constexpr (kTrap) {
            const int c0 = (tid % Cf::kTPT) * Cf::kCPT;
            int tb, s0;
            bc_thread<R, kTrap>(tid, tb, s0);
            (void)tb;
            pr.lam = static_cast<const S *>(tr.lam) + (int64_t)b * L * D + d0;
            pr.x = prev_given ? static_cast<const S *>(tr.x_prev) + ((int64_t)b * D + d0 + c0) * R : xb + c0 * R;
            pr.bc = prev_given ? static_cast<const S *>(tr.B_prev) + ((int64_t)b * kDState + s0) * R : bcb + s0 * R;
        }
        MimoTileRegs<E, R, kTrap> Rg[2];
        mimo_load_tile<E, R, kTrap>(Rg[0], xb, db, bcb, 0, L, D, tid, pr);
        mimo_stage_tile<E, R, AF, kTrap>(Rg[0], dx_s[0], dl_s[0], bc_s[0], p_s[0], 0, L, tid, a2c, prev_given);
        mimo_load_tile<E, R, kTrap>(Rg[1], xb, db, bcb, kT, L, D, tid, pr);
        mimo_load_tile<E, R, kTrap>(Rg[0], xb, db, bcb, 2 * kT, L, D, tid, pr);
        __syncthreads();
        auto tile = [&](auto cur_c, int k) {
            constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
            if (k + 1 < ntiles) {
                mimo_stage_tile<E, R, AF, kTrap>(Rg[nxt], dx_s[nxt], dl_s[nxt], bc_s[nxt], p_s[nxt],
                                                 (int64_t)(k + 1) * kT, L, tid, a2c, prev_given);
                if (k + 3 < ntiles)
                    mimo_load_tile<E, R, kTrap>(Rg[nxt], xb, db, bcb, (int64_t)(k + 3) * kT, L, D, tid, pr);
            }
            if (k > 0) mimo_write_final<E, R, kTrap>(y_s[nxt], yb, (int64_t)(k - 1) * kT, L, D, tid);
            __syncthreads();
        };
        for (int k = 0; k < ntiles; k += 2) {
            tile(IntConst<0>{}, k);
            if (k + 1 < ntiles) tile(IntConst<1>{}, k + 1);
        }
        mimo_write_final<E, R, kTrap>(y_s[(ntiles - 1) & 1], yb, (int64_t)(ntiles - 1) * kT, L, D, tid);
        return;
    }

    // ---------------- scan waves ----------------
    __builtin_amdgcn_s_setprio(3);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;
    const int cg = wave >> 1, sh = wave & 1;
    const int ch = 16 * cg + c;
    const int d = d0 + ch;
    const int n0 = 8 * sh + 2 * r;
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
        const float2 hv = *reinterpret_cast<const float2 *>(h0 + ((int64_t)b * D + d) * kDState + n0);
        h_0 = hv.x;
        h_1 = hv.y;
    }
    const int rt = (r == 1) ? 2 : (r == 2) ? 1 : r;   // partial slot of this row after reduce_rows4
    __syncthreads();   // tile 0 staged
    auto tile = [&](auto cur_c, int k) {
        constexpr int cur = decltype(cur_c)::value;
        float *ys = y_s[cur] + sh * kT * Cf::kYS;
        const float *dxc = dx_s[cur], *dlc = dl_s[cur], *bcc = bc_s[cur], *psc = p_s[cur];
        BcRegs<R> g[2];
        QuarterRegs<R> qa, qb;
        mimo_load_bc<R, kTrap>(g[0], bcc, 0, n0, c);
        mimo_load_quarter<R, kTrap>(qa, dxc, dlc, psc, 0, ch);
        mimo_load_quarter<R, kTrap>(qb, dxc, dlc, psc, 4, ch);
#pragma unroll
        for (int tg = 0; tg < kT; tg += 16) {
            const BcRegs<R> &gc = g[(tg >> 4) & 1];
            mimo_quarter<0, R, AF, kTrap>(gc, qa, h_0, h_1, a2_0, a2_1, ys, tg, rt, ch);
            mimo_load_quarter<R, kTrap>(qa, dxc, dlc, psc, tg + 8, ch);
            if (tg + 16 < kT) mimo_load_bc<R, kTrap>(g[((tg >> 4) + 1) & 1], bcc, tg + 16, n0, c);
            mimo_quarter<4, R, AF, kTrap>(gc, qb, h_0, h_1, a2_0, a2_1, ys, tg + 4, rt, ch);
            mimo_load_quarter<R, kTrap>(qb, dxc, dlc, psc, tg + 12, ch);
            mimo_quarter<8, R, AF, kTrap>(gc, qa, h_0, h_1, a2_0, a2_1, ys, tg + 8, rt, ch);
            if (tg + 16 < kT) mimo_load_quarter<R, kTrap>(qa, dxc, dlc, psc, tg + 16, ch);
            mimo_quarter<12, R, AF, kTrap>(gc, qb, h_0, h_1, a2_0, a2_1, ys, tg + 12, rt, ch);
            if (tg + 16 < kT) mimo_load_quarter<R, kTrap>(qb, dxc, dlc, psc, tg + 20, ch);
        }
        __syncthreads();
        (void)k;
    };
    for (int k = 0; k < ntiles; k += 2) {
        tile(IntConst<0>{}, k);
        if (k + 1 < ntiles) tile(IntConst<1>{}, k + 1);
    }
    *reinterpret_cast<float2 *>(h_final + ((int64_t)b * D + d) * kDState + n0) = make_float2(h_0, h_1);
}

// The row-mapped MIMO kernel needs whole 32-channel blocks (and, with the trapezoidal rule,
// rank 2 or 4: rank 8 would not fit its LDS areas).
inline bool mimo_rows_kernel_applies(int64_t D, int64_t R, bool trap = false) {
    return D % 32 == 0 && (R == 2 || R == 4 || (R == 8 && !trap));
}

template <typename E, AForm AF, int R, bool kTrap = false>
void launch_prefill_mimo_rows(const typename E::store_t *x, const typename E::store_t *dl, const float *A,
                              const typename E::store_t *B, const typename E::store_t *C, const float *h0,
                              typename E::store_t *y, float *h_final, int64_t batch, int64_t L, int D,
                              hipStream_t stream, Trap tr = Trap{nullptr, nullptr, nullptr}) {
    const int blocks_per_row = D / mrows::Cfg<R, kTrap>::kCh;
    const int64_t blocks = batch * blocks_per_row;
    const int xcd_stride = (blocks % 8 == 0) ? (int)(blocks / 8) : 0;
    hipLaunchKernelGGL((prefill_mimo_rows_kernel<E, AF, R, kTrap>), dim3((unsigned)blocks),
                       dim3(mrows::Cfg<R, kTrap>::kThreads), 0, stream, x, dl, A, B, C, h0, y, h_final, L, D,
                       blocks_per_row, xcd_stride, tr);
}

}  // namespace jscan
