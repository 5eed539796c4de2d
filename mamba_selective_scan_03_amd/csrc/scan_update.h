// scan_update.h - the one definition of how a state element advances by one token.
//
// Every kernel of the library (prefill, resume, decode step) advances state elements only
// through the functions below (`advance()` for the diagonal A), so they all compute
// bit-identical fp32 states for the same tokens.  That is what lets a prefill's final state equal, bit for bit, the state after
// the same tokens fed one at a time through the decode step.
//
// With a scaled-identity A (one value a[d] for all 16 states of a channel, the Mamba-2 form)
// the decay 2^(delta * a2[d]) is the same for the whole channel.  The kernels for that form
// evaluate it once per (token, channel) with the same `decay()` and hand it to
// `advance_decayed()`, which is the second half of `advance()`: their states are therefore
// bit-identical to the general kernels' run on A[d][n] = a[d].  A complex-valued state (the
// Mamba-3 form) advances through `advance_complex()`, the one definition of that update.  The
// exponential-trapezoidal rule takes the previous token's input in first (`trap_left_in()`,
// `mimo_left_in()`), and a MIMO scan forms its rank-R input with `mimo_input()` and advances
// through `advance_input()` / `advance_complex_input()`: each form has one definition here.
//
// The recurrence is the S6 equation of the Jamba notes page ("Jamba: A Hybrid
// Transformer-Mamba Language Model", section "Mamba layer"):
//     h_t = Abar_t h_{t-1} + Bbar_t x_t,   Abar_t = exp(delta_t A),   Bbar_t x_t = delta_t B_t x_t
// with A real and diagonal (lesson page "Jamba - Hybrid SSM-Transformer", section "Mamba-3").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jscan {

constexpr int kDState = 16;
constexpr float kLog2e = 1.44269504088896340736f;

// A2 = A * log2(e), rounded once to fp32, so that exp(delta * A) = 2^(delta * A2).
__device__ __forceinline__ float scaled_A(float a) { return a * kLog2e; }

// The decay Abar = exp(delta * A), evaluated by the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float decay(float delta, float a2) {
    return __builtin_amdgcn_exp2f(delta * a2);
}

// The fp32 product delta * x, shared by the 16 states of one channel.
__device__ __forceinline__ float delta_x(float delta, float x) { return delta * x; }

// One state element advanced by one token, given its decay and its input term u:  h <- Abar * h + u.
__device__ __forceinline__ float advance_input(float h, float abar, float u) { return __builtin_fmaf(abar, h, u); }

// The same with the single-input term u = (delta * x) * B.
__device__ __forceinline__ float advance_decayed(float h, float abar, float dx, float b) {
    return advance_input(h, abar, dx * b);
}

// Multi-input (MIMO) term of one state element: u = sum_r (delta * x_r) * B[r], accumulated in
// increasing r (the first product rounded, then one fused multiply-add per rank).  With R = 1
// it is the single-input term (delta * x) * B.
template <int R>
__device__ __forceinline__ float mimo_input(const float (&dx)[R], const float *b) {
    float u = dx[0] * b[0];
#pragma unroll
    for (int r = 1; r < R; ++r) u = __builtin_fmaf(dx[r], b[r], u);
    return u;
}

// The same with the decay evaluated here, from delta and A2.
__device__ __forceinline__ float advance(float h, float delta, float a2, float dx, float b) {
    return advance_decayed(h, decay(delta, a2), dx, b);
}

// ---- forms of A -------------------------------------------------------------------------
// Diagonal: one value per (channel, state), the Mamba-1 form.  ScaledIdentity: one value per
// channel for all its states, the Mamba-2 form (A[d][n] = a[d]).  ComplexPairs: the state is
// complex, the Mamba-3 form (lesson page "Jamba - Hybrid SSM-Transformer", section "Mamba-3",
// item 2): states 2k and 2k+1 of a channel are the real and imaginary parts of one complex
// state, and A[d][2k], A[d][2k+1] the real and imaginary parts of its diagonal entry; B and C
// pair up the same way.
enum class AForm : int { Diagonal, ScaledIdentity, ComplexPairs };

constexpr float kInv2Pi = 0.159154943091895335769f;   // 1 / (2 pi), rounded to fp32

// A complex diagonal entry a = re + i im, prepared once: A2 = re * log2(e) for the modulus of
// the decay and im / (2 pi) for its angle in turns (what v_sin_f32 / v_cos_f32 take).
struct ComplexA {
    float a2, turns;
};
__device__ __forceinline__ ComplexA complex_A(float re, float im) { return ComplexA{re * kLog2e, im * kInv2Pi}; }

// One complex state (h_re, h_im) advanced by one token:  h <- exp(delta a) h + (delta x) b, with
// exp(delta a) = 2^(delta A2) (cos phi + i sin phi), phi = delta im in turns, reduced to [0, 1)
// first so that the hardware sine and cosine see a small argument.  The real-part update is
// fma(r cos, h_re, fma(-r sin, h_im, (delta x) b_re)), the imaginary one mirrors it.
// The same given the complex input term u = (u_re, u_im), which is (delta x) b above and the
// rank-R sum of such terms in a MIMO scan.
__device__ __forceinline__ void advance_complex_input(float &h_re, float &h_im, float delta, ComplexA a, float u_re,
                                                      float u_im) {
    const float r = decay(delta, a.a2);
    const float phi = __builtin_amdgcn_fractf(delta * a.turns);
    const float rc = r * __builtin_amdgcn_cosf(phi), rs = r * __builtin_amdgcn_sinf(phi);
    const float re = __builtin_fmaf(rc, h_re, __builtin_fmaf(-rs, h_im, u_re));
    const float im = __builtin_fmaf(rc, h_im, __builtin_fmaf(rs, h_re, u_im));
    h_re = re;
    h_im = im;
}
__device__ __forceinline__ void advance_complex(float &h_re, float &h_im, float delta, ComplexA a, float dx,
                                                float b_re, float b_im) {
    advance_complex_input(h_re, h_im, delta, a, dx * b_re, dx * b_im);
}

// ---- exponential-trapezoidal rule (the Mamba-3 discretisation) ------------------------------
// Lesson page "Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 1: the input term mixes
// neighbouring tokens.  Over step t the input integral is weighted lam_t at the right end point
// (this token) and 1 - lam_t at the left end point (the previous token), which decays with the
// state over the whole step:
//     h_t = Abar_t (h_{t-1} + p_t B_{t-1}) + q_t B_t,   p_t = ((1 - lam_t) delta_t) x_{t-1},
//                                                     q_t = (lam_t delta_t) x_t
// Every kernel takes the left end point in first, k = fma(p_t, B_{t-1}, h), then advances k by
// its form's update with q_t in place of delta_t * x_t.  lam = 1 gives p = 0 and q = delta * x.
__device__ __forceinline__ float trap_right(float delta, float lam, float x) { return (lam * delta) * x; }
__device__ __forceinline__ float trap_left(float delta, float lam, float x_prev) {
    return ((1.0f - lam) * delta) * x_prev;
}
__device__ __forceinline__ float trap_left_in(float h, float p, float b_prev) { return __builtin_fmaf(p, b_prev, h); }

// The left end point of a MIMO step: k = h + sum_r p_r B_prev[r], taken in onto h in increasing r
// (one fused multiply-add per rank).  With R = 1 it is trap_left_in().
template <int R>
__device__ __forceinline__ float mimo_left_in(float h, const float (&p)[R], const float *b_prev) {
    float k = h;
#pragma unroll
    for (int r = 0; r < R; ++r) k = __builtin_fmaf(p[r], b_prev[r], k);
    return k;
}

// The extra inputs of a trapezoidal prefill, in the dtype of x: lam [tokens][D] like delta, and
// the token before each row's first one, x_prev [rows][D] and B_prev [rows][16] (both null when
// there is none: its term is then zero).
struct Trap {
    const void *lam;
    const void *x_prev;
    const void *B_prev;
};

// A compile-time integer as a value: lets an unrolled loop body pick register sets and LDS
// buffers by constant index.
template <int V> struct IntConst {
    static constexpr int value = V;
};

// ---- rows of work ----------------------------------------------------------------------

// The prefill kernels walk "rows": a run of consecutive tokens of one sequence, scanned in
// order from a given initial state.  A plain prefill has one row per sequence.  The
// time-parallel prefill cuts each sequence into segments of seg_len tokens (the last one may
// be shorter) and gives every segment a row of its own; row v is segment v % n_seg of
// sequence v / n_seg.  Initial states are indexed by row.  Final states are indexed by row
// too, unless final_by_sequence is set: then only the last segment of each sequence writes
// its final state, at that sequence's index.
struct Segments {
    int64_t L;              // tokens per sequence
    int64_t seg_len;        // tokens per segment (L for a plain prefill)
    int n_seg;              // segments per sequence, ceil(L / seg_len)
    int final_by_sequence;  // see above
};

struct RowSpan {
    int64_t tok0;  // index of the row's first token in the [batch][L] token order
    int64_t len;   // tokens in the row (>= 1)
    int state;     // index of the row's final state, or -1 if it writes none
};

__device__ __forceinline__ RowSpan row_span(const Segments &sg, int row) {
    const int seq = row / sg.n_seg, seg = row - seq * sg.n_seg;
    const int64_t t_begin = (int64_t)seg * sg.seg_len;
    RowSpan r;
    r.tok0 = (int64_t)seq * sg.L + t_begin;
    r.len = min(sg.seg_len, sg.L - t_begin);
    r.state = !sg.final_by_sequence ? row : (seg == sg.n_seg - 1 ? seq : -1);
    return r;
}

// ---- element formats -------------------------------------------------------------------

// bf16 -> fp32 is exact: the 16 stored bits are the high half of the fp32 pattern.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Storage traits: F32 stores float, BF16 stores the 16-bit pattern.
struct F32 {
    using store_t = float;
    static __device__ __forceinline__ float load(const store_t *p) { return *p; }
    static __device__ __forceinline__ void store(store_t *p, float v) { *p = v; }
};
struct BF16 {
    using store_t = uint16_t;
    static __device__ __forceinline__ float load(const store_t *p) { return bf16_bits_to_f32(*p); }
    static __device__ __forceinline__ void store(store_t *p, float v) { *p = f32_to_bf16_bits(v); }
};

}  // namespace jscan
