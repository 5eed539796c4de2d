/*
 * jscan.h - C ABI of libjscan, the Mamba-1 (S6) selective state-space scan on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  For every batch row b, channel d < D and state n < N = 16, the scan
 * runs the selective recurrence of the Jamba notes page ("Jamba: A Hybrid
 * Transformer-Mamba Language Model", section "Mamba layer", the S6 equation):
 *
 *     h_t[d,n] = exp(delta_t[d] * A[d,n]) * h_{t-1}[d,n] + (delta_t[d] * x_t[d]) * B_t[n]
 *     y_t[d]   = sum_n C_t[n] * h_t[d,n]
 *
 * The decay exp(delta A) and the input term delta B x are the discretised A-bar and
 * B-bar x of that equation.  delta, B and C are inputs that depend on the token (same
 * section).  A is real and diagonal, one value per (channel, state) (lesson page
 * "Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 2).  d_state is 16 (notes
 * page, "Mamba layer").  Only h_{t-1} and the current token are needed to advance one
 * token, so decoding runs in constant memory (lesson page, section "SSM on one page").
 *
 * Arithmetic.  The state is fp32 and is never rounded to the input dtype.  Every state
 * element is advanced by the same fp32 expression in every entry point:
 *     h = fmaf(exp2(delta * A2), h, (delta * x) * B),   with A2 = A * log2(e) in fp32,
 * and exp2 is the hardware v_exp_f32.  Tokens are visited in increasing t, one after the
 * other.  So the state that jscan_prefill returns is bit-identical to the state after L
 * calls of jscan_step on the same tokens, starting from +0.0.  y accumulates in fp32 and is
 * rounded to nearest even to the output dtype.  With bf16 output the prefill's sum over the
 * states runs on the matrix cores: its terms are rounded to bf16 once (2^-9 relative) and
 * summed in fp32 (the products C_t[n] h_t[d,n] with h rounded, or, in jscan_prefill_fused, the
 * lanes' fp32 partial sums over two states).  A NaN in a channel's state then also reaches
 * that channel's outputs earlier in the same 16-token group (a NaN term times a zero weight of
 * the summing matrix), never another channel.
 *
 * Layouts.  All arrays are row-major with the last index contiguous:
 *     x, delta, y : [batch][L][D]      B, C : [batch][L][N]
 *     A           : [D][N] fp32        h0, h, h_final : [batch][D][N] fp32
 * x, delta, B, C and y share one dtype (jscan_dtype).
 *
 * Ownership and execution.  Every array pointer is a DEVICE pointer that the caller
 * allocates, owns and frees.  The library allocates no memory, keeps no state between
 * calls and never synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL means
 * the default stream), and results are valid once that stream has been synchronised.
 * Calls on different streams may run from different host threads.
 *
 * Errors.  Arguments are checked before anything is launched.  On any error nothing is
 * launched and no output is touched.
 *     JSCAN_ERR_NULL   a required pointer is NULL
 *     JSCAN_ERR_SHAPE  negative sizes, N != 16, D not a multiple of 8, a row stride
 *                      shorter than its row or not a multiple of 8, D above 2^24 or batch
 *                      above 2^20 (the kernels index channels and rows in 32 bits)
 *     JSCAN_ERR_DTYPE  unknown dtype
 *     JSCAN_ERR_ALIGN  an array pointer not 16-byte aligned
 *     JSCAN_ERR_ALIAS  an output overlaps an input or another output (the exceptions are
 *                      the in-place state of jscan_step, and h0 == h_final exactly for
 *                      jscan_prefill_resume)
 *     JSCAN_ERR_HIP    the launch failed; jscan_last_hip_error() gives the hipError_t
 *     JSCAN_ERR_WORKSPACE  the workspace passed to jscan_prefill_chunked is too small
 *     JSCAN_ERR_FORM   unknown form of A (jscan_a_form)
 * Faults inside a kernel surface at the caller's next synchronisation.  A is not
 * range-checked.  With delta >= 0 and A <= 0 the decay lies in (0, 1] and the recurrence
 * is stable; other values may overflow.  Zero-sized work (batch == 0 or D == 0) returns
 * JSCAN_OK without touching anything.
 */
#ifndef JSCAN_H
#define JSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JSCAN_OK = 0,
    JSCAN_ERR_NULL = 1,
    JSCAN_ERR_SHAPE = 2,
    JSCAN_ERR_DTYPE = 3,
    JSCAN_ERR_ALIGN = 4,
    JSCAN_ERR_ALIAS = 5,
    JSCAN_ERR_HIP = 6,
    JSCAN_ERR_WORKSPACE = 7,
    JSCAN_ERR_FORM = 8
} jscan_status;

/* dtype of x, delta, B, C and y.  A and every state are always fp32. */
typedef enum { JSCAN_F32 = 0, JSCAN_BF16 = 1 } jscan_dtype;

#define JSCAN_D_STATE 16

/*
 * Prefill: scan L tokens from the zero state.  Writes y for every token and the state after
 * the last token.
 *   x, delta [batch][L][D]   inputs (delta is used as given: no softplus or bias is applied)
 *   A        [D][N]          fp32 diagonal of A
 *   B, C     [batch][L][N]   inputs
 *   y        [batch][L][D]   output, same dtype as x
 *   h_final  [batch][D][N]   output fp32 state after token L-1 (zeros when L == 0)
 * With L == 0, x, delta, B, C and y may be NULL.
 */
jscan_status jscan_prefill(const void *x, const void *delta, const float *A, const void *B,
                           const void *C, void *y, float *h_final, int64_t batch, int64_t L,
                           int64_t D, int64_t N, jscan_dtype dtype, void *stream);

/*
 * Prefill from a caller-supplied state h0 [batch][D][N] fp32 instead of zeros.  This resumes
 * a scan: scanning tokens [0, L1) and then resuming over [L1, L) gives bit-identical y and
 * h_final to one prefill over [0, L).  h0 may equal h_final (an in-place update of the
 * state) but must not partly overlap it.  The other arguments are as for jscan_prefill.
 */
jscan_status jscan_prefill_resume(const void *x, const void *delta, const float *A,
                                  const void *B, const void *C, const float *h0, void *y,
                                  float *h_final, int64_t batch, int64_t L, int64_t D,
                                  int64_t N, jscan_dtype dtype, void *stream);

/*
 * Time-parallel prefill, for shapes whose batch * D channels are too few to fill the GPU
 * (a single sequence of a channel-sharded layer, for example).  Same inputs and outputs as
 * jscan_prefill_resume (h0 may be NULL for the zero state, and may equal h_final), computed
 * in three passes over segments of `chunk` tokens:
 *   1. every segment is scanned from the zero state, giving its end state h_loc[s] and,
 *      per channel, the sum of its delta values S[s];
 *   2. the segments' starting states follow in order from h_in[0] = h0 by composing the
 *      per-segment maps: h_in[s+1] = exp(A * S[s]) * h_in[s] + h_loc[s];
 *   3. every segment is scanned again from h_in[s], writing y and (last segment) h_final.
 * Pass 2 rests on the recurrence being affine in h: over a run of tokens the map
 * h -> exp(delta A) h + delta B x composes to h -> exp(A * sum delta) h + h_loc, where h_loc
 * is the run's end state from zero (S6 equation, notes page "Jamba: A Hybrid
 * Transformer-Mamba Language Model", section "Mamba layer").
 * Rounding: with fp32 output the first segment's y is bit-identical to jscan_prefill_resume's
 * (with bf16 output it agrees to the rounding of the prefill's sum over states); later
 * segments start from composed states whose rounding differs from the token-by-token walk,
 * so their y and h_final agree with it to within fp32 rounding of the composition, not bit
 * for bit.  Results are deterministic (no atomics; fixed summation orders).
 *   chunk      tokens per segment; 0 picks enough segments for four waves per SIMD (262144
 *              segment-channel lanes, segments of at least 256 tokens), or one segment when
 *              batch * D already fills the GPU (at least 8192 channels, D a multiple of 32).  When it yields a
 *              single segment the call is exactly jscan_prefill_resume (and needs no
 *              workspace).
 *   workspace  device memory of at least jscan_prefill_chunked_workspace(...) bytes,
 *              16-byte aligned, owned by the caller, not overlapping any other array;
 *              may be NULL when that size is 0.  Its contents on entry do not matter.
 * Calls that share a workspace must be ordered on one stream.
 */
jscan_status jscan_prefill_chunked(const void *x, const void *delta, const float *A,
                                   const void *B, const void *C, const float *h0, void *y,
                                   float *h_final, int64_t batch, int64_t L, int64_t D,
                                   int64_t N, int64_t chunk, void *workspace,
                                   int64_t workspace_bytes, jscan_dtype dtype, void *stream);

/*
 * Workspace bytes jscan_prefill_chunked needs for this shape and chunk (0 when it runs as
 * a single segment), or -1 if the shape or chunk is invalid.  Host-only; launches nothing.
 */
int64_t jscan_prefill_chunked_workspace(int64_t batch, int64_t L, int64_t D, int64_t N,
                                        int64_t chunk);

/*
 * Producer side: the scan's delta, B and C computed from x (bf16 only), for M tokens.
 * The notes page ("Jamba: A Hybrid Transformer-Mamba Language Model", section "Mamba layer")
 * makes these parameters functions of the input and applies RMSNorm in the Mamba layer;
 * they are computed as the selective projection of Mamba-1:
 *     [d_low | B | C] = W_x x_t                          (fp32 accumulation of bf16 products)
 *     d_low = rmsnorm(d_low) * g_delta,  B = rmsnorm(B) * g_B,  C = rmsnorm(C) * g_C,
 *             rmsnorm(v) = v / sqrt(mean(v^2) + eps) over each vector's own width
 *     delta = softplus(W_dt d_low + b_dt)
 * Each output is rounded once, to nearest even, from its fp32 value.  The products run on the
 * matrix cores (MFMA 16x16x32 bf16); the normalisation, bias and softplus run on the fp32
 * accumulators before the rounding.
 *   x          [M][D]      bf16, M = batch * L tokens in any order (rows are independent)
 *   w_x        [R + 2N][D] bf16: rows 0..R-1 give d_low, R..R+N-1 give B, R+N.. give C
 *   g_delta [R], g_B [N], g_C [N]   fp32 gains
 *   w_dt       [D][R]      bf16 (row d produces channel d)
 *   b_dt       [D]         fp32
 *   delta_low  [M][R]      out, bf16, the normalised d_low (also the input of the second product)
 *   delta      [M][D]      out, bf16;   B, C [M][N] out, bf16
 * R must be 64, 128 or 256; N = 16; D a multiple of 128; 0 <= M <= 2^31; eps in [0, 1].  dtype must be
 * JSCAN_BF16 (JSCAN_ERR_DTYPE otherwise).  Outputs must not overlap inputs or each other.
 * Two kernels are launched on `stream`, in order.  With delta == NULL only the first
 * product runs (delta_low, B and C; w_dt and b_dt may then be NULL): the input of
 * jscan_prefill_fused, which computes delta itself.
 */
jscan_status jscan_ssm_inputs(const void *x, const void *w_x, const float *g_delta, const float *g_B,
                              const float *g_C, const void *w_dt, const float *b_dt, void *delta_low,
                              void *delta, void *B, void *C, int64_t M, int64_t D, int64_t R,
                              int64_t N, float eps, jscan_dtype dtype, void *stream);

/*
 * Prefill with the second product of jscan_ssm_inputs folded into the scan's load path: delta
 * is never stored.  The kernel computes, tile by tile, delta = softplus(W_dt delta_low + b_dt)
 * with the same matrix-core sequence, bias add, softplus and bf16 rounding as
 * jscan_ssm_inputs, so h_final is bit-identical to jscan_ssm_inputs followed by
 * jscan_prefill_resume (jscan_prefill when h0 is NULL).  y agrees with it to the rounding of the
 * sum over states: this kernel's matrix cores also compute delta, so it sums the lanes' partials
 * there (half the MFMAs) rather than contracting the states with C.
 *   x          [batch][L][D] bf16      delta_low [batch][L][R] bf16 (from jscan_ssm_inputs)
 *   w_dt       [D][R] bf16             b_dt [D] fp32
 *   A, B, C, h0 (may be NULL), y, h_final as for jscan_prefill_resume
 * Limits: bf16 only, R = 256, D a multiple of 32 (the shapes of the row-mapped prefill);
 * other shapes return JSCAN_ERR_SHAPE and are served by jscan_ssm_inputs then jscan_prefill.
 */
jscan_status jscan_prefill_fused(const void *x, const void *delta_low, const void *w_dt,
                                 const float *b_dt, const float *A, const void *B, const void *C,
                                 const float *h0, void *y, float *h_final, int64_t batch,
                                 int64_t L, int64_t D, int64_t N, int64_t R, jscan_dtype dtype,
                                 void *stream);

/*
 * Decode step: advance the state by one token, in place, and write that token's output.
 *   h        [batch][D][N] fp32, read and overwritten with the new state
 *   x_t, delta_t: batch rows of D values; row b starts at element b * ld_xd
 *   A        [D][N] fp32
 *   B_t, C_t: batch rows of N values; row b starts at element b * ld_bc
 *   y_t      batch rows of D values; row b starts at element b * ld_y; same dtype as x_t
 * The strides let a caller pass token t of prefill-layout tensors without a copy
 * (x + t*D with ld_xd = L*D, B + t*N with ld_bc = L*N), and write y_t either into a
 * prefill-layout output (y + t*D with ld_y = L*D) or into a contiguous [batch][D] (ld_y = D).
 * ld_xd >= D, ld_bc >= N, ld_y >= D, and all three must be multiples of 8.
 */
jscan_status jscan_step(float *h, const void *x_t, const void *delta_t, const float *A,
                        const void *B_t, const void *C_t, void *y_t, int64_t batch, int64_t D,
                        int64_t N, int64_t ld_xd, int64_t ld_bc, int64_t ld_y, jscan_dtype dtype,
                        void *stream);

/*
 * Scaled-identity A (the Mamba-2 form).  The lesson page ("Jamba - Hybrid SSM-Transformer",
 * section "Mamba-3", item 2) describes Mamba-2's state matrix as a scaled identity instead of
 * Mamba-1's real diagonal; everything else about the layer is taken to be unchanged (same
 * Euler-style input term, same delta, B, C and y).  So A is one value per channel:
 *     A[d][n] = a[d] for every n,   a [D] fp32.
 * The decay exp(delta_t[d] * a[d]) is then the same for all 16 states of a channel, and these
 * kernels evaluate it once per (token, channel) instead of once per state element, by the
 * same fp32 expression as the general kernels.  Their y, h_final and decode states are
 * therefore bit-identical to jscan_prefill_resume / jscan_step run on the expanded A[d][n] =
 * a[d], only faster.
 *
 * Prefill from h0 (NULL for the zero state; h0 may equal h_final).  The other arguments,
 * layouts and errors are those of jscan_prefill_resume, with `a` [D] fp32 in place of A.
 */
jscan_status jscan_prefill_scalar_a(const void *x, const void *delta, const float *a,
                                    const void *B, const void *C, const float *h0, void *y,
                                    float *h_final, int64_t batch, int64_t L, int64_t D,
                                    int64_t N, jscan_dtype dtype, void *stream);

/* Decode step with a scaled-identity A: jscan_step with `a` [D] fp32 in place of A. */
jscan_status jscan_step_scalar_a(float *h, const void *x_t, const void *delta_t, const float *a,
                                 const void *B_t, const void *C_t, void *y_t, int64_t batch,
                                 int64_t D, int64_t N, int64_t ld_xd, int64_t ld_bc,
                                 int64_t ld_y, jscan_dtype dtype, void *stream);

/*
 * Complex-valued state (the Mamba-3 form).  The lesson page ("Jamba - Hybrid SSM-Transformer",
 * section "Mamba-3", item 2) has Mamba-3 bring back a complex state matrix, which amounts to
 * multiplying the state by a data-dependent rotation.  Here the 16 real state components of a
 * channel are read as 8 complex states, h[k] = h[2k] + i h[2k+1], and A[d][2k], A[d][2k+1] as
 * the real and imaginary parts of its complex diagonal entry a; B and C pair up the same way.
 * The S6 equation in complex arithmetic then reads
 *     h_t[k] = exp(delta_t a) h_{t-1}[k] + (delta_t x_t) (B_t[2k] + i B_t[2k+1])
 *     y_t    = sum_n C_t[n] h_t[n]            (= sum_k Re(conj(c_k) h_t[k]))
 * with exp(delta a) = 2^(delta Re(a) log2 e) (cos(delta Im a) + i sin(delta Im a)): a decay by
 * the real part and a rotation by the imaginary part.  With every Im a = 0 this is the real
 * diagonal scan with A[d][2k+1] = A[d][2k].  Every entry point advances the pairs with the same
 * fp32 expression (hardware sine and cosine of the angle in turns, reduced to [0, 1)), so the
 * prefill's final state equals the step chain's bit for bit.  States, h0 and h_final keep the
 * [batch][D][16] fp32 layout with the pairs interleaved.  Re(a) <= 0 keeps the recurrence
 * stable; Im(a) is an angle rate in radians per unit of delta.  The other arguments, layouts
 * and errors are those of jscan_prefill_resume (h0 may be NULL) and jscan_step.
 */
jscan_status jscan_prefill_complex(const void *x, const void *delta, const float *A,
                                   const void *B, const void *C, const float *h0, void *y,
                                   float *h_final, int64_t batch, int64_t L, int64_t D,
                                   int64_t N, jscan_dtype dtype, void *stream);

/* Decode step with the complex-valued state (see jscan_prefill_complex). */
jscan_status jscan_step_complex(float *h, const void *x_t, const void *delta_t, const float *A,
                                const void *B_t, const void *C_t, void *y_t, int64_t batch,
                                int64_t D, int64_t N, int64_t ld_xd, int64_t ld_bc,
                                int64_t ld_y, jscan_dtype dtype, void *stream);

/*
 * Exponential-trapezoidal discretisation, the Mamba-3 replacement of the Euler rule (lesson
 * page "Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 1: the input term of the
 * recurrence mixes neighbouring tokens).  The input integral over step t is weighted lam_t at
 * the step's right end (this token) and 1 - lam_t at its left end (the previous token), which
 * decays with the state over the step:
 *
 *     h_t = exp(delta_t a) (h_{t-1} + ((1 - lam_t) delta_t) x_{t-1} B_{t-1}) + ((lam_t delta_t) x_t) B_t
 *
 * in fp32 as k = fmaf(p, B_{t-1}, h), p = ((1 - lam) * delta) * x_{t-1}, then the form's usual
 * update of k with q = (lam * delta) * x_t in place of delta * x_t.  y_t = C_t h_t as before.
 * lam = 1 is the Euler rule of the other entry points, bit for bit.  lam_t in [0, 1] is
 * expected (not checked).  The rule combines with every form of A:
 *     JSCAN_A_DIAGONAL         A [D][N]: the Mamba-1 form of jscan_prefill
 *     JSCAN_A_SCALED_IDENTITY  a [D]: the Mamba-2 form of jscan_prefill_scalar_a
 *     JSCAN_A_COMPLEX          A [D][N] as (real, imaginary) pairs: jscan_prefill_complex
 */
typedef enum { JSCAN_A_DIAGONAL = 0, JSCAN_A_SCALED_IDENTITY = 1, JSCAN_A_COMPLEX = 2 } jscan_a_form;

/*
 * Prefill with the exponential-trapezoidal rule, from h0 (NULL: zero state).
 *   lam     [batch][L][D], the dtype of x: the right-end weight of each (token, channel).
 *   x_prev  [batch][D] and B_prev [batch][N], the dtype of x: the token before the first one,
 *           whose input is the first step's left end point.  Both NULL when the sequence
 *           starts here (that term is then zero); a resumed sequence passes its last token.
 * Other arguments, layouts, errors and the bit-identity of h_final with the step chain are
 * as for jscan_prefill_resume (with jscan_step_trapezoid as the step).  Added errors:
 * JSCAN_ERR_NULL when lam is NULL or only one of x_prev and B_prev is, JSCAN_ERR_FORM for an
 * unknown a_form, JSCAN_ERR_ALIAS when y or h_final overlaps lam, x_prev or B_prev.
 */
jscan_status jscan_prefill_trapezoid(const void *x, const void *delta, const void *lam, const float *A,
                                     const void *B, const void *C, const float *h0, const void *x_prev,
                                     const void *B_prev, void *y, float *h_final, int64_t batch, int64_t L,
                                     int64_t D, int64_t N, jscan_a_form a_form, jscan_dtype dtype,
                                     void *stream);

/*
 * Decode step with the exponential-trapezoidal rule.  x_prev (rows of D, stride ld_xd) and
 * B_prev (rows of N, stride ld_bc) are the previous token's x and B, required: zeros for a
 * sequence's first token.  lam_t has the rows of x_t.  Otherwise as jscan_step (h in place).
 */
jscan_status jscan_step_trapezoid(float *h, const void *x_prev, const void *B_prev, const void *x_t,
                                  const void *delta_t, const void *lam_t, const float *A, const void *B_t,
                                  const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t N,
                                  int64_t ld_xd, int64_t ld_bc, int64_t ld_y, jscan_a_form a_form,
                                  jscan_dtype dtype, void *stream);

/*
 * Multi-input, multi-output (MIMO) scan, the Mamba-3 replacement of the per-channel scalar
 * projections by matrix-valued ones (lesson page "Jamba - Hybrid SSM-Transformer", section
 * "Mamba-3", item 3).  Each channel takes R inputs and gives R outputs; B_t and C_t are N x R
 * matrices shared by the channels; the state keeps its [batch][D][N] size:
 *
 *     h_t[d][n] = exp(delta_t[d] a) h_{t-1}[d][n] + sum_r (delta_t[d] * x_t[d][r]) * B_t[n][r]
 *     y_t[d][r] = sum_n C_t[n][r] * h_t[d][n]
 *
 * with the sum over r accumulated in increasing r (first product, then fmaf), and the decay a
 * of any form of A (jscan_a_form; with JSCAN_A_COMPLEX the state pairs, and B's and C's row
 * pairs for each r, are complex numbers).  R = 1 is the single-input scan of the form's
 * entry point, bit for bit in the state.  R must be 1, 2, 4 or 8 (else JSCAN_ERR_SHAPE).
 *
 * Prefill from h0 (NULL: zero state).  Layouts:
 *     x, y : [batch][L][D][R]     delta : [batch][L][D]     B, C : [batch][L][N][R]
 * Other arguments, ownership, errors (plus JSCAN_ERR_FORM) and the bit-identity of h_final
 * with the jscan_step_mimo chain are as for jscan_prefill_resume.
 */
jscan_status jscan_prefill_mimo(const void *x, const void *delta, const float *A, const void *B,
                                const void *C, const float *h0, void *y, float *h_final,
                                int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R,
                                jscan_a_form a_form, jscan_dtype dtype, void *stream);

/*
 * One MIMO decode token for a batch, h [batch][D][N] in place.  x_t is rows of D * R with
 * row stride ld_x; delta_t rows of D with stride ld_d; B_t and C_t rows of N * R with stride
 * ld_bc; y_t rows of D * R with stride ld_y (strides in elements, multiples of 8, at least the
 * row length).
 */
jscan_status jscan_step_mimo(float *h, const void *x_t, const void *delta_t, const float *A,
                             const void *B_t, const void *C_t, void *y_t, int64_t batch, int64_t D,
                             int64_t N, int64_t R, int64_t ld_x, int64_t ld_d, int64_t ld_bc,
                             int64_t ld_y, jscan_a_form a_form, jscan_dtype dtype, void *stream);

/*
 * The MIMO scan with the exponential-trapezoidal rule: both Mamba-3 changes together.  The
 * rank-R input u_t[n] = sum_r x_t[d][r] B_t[n][r] takes the place of x_t B_t at both end
 * points of the step, in fp32 as
 *     k = h;  k = fmaf(p_r, B_{t-1}[n][r], k) for r = 0 .. R-1,   p_r = ((1 - lam) * delta) * x_{t-1}[d][r]
 * then the MIMO update of k with q_r = (lam * delta) * x_t[d][r] in place of delta * x_t[d][r].
 * lam = 1 is jscan_prefill_mimo bit for bit; R = 1 is jscan_prefill_trapezoid bit for bit.
 * lam [batch][L][D] (delta's layout); x_prev [batch][D][R] and B_prev [batch][N][R] are the token
 * before the first (both NULL when there is none).  Other arguments, layouts and errors as for
 * jscan_prefill_mimo and jscan_prefill_trapezoid.
 */
jscan_status jscan_prefill_mimo_trapezoid(const void *x, const void *delta, const void *lam,
                                          const float *A, const void *B, const void *C,
                                          const float *h0, const void *x_prev, const void *B_prev,
                                          void *y, float *h_final, int64_t batch, int64_t L,
                                          int64_t D, int64_t N, int64_t R, jscan_a_form a_form,
                                          jscan_dtype dtype, void *stream);

/*
 * One MIMO decode token with the exponential-trapezoidal rule.  x_prev has x_t's rows (stride
 * ld_x), B_prev B_t's (ld_bc), lam_t delta_t's (ld_d); all three required (zeros before a
 * sequence's first token).  Otherwise as jscan_step_mimo.
 */
jscan_status jscan_step_mimo_trapezoid(float *h, const void *x_prev, const void *B_prev,
                                       const void *x_t, const void *delta_t, const void *lam_t,
                                       const float *A, const void *B_t, const void *C_t, void *y_t,
                                       int64_t batch, int64_t D, int64_t N, int64_t R, int64_t ld_x,
                                       int64_t ld_d, int64_t ld_bc, int64_t ld_y,
                                       jscan_a_form a_form, jscan_dtype dtype, void *stream);

/*
 * jscan_prefill_chunked without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It runs the same three passes on the same kernels, with the segment states and
 * delta sums in a library-owned scratch array of JSCAN_NOALLOC_SCRATCH_BYTES in each GPU's
 * memory (a static device array, held until the process ends).  The call itself allocates
 * nothing; the first call on a device looks up that device's copy of the array once.
 *   - A shape and chunk whose jscan_prefill_chunked_workspace(...) exceeds
 *     JSCAN_NOALLOC_SCRATCH_BYTES returns JSCAN_ERR_WORKSPACE and launches nothing (24 MiB
 *     holds every automatic plan, which needs at most 262144 * 68 bytes = 17 MiB; explicit
 *     chunks need batch * n_seg * D * 68 bytes).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in time on one GPU
 *     (from different streams or threads, or an unordered graph) race and give wrong results.
 *     Order them on one stream.  The array's contents on entry do not matter (every element
 *     the passes read was written earlier in the same call).
 * The other arguments, the results and the errors are those of jscan_prefill_chunked; a
 * failure to look up the array returns JSCAN_ERR_HIP.
 */
#define JSCAN_NOALLOC_SCRATCH_BYTES (24 * 1024 * 1024)
jscan_status jscan_prefill_chunked_noalloc(const void *x, const void *delta, const float *A,
                                           const void *B, const void *C, const float *h0, void *y,
                                           float *h_final, int64_t batch, int64_t L, int64_t D,
                                           int64_t N, int64_t chunk, jscan_dtype dtype, void *stream);

/* Static, human-readable name of a status code. */
const char *jscan_status_string(jscan_status s);

/* hipError_t behind the last JSCAN_ERR_HIP returned on the calling thread (0 if none). */
int jscan_last_hip_error(void);

/* Library ABI version: 100 * major + minor (101 adds the time-parallel prefill, 102 the
 * producer side, 103 the fused prefill, 104 the scaled-identity A entry points, 105 the
 * complex-valued state, 106 the exponential-trapezoidal rule, 107 the MIMO scan, 108 MIMO with the
 * trapezoidal rule, 109 the output row stride ld_y of the decode steps). */
int jscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JSCAN_H */
