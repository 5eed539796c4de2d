// jscan.hip - libjscan: host entry points of the C ABI declared in include/jscan.h, plus
// the kernels they launch (included below).  Everything runs on the caller's stream; the
// library allocates nothing and keeps no state except the calling thread's last HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/jscan.h"
#include "prefill_lane_kernel.h"
#include "prefill_rows_kernel.h"
#include "chunk_carry_kernel.h"
#include "prefill_seg_lane_kernel.h"
#include "project_kernels.h"
#include "step_kernel.h"
#include "mimo_kernels.h"
#include "prefill_mimo_rows_kernel.h"

namespace {

thread_local int g_last_hip_error = 0;

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi), empty when lo == hi
};

Span span(const void *p, int64_t bytes) {
    Span s;
    if (p && bytes > 0) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + static_cast<uintptr_t>(bytes);
    }
    return s;
}

bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t elem_bytes(jscan_dtype dt) { return dt == JSCAN_BF16 ? 2 : 4; }

jscan_status launch_status() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return JSCAN_ERR_HIP;
    }
    return JSCAN_OK;
}

// ---- prefill ----------------------------------------------------------------------------

// Largest grid the launchers accept (work-group counts and row indices are 32-bit ints).
constexpr int64_t kMaxBlocks = (int64_t)1 << 30;

// Scans `nrows` rows (see Segments) with the row-mapped kernel when it applies, otherwise
// with one lane per (row, channel).  AF: the form of A; kTrap: the trapezoidal rule (inputs tr).
template <typename E, jscan::AForm AF = jscan::AForm::Diagonal, bool kTrap = false>
void launch_rows(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *h0,
                 void *y, float *h_final, const jscan::Segments &sg, int64_t nrows, int64_t D, hipStream_t stream,
                 jscan::Trap tr = jscan::Trap{nullptr, nullptr, nullptr}) {
    using T = typename E::store_t;
    const T *xt = static_cast<const T *>(x), *dt = static_cast<const T *>(delta);
    const T *bt = static_cast<const T *>(B), *ct = static_cast<const T *>(C);
    T *yt = static_cast<T *>(y);
    if (jscan::rows_kernel_applies(nrows, D)) {
        jscan::launch_prefill_rows<E, false, AF, kTrap>(xt, dt, A, bt, ct, h0, yt, h_final, sg, nrows, (int)D, stream,
                                                        jscan::DeltaProj{nullptr, nullptr, nullptr}, tr);
        return;
    }
    const int blocks_per_row = (int)((D + 63) / 64);
    hipLaunchKernelGGL((jscan::prefill_lane_kernel<E, AF, kTrap>), dim3((unsigned)(nrows * blocks_per_row)), dim3(64),
                       0, stream, xt, dt, A, bt, ct, h0, yt, h_final, sg, (int)D, blocks_per_row, tr);
}

// Token-by-token prefill of whole sequences (one row per sequence).
template <typename E, jscan::AForm AF = jscan::AForm::Diagonal, bool kTrap = false>
jscan_status launch_prefill(const void *x, const void *delta, const float *A, const void *B, const void *C,
                            const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                            hipStream_t stream, jscan::Trap tr = jscan::Trap{nullptr, nullptr, nullptr}) {
    if (L == 0) {
        const int64_t count = batch * D * jscan::kDState;
        const int64_t blocks = (count + 255) / 256;
        hipLaunchKernelGGL(jscan::copy_state_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, h0, h_final, count);
        return launch_status();
    }
    const jscan::Segments sg{L, L, 1, 0};
    launch_rows<E, AF, kTrap>(x, delta, A, B, C, h0, y, h_final, sg, batch, D, stream, tr);
    return launch_status();
}

// Argument checks shared by every prefill entry point.  af: the form of A, which fixes its
// size (D values for the scaled identity, D * N otherwise).  Sets *nothing_to_do for zero-sized
// work (which is then OK without a launch).
jscan_status check_prefill(const void *x, const void *delta, const float *A, const void *B, const void *C,
                           const float *h0, bool h0_required, const void *y, const float *h_final, int64_t batch,
                           int64_t L, int64_t D, int64_t N, jscan_dtype dtype, bool *nothing_to_do,
                           jscan::AForm af = jscan::AForm::Diagonal) {
    *nothing_to_do = false;
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (batch < 0 || L < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0) return JSCAN_ERR_SHAPE;
    // index arithmetic inside the kernels: rows of D fit in int, grid sizes in 32 bits
    if (D > (1 << 24) || batch > (1 << 20) || batch * ((D + 63) / 64) > kMaxBlocks) return JSCAN_ERR_SHAPE;
    // the state-wide kernels (empty-sequence copy, segment carry) run one thread per element
    if (batch * D * JSCAN_D_STATE / 256 > kMaxBlocks) return JSCAN_ERR_SHAPE;
    if (batch == 0 || D == 0) {
        *nothing_to_do = true;
        return JSCAN_OK;
    }
    if (!A || !h_final || (h0_required && !h0)) return JSCAN_ERR_NULL;
    if (L > 0 && (!x || !delta || !B || !C || !y)) return JSCAN_ERR_NULL;

    const int64_t es = elem_bytes(dtype);
    const void *arrays[] = {x, delta, A, B, C, h0, y, h_final};
    for (const void *p : arrays)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;

    const int64_t seq = batch * L * D * es, bc = batch * L * N * es;
    const int64_t state = batch * D * N * 4, a_bytes = D * (af == jscan::AForm::ScaledIdentity ? 1 : N) * 4;
    const Span sy = span(y, L > 0 ? seq : 0), sh = span(h_final, state);
    const Span inputs[] = {span(x, seq), span(delta, seq), span(A, a_bytes), span(B, bc), span(C, bc)};
    for (const Span &s : inputs)
        if (overlaps(sy, s) || overlaps(sh, s)) return JSCAN_ERR_ALIAS;
    if (overlaps(sy, sh)) return JSCAN_ERR_ALIAS;
    if (h0) {
        const Span s0 = span(h0, state);
        if (overlaps(sy, s0)) return JSCAN_ERR_ALIAS;
        if (overlaps(sh, s0) && h0 != h_final) return JSCAN_ERR_ALIAS;  // exact in-place is allowed
    }
    return JSCAN_OK;
}

jscan_status prefill_impl(const void *x, const void *delta, const float *A, const void *B,
                          const void *C, const float *h0, bool resume, void *y, float *h_final,
                          int64_t batch, int64_t L, int64_t D, int64_t N, jscan_dtype dtype,
                          void *stream, jscan::AForm af = jscan::AForm::Diagonal) {
    using jscan::AForm;
    bool empty = false;
    const jscan_status st =
        check_prefill(x, delta, A, B, C, h0, resume, y, h_final, batch, L, D, N, dtype, &empty, af);
    if (st != JSCAN_OK || empty) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (af == AForm::ScaledIdentity) {
        if (dtype == JSCAN_BF16)
            return launch_prefill<jscan::BF16, AForm::ScaledIdentity>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
        return launch_prefill<jscan::F32, AForm::ScaledIdentity>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
    }
    if (af == AForm::ComplexPairs) {
        if (dtype == JSCAN_BF16)
            return launch_prefill<jscan::BF16, AForm::ComplexPairs>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
        return launch_prefill<jscan::F32, AForm::ComplexPairs>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
    }
    if (dtype == JSCAN_BF16)
        return launch_prefill<jscan::BF16>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
    return launch_prefill<jscan::F32>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
}

// ---- exponential-trapezoidal rule --------------------------------------------------------

template <typename E>
jscan_status launch_prefill_trap(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                 const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                                 hipStream_t s, jscan::AForm af, jscan::Trap tr) {
    using jscan::AForm;
    if (af == AForm::ScaledIdentity)
        return launch_prefill<E, AForm::ScaledIdentity, true>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s, tr);
    if (af == AForm::ComplexPairs)
        return launch_prefill<E, AForm::ComplexPairs, true>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s, tr);
    return launch_prefill<E, AForm::Diagonal, true>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s, tr);
}

bool form_of(jscan_a_form f, jscan::AForm *af) {
    switch (f) {
    case JSCAN_A_DIAGONAL: *af = jscan::AForm::Diagonal; return true;
    case JSCAN_A_SCALED_IDENTITY: *af = jscan::AForm::ScaledIdentity; return true;
    case JSCAN_A_COMPLEX: *af = jscan::AForm::ComplexPairs; return true;
    }
    return false;
}

// ---- multi-input, multi-output (MIMO) ------------------------------------------------------

bool mimo_rank_ok(int64_t R) { return R == 1 || R == 2 || R == 4 || R == 8; }

// Rank 1 is the single-input scan (same layouts), rank 2-8 the row-mapped MIMO kernel when it
// applies, else one lane per channel.  kTrap: the exponential-trapezoidal rule (inputs tr).
template <typename E, jscan::AForm AF, int R, bool kTrap>
void launch_prefill_mimo_r(const void *x, const void *delta, const float *A, const void *B, const void *C,
                           const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                           jscan::Trap tr, hipStream_t s) {
    using T = typename E::store_t;
    if constexpr (R == 1) {
        launch_prefill<E, AF, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s, tr);
    } else if constexpr (R == 8 && kTrap) {
        const int blocks_per_row = (int)((D + 63) / 64);
        hipLaunchKernelGGL((jscan::prefill_mimo_lane_kernel<E, AF, R, kTrap>), dim3((unsigned)(batch * blocks_per_row)),
                           dim3(64), 0, s, static_cast<const T *>(x), static_cast<const T *>(delta), A,
                           static_cast<const T *>(B), static_cast<const T *>(C), h0, static_cast<T *>(y), h_final, L,
                           (int)D, blocks_per_row, tr);
    } else {
        if (jscan::mimo_rows_kernel_applies(D, R, kTrap)) {
            jscan::launch_prefill_mimo_rows<E, AF, R, kTrap>(static_cast<const T *>(x), static_cast<const T *>(delta),
                                                             A, static_cast<const T *>(B), static_cast<const T *>(C),
                                                             h0, static_cast<T *>(y), h_final, batch, L, (int)D, s, tr);
        } else {
            const int blocks_per_row = (int)((D + 63) / 64);
            hipLaunchKernelGGL((jscan::prefill_mimo_lane_kernel<E, AF, R, kTrap>),
                               dim3((unsigned)(batch * blocks_per_row)), dim3(64), 0, s, static_cast<const T *>(x),
                               static_cast<const T *>(delta), A, static_cast<const T *>(B), static_cast<const T *>(C),
                               h0, static_cast<T *>(y), h_final, L, (int)D, blocks_per_row, tr);
        }
    }
}
template <typename E, jscan::AForm AF, bool kTrap>
void launch_prefill_mimo_af(const void *x, const void *delta, const float *A, const void *B, const void *C,
                            const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D, int64_t R,
                            jscan::Trap tr, hipStream_t s) {
    switch (R) {
    case 1: launch_prefill_mimo_r<E, AF, 1, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, tr, s); break;
    case 2: launch_prefill_mimo_r<E, AF, 2, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, tr, s); break;
    case 4: launch_prefill_mimo_r<E, AF, 4, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, tr, s); break;
    default: launch_prefill_mimo_r<E, AF, 8, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, tr, s); break;
    }
}
template <typename E, bool kTrap>
void launch_prefill_mimo(const void *x, const void *delta, const float *A, const void *B, const void *C,
                         const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D, int64_t R,
                         jscan::AForm af, jscan::Trap tr, hipStream_t s) {
    using jscan::AForm;
    if (af == AForm::ScaledIdentity)
        launch_prefill_mimo_af<E, AForm::ScaledIdentity, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, tr,
                                                                s);
    else if (af == AForm::ComplexPairs)
        launch_prefill_mimo_af<E, AForm::ComplexPairs, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, tr, s);
    else
        launch_prefill_mimo_af<E, AForm::Diagonal, kTrap>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, tr, s);
}

template <typename E, jscan::AForm AF, int R, bool kTrap>
void launch_step_mimo_r(float *h, const void *x, const void *delta, const float *A, const void *B, const void *C,
                        void *y, int64_t batch, int64_t D, int64_t ld_x, int64_t ld_d, int64_t ld_bc, int64_t ld_y,
                        jscan::Trap tr, hipStream_t s) {
    using T = typename E::store_t;
    const int blocks_per_rows = (int)((D * 4 + 255) / 256);
    const int64_t row_groups = (batch + jscan::mimo_step::kRows - 1) / jscan::mimo_step::kRows;
    hipLaunchKernelGGL((jscan::step_mimo_kernel<E, AF, R, kTrap>), dim3((unsigned)(row_groups * blocks_per_rows)),
                       dim3(256), 0, s, h, static_cast<const T *>(x), static_cast<const T *>(delta), A,
                       static_cast<const T *>(B), static_cast<const T *>(C), static_cast<T *>(y), (int)batch, (int)D,
                       blocks_per_rows, ld_x, ld_d, ld_bc, ld_y, static_cast<const T *>(tr.lam),
                       static_cast<const T *>(tr.x_prev), static_cast<const T *>(tr.B_prev));
}
template <typename E, jscan::AForm AF, bool kTrap>
void launch_step_mimo_af(float *h, const void *x, const void *delta, const float *A, const void *B, const void *C,
                         void *y, int64_t batch, int64_t D, int64_t R, int64_t ld_x, int64_t ld_d, int64_t ld_bc,
                         int64_t ld_y, jscan::Trap tr, hipStream_t s) {
    switch (R) {
    case 1: launch_step_mimo_r<E, AF, 1, kTrap>(h, x, delta, A, B, C, y, batch, D, ld_x, ld_d, ld_bc, ld_y, tr, s); break;
    case 2: launch_step_mimo_r<E, AF, 2, kTrap>(h, x, delta, A, B, C, y, batch, D, ld_x, ld_d, ld_bc, ld_y, tr, s); break;
    case 4: launch_step_mimo_r<E, AF, 4, kTrap>(h, x, delta, A, B, C, y, batch, D, ld_x, ld_d, ld_bc, ld_y, tr, s); break;
    default: launch_step_mimo_r<E, AF, 8, kTrap>(h, x, delta, A, B, C, y, batch, D, ld_x, ld_d, ld_bc, ld_y, tr, s); break;
    }
}
template <typename E, bool kTrap>
void launch_step_mimo(float *h, const void *x, const void *delta, const float *A, const void *B, const void *C,
                      void *y, int64_t batch, int64_t D, int64_t R, int64_t ld_x, int64_t ld_d, int64_t ld_bc,
                      int64_t ld_y, jscan::AForm af, jscan::Trap tr, hipStream_t s) {
    using jscan::AForm;
    if (af == AForm::ScaledIdentity)
        launch_step_mimo_af<E, AForm::ScaledIdentity, kTrap>(h, x, delta, A, B, C, y, batch, D, R, ld_x, ld_d, ld_bc,
                                                             ld_y, tr, s);
    else if (af == AForm::ComplexPairs)
        launch_step_mimo_af<E, AForm::ComplexPairs, kTrap>(h, x, delta, A, B, C, y, batch, D, R, ld_x, ld_d, ld_bc,
                                                           ld_y, tr, s);
    else
        launch_step_mimo_af<E, AForm::Diagonal, kTrap>(h, x, delta, A, B, C, y, batch, D, R, ld_x, ld_d, ld_bc, ld_y,
                                                       tr, s);
}

// Checks and launch shared by the MIMO prefill entry points; trap: the trapezoidal rule.
jscan_status prefill_mimo_impl(const void *x, const void *delta, const void *lam, const float *A, const void *B,
                               const void *C, const float *h0, const void *x_prev, const void *B_prev, void *y,
                               float *h_final, int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R,
                               jscan_a_form a_form, jscan_dtype dtype, void *stream, bool trap) {
    jscan::AForm af;
    if (!form_of(a_form, &af)) return JSCAN_ERR_FORM;
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (batch < 0 || L < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0 || !mimo_rank_ok(R)) return JSCAN_ERR_SHAPE;
    if (D > (1 << 24) || batch > (1 << 20) || batch * ((D + 63) / 64) > kMaxBlocks) return JSCAN_ERR_SHAPE;
    if (batch * D * JSCAN_D_STATE / 256 > kMaxBlocks) return JSCAN_ERR_SHAPE;
    if (batch == 0 || D == 0) return JSCAN_OK;
    if (!A || !h_final) return JSCAN_ERR_NULL;
    if (L > 0 && (!x || !delta || !B || !C || !y)) return JSCAN_ERR_NULL;
    if (trap && ((L > 0 && !lam) || ((x_prev == nullptr) != (B_prev == nullptr)))) return JSCAN_ERR_NULL;
    const void *arrays[] = {x, delta, A, B, C, h0, y, h_final, lam, x_prev, B_prev};
    for (const void *p : arrays)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;
    const int64_t es = elem_bytes(dtype);
    const int64_t xs = batch * L * D * R * es, ds = batch * L * D * es, bc = batch * L * N * R * es;
    const int64_t state = batch * D * N * 4, a_bytes = D * (af == jscan::AForm::ScaledIdentity ? 1 : N) * 4;
    const Span sy = span(y, L > 0 ? xs : 0), sh = span(h_final, state);
    const Span inputs[] = {span(x, xs), span(delta, ds), span(A, a_bytes), span(B, bc), span(C, bc),
                           span(trap ? lam : nullptr, L > 0 ? ds : 0), span(trap ? x_prev : nullptr, batch * D * R * es),
                           span(trap ? B_prev : nullptr, batch * N * R * es)};
    for (const Span &sp : inputs)
        if (overlaps(sy, sp) || overlaps(sh, sp)) return JSCAN_ERR_ALIAS;
    if (overlaps(sy, sh)) return JSCAN_ERR_ALIAS;
    if (h0) {
        const Span s0 = span(h0, state);
        if (overlaps(sy, s0)) return JSCAN_ERR_ALIAS;
        if (overlaps(sh, s0) && h0 != h_final) return JSCAN_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (L == 0) {
        const int64_t count = batch * D * jscan::kDState;
        hipLaunchKernelGGL(jscan::copy_state_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, h0,
                           h_final, count);
        return launch_status();
    }
    const jscan::Trap tr{lam, x_prev, B_prev};
    if (dtype == JSCAN_BF16) {
        if (trap) launch_prefill_mimo<jscan::BF16, true>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, af, tr, s);
        else launch_prefill_mimo<jscan::BF16, false>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, af, tr, s);
    } else {
        if (trap) launch_prefill_mimo<jscan::F32, true>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, af, tr, s);
        else launch_prefill_mimo<jscan::F32, false>(x, delta, A, B, C, h0, y, h_final, batch, L, D, R, af, tr, s);
    }
    return launch_status();
}

// Checks and launch shared by the MIMO step entry points; trap: the trapezoidal rule (lam has
// delta's rows, x_prev x's rows, B_prev B's rows).
jscan_status step_mimo_impl(float *h, const void *x_prev, const void *B_prev, const void *x_t, const void *delta_t,
                            const void *lam_t, const float *A, const void *B_t, const void *C_t, void *y_t,
                            int64_t batch, int64_t D, int64_t N, int64_t R, int64_t ld_x, int64_t ld_d, int64_t ld_bc,
                            int64_t ld_y, jscan_a_form a_form, jscan_dtype dtype, void *stream, bool trap) {
    jscan::AForm af;
    if (!form_of(a_form, &af)) return JSCAN_ERR_FORM;
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (batch < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0 || !mimo_rank_ok(R)) return JSCAN_ERR_SHAPE;
    if (D > (1 << 24) || batch > (1 << 20)) return JSCAN_ERR_SHAPE;
    if ((batch + jscan::mimo_step::kRows - 1) / jscan::mimo_step::kRows * ((D * 4 + 255) / 256) > kMaxBlocks)
        return JSCAN_ERR_SHAPE;
    if (batch == 0 || D == 0) return JSCAN_OK;
    if (ld_x < D * R || ld_d < D || ld_bc < N * R || ld_y < D * R || ld_x % 8 != 0 || ld_d % 8 != 0 ||
        ld_bc % 8 != 0 || ld_y % 8 != 0)
        return JSCAN_ERR_SHAPE;
    if (!h || !x_t || !delta_t || !A || !B_t || !C_t || !y_t) return JSCAN_ERR_NULL;
    if (trap && (!x_prev || !B_prev || !lam_t)) return JSCAN_ERR_NULL;
    const void *arrays[] = {h, x_t, delta_t, A, B_t, C_t, y_t};
    for (const void *p : arrays)
        if (!aligned16(p)) return JSCAN_ERR_ALIGN;
    const void *extra[] = {x_prev, B_prev, lam_t};
    for (const void *p : extra)
        if (trap && !aligned16(p)) return JSCAN_ERR_ALIGN;
    const int64_t es = elem_bytes(dtype);
    const int64_t rows_x = ((batch - 1) * ld_x + D * R) * es, rows_d = ((batch - 1) * ld_d + D) * es;
    const int64_t rows_bc = ((batch - 1) * ld_bc + N * R) * es;
    const Span sh = span(h, batch * D * N * 4), sy = span(y_t, ((batch - 1) * ld_y + D * R) * es);
    const Span inputs[] = {span(x_t, rows_x), span(delta_t, rows_d),
                           span(A, D * (af == jscan::AForm::ScaledIdentity ? 1 : N) * 4), span(B_t, rows_bc),
                           span(C_t, rows_bc), span(trap ? x_prev : nullptr, rows_x),
                           span(trap ? B_prev : nullptr, rows_bc), span(trap ? lam_t : nullptr, rows_d)};
    for (const Span &sp : inputs)
        if (overlaps(sy, sp) || overlaps(sh, sp)) return JSCAN_ERR_ALIAS;
    if (overlaps(sy, sh)) return JSCAN_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const jscan::Trap tr{lam_t, x_prev, B_prev};
    if (dtype == JSCAN_BF16) {
        if (trap) launch_step_mimo<jscan::BF16, true>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, R, ld_x, ld_d,
                                                      ld_bc, ld_y, af, tr, s);
        else launch_step_mimo<jscan::BF16, false>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, R, ld_x, ld_d, ld_bc,
                                                  ld_y, af, tr, s);
    } else {
        if (trap) launch_step_mimo<jscan::F32, true>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, R, ld_x, ld_d,
                                                     ld_bc, ld_y, af, tr, s);
        else launch_step_mimo<jscan::F32, false>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, R, ld_x, ld_d, ld_bc,
                                                 ld_y, af, tr, s);
    }
    return launch_status();
}

// ---- time-parallel prefill ---------------------------------------------------------------

struct ChunkPlan {
    int64_t seg_len = 0;
    int64_t n_seg = 1;
};

// Segments of `chunk` tokens, or (chunk == 0) as many as it takes to give the segment-lane
// kernel kSegLanes (segment, channel) lanes, four waves on each of the 1024 SIMDs, when the
// sequences' channels are too few for the token-by-token kernel to fill the GPU (fewer than
// 8192 channels, or D not a multiple of 32).  Automatic segments are at least 256 tokens long
// and a multiple of 64.
constexpr int64_t kSegLanes = (int64_t)1024 * jscan::seglane::kWavesPerSimd * 64;
ChunkPlan plan_chunks(int64_t batch, int64_t L, int64_t D, int64_t chunk) {
    ChunkPlan p;
    p.seg_len = L;
    if (L <= 0 || batch <= 0 || D <= 0) return p;
    if (chunk > 0) {
        p.seg_len = chunk < L ? chunk : L;
    } else {
        const int64_t channels = batch * D;
        const bool filled = channels >= 8192 && D % jscan::rows::kCh == 0;
        int64_t n = (filled || channels >= kSegLanes) ? 1 : kSegLanes / channels;
        const int64_t by_length = L / 256 > 1 ? L / 256 : 1;
        if (n > by_length) n = by_length;
        p.seg_len = (L + n - 1) / n;
        p.seg_len = (p.seg_len + 63) / 64 * 64;
        if (p.seg_len > L) p.seg_len = L;
    }
    p.n_seg = (L + p.seg_len - 1) / p.seg_len;
    return p;
}

// Whether the plan's grids fit the launchers: segment rows and scan work-groups, the carry
// pass's work-groups of carry::kPairs (channel, state) pairs, and 32-bit token indexes.
bool chunk_grids_fit(int64_t batch, int64_t D, const ChunkPlan &p) {
    return batch * p.n_seg <= (1 << 24) && batch * p.n_seg * ((D + 63) / 64) <= kMaxBlocks &&
           batch * D * JSCAN_D_STATE / jscan::carry::kPairs <= kMaxBlocks && p.seg_len < ((int64_t)1 << 31);
}

// Workspace bytes of a plan: h_loc / h_in [batch * n_seg][D][N] and delta sums [batch * n_seg][D].
int64_t chunk_workspace_bytes(const ChunkPlan &p, int64_t batch, int64_t D) {
    if (p.n_seg <= 1) return 0;
    return batch * p.n_seg * D * (JSCAN_D_STATE + 1) * 4;
}

template <typename E>
jscan_status launch_chunked(const void *x, const void *delta, const float *A, const void *B, const void *C,
                            const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                            const ChunkPlan &p, void *workspace, hipStream_t stream) {
    float *hbuf = static_cast<float *>(workspace);
    float *dsum = hbuf + batch * p.n_seg * D * jscan::kDState;
    const int64_t nrows = batch * p.n_seg;
    using T = typename E::store_t;
    const T *xt = static_cast<const T *>(x), *dt = static_cast<const T *>(delta);
    const T *bt = static_cast<const T *>(B), *ct = static_cast<const T *>(C);
    // 1. every segment from zero: end states into hbuf, delta sums into dsum (no y)
    const jscan::Segments each{L, p.seg_len, (int)p.n_seg, 0};
    jscan::launch_prefill_seg_lane<E, true, true>(xt, dt, A, bt, ct, nullptr, nullptr, hbuf, dsum, each, nrows,
                                                  (int)D, stream);
    if (launch_status() != JSCAN_OK) return JSCAN_ERR_HIP;
    // 2. starting state of every segment, in place in hbuf
    const int64_t count = batch * D * jscan::kDState;
    jscan::launch_chunk_carry(hbuf, dsum, A, h0, count, (int)D, (int)p.n_seg, stream);
    if (launch_status() != JSCAN_OK) return JSCAN_ERR_HIP;
    // 3. every segment again from its starting state: y, and h_final from the last segments
    const jscan::Segments again{L, p.seg_len, (int)p.n_seg, 1};
    // y summed in the order the sequential prefill uses for this D, so segment 0 matches it
    if (jscan::rows_kernel_applies(batch, D))
        jscan::launch_prefill_seg_lane<E, false, true>(xt, dt, A, bt, ct, hbuf, static_cast<T *>(y), h_final,
                                                       nullptr, again, nrows, (int)D, stream);
    else
        jscan::launch_prefill_seg_lane<E, false, false>(xt, dt, A, bt, ct, hbuf, static_cast<T *>(y), h_final,
                                                        nullptr, again, nrows, (int)D, stream);
    return launch_status();
}

// ---- the time-parallel prefill's library-owned scratch -----------------------------------
// One array per GPU for jscan_prefill_chunked_noalloc.  Host code never passes `scratch`
// itself to a kernel (on the host the name only stands for the symbol); it looks up each
// device's address once with hipGetSymbolAddress and uses that.
static __device__ __align__(256) unsigned char scratch[JSCAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that owns `stream` (the current device for NULL).
jscan_status scratch_on_stream_device(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int>(e);
        return JSCAN_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        g_last_hip_error = static_cast<int>(hipErrorInvalidDevice);
        return JSCAN_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess || !p) {
            g_last_hip_error = static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return JSCAN_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return JSCAN_OK;
}

// ---- producer side: delta, B and C from x ---------------------------------------------

template <int R>
void launch_ssm_inputs(const uint16_t *x, const uint16_t *w_x, const float *g_d, const float *g_b, const float *g_c,
                       const uint16_t *w_dt, const float *b_dt, uint16_t *d_low, uint16_t *delta, uint16_t *B,
                       uint16_t *C, int64_t M, int D, float eps, hipStream_t stream) {
    const int64_t row_tiles = (M + jscan::proj::kRowsX - 1) / jscan::proj::kRowsX;
    hipLaunchKernelGGL((jscan::xproj_kernel<R / 16, jscan::proj::kXRowTiles>), dim3((unsigned)row_tiles),
                       dim3(jscan::proj::xproj_threads(jscan::proj::kXRowTiles)), 0, stream,
                       x, w_x, g_d,
                       g_b, g_c, d_low, B, C, M, D, eps);
    if (!delta) return;   // x projection only: delta is computed inside jscan_prefill_fused
    // one work-group per CU (the registers allow one): 256 groups of (channel slice, token tiles)
    const int ch_tiles = (D + jscan::proj::kDtCh - 1) / jscan::proj::kDtCh;
    const int64_t tok_tiles = (M + jscan::proj::kDtTok - 1) / jscan::proj::kDtTok;
    int64_t groups = ch_tiles >= 256 ? 1 : 256 / ch_tiles;
    if (groups > tok_tiles) groups = tok_tiles;
    hipLaunchKernelGGL((jscan::dtproj_kernel<R>), dim3((unsigned)(groups * ch_tiles)), dim3(512), 0, stream, d_low,
                       w_dt, b_dt, delta, M, D, ch_tiles, (int)groups);
}

// ---- decode step -----------------------------------------------------------------------

// tr: the trapezoidal rule's lam_t, x_prev and B_prev (rows like x_t, x_t and B_t), when kTrap.
template <typename E, jscan::AForm AF, bool kTrap = false>
jscan_status launch_step(float *h, const void *x_t, const void *delta_t, const float *A,
                         const void *B_t, const void *C_t, void *y_t, int64_t batch, int64_t D,
                         int64_t ld_xd, int64_t ld_bc, int64_t ld_y, hipStream_t stream,
                         jscan::Trap tr = jscan::Trap{nullptr, nullptr, nullptr}) {
    using T = typename E::store_t;
    const int blocks_per_rows = (int)((D * 4 + 255) / 256);
    const int64_t row_groups = (batch + jscan::step::kRows - 1) / jscan::step::kRows;
    hipLaunchKernelGGL((jscan::step_kernel<E, AF, kTrap>), dim3((unsigned)(row_groups * blocks_per_rows)), dim3(256), 0,
                       stream, h, static_cast<const T *>(x_t), static_cast<const T *>(delta_t), A,
                       static_cast<const T *>(B_t), static_cast<const T *>(C_t), static_cast<T *>(y_t), (int)batch,
                       (int)D, blocks_per_rows, ld_xd, ld_bc, ld_y, static_cast<const T *>(tr.lam),
                       static_cast<const T *>(tr.x_prev), static_cast<const T *>(tr.B_prev));
    return launch_status();
}

template <typename E>
jscan_status dispatch_step_trap_e(float *h, const void *x_t, const void *delta_t, const float *A, const void *B_t,
                                  const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t ld_xd, int64_t ld_bc,
                                  int64_t ld_y, hipStream_t s, jscan::AForm af, jscan::Trap tr) {
    using jscan::AForm;
    if (af == AForm::ScaledIdentity)
        return launch_step<E, AForm::ScaledIdentity, true>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc,
                                                           ld_y, s, tr);
    if (af == AForm::ComplexPairs)
        return launch_step<E, AForm::ComplexPairs, true>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc,
                                                         ld_y, s, tr);
    return launch_step<E, AForm::Diagonal, true>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, ld_y, s,
                                                 tr);
}
jscan_status dispatch_step_trap(float *h, const void *x_t, const void *delta_t, const float *A, const void *B_t,
                                const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t ld_xd, int64_t ld_bc,
                                int64_t ld_y, jscan_dtype dtype, hipStream_t s, jscan::AForm af, jscan::Trap tr) {
    if (dtype == JSCAN_BF16)
        return dispatch_step_trap_e<jscan::BF16>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, ld_y, s,
                                                 af, tr);
    return dispatch_step_trap_e<jscan::F32>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, ld_y, s, af, tr);
}

// Checks and launch shared by the decode-step entry points.  af: the form of A.
// With tr.lam set, the trapezoidal rule: lam_t and x_prev have the rows of x_t, B_prev those of B_t.
jscan_status step_impl(float *h, const void *x_t, const void *delta_t, const float *A, const void *B_t, const void *C_t,
                       void *y_t, int64_t batch, int64_t D, int64_t N, int64_t ld_xd, int64_t ld_bc, int64_t ld_y,
                       jscan_dtype dtype, void *stream, jscan::AForm af, jscan::Trap tr = jscan::Trap{nullptr, nullptr, nullptr},
                       bool trap = false) {
    using jscan::AForm;
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (batch < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0) return JSCAN_ERR_SHAPE;
    if (D > (1 << 24) || batch > (1 << 20)) return JSCAN_ERR_SHAPE;
    if ((batch + jscan::step::kRows - 1) / jscan::step::kRows * ((D * 4 + 255) / 256) > kMaxBlocks)
        return JSCAN_ERR_SHAPE;
    if (batch == 0 || D == 0) return JSCAN_OK;
    if (ld_xd < D || ld_bc < N || ld_y < D || ld_xd % 8 != 0 || ld_bc % 8 != 0 || ld_y % 8 != 0)
        return JSCAN_ERR_SHAPE;
    if (!h || !x_t || !delta_t || !A || !B_t || !C_t || !y_t) return JSCAN_ERR_NULL;
    if (trap && (!tr.lam || !tr.x_prev || !tr.B_prev)) return JSCAN_ERR_NULL;
    const void *arrays[] = {h, x_t, delta_t, A, B_t, C_t, y_t};
    for (const void *p : arrays)
        if (!aligned16(p)) return JSCAN_ERR_ALIGN;
    const void *extra[] = {tr.lam, tr.x_prev, tr.B_prev};
    for (const void *p : extra)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;

    const int64_t es = elem_bytes(dtype);
    const int64_t rows_xd = ((batch - 1) * ld_xd + D) * es, rows_bc = ((batch - 1) * ld_bc + N) * es;
    const Span sh = span(h, batch * D * N * 4), sy = span(y_t, ((batch - 1) * ld_y + D) * es);
    const Span inputs[] = {span(x_t, rows_xd), span(delta_t, rows_xd), span(A, D * (af == AForm::ScaledIdentity ? 1 : N) * 4), span(B_t, rows_bc),
                           span(C_t, rows_bc)};
    for (const Span &s : inputs)
        if (overlaps(sy, s) || overlaps(sh, s)) return JSCAN_ERR_ALIAS;
    if (overlaps(sy, sh)) return JSCAN_ERR_ALIAS;
    if (trap) {
        const Span more[] = {span(tr.lam, rows_xd), span(tr.x_prev, rows_xd), span(tr.B_prev, rows_bc)};
        for (const Span &s : more)
            if (overlaps(sy, s) || overlaps(sh, s)) return JSCAN_ERR_ALIAS;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (trap)
        return dispatch_step_trap(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, ld_y, dtype, s, af, tr);
    if (af == AForm::ScaledIdentity) {
        if (dtype == JSCAN_BF16)
            return launch_step<jscan::BF16, AForm::ScaledIdentity>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd,
                                                                    ld_bc, ld_y, s);
        return launch_step<jscan::F32, AForm::ScaledIdentity>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd,
                                                              ld_bc, ld_y, s);
    }
    if (af == AForm::ComplexPairs) {
        if (dtype == JSCAN_BF16)
            return launch_step<jscan::BF16, AForm::ComplexPairs>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd,
                                                                  ld_bc, ld_y, s);
        return launch_step<jscan::F32, AForm::ComplexPairs>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc,
                                                            ld_y, s);
    }
    if (dtype == JSCAN_BF16)
        return launch_step<jscan::BF16, AForm::Diagonal>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc,
                                                         ld_y, s);
    return launch_step<jscan::F32, AForm::Diagonal>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, ld_y, s);
}

}  // namespace

extern "C" {

jscan_status jscan_prefill(const void *x, const void *delta, const float *A, const void *B,
                           const void *C, void *y, float *h_final, int64_t batch, int64_t L,
                           int64_t D, int64_t N, jscan_dtype dtype, void *stream) {
    return prefill_impl(x, delta, A, B, C, nullptr, false, y, h_final, batch, L, D, N, dtype, stream);
}

jscan_status jscan_prefill_resume(const void *x, const void *delta, const float *A,
                                  const void *B, const void *C, const float *h0, void *y,
                                  float *h_final, int64_t batch, int64_t L, int64_t D,
                                  int64_t N, jscan_dtype dtype, void *stream) {
    return prefill_impl(x, delta, A, B, C, h0, true, y, h_final, batch, L, D, N, dtype, stream);
}

int64_t jscan_prefill_chunked_workspace(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t chunk) {
    if (batch < 0 || L < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0 || chunk < 0) return -1;
    if (D > (1 << 24) || batch > (1 << 20)) return -1;
    const ChunkPlan p = plan_chunks(batch, L, D, chunk);
    if (!chunk_grids_fit(batch, D, p)) return -1;
    return chunk_workspace_bytes(p, batch, D);
}

jscan_status jscan_prefill_chunked(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                   const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                                   int64_t N, int64_t chunk, void *workspace, int64_t workspace_bytes,
                                   jscan_dtype dtype, void *stream) {
    bool empty = false;
    jscan_status st = check_prefill(x, delta, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, &empty);
    if (st != JSCAN_OK) return st;
    if (chunk < 0) return JSCAN_ERR_SHAPE;
    if (empty) return JSCAN_OK;
    const ChunkPlan p = plan_chunks(batch, L, D, chunk);
    if (p.n_seg <= 1) return prefill_impl(x, delta, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, stream);
    if (!chunk_grids_fit(batch, D, p)) return JSCAN_ERR_SHAPE;
    const int64_t need = chunk_workspace_bytes(p, batch, D);
    if (!workspace) return JSCAN_ERR_NULL;
    if (workspace_bytes < need) return JSCAN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return JSCAN_ERR_ALIGN;
    const int64_t es = elem_bytes(dtype);
    const int64_t seq = batch * L * D * es, bc = batch * L * N * es, state = batch * D * N * 4;
    const Span sw = span(workspace, need);
    const Span others[] = {span(x, seq), span(delta, seq), span(A, D * N * 4), span(B, bc), span(C, bc),
                           span(h0, state), span(y, seq), span(h_final, state)};
    for (const Span &o : others)
        if (overlaps(sw, o)) return JSCAN_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == JSCAN_BF16)
        return launch_chunked<jscan::BF16>(x, delta, A, B, C, h0, y, h_final, batch, L, D, p, workspace, s);
    return launch_chunked<jscan::F32>(x, delta, A, B, C, h0, y, h_final, batch, L, D, p, workspace, s);
}

jscan_status jscan_prefill_chunked_noalloc(const void *x, const void *delta, const float *A, const void *B,
                                           const void *C, const float *h0, void *y, float *h_final, int64_t batch,
                                           int64_t L, int64_t D, int64_t N, int64_t chunk, jscan_dtype dtype,
                                           void *stream) {
    bool empty = false;
    jscan_status st = check_prefill(x, delta, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, &empty);
    if (st != JSCAN_OK) return st;
    if (chunk < 0) return JSCAN_ERR_SHAPE;
    if (empty) return JSCAN_OK;
    const ChunkPlan p = plan_chunks(batch, L, D, chunk);
    if (p.n_seg <= 1) return prefill_impl(x, delta, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, stream);
    if (!chunk_grids_fit(batch, D, p)) return JSCAN_ERR_SHAPE;
    if (chunk_workspace_bytes(p, batch, D) > JSCAN_NOALLOC_SCRATCH_BYTES) return JSCAN_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    st = scratch_on_stream_device(s, &ws);
    if (st != JSCAN_OK) return st;
    if (dtype == JSCAN_BF16)
        return launch_chunked<jscan::BF16>(x, delta, A, B, C, h0, y, h_final, batch, L, D, p, ws, s);
    return launch_chunked<jscan::F32>(x, delta, A, B, C, h0, y, h_final, batch, L, D, p, ws, s);
}

jscan_status jscan_step(float *h, const void *x_t, const void *delta_t, const float *A,
                        const void *B_t, const void *C_t, void *y_t, int64_t batch, int64_t D,
                        int64_t N, int64_t ld_xd, int64_t ld_bc, int64_t ld_y, jscan_dtype dtype,
                        void *stream) {
    return step_impl(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, N, ld_xd, ld_bc, ld_y, dtype, stream,
                     jscan::AForm::Diagonal);
}

jscan_status jscan_prefill_scalar_a(const void *x, const void *delta, const float *a, const void *B, const void *C,
                                    const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                                    int64_t N, jscan_dtype dtype, void *stream) {
    return prefill_impl(x, delta, a, B, C, h0, false, y, h_final, batch, L, D, N, dtype, stream,
                        jscan::AForm::ScaledIdentity);
}

jscan_status jscan_step_scalar_a(float *h, const void *x_t, const void *delta_t, const float *a, const void *B_t,
                                 const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t N, int64_t ld_xd,
                                 int64_t ld_bc, int64_t ld_y, jscan_dtype dtype, void *stream) {
    return step_impl(h, x_t, delta_t, a, B_t, C_t, y_t, batch, D, N, ld_xd, ld_bc, ld_y, dtype, stream,
                     jscan::AForm::ScaledIdentity);
}

jscan_status jscan_prefill_complex(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                   const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                                   int64_t N, jscan_dtype dtype, void *stream) {
    return prefill_impl(x, delta, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, stream,
                        jscan::AForm::ComplexPairs);
}

jscan_status jscan_step_complex(float *h, const void *x_t, const void *delta_t, const float *A, const void *B_t,
                                const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t N, int64_t ld_xd,
                                int64_t ld_bc, int64_t ld_y, jscan_dtype dtype, void *stream) {
    return step_impl(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, N, ld_xd, ld_bc, ld_y, dtype, stream,
                     jscan::AForm::ComplexPairs);
}

jscan_status jscan_prefill_trapezoid(const void *x, const void *delta, const void *lam, const float *A, const void *B,
                                     const void *C, const float *h0, const void *x_prev, const void *B_prev, void *y,
                                     float *h_final, int64_t batch, int64_t L, int64_t D, int64_t N,
                                     jscan_a_form a_form, jscan_dtype dtype, void *stream) {
    jscan::AForm af;
    if (!form_of(a_form, &af)) return JSCAN_ERR_FORM;
    bool empty = false;
    const jscan_status st = check_prefill(x, delta, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, &empty, af);
    if (st != JSCAN_OK || empty) return st;
    if ((L > 0 && !lam) || ((x_prev == nullptr) != (B_prev == nullptr))) return JSCAN_ERR_NULL;
    const void *more[] = {lam, x_prev, B_prev};
    for (const void *p : more)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;
    const int64_t es = elem_bytes(dtype);
    const Span outs[] = {span(y, L > 0 ? batch * L * D * es : 0), span(h_final, batch * D * N * 4)};
    const Span ins[] = {span(lam, L > 0 ? batch * L * D * es : 0), span(x_prev, batch * D * es),
                        span(B_prev, batch * N * es)};
    for (const Span &o : outs)
        for (const Span &i : ins)
            if (overlaps(o, i)) return JSCAN_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const jscan::Trap tr{lam, x_prev, B_prev};
    if (dtype == JSCAN_BF16)
        return launch_prefill_trap<jscan::BF16>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s, af, tr);
    return launch_prefill_trap<jscan::F32>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s, af, tr);
}

jscan_status jscan_step_trapezoid(float *h, const void *x_prev, const void *B_prev, const void *x_t,
                                  const void *delta_t, const void *lam_t, const float *A, const void *B_t,
                                  const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t N, int64_t ld_xd,
                                  int64_t ld_bc, int64_t ld_y, jscan_a_form a_form, jscan_dtype dtype, void *stream) {
    jscan::AForm af;
    if (!form_of(a_form, &af)) return JSCAN_ERR_FORM;
    return step_impl(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, N, ld_xd, ld_bc, ld_y, dtype, stream, af,
                     jscan::Trap{lam_t, x_prev, B_prev}, true);
}

jscan_status jscan_prefill_mimo(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                const float *h0, void *y, float *h_final, int64_t batch, int64_t L, int64_t D,
                                int64_t N, int64_t R, jscan_a_form a_form, jscan_dtype dtype, void *stream) {
    return prefill_mimo_impl(x, delta, nullptr, A, B, C, h0, nullptr, nullptr, y, h_final, batch, L, D, N, R, a_form,
                             dtype, stream, false);
}

jscan_status jscan_step_mimo(float *h, const void *x_t, const void *delta_t, const float *A, const void *B_t,
                             const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t N, int64_t R, int64_t ld_x,
                             int64_t ld_d, int64_t ld_bc, int64_t ld_y, jscan_a_form a_form, jscan_dtype dtype,
                             void *stream) {
    return step_mimo_impl(h, nullptr, nullptr, x_t, delta_t, nullptr, A, B_t, C_t, y_t, batch, D, N, R, ld_x, ld_d,
                          ld_bc, ld_y, a_form, dtype, stream, false);
}

jscan_status jscan_prefill_mimo_trapezoid(const void *x, const void *delta, const void *lam, const float *A,
                                          const void *B, const void *C, const float *h0, const void *x_prev,
                                          const void *B_prev, void *y, float *h_final, int64_t batch, int64_t L,
                                          int64_t D, int64_t N, int64_t R, jscan_a_form a_form, jscan_dtype dtype,
                                          void *stream) {
    return prefill_mimo_impl(x, delta, lam, A, B, C, h0, x_prev, B_prev, y, h_final, batch, L, D, N, R, a_form, dtype,
                             stream, true);
}

jscan_status jscan_step_mimo_trapezoid(float *h, const void *x_prev, const void *B_prev, const void *x_t,
                                       const void *delta_t, const void *lam_t, const float *A, const void *B_t,
                                       const void *C_t, void *y_t, int64_t batch, int64_t D, int64_t N, int64_t R,
                                       int64_t ld_x, int64_t ld_d, int64_t ld_bc, int64_t ld_y, jscan_a_form a_form,
                                       jscan_dtype dtype, void *stream) {
    return step_mimo_impl(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t, y_t, batch, D, N, R, ld_x, ld_d, ld_bc,
                          ld_y, a_form, dtype, stream, true);
}

jscan_status jscan_ssm_inputs(const void *x, const void *w_x, const float *g_delta, const float *g_B,
                              const float *g_C, const void *w_dt, const float *b_dt, void *delta_low, void *delta,
                              void *B, void *C, int64_t M, int64_t D, int64_t R, int64_t N, float eps,
                              jscan_dtype dtype, void *stream) {
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;   // the matrix-core path is bf16 in, fp32 accumulate
    if (M < 0 || D <= 0 || N != JSCAN_D_STATE || (R != 64 && R != 128 && R != 256)) return JSCAN_ERR_SHAPE;
    if (D % 128 != 0 || D > (1 << 24)) return JSCAN_ERR_SHAPE;   // channels go in pairs of 64-channel waves
    if (!(eps >= 0.0f) || eps > 1.0f) return JSCAN_ERR_SHAPE;
    if (M > ((int64_t)1 << 31)) return JSCAN_ERR_SHAPE;   // keeps the kernels' per-group tile counts in int
    if (M == 0) return JSCAN_OK;
    // delta == NULL: the x projection alone (w_dt and b_dt are then not used and may be NULL)
    const void *arrays[] = {x, w_x, g_delta, g_B, g_C, delta_low, B, C};
    for (const void *p : arrays)
        if (!p) return JSCAN_ERR_NULL;
    if (delta && (!w_dt || !b_dt)) return JSCAN_ERR_NULL;
    const void *maybe[] = {x, w_x, g_delta, g_B, g_C, delta_low, B, C, delta, w_dt, b_dt};
    for (const void *p : maybe)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;
    const Span outs[] = {span(delta_low, M * R * 2), span(delta, M * D * 2), span(B, M * N * 2), span(C, M * N * 2)};
    const Span ins[] = {span(x, M * D * 2),     span(w_x, (R + 2 * N) * D * 2), span(g_delta, R * 4),
                        span(g_B, N * 4),       span(g_C, N * 4),               span(w_dt, D * R * 2),
                        span(b_dt, D * 4)};
    for (int i = 0; i < 4; ++i) {
        for (const Span &in : ins)
            if (overlaps(outs[i], in)) return JSCAN_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return JSCAN_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    using U = uint16_t;
    auto xs = static_cast<const U *>(x), wx = static_cast<const U *>(w_x), wd = static_cast<const U *>(w_dt);
    auto dl = static_cast<U *>(delta_low), de = static_cast<U *>(delta), bo = static_cast<U *>(B), co = static_cast<U *>(C);
    if (R == 64) launch_ssm_inputs<64>(xs, wx, g_delta, g_B, g_C, wd, b_dt, dl, de, bo, co, M, (int)D, eps, s);
    else if (R == 128) launch_ssm_inputs<128>(xs, wx, g_delta, g_B, g_C, wd, b_dt, dl, de, bo, co, M, (int)D, eps, s);
    else launch_ssm_inputs<256>(xs, wx, g_delta, g_B, g_C, wd, b_dt, dl, de, bo, co, M, (int)D, eps, s);
    return launch_status();
}

jscan_status jscan_prefill_fused(const void *x, const void *delta_low, const void *w_dt, const float *b_dt,
                                 const float *A, const void *B, const void *C, const float *h0, void *y,
                                 float *h_final, int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R,
                                 jscan_dtype dtype, void *stream) {
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    bool empty = false;
    // the usual prefill checks, with x standing in for delta (same shape)
    jscan_status st = check_prefill(x, x, A, B, C, h0, false, y, h_final, batch, L, D, N, dtype, &empty);
    if (st != JSCAN_OK) return st;
    if (R != jscan::fused::kRank) return JSCAN_ERR_SHAPE;
    if (empty) return JSCAN_OK;
    if (!jscan::rows_kernel_applies(batch, D)) return JSCAN_ERR_SHAPE;
    if (!w_dt || !b_dt || (L > 0 && !delta_low)) return JSCAN_ERR_NULL;
    const void *more[] = {delta_low, w_dt, b_dt};
    for (const void *p : more)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;
    const int64_t seq = batch * L * D * 2, state = batch * D * N * 4;
    const Span outs[] = {span(y, L > 0 ? seq : 0), span(h_final, state)};
    const Span ins[] = {span(delta_low, batch * L * R * 2), span(w_dt, D * R * 2), span(b_dt, D * 4)};
    for (const Span &o : outs)
        for (const Span &i : ins)
            if (overlaps(o, i)) return JSCAN_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (L == 0) return launch_prefill<jscan::BF16>(x, x, A, B, C, h0, y, h_final, batch, L, D, s);
    using U = uint16_t;
    const jscan::Segments sg{L, L, 1, 0};
    const jscan::DeltaProj dp{static_cast<const U *>(delta_low), static_cast<const U *>(w_dt), b_dt};
    jscan::launch_prefill_rows<jscan::BF16, true>(static_cast<const U *>(x), nullptr, A, static_cast<const U *>(B),
                                                  static_cast<const U *>(C), h0, static_cast<U *>(y), h_final, sg,
                                                  batch, (int)D, s, dp);
    return launch_status();
}

const char *jscan_status_string(jscan_status s) {
    switch (s) {
    case JSCAN_OK: return "ok";
    case JSCAN_ERR_NULL: return "a required pointer is NULL";
    case JSCAN_ERR_SHAPE: return "bad shape (negative size, N != 16, D not a multiple of 8, or bad row stride)";
    case JSCAN_ERR_DTYPE: return "unknown dtype";
    case JSCAN_ERR_ALIGN: return "array pointer not 16-byte aligned";
    case JSCAN_ERR_ALIAS: return "an output overlaps an input or another output";
    case JSCAN_ERR_HIP: return "HIP launch failed (see jscan_last_hip_error)";
    case JSCAN_ERR_WORKSPACE: return "workspace smaller than jscan_prefill_chunked_workspace() bytes";
    case JSCAN_ERR_FORM: return "unknown form of A";
    }
    return "unknown status";
}

int jscan_last_hip_error(void) { return g_last_hip_error; }

int jscan_version(void) { return 109; }

}  // extern "C"
