// jscan.hip - libjscan: host entry points of the C ABI declared in include/jscan.h, plus
// the kernels they launch (included below).  Everything runs on the caller's stream; the
// library allocates nothing and keeps no state except the calling thread's last HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/jscan.h"
#include "prefill_lane_kernel.h"
#include "prefill_rows_kernel.h"
#include "step_kernel.h"

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

// ---- prefill ---------------------------------------------------------------------------

template <typename E>
jscan_status launch_prefill(const void *x, const void *delta, const float *A, const void *B,
                            const void *C, const float *h0, void *y, float *h_final,
                            int64_t batch, int64_t L, int64_t D, hipStream_t stream) {
    using T = typename E::store_t;
    if (L == 0) {
        const int64_t count = batch * D * jscan::kDState;
        const int64_t blocks = (count + 255) / 256;
        hipLaunchKernelGGL(jscan::copy_state_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           h0, h_final, count);
        return launch_status();
    }
    if (jscan::rows_kernel_applies(batch, D)) {
        return jscan::launch_prefill_rows<E>(static_cast<const T *>(x), static_cast<const T *>(delta), A,
                                             static_cast<const T *>(B), static_cast<const T *>(C), h0,
                                             static_cast<T *>(y), h_final, batch, L, (int)D, stream)
                   ? launch_status()
                   : JSCAN_ERR_HIP;
    }
    const int blocks_per_row = (int)((D + 63) / 64);
    hipLaunchKernelGGL(jscan::prefill_lane_kernel<E>, dim3((unsigned)(batch * blocks_per_row)), dim3(64), 0,
                       stream, static_cast<const T *>(x), static_cast<const T *>(delta), A,
                       static_cast<const T *>(B), static_cast<const T *>(C), h0, static_cast<T *>(y),
                       h_final, L, (int)D, blocks_per_row);
    return launch_status();
}

jscan_status prefill_impl(const void *x, const void *delta, const float *A, const void *B,
                          const void *C, const float *h0, bool resume, void *y, float *h_final,
                          int64_t batch, int64_t L, int64_t D, int64_t N, jscan_dtype dtype,
                          void *stream) {
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (batch < 0 || L < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0) return JSCAN_ERR_SHAPE;
    // index arithmetic inside the kernels: rows of D fit in int, grid sizes in 32 bits
    if (D > (1 << 24) || batch > (1 << 20)) return JSCAN_ERR_SHAPE;
    if (batch == 0 || D == 0) return JSCAN_OK;
    if (!A || !h_final || (resume && !h0)) return JSCAN_ERR_NULL;
    if (L > 0 && (!x || !delta || !B || !C || !y)) return JSCAN_ERR_NULL;

    const int64_t es = elem_bytes(dtype);
    const void *arrays[] = {x, delta, A, B, C, h0, y, h_final};
    for (const void *p : arrays)
        if (p && !aligned16(p)) return JSCAN_ERR_ALIGN;

    const int64_t seq = batch * L * D * es, bc = batch * L * N * es;
    const int64_t state = batch * D * N * 4, a_bytes = D * N * 4;
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

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == JSCAN_BF16)
        return launch_prefill<jscan::BF16>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
    return launch_prefill<jscan::F32>(x, delta, A, B, C, h0, y, h_final, batch, L, D, s);
}

// ---- decode step -----------------------------------------------------------------------

template <typename E>
jscan_status launch_step(float *h, const void *x_t, const void *delta_t, const float *A,
                         const void *B_t, const void *C_t, void *y_t, int64_t batch, int64_t D,
                         int64_t ld_xd, int64_t ld_bc, hipStream_t stream) {
    using T = typename E::store_t;
    const int blocks_per_rows = (int)((D * 4 + 255) / 256);
    const int64_t row_groups = (batch + jscan::step::kRows - 1) / jscan::step::kRows;
    hipLaunchKernelGGL(jscan::step_kernel<E>, dim3((unsigned)(row_groups * blocks_per_rows)), dim3(256), 0, stream,
                       h, static_cast<const T *>(x_t), static_cast<const T *>(delta_t), A,
                       static_cast<const T *>(B_t), static_cast<const T *>(C_t), static_cast<T *>(y_t), (int)batch,
                       (int)D, blocks_per_rows, ld_xd, ld_bc);
    return launch_status();
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

jscan_status jscan_step(float *h, const void *x_t, const void *delta_t, const float *A,
                        const void *B_t, const void *C_t, void *y_t, int64_t batch, int64_t D,
                        int64_t N, int64_t ld_xd, int64_t ld_bc, jscan_dtype dtype,
                        void *stream) {
    if (dtype != JSCAN_F32 && dtype != JSCAN_BF16) return JSCAN_ERR_DTYPE;
    if (batch < 0 || D < 0 || N != JSCAN_D_STATE || D % 8 != 0) return JSCAN_ERR_SHAPE;
    if (D > (1 << 24) || batch > (1 << 20)) return JSCAN_ERR_SHAPE;
    if (batch == 0 || D == 0) return JSCAN_OK;
    if (ld_xd < D || ld_bc < N || ld_xd % 8 != 0 || ld_bc % 8 != 0) return JSCAN_ERR_SHAPE;
    if (!h || !x_t || !delta_t || !A || !B_t || !C_t || !y_t) return JSCAN_ERR_NULL;
    const void *arrays[] = {h, x_t, delta_t, A, B_t, C_t, y_t};
    for (const void *p : arrays)
        if (!aligned16(p)) return JSCAN_ERR_ALIGN;

    const int64_t es = elem_bytes(dtype);
    const int64_t rows_xd = ((batch - 1) * ld_xd + D) * es, rows_bc = ((batch - 1) * ld_bc + N) * es;
    const Span sh = span(h, batch * D * N * 4), sy = span(y_t, rows_xd);
    const Span inputs[] = {span(x_t, rows_xd), span(delta_t, rows_xd), span(A, D * N * 4), span(B_t, rows_bc),
                           span(C_t, rows_bc)};
    for (const Span &s : inputs)
        if (overlaps(sy, s) || overlaps(sh, s)) return JSCAN_ERR_ALIAS;
    if (overlaps(sy, sh)) return JSCAN_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == JSCAN_BF16)
        return launch_step<jscan::BF16>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, s);
    return launch_step<jscan::F32>(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, s);
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
    }
    return "unknown status";
}

int jscan_last_hip_error(void) { return g_last_hip_error; }

int jscan_version(void) { return 100; }

}  // extern "C"
