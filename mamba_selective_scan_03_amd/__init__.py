"""libjscan: the Mamba-1 (S6) selective state-space scan on AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of ``include/jscan.h``;
this package only marshals torch tensors (device memory and streams) into those calls.
There is no CPU fallback: without the built library every call raises.

    y, h_final = prefill(x, delta, A, B, C)                # scan from the zero state
    y, h_final = prefill(x, delta, A, B, C, h0=h)          # resume from a state
    y_t = step(h, x_t, delta_t, A, B_t, C_t)               # one decode token, h in place
    y, h_final = prefill_chunked(x, delta, A, B, C)        # time-parallel, for few channels
    delta, B, C, d_low = ssm_inputs(x, w_x, g_d, g_B, g_C, w_dt, b_dt)   # producer side (MFMA)
    y, h_final = prefill_fused(x, d_low, w_dt, b_dt, A, B, C)             # delta computed in the scan
    y, h_final = prefill_scalar_a(x, delta, a, B, C)       # scaled-identity A (a: [D])
    y_t = step_scalar_a(h, x_t, delta_t, a, B_t, C_t)
    y, h_final = prefill_complex(x, delta, A, B, C)        # complex-valued state (pairs of states)
    y_t = step_complex(h, x_t, delta_t, A, B_t, C_t)
    y, h_final = prefill_trapezoid(x, delta, lam, A, B, C, form="diagonal")   # exponential-trapezoidal rule
    y_t = step_trapezoid(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t)
    y, h_final = prefill_mimo(x, delta, A, B, C)          # R inputs and outputs per channel (MIMO)
    y_t = step_mimo(h, x_t, delta_t, A, B_t, C_t)
    y, h_final = prefill_mimo_trapezoid(x, delta, lam, A, B, C)   # both Mamba-3 changes together
    y_t = step_mimo_trapezoid(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t)
"""
from ._binding import (  # noqa: F401
    A_FORMS,
    D_STATE,
    JScanError,
    chunked_workspace_bytes,
    library,
    library_path,
    prefill,
    prefill_chunked,
    prefill_chunked_noalloc,
    prefill_complex,
    prefill_fused,
    prefill_mimo,
    prefill_mimo_trapezoid,
    prefill_scalar_a,
    prefill_trapezoid,
    ssm_inputs,
    step,
    step_complex,
    step_mimo,
    step_mimo_trapezoid,
    step_raw,
    step_scalar_a,
    step_trapezoid,
)
