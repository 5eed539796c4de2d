"""libjscan: the Mamba-1 (S6) selective state-space scan on AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI of ``include/jscan.h``;
this package only marshals torch tensors (device memory and streams) into those calls.
There is no CPU fallback: without the built library every call raises.

    y, h_final = prefill(x, delta, A, B, C)                # scan from the zero state
    y, h_final = prefill(x, delta, A, B, C, h0=h)          # resume from a state
    y_t = step(h, x_t, delta_t, A, B_t, C_t)               # one decode token, h in place
    y, h_final = prefill_chunked(x, delta, A, B, C)        # time-parallel, for few channels
"""
from ._binding import (  # noqa: F401
    D_STATE,
    JScanError,
    chunked_workspace_bytes,
    library,
    library_path,
    prefill,
    prefill_chunked,
    step,
    step_raw,
)
