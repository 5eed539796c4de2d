"""ctypes binding of libjscan (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libjscan.so")

D_STATE = 16
JSCAN_F32, JSCAN_BF16 = 0, 1
_DTYPES = {torch.float32: JSCAN_F32, torch.bfloat16: JSCAN_BF16}
_lib = None


class JScanError(RuntimeError):
    """A libjscan call returned an error status."""

    def __init__(self, status: int, msg: str, hip_error: int = 0):
        super().__init__(f"libjscan: {msg} (status {status}" + (f", hipError {hip_error})" if hip_error else ")"))
        self.status = status
        self.hip_error = hip_error


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libjscan.so (building it first if it is missing) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build

        build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, i64, i32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.jscan_prefill.argtypes = [vp, vp, fp, vp, vp, vp, fp, i64, i64, i64, i64, i32, vp]
    lib.jscan_prefill_resume.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i32, vp]
    lib.jscan_step.argtypes = [fp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.jscan_prefill_chunked.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i64, vp, i64, i32, vp]
    lib.jscan_prefill_chunked_workspace.argtypes = [i64, i64, i64, i64, i64]
    lib.jscan_prefill_chunked_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i64, i32, vp]
    lib.jscan_prefill_chunked_noalloc.restype = i32
    lib.jscan_ssm_inputs.argtypes = [vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, i32,
                                     vp]
    lib.jscan_ssm_inputs.restype = i32
    lib.jscan_prefill_fused.argtypes = [vp, vp, vp, fp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i64, i32, vp]
    lib.jscan_prefill_fused.restype = i32
    lib.jscan_prefill_scalar_a.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i32, vp]
    lib.jscan_step_scalar_a.argtypes = [fp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.jscan_prefill_complex.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i32, vp]
    lib.jscan_step_complex.argtypes = [fp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.jscan_prefill_trapezoid.argtypes = [vp, vp, vp, fp, vp, vp, fp, vp, vp, vp, fp, i64, i64, i64, i64, i32, i32, vp]
    lib.jscan_step_trapezoid.argtypes = [fp, vp, vp, vp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32,
                                         vp]
    lib.jscan_prefill_mimo.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i64, i64, i64, i64, i64, i32, i32, vp]
    lib.jscan_step_mimo.argtypes = [fp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp]
    lib.jscan_prefill_mimo_trapezoid.argtypes = [vp, vp, vp, fp, vp, vp, fp, vp, vp, vp, fp, i64, i64, i64, i64, i64,
                                                 i32, i32, vp]
    lib.jscan_step_mimo_trapezoid.argtypes = [fp, vp, vp, vp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                              i64, i32, i32, vp]
    lib.jscan_prefill_chunked_workspace.restype = i64
    for f in (lib.jscan_prefill, lib.jscan_prefill_resume, lib.jscan_step, lib.jscan_prefill_chunked,
              lib.jscan_prefill_scalar_a, lib.jscan_step_scalar_a, lib.jscan_prefill_complex, lib.jscan_step_complex,
              lib.jscan_prefill_trapezoid, lib.jscan_step_trapezoid, lib.jscan_prefill_mimo, lib.jscan_step_mimo,
              lib.jscan_prefill_mimo_trapezoid, lib.jscan_step_mimo_trapezoid):
        f.restype = i32
    lib.jscan_status_string.argtypes = [i32]
    lib.jscan_status_string.restype = ctypes.c_char_p
    lib.jscan_last_hip_error.restype = i32
    lib.jscan_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = library()
        raise JScanError(status, lib.jscan_status_string(status).decode(), lib.jscan_last_hip_error())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_prefill_args(x, delta, A, B, C, h0, scalar_a=False):
    _require(x.is_cuda, "inputs must be CUDA (HIP) tensors")
    _require(x.dtype in _DTYPES, "x must be bfloat16 or float32")
    _require(x.dim() == 3, "x must be [batch, L, D]")
    batch, L, D = x.shape
    a_shape = (D,) if scalar_a else (D, D_STATE)
    for name, t, shape, dt in (("delta", delta, (batch, L, D), x.dtype), ("A", A, a_shape, torch.float32),
                               ("B", B, (batch, L, D_STATE), x.dtype), ("C", C, (batch, L, D_STATE), x.dtype)):
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt, f"{name} must be {dt}")
        _require(t.device == x.device, f"{name} is on another device")
        _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(x.is_contiguous(), "x must be contiguous")
    if h0 is not None:
        _require(tuple(h0.shape) == (batch, D, D_STATE) and h0.dtype == torch.float32 and h0.is_contiguous()
                 and h0.device == x.device, "h0 must be a contiguous fp32 [batch, D, 16] tensor on x's device")
    return batch, L, D


def prefill(x, delta, A, B, C, h0=None, y=None, h_final=None):
    """Scan ``L`` tokens.  x, delta ``[batch, L, D]``, B, C ``[batch, L, 16]`` (bf16 or fp32, one
    dtype), A ``[D, 16]`` fp32, optional h0 ``[batch, D, 16]`` fp32 to resume from.
    Returns ``(y [batch, L, D] in the input dtype, h_final [batch, D, 16] fp32)``.
    ``h_final`` may be passed as ``h0`` itself to update a state in place."""
    batch, L, D = _check_prefill_args(x, delta, A, B, C, h0)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    args_tail = (ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(h_final.data_ptr()), batch, L, D, D_STATE,
                 _DTYPES[x.dtype], _stream(x.device))
    with torch.cuda.device(x.device):
        if h0 is None:
            st = lib.jscan_prefill(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), *args_tail)
        else:
            st = lib.jscan_prefill_resume(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), *args_tail)
    _check(st)
    return y, h_final


def prefill_scalar_a(x, delta, a, B, C, h0=None, y=None, h_final=None):
    """Prefill with a scaled-identity A (``jscan_prefill_scalar_a``): ``a`` ``[D]`` fp32 stands
    for ``A[d, n] = a[d]``.  Bit-identical to :func:`prefill` on that expanded A, and faster
    (one decay per token and channel).  Other arguments and results as for :func:`prefill`."""
    batch, L, D = _check_prefill_args(x, delta, a, B, C, h0, scalar_a=True)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_scalar_a(_ptr(x), _ptr(delta), _ptr(a), _ptr(B), _ptr(C), _ptr(h0), _ptr(y),
                                        _ptr(h_final), batch, L, D, D_STATE, _DTYPES[x.dtype], _stream(x.device))
    _check(st)
    return y, h_final


def prefill_complex(x, delta, A, B, C, h0=None, y=None, h_final=None):
    """Prefill with the complex-valued state (``jscan_prefill_complex``): states 2k, 2k+1 of a
    channel are one complex state and ``A[d, 2k], A[d, 2k+1]`` the real and imaginary parts of
    its diagonal entry.  Arguments and results as for :func:`prefill`."""
    batch, L, D = _check_prefill_args(x, delta, A, B, C, h0)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_complex(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y),
                                       _ptr(h_final), batch, L, D, D_STATE, _DTYPES[x.dtype], _stream(x.device))
    _check(st)
    return y, h_final


def chunked_workspace_bytes(batch: int, L: int, D: int, chunk: int = 0) -> int:
    """Bytes of workspace ``prefill_chunked`` needs (0 when it runs as one segment)."""
    n = library().jscan_prefill_chunked_workspace(batch, L, D, D_STATE, chunk)
    if n < 0:
        raise ValueError(f"invalid shape or chunk: batch={batch} L={L} D={D} chunk={chunk}")
    return n


def prefill_chunked(x, delta, A, B, C, h0=None, y=None, h_final=None, chunk=0, workspace=None):
    """Time-parallel prefill (``jscan_prefill_chunked``): the same result as :func:`prefill` up
    to fp32 rounding of the segment composition, for shapes with too few channels to fill
    the GPU.  ``chunk`` is the segment length in tokens (0 = automatic).  ``workspace`` is a
    CUDA tensor of at least :func:`chunked_workspace_bytes` bytes; one is allocated if None."""
    batch, L, D = _check_prefill_args(x, delta, A, B, C, h0)
    need = chunked_workspace_bytes(batch, L, D, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_chunked(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y),
                                       _ptr(h_final), batch, L, D, D_STATE, chunk, _ptr(workspace), ws_bytes,
                                       _DTYPES[x.dtype], _stream(x.device))
    _check(st)
    return y, h_final


NOALLOC_SCRATCH_BYTES = 24 * 1024 * 1024   # JSCAN_NOALLOC_SCRATCH_BYTES


def prefill_chunked_noalloc(x, delta, A, B, C, h0=None, y=None, h_final=None, chunk=0):
    """:func:`prefill_chunked` through ``jscan_prefill_chunked_noalloc``: the library's own
    scratch array instead of a workspace (calls on one GPU must not overlap in time).  Pass
    ``y`` and ``h_final`` to allocate nothing here either."""
    batch, L, D = _check_prefill_args(x, delta, A, B, C, h0)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_chunked_noalloc(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y),
                                               _ptr(h_final), batch, L, D, D_STATE, chunk, _DTYPES[x.dtype],
                                               _stream(x.device))
    _check(st)
    return y, h_final


def ssm_inputs(x, w_x, g_delta, g_B, g_C, w_dt, b_dt, eps=1e-6, delta=None, B=None, C=None, delta_low=None,
               skip_delta=False):
    """Producer side (``jscan_ssm_inputs``): delta, B and C of the scan computed from x.
    x ``[..., D]`` bf16; w_x ``[R + 32, D]`` bf16; gains fp32 ``[R]``, ``[16]``, ``[16]``;
    w_dt ``[D, R]`` bf16; b_dt ``[D]`` fp32.  Returns ``(delta [..., D], B [..., 16], C [..., 16],
    delta_low [..., R])``, all bf16, with x's leading shape.  ``skip_delta`` runs only the first
    product (delta is then None): the input of :func:`prefill_fused`."""
    _require(x.is_cuda and x.dtype == torch.bfloat16 and x.is_contiguous(), "x must be a contiguous bf16 CUDA tensor")
    D = x.shape[-1]
    lead = tuple(x.shape[:-1])
    M = x.numel() // D if D else 0
    R = w_dt.shape[1] if w_dt.dim() == 2 else -1
    for name, t, shape, dt in (("w_x", w_x, (R + 2 * D_STATE, D), torch.bfloat16),
                               ("g_delta", g_delta, (R,), torch.float32), ("g_B", g_B, (D_STATE,), torch.float32),
                               ("g_C", g_C, (D_STATE,), torch.float32), ("w_dt", w_dt, (D, R), torch.bfloat16),
                               ("b_dt", b_dt, (D,), torch.float32)):
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt and t.is_contiguous() and t.device == x.device, f"{name} must be contiguous {dt} on x's device")
    dev = x.device
    if skip_delta:
        delta = None
    elif delta is None:
        delta = torch.empty(lead + (D,), dtype=torch.bfloat16, device=dev)
    B = torch.empty(lead + (D_STATE,), dtype=torch.bfloat16, device=dev) if B is None else B
    C = torch.empty(lead + (D_STATE,), dtype=torch.bfloat16, device=dev) if C is None else C
    delta_low = torch.empty(lead + (R,), dtype=torch.bfloat16, device=dev) if delta_low is None else delta_low
    lib = library()
    with torch.cuda.device(dev):
        st = lib.jscan_ssm_inputs(_ptr(x), _ptr(w_x), _ptr(g_delta), _ptr(g_B), _ptr(g_C), _ptr(w_dt), _ptr(b_dt),
                                  _ptr(delta_low), _ptr(delta), _ptr(B), _ptr(C), M, D, R, D_STATE, float(eps),
                                  JSCAN_BF16, _stream(dev))
    _check(st)
    return delta, B, C, delta_low


def prefill_fused(x, delta_low, w_dt, b_dt, A, B, C, h0=None, y=None, h_final=None):
    """Prefill with delta computed inside the scan from delta_low (``jscan_prefill_fused``):
    bit-identical to ``ssm_inputs`` then ``prefill``.  bf16, rank 256, long-sequence shapes."""
    _require(x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 3 and x.is_contiguous(),
             "x must be a contiguous bf16 [batch, L, D] CUDA tensor")
    batch, L, D = x.shape
    R = delta_low.shape[-1]
    for name, t, shape, dt in (("delta_low", delta_low, (batch, L, R), torch.bfloat16),
                               ("w_dt", w_dt, (D, R), torch.bfloat16), ("b_dt", b_dt, (D,), torch.float32),
                               ("A", A, (D, D_STATE), torch.float32), ("B", B, (batch, L, D_STATE), torch.bfloat16),
                               ("C", C, (batch, L, D_STATE), torch.bfloat16)):
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt and t.is_contiguous() and t.device == x.device, f"{name} must be contiguous {dt}")
    if h0 is not None:
        _require(tuple(h0.shape) == (batch, D, D_STATE) and h0.dtype == torch.float32 and h0.is_contiguous(),
                 "h0 must be a contiguous fp32 [batch, D, 16] tensor")
    y = torch.empty_like(x) if y is None else y
    h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device) if h_final is None else h_final
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_fused(_ptr(x), _ptr(delta_low), _ptr(w_dt), _ptr(b_dt), _ptr(A), _ptr(B), _ptr(C),
                                     _ptr(h0), _ptr(y), _ptr(h_final), batch, L, D, D_STATE, R, JSCAN_BF16,
                                     _stream(x.device))
    _check(st)
    return y, h_final


def _step_output(y_t, shape, dtype, device):
    """The output of a decode step and its row stride in elements: a new contiguous tensor, or
    the caller's ``y_t`` of that shape and dtype whose rows are contiguous (the row stride of a
    strided view, e.g. ``y[:, t]``, is passed to the library, which checks it)."""
    if y_t is None:
        y_t = torch.empty(shape, dtype=dtype, device=device)
    _require(tuple(y_t.shape) == tuple(shape) and y_t.dtype == dtype and y_t.device == device,
             f"y_t must be {tuple(shape)} of dtype {dtype} on {device}")
    row = 1
    for k in range(len(shape) - 1, 0, -1):
        _require(y_t.stride(k) == row, "y_t rows must be contiguous")
        row *= shape[k]
    return y_t, (y_t.stride(0) if shape[0] > 1 else row)


def step_raw(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, dtype, scalar_a=False, complex_a=False,
             ld_y=None):
    """Direct call of ``jscan_step`` (``jscan_step_scalar_a`` with ``scalar_a``,
    ``jscan_step_complex`` with ``complex_a``) on raw tensors/pointers with explicit row strides
    (no checks beyond the library's own; ``ld_y`` defaults to ``ld_xd``).  ``x_t`` etc. may be
    tensors or integer device addresses."""
    lib = library()

    def p(v):
        return ctypes.c_void_p(v if isinstance(v, int) else v.data_ptr())

    dev = h.device if hasattr(h, "device") else torch.device("cuda")
    fn = lib.jscan_step_scalar_a if scalar_a else lib.jscan_step_complex if complex_a else lib.jscan_step
    st = fn(p(h), p(x_t), p(delta_t), p(A), p(B_t), p(C_t), p(y_t), batch, D, D_STATE, ld_xd, ld_bc,
            ld_xd if ld_y is None else ld_y, _DTYPES[dtype], _stream(dev))
    _check(st)


def step_scalar_a(h, x_t, delta_t, a, B_t, C_t, y_t=None):
    """:func:`step` with a scaled-identity A, ``a`` ``[D]`` fp32 (``jscan_step_scalar_a``)."""
    return step(h, x_t, delta_t, a, B_t, C_t, y_t, _scalar_a=True)


def step_complex(h, x_t, delta_t, A, B_t, C_t, y_t=None):
    """:func:`step` with the complex-valued state (``jscan_step_complex``)."""
    return step(h, x_t, delta_t, A, B_t, C_t, y_t, _complex_a=True)


def step(h, x_t, delta_t, A, B_t, C_t, y_t=None, _scalar_a=False, _complex_a=False):
    """One decode token for a batch: h ``[batch, D, 16]`` fp32 is updated in place; x_t, delta_t
    ``[batch, D]`` and B_t, C_t ``[batch, 16]`` (rows may be strided views of prefill tensors,
    e.g. ``x[:, t]``).  Returns y_t ``[batch, D]``: a new contiguous tensor, or the given ``y_t``,
    whose rows may be strided too (for example ``y[:, t]`` of a ``[batch, L, D]`` output)."""
    _require(h.is_cuda and h.dtype == torch.float32 and h.dim() == 3 and h.shape[2] == D_STATE and h.is_contiguous(),
             "h must be a contiguous fp32 [batch, D, 16] CUDA tensor")
    batch, D, _ = h.shape
    _require(x_t.dtype in _DTYPES, "x_t must be bfloat16 or float32")
    for name, t, shape in (("x_t", x_t, (batch, D)), ("delta_t", delta_t, (batch, D)),
                           ("B_t", B_t, (batch, D_STATE)), ("C_t", C_t, (batch, D_STATE))):
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}")
        _require(t.dtype == x_t.dtype, f"{name} must be {x_t.dtype}")
        _require(t.stride(1) == 1, f"{name} rows must be contiguous")
        _require(t.device == h.device, f"{name} is on another device")
    a_shape = (D,) if _scalar_a else (D, D_STATE)
    _require(A.dtype == torch.float32 and tuple(A.shape) == a_shape and A.is_contiguous(),
             f"A must be a contiguous fp32 tensor of shape {a_shape}")
    ld_xd = x_t.stride(0) if batch > 1 else D
    _require(batch <= 1 or delta_t.stride(0) == ld_xd, "x_t and delta_t must share a row stride")
    ld_bc = B_t.stride(0) if batch > 1 else D_STATE
    _require(batch <= 1 or C_t.stride(0) == ld_bc, "B_t and C_t must share a row stride")
    y_t, ld_y = _step_output(y_t, (batch, D), x_t.dtype, h.device)
    with torch.cuda.device(h.device):
        step_raw(h, x_t, delta_t, A, B_t, C_t, y_t, batch, D, ld_xd, ld_bc, x_t.dtype, scalar_a=_scalar_a,
                 complex_a=_complex_a, ld_y=ld_y)
    return y_t


# ---- exponential-trapezoidal rule ----------------------------------------------------------
# jscan_a_form values: the form of A that the trapezoidal entry points take.
A_FORMS = {"diagonal": 0, "scalar": 1, "complex": 2}


def prefill_trapezoid(x, delta, lam, A, B, C, h0=None, x_prev=None, B_prev=None, form="diagonal", y=None,
                      h_final=None):
    """Prefill with the exponential-trapezoidal rule (``jscan_prefill_trapezoid``).  ``lam``
    ``[batch, L, D]`` (x's dtype) weights each step's right end; the left end, the previous
    token's input, gets ``1 - lam`` and decays over the step.  ``x_prev [batch, D]`` and
    ``B_prev [batch, 16]`` are the token before the first (omit both for a fresh sequence).
    ``form``: "diagonal" (A ``[D, 16]``), "scalar" (a ``[D]``) or "complex" (A ``[D, 16]`` as
    (real, imaginary) pairs).  Other arguments and results as for :func:`prefill`."""
    _require(form in A_FORMS, f"form must be one of {tuple(A_FORMS)}")
    batch, L, D = _check_prefill_args(x, delta, A, B, C, h0, scalar_a=form == "scalar")
    _require(tuple(lam.shape) == (batch, L, D) and lam.dtype == x.dtype and lam.is_contiguous()
             and lam.device == x.device, "lam must be a contiguous [batch, L, D] tensor like x")
    _require((x_prev is None) == (B_prev is None), "x_prev and B_prev go together")
    if x_prev is not None:
        for name, t, shape in (("x_prev", x_prev, (batch, D)), ("B_prev", B_prev, (batch, D_STATE))):
            _require(tuple(t.shape) == shape and t.dtype == x.dtype and t.is_contiguous() and t.device == x.device,
                     f"{name} must be a contiguous {shape} tensor like x")
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_trapezoid(_ptr(x), _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(h0),
                                         _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(h_final), batch, L, D, D_STATE,
                                         A_FORMS[form], _DTYPES[x.dtype], _stream(x.device))
    _check(st)
    return y, h_final


def step_trapezoid(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t, form="diagonal", y_t=None):
    """One decode token with the exponential-trapezoidal rule (``jscan_step_trapezoid``): as
    :func:`step`, plus the previous token's ``x_prev [batch, D]`` and ``B_prev [batch, 16]``
    (zeros before a sequence's first token) and this token's ``lam_t [batch, D]``.  x_prev and
    lam_t share x_t's row stride, B_prev shares B_t's."""
    _require(form in A_FORMS, f"form must be one of {tuple(A_FORMS)}")
    _require(h.is_cuda and h.dtype == torch.float32 and h.dim() == 3 and h.shape[2] == D_STATE and h.is_contiguous(),
             "h must be a contiguous fp32 [batch, D, 16] CUDA tensor")
    batch, D, _ = h.shape
    _require(x_t.dtype in _DTYPES, "x_t must be bfloat16 or float32")
    ld_xd = x_t.stride(0) if batch > 1 else D
    ld_bc = B_t.stride(0) if batch > 1 else D_STATE
    for name, t, shape, ld in (("x_t", x_t, (batch, D), ld_xd), ("delta_t", delta_t, (batch, D), ld_xd),
                               ("lam_t", lam_t, (batch, D), ld_xd), ("x_prev", x_prev, (batch, D), ld_xd),
                               ("B_t", B_t, (batch, D_STATE), ld_bc), ("C_t", C_t, (batch, D_STATE), ld_bc),
                               ("B_prev", B_prev, (batch, D_STATE), ld_bc)):
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}")
        _require(t.dtype == x_t.dtype, f"{name} must be {x_t.dtype}")
        _require(t.stride(1) == 1 and (batch <= 1 or t.stride(0) == ld), f"{name} rows must be contiguous with "
                 f"the row stride of {'x_t' if ld is ld_xd else 'B_t'}")
        _require(t.device == h.device, f"{name} is on another device")
    a_shape = (D,) if form == "scalar" else (D, D_STATE)
    _require(A.dtype == torch.float32 and tuple(A.shape) == a_shape and A.is_contiguous(),
             f"A must be a contiguous fp32 tensor of shape {a_shape}")
    y_t, ld_y = _step_output(y_t, (batch, D), x_t.dtype, h.device)
    lib = library()
    with torch.cuda.device(h.device):
        st = lib.jscan_step_trapezoid(_ptr(h), _ptr(x_prev), _ptr(B_prev), _ptr(x_t), _ptr(delta_t), _ptr(lam_t),
                                      _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y_t), batch, D, D_STATE, ld_xd, ld_bc,
                                      ld_y, A_FORMS[form], _DTYPES[x_t.dtype], _stream(h.device))
    _check(st)
    return y_t


# ---- multi-input, multi-output (MIMO) --------------------------------------------------------

def prefill_mimo(x, delta, A, B, C, h0=None, form="diagonal", y=None, h_final=None):
    """MIMO prefill (``jscan_prefill_mimo``): each channel takes R inputs and gives R outputs.
    x ``[batch, L, D, R]``, delta ``[batch, L, D]``, B, C ``[batch, L, 16, R]`` (one dtype),
    A as for ``form`` ("diagonal" ``[D, 16]``, "scalar" ``[D]``, "complex" ``[D, 16]``), optional
    h0 ``[batch, D, 16]``; R is 1, 2, 4 or 8.  Returns ``(y [batch, L, D, R], h_final)``."""
    batch, L, D, R = _check_mimo_args(x, delta, A, B, C, h0, form)
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_mimo(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y), _ptr(h_final),
                                    batch, L, D, D_STATE, R, A_FORMS[form], _DTYPES[x.dtype], _stream(x.device))
    _check(st)
    return y, h_final


def _check_mimo_args(x, delta, A, B, C, h0, form):
    _require(form in A_FORMS, f"form must be one of {tuple(A_FORMS)}")
    _require(x.is_cuda and x.dtype in _DTYPES and x.dim() == 4 and x.is_contiguous(),
             "x must be a contiguous [batch, L, D, R] CUDA tensor (bfloat16 or float32)")
    batch, L, D, R = x.shape
    a_shape = (D,) if form == "scalar" else (D, D_STATE)
    for name, t, shape, dt in (("delta", delta, (batch, L, D), x.dtype), ("A", A, a_shape, torch.float32),
                               ("B", B, (batch, L, D_STATE, R), x.dtype), ("C", C, (batch, L, D_STATE, R), x.dtype)):
        _require(tuple(t.shape) == shape, f"{name} must have shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt and t.is_contiguous() and t.device == x.device, f"{name} must be a contiguous {dt} "
                 "tensor on x's device")
    if h0 is not None:
        _require(tuple(h0.shape) == (batch, D, D_STATE) and h0.dtype == torch.float32 and h0.is_contiguous()
                 and h0.device == x.device, "h0 must be a contiguous fp32 [batch, D, 16] tensor on x's device")
    return batch, L, D, R


def prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0=None, x_prev=None, B_prev=None, form="diagonal", y=None,
                           h_final=None):
    """MIMO prefill with the exponential-trapezoidal rule (``jscan_prefill_mimo_trapezoid``): as
    :func:`prefill_mimo`, plus ``lam`` ``[batch, L, D]`` (the right-end weight, x's dtype) and the
    token before the first, ``x_prev [batch, D, R]`` and ``B_prev [batch, 16, R]`` (omit both for a
    fresh sequence)."""
    batch, L, D, R = _check_mimo_args(x, delta, A, B, C, h0, form)
    _require(tuple(lam.shape) == (batch, L, D) and lam.dtype == x.dtype and lam.is_contiguous()
             and lam.device == x.device, "lam must be a contiguous [batch, L, D] tensor like x")
    _require((x_prev is None) == (B_prev is None), "x_prev and B_prev go together")
    if x_prev is not None:
        for name, t, shape in (("x_prev", x_prev, (batch, D, R)), ("B_prev", B_prev, (batch, D_STATE, R))):
            _require(tuple(t.shape) == shape and t.dtype == x.dtype and t.is_contiguous() and t.device == x.device,
                     f"{name} must be a contiguous {shape} tensor like x")
    if y is None:
        y = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((batch, D, D_STATE), dtype=torch.float32, device=x.device)
    lib = library()
    with torch.cuda.device(x.device):
        st = lib.jscan_prefill_mimo_trapezoid(_ptr(x), _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(h0),
                                              _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(h_final), batch, L, D, D_STATE,
                                              R, A_FORMS[form], _DTYPES[x.dtype], _stream(x.device))
    _check(st)
    return y, h_final


def step_mimo_trapezoid(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t, form="diagonal", y_t=None):
    """One MIMO decode token with the exponential-trapezoidal rule (``jscan_step_mimo_trapezoid``):
    as :func:`step_mimo`, plus the previous token's ``x_prev [batch, D, R]`` (x_t's row stride) and
    ``B_prev [batch, 16, R]`` (B_t's) and this token's ``lam_t [batch, D]`` (delta_t's)."""
    return step_mimo(h, x_t, delta_t, A, B_t, C_t, form=form, y_t=y_t, _trap=(x_prev, B_prev, lam_t))


def step_mimo(h, x_t, delta_t, A, B_t, C_t, form="diagonal", y_t=None, _trap=None):
    """One MIMO decode token (``jscan_step_mimo``): h ``[batch, D, 16]`` fp32 in place; x_t
    ``[batch, D, R]``, delta_t ``[batch, D]``, B_t, C_t ``[batch, 16, R]`` (each row contiguous;
    rows may be strided views of prefill tensors, e.g. ``x[:, t]``).  Returns y_t ``[batch, D, R]``."""
    _require(form in A_FORMS, f"form must be one of {tuple(A_FORMS)}")
    _require(h.is_cuda and h.dtype == torch.float32 and h.dim() == 3 and h.shape[2] == D_STATE and h.is_contiguous(),
             "h must be a contiguous fp32 [batch, D, 16] CUDA tensor")
    batch, D, _ = h.shape
    _require(x_t.dim() == 3 and x_t.shape[:2] == (batch, D) and x_t.dtype in _DTYPES, "x_t must be [batch, D, R]")
    R = x_t.shape[2]
    _require(x_t.stride(2) == 1 and x_t.stride(1) == R, "x_t rows must be contiguous")
    _require(tuple(delta_t.shape) == (batch, D) and delta_t.stride(1) == 1 and delta_t.dtype == x_t.dtype,
             "delta_t must be [batch, D] with contiguous rows, x_t's dtype")
    for name, t in (("B_t", B_t), ("C_t", C_t)):
        _require(tuple(t.shape) == (batch, D_STATE, R) and t.dtype == x_t.dtype and t.stride(2) == 1
                 and t.stride(1) == R, f"{name} must be [batch, 16, R] with contiguous rows, x_t's dtype")
    a_shape = (D,) if form == "scalar" else (D, D_STATE)
    _require(A.dtype == torch.float32 and tuple(A.shape) == a_shape and A.is_contiguous(),
             f"A must be a contiguous fp32 tensor of shape {a_shape}")
    ld_x = x_t.stride(0) if batch > 1 else D * R
    ld_d = delta_t.stride(0) if batch > 1 else D
    ld_bc = B_t.stride(0) if batch > 1 else D_STATE * R
    _require(batch <= 1 or C_t.stride(0) == ld_bc, "B_t and C_t must share a row stride")
    if _trap is not None:
        x_prev, B_prev, lam_t = _trap
        for name, t, shape, ld in (("x_prev", x_prev, (batch, D, R), ld_x), ("B_prev", B_prev, (batch, D_STATE, R), ld_bc),
                                   ("lam_t", lam_t, (batch, D), ld_d)):
            _require(tuple(t.shape) == shape and t.dtype == x_t.dtype and t.device == h.device
                     and t.stride(-1) == 1 and (t.dim() == 2 or t.stride(1) == R) and (batch <= 1 or t.stride(0) == ld),
                     f"{name} must be {shape} with contiguous rows and the row stride of the matching input")
    y_t, ld_y = _step_output(y_t, (batch, D, R), x_t.dtype, h.device)
    lib = library()
    with torch.cuda.device(h.device):
        if _trap is None:
            st = lib.jscan_step_mimo(_ptr(h), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y_t), batch,
                                     D, D_STATE, R, ld_x, ld_d, ld_bc, ld_y, A_FORMS[form], _DTYPES[x_t.dtype],
                                     _stream(h.device))
        else:
            st = lib.jscan_step_mimo_trapezoid(_ptr(h), _ptr(_trap[0]), _ptr(_trap[1]), _ptr(x_t), _ptr(delta_t),
                                               _ptr(_trap[2]), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y_t), batch, D,
                                               D_STATE, R, ld_x, ld_d, ld_bc, ld_y, A_FORMS[form],
                                               _DTYPES[x_t.dtype], _stream(h.device))
    _check(st)
    return y_t
