"""fp64 CPU oracle for the Mamba-1 (S6) selective scan -- test infrastructure only.

Only the test suite, the smoke check of the repository's entry module and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library never links, loads or calls it,
and it imports nothing from the GPU library.

The arithmetic lives in ``jscan_oracle.c`` (plain C, fp64, compiled with
``-O2 -fno-fast-math -ffp-contract=off``); this module only widens inputs exactly to
float64, allocates outputs and calls it through ctypes.  The recurrence it computes is the
S6 equation of the Jamba notes page ("Jamba: A Hybrid Transformer-Mamba Language Model",
section "Mamba layer"):

    h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,     y_t = C_t h_t

for every (batch, channel, state) with diagonal A (lesson page "Jamba - Hybrid
SSM-Transformer", section "Mamba-3", item 2).  Shapes: x, delta, y ``[batch, L, D]``;
A ``[D, N]``; B, C ``[batch, L, N]``; states ``[batch, D, N]``.

``prefill_scalar_a`` / ``step_scalar_a`` are the same recurrence with a scaled-identity A
(one value per channel, the Mamba-2 form); ``prefill_complex`` / ``step_complex`` run it with a
complex-valued state (the Mamba-3 change); ``prefill_trapezoid`` / ``step_trapezoid`` replace the
Euler rule by the exponential-trapezoidal one (the other Mamba-3 change), for any of the three
forms of A; ``prefill_mimo`` / ``step_mimo`` give each channel R inputs and R outputs (MIMO, the third
Mamba-3 change).  ``oracle.producer`` is the fp64 (numpy) oracle
of the producer side that computes delta, B and C from x.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jscan_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_jscan.so")
_lib = None

GCC_FLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]


def build() -> str:
    """Compile the C oracle in place (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_prefill_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int]
    lib.oracle_prefill_chunked_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, ctypes.c_int]
    lib.oracle_step_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64]
    lib.oracle_prefill_complex_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int]
    lib.oracle_step_complex_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64]
    ci = ctypes.c_int
    lib.oracle_prefill_trapezoid_f64.argtypes = [dp] * 11 + [i64, i64, i64, i64, ci, ci]
    lib.oracle_step_trapezoid_f64.argtypes = [dp] * 10 + [i64, i64, i64, ci]
    lib.oracle_prefill_mimo_f64.argtypes = [dp] * 8 + [i64, i64, i64, i64, i64, ci, ci]
    lib.oracle_step_mimo_f64.argtypes = [dp] * 7 + [i64, i64, i64, i64, ci]
    lib.oracle_prefill_mimo_trapezoid_f64.argtypes = [dp] * 11 + [i64, i64, i64, i64, i64, ci, ci]
    for f in (lib.oracle_prefill_f64, lib.oracle_prefill_chunked_f64, lib.oracle_step_f64,
              lib.oracle_prefill_complex_f64, lib.oracle_step_complex_f64, lib.oracle_prefill_trapezoid_f64,
              lib.oracle_step_trapezoid_f64, lib.oracle_prefill_mimo_f64, lib.oracle_step_mimo_f64,
              lib.oracle_prefill_mimo_trapezoid_f64):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    """Exact widening to a contiguous float64 numpy array (bf16 and fp32 are exact in fp64)."""
    if hasattr(a, "detach"):  # torch tensor
        import torch

        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check_shapes(x, delta, A, B, C, h0):
    if x.ndim != 3 or delta.shape != x.shape:
        raise ValueError("x and delta must both be [batch, L, D]")
    batch, L, D = x.shape
    if A.ndim != 2 or A.shape[0] != D:
        raise ValueError("A must be [D, N]")
    N = A.shape[1]
    if B.shape != (batch, L, N) or C.shape != (batch, L, N):
        raise ValueError("B and C must be [batch, L, N]")
    if h0 is not None and h0.shape != (batch, D, N):
        raise ValueError("h0 must be [batch, D, N]")
    return batch, L, D, N


def prefill(x, delta, A, B, C, h0=None, nthreads: int = 0):
    """Sequential fp64 scan.  Returns ``(y [batch,L,D], h_final [batch,D,N])`` as float64."""
    lib = _load()
    x, delta, A, B, C = (_f64(v) for v in (x, delta, A, B, C))
    h0 = None if h0 is None else _f64(h0)
    batch, L, D, N = _check_shapes(x, delta, A, B, C, h0)
    y = np.empty((batch, L, D), np.float64)
    h = np.empty((batch, D, N), np.float64)
    rc = lib.oracle_prefill_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y), _ptr(h),
                                batch, L, D, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_f64 failed ({rc})")
    return y, h


def prefill_chunked(x, delta, A, B, C, chunk: int, h0=None, nthreads: int = 0):
    """The same scan evaluated chunk by chunk through the associative combine."""
    lib = _load()
    x, delta, A, B, C = (_f64(v) for v in (x, delta, A, B, C))
    h0 = None if h0 is None else _f64(h0)
    batch, L, D, N = _check_shapes(x, delta, A, B, C, h0)
    y = np.empty((batch, L, D), np.float64)
    h = np.empty((batch, D, N), np.float64)
    rc = lib.oracle_prefill_chunked_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y),
                                        _ptr(h), batch, L, D, N, int(chunk), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_chunked_f64 failed ({rc})")
    return y, h


def step(h, x_t, delta_t, A, B_t, C_t):
    """One decode step.  Returns ``(y_t [batch,D], h_new [batch,D,N])``; the input h is not modified."""
    lib = _load()
    h = _f64(h).copy()
    x_t, delta_t, A, B_t, C_t = (_f64(v) for v in (x_t, delta_t, A, B_t, C_t))
    batch, D, N = h.shape
    if x_t.shape != (batch, D) or delta_t.shape != (batch, D) or A.shape != (D, N):
        raise ValueError("step: x_t, delta_t must be [batch, D] and A [D, N]")
    if B_t.shape != (batch, N) or C_t.shape != (batch, N):
        raise ValueError("step: B_t and C_t must be [batch, N]")
    y = np.empty((batch, D), np.float64)
    rc = lib.oracle_step_f64(_ptr(h), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y),
                             batch, D, N)
    if rc != 0:
        raise RuntimeError(f"oracle_step_f64 failed ({rc})")
    return y, h


# ---- scaled-identity A (the Mamba-2 form) ------------------------------------------------
# The lesson page ("Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 2) says Mamba-2
# reduced the state matrix to a scaled identity.  Nothing else about the layer is stated to
# change, so the scan is the same diagonal recurrence with A[d, n] = a[d] for every state n:
# these functions write out exactly that and run the general recurrence above.


def expand_scalar_a(a, N: int = 16) -> np.ndarray:
    """The scaled identity a[d] * I as the diagonal [D, N]: A[d, n] = a[d]."""
    a = _f64(a)
    if a.ndim != 1:
        raise ValueError("a must be [D]")
    return np.ascontiguousarray(np.repeat(a[:, None], N, axis=1))


def prefill_scalar_a(x, delta, a, B, C, h0=None, nthreads: int = 0):
    """:func:`prefill` with A[d, n] = a[d]."""
    return prefill(x, delta, expand_scalar_a(a, np.shape(B)[-1]), B, C, h0, nthreads)


def step_scalar_a(h, x_t, delta_t, a, B_t, C_t):
    """:func:`step` with A[d, n] = a[d]."""
    return step(h, x_t, delta_t, expand_scalar_a(a, np.shape(B_t)[-1]), B_t, C_t)


# ---- complex-valued state (the Mamba-3 change) ----------------------------------------------
# The lesson page ("Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 2) names a complex
# state matrix again, equivalent to a data-dependent rotation of the state.  The N real state
# components of a channel are read as N/2 complex states (h[2k] + i h[2k+1]); A, B and C pair
# up the same way, A[2k] and A[2k+1] being the real and imaginary parts of the diagonal entry.


def prefill_complex(x, delta, A, B, C, h0=None, nthreads: int = 0):
    """Sequential fp64 scan with the complex-valued state.  Returns ``(y, h_final)`` as float64,
    h_final in the same paired layout as h0."""
    lib = _load()
    x, delta, A, B, C = (_f64(v) for v in (x, delta, A, B, C))
    h0 = None if h0 is None else _f64(h0)
    batch, L, D, N = _check_shapes(x, delta, A, B, C, h0)
    if N % 2:
        raise ValueError("the complex state needs an even N")
    y = np.empty((batch, L, D), np.float64)
    h = np.empty((batch, D, N), np.float64)
    rc = lib.oracle_prefill_complex_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y),
                                        _ptr(h), batch, L, D, N, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_complex_f64 failed ({rc})")
    return y, h


def step_complex(h, x_t, delta_t, A, B_t, C_t):
    """One decode step with the complex-valued state.  Returns ``(y_t, h_new)``."""
    lib = _load()
    h = _f64(h).copy()
    x_t, delta_t, A, B_t, C_t = (_f64(v) for v in (x_t, delta_t, A, B_t, C_t))
    batch, D, N = h.shape
    if x_t.shape != (batch, D) or delta_t.shape != (batch, D) or A.shape != (D, N) or N % 2:
        raise ValueError("step_complex: x_t, delta_t must be [batch, D] and A [D, N] with N even")
    if B_t.shape != (batch, N) or C_t.shape != (batch, N):
        raise ValueError("step_complex: B_t and C_t must be [batch, N]")
    y = np.empty((batch, D), np.float64)
    rc = lib.oracle_step_complex_f64(_ptr(h), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y),
                                     batch, D, N)
    if rc != 0:
        raise RuntimeError(f"oracle_step_complex_f64 failed ({rc})")
    return y, h


# ---- exponential-trapezoidal rule (the Mamba-3 discretisation) ----------------------------
# The lesson page ("Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 1) replaces the
# Euler rule by a recurrence that mixes neighbouring tokens' state input inside the scan.  Read
# as a two-point rule for the input integral over one step (jscan_oracle.c,
# scan_chain_trapezoid):
#     h_t = Abar_t h_{t-1} + (1 - lam_t) Delta_t Abar_t B_{t-1} x_{t-1} + lam_t Delta_t B_t x_t
# lam is [batch, L, D] like delta; lam = 1 is the Euler rule, lam = 1/2 the trapezoid rule.
# The token before the first is (x_prev [batch, D], B_prev [batch, N]) when given, else none.
# ``form`` picks A: "diagonal" ([D, N]), "scalar" (a [D], A[d, n] = a[d]) or "complex"
# ([D, N] as (real, imaginary) pairs, the complex-valued state).

_FORMS = ("diagonal", "scalar", "complex")


def _form_A(A, form: str, N: int):
    if form not in _FORMS:
        raise ValueError(f"form must be one of {_FORMS}")
    return expand_scalar_a(A, N) if form == "scalar" else _f64(A)


def prefill_trapezoid(x, delta, lam, A, B, C, h0=None, x_prev=None, B_prev=None, form: str = "diagonal",
                      nthreads: int = 0):
    """Sequential fp64 scan with the exponential-trapezoidal rule.  Returns ``(y, h_final)``."""
    lib = _load()
    x, delta, lam, B, C = (_f64(v) for v in (x, delta, lam, B, C))
    A = _form_A(A, form, B.shape[-1])
    h0 = None if h0 is None else _f64(h0)
    batch, L, D, N = _check_shapes(x, delta, A, B, C, h0)
    if lam.shape != x.shape:
        raise ValueError("lam must be [batch, L, D]")
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev go together")
    if x_prev is not None:
        x_prev, B_prev = _f64(x_prev), _f64(B_prev)
        if x_prev.shape != (batch, D) or B_prev.shape != (batch, N):
            raise ValueError("x_prev must be [batch, D] and B_prev [batch, N]")
    cplx = form == "complex"
    if cplx and N % 2:
        raise ValueError("the complex state needs an even N")
    y = np.empty((batch, L, D), np.float64)
    h = np.empty((batch, D, N), np.float64)
    rc = lib.oracle_prefill_trapezoid_f64(_ptr(x), _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(h0),
                                          _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(h), batch, L, D, N, int(cplx),
                                          int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_trapezoid_f64 failed ({rc})")
    return y, h


def step_trapezoid(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t, form: str = "diagonal"):
    """One decode step with the exponential-trapezoidal rule; (x_prev, B_prev) is the previous
    token.  Returns ``(y_t, h_new)``; the input h is not modified."""
    lib = _load()
    h = _f64(h).copy()
    x_prev, B_prev, x_t, delta_t, lam_t, B_t, C_t = (_f64(v) for v in (x_prev, B_prev, x_t, delta_t, lam_t, B_t,
                                                                       C_t))
    batch, D, N = h.shape
    A = _form_A(A, form, N)
    for v in (x_prev, x_t, delta_t, lam_t):
        if v.shape != (batch, D):
            raise ValueError("step_trapezoid: x_prev, x_t, delta_t, lam_t must be [batch, D]")
    if B_prev.shape != (batch, N) or B_t.shape != (batch, N) or C_t.shape != (batch, N) or A.shape != (D, N):
        raise ValueError("step_trapezoid: B_prev, B_t, C_t must be [batch, N] and A [D, N]")
    cplx = form == "complex"
    if cplx and N % 2:
        raise ValueError("the complex state needs an even N")
    y = np.empty((batch, D), np.float64)
    rc = lib.oracle_step_trapezoid_f64(_ptr(h), _ptr(x_prev), _ptr(B_prev), _ptr(x_t), _ptr(delta_t), _ptr(lam_t),
                                       _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y), batch, D, N, int(cplx))
    if rc != 0:
        raise RuntimeError(f"oracle_step_trapezoid_f64 failed ({rc})")
    return y, h


# ---- multi-input, multi-output (MIMO, the third Mamba-3 change) ----------------------------
# The lesson page ("Jamba - Hybrid SSM-Transformer", section "Mamba-3", item 3) replaces the
# per-channel scalar projections by matrix-valued ones.  Each channel takes R inputs and gives
# R outputs; B_t and C_t are N x R (jscan_oracle.c, scan_chain_mimo):
#     h_t[d, n] = Abar_t[d, n] h_{t-1}[d, n] + Delta_t[d] sum_r B_t[n, r] x_t[d, r]
#     y_t[d, r] = sum_n C_t[n, r] h_t[d, n]
# Shapes: x, y [batch, L, D, R]; delta [batch, L, D]; B, C [batch, L, N, R].


def prefill_mimo(x, delta, A, B, C, h0=None, form: str = "diagonal", nthreads: int = 0):
    """Sequential fp64 MIMO scan.  Returns ``(y [batch, L, D, R], h_final [batch, D, N])``."""
    lib = _load()
    x, delta, B, C = (_f64(v) for v in (x, delta, B, C))
    if x.ndim != 4 or B.ndim != 4:
        raise ValueError("x must be [batch, L, D, R] and B, C [batch, L, N, R]")
    batch, L, D, R = x.shape
    N = B.shape[2]
    A = _form_A(A, form, N)
    h0 = None if h0 is None else _f64(h0)
    if delta.shape != (batch, L, D) or B.shape != (batch, L, N, R) or C.shape != B.shape or A.shape != (D, N):
        raise ValueError("prefill_mimo: inconsistent shapes")
    if h0 is not None and h0.shape != (batch, D, N):
        raise ValueError("h0 must be [batch, D, N]")
    cplx = form == "complex"
    y = np.empty((batch, L, D, R), np.float64)
    h = np.empty((batch, D, N), np.float64)
    rc = lib.oracle_prefill_mimo_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(h0), _ptr(y), _ptr(h),
                                     batch, L, D, N, R, int(cplx), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_mimo_f64 failed ({rc})")
    return y, h


def step_mimo(h, x_t, delta_t, A, B_t, C_t, form: str = "diagonal"):
    """One MIMO decode step.  Returns ``(y_t [batch, D, R], h_new)``; the input h is not modified."""
    lib = _load()
    h = _f64(h).copy()
    x_t, delta_t, B_t, C_t = (_f64(v) for v in (x_t, delta_t, B_t, C_t))
    batch, D, N = h.shape
    A = _form_A(A, form, N)
    if x_t.ndim != 3 or x_t.shape[:2] != (batch, D):
        raise ValueError("step_mimo: x_t must be [batch, D, R]")
    R = x_t.shape[2]
    if delta_t.shape != (batch, D) or B_t.shape != (batch, N, R) or C_t.shape != (batch, N, R) or A.shape != (D, N):
        raise ValueError("step_mimo: inconsistent shapes")
    y = np.empty((batch, D, R), np.float64)
    rc = lib.oracle_step_mimo_f64(_ptr(h), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(y),
                                  batch, D, N, R, int(form == "complex"))
    if rc != 0:
        raise RuntimeError(f"oracle_step_mimo_f64 failed ({rc})")
    return y, h


# ---- MIMO with the exponential-trapezoidal rule ---------------------------------------------
# Both Mamba-3 changes together (jscan_oracle.c, scan_chain_mimo with the trapezoidal flag): the
# trapezoidal rule's input term with the rank-R input u_t[n] = sum_r B_t[n, r] x_t[d, r] in place
# of B_t x_t.  The previous token is (x_prev [batch, D, R], B_prev [batch, N, R]) or none.


def prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0=None, x_prev=None, B_prev=None, form: str = "diagonal",
                           nthreads: int = 0):
    """Sequential fp64 MIMO scan with the exponential-trapezoidal rule.  Returns ``(y, h_final)``."""
    lib = _load()
    x, delta, lam, B, C = (_f64(v) for v in (x, delta, lam, B, C))
    if x.ndim != 4 or B.ndim != 4:
        raise ValueError("x must be [batch, L, D, R] and B, C [batch, L, N, R]")
    batch, L, D, R = x.shape
    N = B.shape[2]
    A = _form_A(A, form, N)
    h0 = None if h0 is None else _f64(h0)
    if (delta.shape != (batch, L, D) or lam.shape != (batch, L, D) or B.shape != (batch, L, N, R)
            or C.shape != B.shape or A.shape != (D, N)):
        raise ValueError("prefill_mimo_trapezoid: inconsistent shapes")
    if (x_prev is None) != (B_prev is None):
        raise ValueError("x_prev and B_prev go together")
    if x_prev is not None:
        x_prev, B_prev = _f64(x_prev), _f64(B_prev)
        if x_prev.shape != (batch, D, R) or B_prev.shape != (batch, N, R):
            raise ValueError("x_prev must be [batch, D, R] and B_prev [batch, N, R]")
    y = np.empty((batch, L, D, R), np.float64)
    h = np.empty((batch, D, N), np.float64)
    rc = lib.oracle_prefill_mimo_trapezoid_f64(_ptr(x), _ptr(delta), _ptr(lam), _ptr(A), _ptr(B), _ptr(C), _ptr(h0),
                                               _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(h), batch, L, D, N, R,
                                               int(form == "complex"), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill_mimo_trapezoid_f64 failed ({rc})")
    return y, h


def step_mimo_trapezoid(h, x_prev, B_prev, x_t, delta_t, lam_t, A, B_t, C_t, form: str = "diagonal"):
    """One MIMO decode step with the exponential-trapezoidal rule: the one-token prefill from h with
    (x_prev, B_prev) as the previous token.  Returns ``(y_t [batch, D, R], h_new)``."""
    y, hn = prefill_mimo_trapezoid(np.asarray(_f64(x_t))[:, None], _f64(delta_t)[:, None], _f64(lam_t)[:, None], A,
                                   _f64(B_t)[:, None], _f64(C_t)[:, None], h0=h, x_prev=x_prev, B_prev=B_prev,
                                   form=form, nthreads=1)
    return y[:, 0], hn
