"""fp64 oracle of the scan's producer side: delta, B and C from x -- test infrastructure only.

Only the test suite and the bench's CPU baseline may use this module; the GPU library never
loads it.  The notes page ("Jamba: A Hybrid Transformer-Mamba Language Model", section
"Mamba layer") makes the scan's parameters functions of the input, B_t, C_t, delta_t =
f(x_t), and applies RMSNorm inside the Mamba layer.  f is read as the selective projection
of Mamba-1, step by step:

    1. [d_low | B | C] = W_x x_t                 W_x: [R + 2N, D] (rows are outputs)
    2. d_low, B and C are each RMS-normalised over their own width, v / sqrt(mean(v^2) + eps),
       and multiplied by their gain vectors g_d [R], g_B [N], g_C [N]
    3. delta_t = softplus(W_dt d_low + b_dt)     W_dt: [D, R], b_dt: [D]

Every stored tensor is bf16, so the oracle rounds each of d_low, B, C and delta exactly once,
from its fp64 value to the nearest bf16 (ties to even): the points where the GPU path rounds
its fp32 accumulators.  Everything else is float64.
"""
from __future__ import annotations

import numpy as np


def round_bf16(a) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of each float64 element, as float64.
    Normal range only (|a| >= 2^-126 or 0), which covers every value here."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                      # a = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)   # np.rint rounds half to even


def rms_norm(v, g, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * g over the last axis."""
    v = np.asarray(v, np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def softplus(z) -> np.ndarray:
    """log(1 + e^z), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(z, np.float64))


def ssm_inputs_low(x, w_x, g_d, g_b, g_c, eps: float, R: int, N: int = 16):
    """Steps 1 and 2 for M tokens: x [M, D] -> (d_low [M, R], B [M, N], C [M, N]), each rounded
    once to bf16 (returned as float64 arrays of bf16 values)."""
    x = np.asarray(x, np.float64)
    w_x = np.asarray(w_x, np.float64)
    if w_x.shape != (R + 2 * N, x.shape[1]):
        raise ValueError("w_x must be [R + 2N, D]")
    proj = x @ w_x.T                                             # step 1
    d_low = round_bf16(rms_norm(proj[:, :R], g_d, eps))          # step 2
    B = round_bf16(rms_norm(proj[:, R:R + N], g_b, eps))
    C = round_bf16(rms_norm(proj[:, R + N:], g_c, eps))
    return d_low, B, C


def ssm_inputs(x, w_x, g_d, g_b, g_c, w_dt, b_dt, eps: float, R: int, N: int = 16):
    """Producer side for M tokens: x [M, D] -> (d_low [M, R], B [M, N], C [M, N], delta [M, D]),
    each rounded once to bf16 (returned as float64 arrays of bf16 values)."""
    w_dt = np.asarray(w_dt, np.float64)
    if w_dt.shape != (np.shape(x)[1], R):
        raise ValueError("w_dt must be [D, R]")
    d_low, B, C = ssm_inputs_low(x, w_x, g_d, g_b, g_c, eps, R, N)
    delta = delta_from_low(d_low, w_dt, b_dt)                    # step 3
    return d_low, B, C, delta


def delta_from_low(d_low, w_dt, b_dt) -> np.ndarray:
    """Step 3 alone, from a given d_low [M, R]: delta [M, D] rounded once to bf16."""
    return round_bf16(softplus(np.asarray(d_low, np.float64) @ np.asarray(w_dt, np.float64).T
                               + np.asarray(b_dt, np.float64)))
