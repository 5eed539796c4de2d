"""Seeded synthetic inputs for the selective-scan workloads.

This module only draws random inputs of the right shapes and distributions; it holds none
of the scan's arithmetic.  Both the GPU path (through the bench and tests) and the CPU
oracle are fed from it, so the two always see the same bytes.

Shapes follow the Jamba-1 Mamba layer: hidden 4096 with expansion factor 2 gives
d_inner D = 8192, and d_state N = 16 (notes page "Jamba: A Hybrid Transformer-Mamba
Language Model", section "Mamba layer"); 28 of the 32 layers are Mamba layers (lesson page
"Jamba - Hybrid SSM-Transformer", section "memory budget").  The prompt lengths (4K, 64K,
256K) span the pages' long-context range (notes page, throughput table; 256K context on
one 80 GB GPU).  prefill_64k_tp8 is the 64K prompt with d_inner split 8 ways, the share of
one GPU under channel (tensor) parallelism; prefill_16x4k is a batched prefill of sixteen 4K
prompts.

Distributions (the same for every workload):
    x, B, C ~ N(0, 1)                              per element
    delta   = softplus(z - 2),  z ~ N(0, 1)        evaluated in fp64, mean ~0.18
    A[d, n] = -(n + 1)                             tiny workload (exact)
    A[d, n] = -(n + 1) * U(0.5, 1.5)               other workloads, one draw per (d, n)
    a[d]    = -(d % 16 + 1)                         scaled-identity A, tiny workload (exact)
    a[d]    = -(k_d + 1) * U(0.5, 1.5), k_d ~ U{0..15}   scaled-identity A, other workloads:
                                                    the channels' decays span the diagonal A's range
    complex A (pairs 2k, 2k+1 = real, imaginary part of entry k):
            real -(k + 1) * U(0.5, 1.5), imaginary pi * U(-1, 1), one draw per (d, k)
    h0      ~ N(0, 0.1)  (0.1 = standard deviation) decode workload's resident state
    lam     = sigmoid(z),  z ~ N(0, 1)             evaluated in fp64: the exponential-trapezoidal
                                                    rule's per-(token, channel) weight in (0, 1)
    MIMO (rank R): x [.., D, R], B, C [.., N, R] ~ N(0, 1) per element, from their own streams;
                   delta, A, h0 as above
bf16 workloads round every drawn value to bf16 by round-to-nearest-even (torch ``.to``).

Seeding: every tensor is drawn block by block from
``numpy.random.default_rng([seed, workload_id, tensor_id, batch_row or layer, block])``
with blocks of 4096 tokens, so generation is reproducible, order-independent and can be
done for any token range on its own.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os

import numpy as np
import torch

BLOCK = 4096  # tokens per seeded block

# tensor ids inside the seed
T_X, T_Z, T_B, T_C, T_A, T_H0 = 0, 1, 2, 3, 4, 5
T_WX, T_GAIN, T_WDT, T_BDT = 6, 7, 8, 9     # producer-side weights
T_ASC = 10                                  # scaled-identity A
T_ACX = 11                                  # complex A
T_LAM = 12                                  # trapezoidal-rule weights
T_XR, T_BR, T_CR = 13, 14, 15               # MIMO inputs and projections


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id inside the seed
    batch: int
    L: int              # tokens handed to prefill (decode: 1 token per step)
    D: int
    N: int
    dtype: str          # "f32" or "bf16": dtype of x, delta, B, C and y
    a_scaled: bool      # A = -(n+1)*U(0.5,1.5) (True) or exactly -(n+1) (False)
    layers: int = 1     # decode: independent Mamba layers per token step
    extra_tokens: int = 0  # tokens generated after the prefill range (step continuation)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elems(self) -> int:
        """B * L * D (decode: batch * D * layers per token step)."""
        if self.layers > 1:
            return self.batch * self.D * self.layers
        return self.batch * self.L * self.D


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 0, 1, 256, 64, 16, "f32", False),
        Workload("prefill_4k", 1, 1, 4096, 8192, 16, "bf16", True),
        Workload("prefill_64k", 2, 1, 65536, 8192, 16, "bf16", True),
        Workload("decode_256x28", 3, 256, 1, 8192, 16, "bf16", True, layers=28),
        Workload("prefill_256k", 4, 1, 262144, 8192, 16, "bf16", True, extra_tokens=64),
        # one GPU's share of the 64K prefill when the 8192 channels are split over 8 GPUs
        # (channels are independent, so each GPU scans D = 1024 of them on its own)
        Workload("prefill_64k_tp8", 5, 1, 65536, 1024, 16, "bf16", True),
        # a batched prefill: sixteen 4K-token prompts at the same width
        Workload("prefill_16x4k", 6, 16, 4096, 8192, 16, "bf16", True),
    ]
}


def get(name_or_wl) -> Workload:
    return name_or_wl if isinstance(name_or_wl, Workload) else WORKLOADS[name_or_wl]


def _rng(seed, wid, tensor, row, block):
    return np.random.default_rng([seed, wid, tensor, row, block])


def _softplus64(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def _to_dtype(a: np.ndarray, wl: Workload) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if wl.dtype == "f32" else t.to(torch.bfloat16)


def _draw_rows(wl: Workload, seed: int, tensor: int, row: int, t0: int, t1: int, width: int) -> np.ndarray:
    """Tokens [t0, t1) of one batch row of a [tokens, width] tensor, as float32."""
    out = np.empty((t1 - t0, width), np.float32)
    for blk in range(t0 // BLOCK, (t1 - 1) // BLOCK + 1):
        b0 = blk * BLOCK
        rng = _rng(seed, wl.wid, tensor, row, blk)
        if tensor == T_Z:
            z = rng.standard_normal((BLOCK, width), dtype=np.float64)
            vals = _softplus64(z - 2.0).astype(np.float32)
        elif tensor == T_LAM:
            z = rng.standard_normal((BLOCK, width), dtype=np.float64)
            vals = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
        else:
            vals = rng.standard_normal((BLOCK, width), dtype=np.float32)
        lo, hi = max(t0, b0), min(t1, b0 + BLOCK)
        out[lo - t0:hi - t0] = vals[lo - b0:hi - b0]
    return out


def _draw_seq(wl: Workload, seed: int, tensor: int, width: int, t0: int, t1: int, threads: int) -> torch.Tensor:
    """[batch, t1-t0, width] tensor, drawn block-parallel and converted to the workload dtype."""
    out = torch.empty((wl.batch, t1 - t0, width), dtype=wl.torch_dtype)
    jobs = []
    for row in range(wl.batch):
        for blk in range(t0 // BLOCK, (t1 - 1) // BLOCK + 1):
            lo, hi = max(t0, blk * BLOCK), min(t1, (blk + 1) * BLOCK)
            jobs.append((row, lo, hi))

    def work(job):
        row, lo, hi = job
        out[row, lo - t0:hi - t0] = _to_dtype(_draw_rows(wl, seed, tensor, row, lo, hi, width), wl)

    if threads <= 1 or len(jobs) == 1:
        for j in jobs:
            work(j)
    else:
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, jobs))
    return out


def draw_A(wl: Workload, seed: int = 0, layer: int = 0) -> torch.Tensor:
    """[D, N] fp32 diagonal of A (always fp32, every entry < 0)."""
    n1 = np.arange(1, wl.N + 1, dtype=np.float64)[None, :]
    if not wl.a_scaled:
        a = -np.broadcast_to(n1, (wl.D, wl.N))
    else:
        u = _rng(seed, wl.wid, T_A, layer, 0).uniform(0.5, 1.5, size=(wl.D, wl.N))
        a = -n1 * u
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def draw_scalar_a(wl: Workload, seed: int = 0, layer: int = 0) -> torch.Tensor:
    """[D] fp32 scaled-identity A (A[d, n] = a[d] for every n; every entry < 0)."""
    wl = get(wl)
    if not wl.a_scaled:
        a = -(np.arange(wl.D) % wl.N + 1).astype(np.float64)
    else:
        rng = _rng(seed, wl.wid, T_ASC, layer, 0)
        k = rng.integers(0, wl.N, size=wl.D)
        a = -(k + 1) * rng.uniform(0.5, 1.5, size=wl.D)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def draw_complex_a(wl: Workload, seed: int = 0, layer: int = 0) -> torch.Tensor:
    """[D, N] fp32 complex diagonal of A as (real, imaginary) pairs: real parts < 0, imaginary
    parts (angle rates) in (-pi, pi)."""
    wl = get(wl)
    K = wl.N // 2
    rng = _rng(seed, wl.wid, T_ACX, layer, 0)
    a = np.empty((wl.D, wl.N), np.float64)
    a[:, 0::2] = -np.arange(1, K + 1)[None, :] * rng.uniform(0.5, 1.5, size=(wl.D, K))
    a[:, 1::2] = np.pi * rng.uniform(-1.0, 1.0, size=(wl.D, K))
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def prefill_inputs(name_or_wl, seed: int = 0, t0: int = 0, t1: int | None = None, threads: int | None = None):
    """Inputs of a prefill workload for tokens [t0, t1) (default: the prefill range [0, L)).

    Returns a dict of CPU tensors: x, delta ``[batch, T, D]``, B, C ``[batch, T, N]`` in the
    workload dtype, and A ``[D, N]`` fp32.  ``t1`` may run past L up to L + extra_tokens.
    """
    wl = get(name_or_wl)
    t1 = wl.L if t1 is None else t1
    if not 0 <= t0 < t1 <= wl.L + wl.extra_tokens:
        raise ValueError("token range outside the workload")
    threads = threads or min(16, os.cpu_count() or 1)
    return {
        "x": _draw_seq(wl, seed, T_X, wl.D, t0, t1, threads),
        "delta": _draw_seq(wl, seed, T_Z, wl.D, t0, t1, threads),
        "A": draw_A(wl, seed),
        "B": _draw_seq(wl, seed, T_B, wl.N, t0, t1, threads),
        "C": _draw_seq(wl, seed, T_C, wl.N, t0, t1, threads),
    }


def lam_inputs(name_or_wl, seed: int = 0, t0: int = 0, t1: int | None = None, threads: int | None = None):
    """The exponential-trapezoidal rule's weights lam ``[batch, T, D]`` (workload dtype) for
    tokens [t0, t1), drawn like the other inputs of :func:`prefill_inputs`."""
    wl = get(name_or_wl)
    t1 = wl.L if t1 is None else t1
    if not 0 <= t0 < t1 <= wl.L + wl.extra_tokens:
        raise ValueError("token range outside the workload")
    return _draw_seq(wl, seed, T_LAM, wl.D, t0, t1, threads or min(16, os.cpu_count() or 1))


def mimo_inputs(name_or_wl, R: int, seed: int = 0, t0: int = 0, t1: int | None = None, threads: int | None = None):
    """Inputs of a MIMO prefill of rank R for tokens [t0, t1): x ``[batch, T, D, R]``, B, C
    ``[batch, T, N, R]`` in the workload dtype, and the workload's delta ``[batch, T, D]`` and A."""
    wl = get(name_or_wl)
    t1 = wl.L if t1 is None else t1
    if not 0 <= t0 < t1 <= wl.L + wl.extra_tokens:
        raise ValueError("token range outside the workload")
    threads = threads or min(16, os.cpu_count() or 1)
    T = t1 - t0
    return {
        "x": _draw_seq(wl, seed, T_XR, wl.D * R, t0, t1, threads).view(wl.batch, T, wl.D, R),
        "delta": _draw_seq(wl, seed, T_Z, wl.D, t0, t1, threads),
        "A": draw_A(wl, seed),
        "B": _draw_seq(wl, seed, T_BR, wl.N * R, t0, t1, threads).view(wl.batch, T, wl.N, R),
        "C": _draw_seq(wl, seed, T_CR, wl.N * R, t0, t1, threads).view(wl.batch, T, wl.N, R),
    }


def decode_layer_inputs(name_or_wl, layer: int, seed: int = 0, token: int = 0):
    """One layer of the batched-decode workload at one token step.

    Returns CPU tensors: h0 ``[batch, D, N]`` fp32 (the resident state, N(0, 0.1)), x_t,
    delta_t ``[batch, D]`` and B_t, C_t ``[batch, N]`` in the workload dtype, A ``[D, N]``.
    Each layer draws from its own seed stream; ``token`` selects the token step.
    """
    wl = get(name_or_wl)
    if not 0 <= layer < wl.layers:
        raise ValueError("layer outside the workload")
    row = layer * 1_000_003 + token  # one stream per (layer, token step)

    def mat(tensor, width):
        rng = _rng(seed, wl.wid, tensor, row, 0)
        if tensor == T_Z:
            v = _softplus64(rng.standard_normal((wl.batch, width), dtype=np.float64) - 2.0).astype(np.float32)
        elif tensor == T_LAM:
            v = (1.0 / (1.0 + np.exp(-rng.standard_normal((wl.batch, width), dtype=np.float64)))).astype(np.float32)
        else:
            v = rng.standard_normal((wl.batch, width), dtype=np.float32)
        return _to_dtype(v, wl)

    h_rng = _rng(seed, wl.wid, T_H0, layer, 0)
    h0 = h_rng.normal(0.0, 0.1, size=(wl.batch, wl.D, wl.N)).astype(np.float32)
    return {
        "h0": torch.from_numpy(h0),
        "x": mat(T_X, wl.D),
        "delta": mat(T_Z, wl.D),
        "A": draw_A(wl, seed, layer),
        "B": mat(T_B, wl.N),
        "C": mat(T_C, wl.N),
        "lam": mat(T_LAM, wl.D),   # used by the exponential-trapezoidal rule only
    }


def decode_layer_mimo_inputs(name_or_wl, layer: int, R: int, seed: int = 0, token: int = 0):
    """One layer of the batched-decode workload at one token step, MIMO of rank R: the state h0,
    delta_t and A of :func:`decode_layer_inputs`, with x_t ``[batch, D, R]`` and B_t, C_t
    ``[batch, N, R]`` from their own streams."""
    wl = get(name_or_wl)
    base = decode_layer_inputs(wl, layer, seed, token)
    row = layer * 1_000_003 + token

    def mat(tensor, shape):
        v = _rng(seed, wl.wid, tensor, row, 0).standard_normal((wl.batch,) + shape, dtype=np.float32)
        return _to_dtype(v, wl)

    return {"h0": base["h0"], "delta": base["delta"], "A": base["A"], "x": mat(T_XR, (wl.D, R)),
            "B": mat(T_BR, (wl.N, R)), "C": mat(T_CR, (wl.N, R))}


def producer_weights(D: int, R: int = 256, N: int = 16, seed: int = 0, wid: int = 50):
    """Synthetic weights of the producer side (delta, B and C computed from x):
        w_x  [R + 2N, D] bf16, N(0, 1/D): unit-variance projections of unit-variance x
        g_d [R], g_b [N], g_c [N] fp32 gains, U(0.75, 1.25)
        w_dt [D, R] bf16, N(0, 1/R): unit-variance pre-activations of a unit-RMS d_low
        b_dt [D] fp32, -2 + 0.25 N(0, 1)
    so that delta = softplus(N(0, ~1) - 2) per channel, the distribution the scan workloads
    draw delta from directly.  R defaults to 256 (d_model 4096 / 16, the usual rank of delta)."""
    def rng(tensor):
        return _rng(seed, wid, tensor, D * 1000 + R, 0)

    w_x = rng(T_WX).standard_normal((R + 2 * N, D), dtype=np.float32) / np.float32(np.sqrt(D))
    gains = rng(T_GAIN).uniform(0.75, 1.25, size=R + 2 * N).astype(np.float32)
    w_dt = rng(T_WDT).standard_normal((D, R), dtype=np.float32) / np.float32(np.sqrt(R))
    b_dt = (-2.0 + 0.25 * rng(T_BDT).standard_normal(D)).astype(np.float32)
    t = torch.from_numpy
    return {
        "w_x": t(np.ascontiguousarray(w_x)).to(torch.bfloat16),
        "g_d": t(gains[:R].copy()), "g_b": t(gains[R:R + N].copy()), "g_c": t(gains[R + N:].copy()),
        "w_dt": t(np.ascontiguousarray(w_dt)).to(torch.bfloat16),
        "b_dt": t(b_dt),
    }


def small_prefill(batch: int, L: int, D: int, dtype: str = "f32", seed: int = 0, a_scaled: bool = True, N: int = 16):
    """An ad-hoc prefill case with the same distributions (for parity cases off the named sizes)."""
    wl = Workload(f"adhoc_{batch}x{L}x{D}", 100 + (batch * 131 + L * 7 + D) % 997, batch, L, D, N, dtype, a_scaled)
    return prefill_inputs(wl, seed=seed, threads=1 if batch * L * D < (1 << 20) else None)
