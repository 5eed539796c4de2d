"""ctypes binding of libjscan_micro (the microbenchmarks of include/jscan_micro.h) and the
rates derived from them.  Measurement only: the scan never uses this module."""
from __future__ import annotations

import ctypes
import os
import struct

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libjscan_micro.so")
_lib = None

VALU_KINDS = {0: "fma", 1: "exp", 2: "exp8+fma8", 3: "exp4+fma12", 4: "mul_dpp_bcast", 5: "permlane32_swap+max",
              6: "permlane16_swap+max", 7: "mul+exp pairs", 10: "fma_distinct_operands"}
SCAN_BODY_KINDS = {8: "sgpr_bc", 9: "dpp_bc"}   # 4 scan tokens per trip (see jscan_micro.h)


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with python -m mamba_selective_scan_03_amd.build")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, fpp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_float)
        lib.jscan_micro_valu.argtypes = [i32, i64, i32, i32, vp, vp, fpp]
        lib.jscan_micro_mfma_valu.argtypes = [i32, i64, i32, i32, vp, vp, fpp]
        lib.jscan_micro_mfma_rounding.argtypes = [i32, vp, vp, vp, vp, vp, vp]
        lib.jscan_micro_lds.argtypes = [i64, i32, i32, i32, vp, vp, fpp]
        lib.jscan_micro_hbm.argtypes = [i32, i32, vp, vp, i64, i32, i32, vp, vp, fpp]
        for f in (lib.jscan_micro_valu, lib.jscan_micro_mfma_valu, lib.jscan_micro_mfma_rounding, lib.jscan_micro_lds,
                  lib.jscan_micro_hbm):
            f.restype = i32
        _lib = lib
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed (return code {rc})")


def _sink(n):
    return torch.zeros(n + 16, dtype=torch.float32, device="cuda")


def _u64(lo: float, hi: float) -> int:
    lo_i = struct.unpack("<I", struct.pack("<f", lo))[0]
    hi_i = struct.unpack("<I", struct.pack("<f", hi))[0]
    return lo_i | (hi_i << 32)


def valu(kind: int, iters: int, blocks: int, threads: int, placement: bool = False):
    """Runs one vector-ALU loop; returns (ms, shader clocks, 100 MHz ticks) of the timed launch
    (the clocks are block 0's first wave's), and with ``placement`` also the largest number of
    waves that shared one SIMD (from the waves' HW_ID and XCC_ID registers)."""
    n = blocks * threads
    sink = _sink(n + 2 * n // 64)
    ms = ctypes.c_float()
    _check(library().jscan_micro_valu(kind, iters, blocks, threads, ctypes.c_void_p(sink.data_ptr()), _stream(),
                                      ctypes.byref(ms)), "jscan_micro_valu")
    c = sink[n:n + 4].cpu().tolist()
    res = (ms.value, _u64(c[0], c[1]), _u64(c[2], c[3]))
    if placement:
        ids = sink[n + 4:n + 4 + 2 * n // 64].cpu().view(torch.int32).view(-1, 2)
        hw, xcc = ids[:, 0].long(), ids[:, 1].long() & 0xF
        # SIMD_ID [5:4], CU_ID [11:8], SH_ID [12], SE_ID [15:13]
        key = (((xcc * 8 + ((hw >> 13) & 7)) * 2 + ((hw >> 12) & 1)) * 16 + ((hw >> 8) & 15)) * 4 + ((hw >> 4) & 3)
        res = res + (int(torch.bincount(key).max()),)
    return res


def mfma_valu(mode: int, iters: int, blocks: int, threads: int) -> float:
    sink = _sink(blocks * threads)
    ms = ctypes.c_float()
    _check(library().jscan_micro_mfma_valu(mode, iters, blocks, threads, ctypes.c_void_p(sink.data_ptr()), _stream(),
                                           ctypes.byref(ms)), "jscan_micro_mfma_valu")
    return ms.value


def mfma_rounding(variant: int, a: torch.Tensor, b: torch.Tensor, c: torch.Tensor):
    """(d_mfma, d_fma) for 64 values of a and b and 256 of c (fp32 CUDA tensors)."""
    d1 = torch.empty(256, dtype=torch.float32, device="cuda")
    d2 = torch.empty_like(d1)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _check(library().jscan_micro_mfma_rounding(variant, p(a), p(b), p(c), p(d1), p(d2), _stream()),
           "jscan_micro_mfma_rounding")
    return d1, d2


def lds(iters: int, blocks: int, threads: int, unique: int = 64) -> float:
    sink = _sink(blocks * threads)
    ms = ctypes.c_float()
    _check(library().jscan_micro_lds(iters, unique, blocks, threads, ctypes.c_void_p(sink.data_ptr()), _stream(),
                                     ctypes.byref(ms)), "jscan_micro_lds")
    return ms.value


def hbm(kind: int, nontemporal: bool, src: torch.Tensor, dst: torch.Tensor, nbytes: int, blocks: int,
        reps: int) -> float:
    sink = _sink(blocks * 256)
    ms = ctypes.c_float()
    _check(library().jscan_micro_hbm(kind, int(nontemporal), ctypes.c_void_p(src.data_ptr()),
                                     ctypes.c_void_p(dst.data_ptr()), nbytes, blocks, reps,
                                     ctypes.c_void_p(sink.data_ptr()), _stream(), ctypes.byref(ms)),
           "jscan_micro_hbm")
    return ms.value
