"""The C ABI loads, exports every symbol declared in include/jscan.h and rejects bad
arguments before touching the GPU (pointers below are never dereferenced: every call
fails validation first).  CPU only."""
import ctypes
import os
import re

import pytest
import torch

import mamba_selective_scan_03_amd as jscan
from mamba_selective_scan_03_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, ENULL, ESHAPE, EDTYPE, EALIGN, EALIAS, EHIP, EWORKSPACE, EFORM = range(9)
F32, BF16 = 0, 1
P = 0x10000000  # a 16-byte aligned address that is never dereferenced


def header_symbols():
    text = open(os.path.join(ROOT, "include", "jscan.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(jscan_\w+)\s*\(", text, re.M)))


def test_header_symbols_are_exported():
    lib = jscan.library()
    names = header_symbols()
    assert {"jscan_prefill", "jscan_prefill_resume", "jscan_step", "jscan_status_string",
            "jscan_last_hip_error", "jscan_version", "jscan_prefill_chunked",
            "jscan_prefill_chunked_workspace", "jscan_ssm_inputs", "jscan_prefill_fused", "jscan_prefill_scalar_a",
            "jscan_step_scalar_a", "jscan_prefill_complex", "jscan_step_complex", "jscan_prefill_trapezoid",
            "jscan_step_trapezoid", "jscan_prefill_mimo", "jscan_step_mimo", "jscan_prefill_mimo_trapezoid",
            "jscan_step_mimo_trapezoid", "jscan_prefill_chunked_noalloc"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_micro_header_symbols_are_exported():
    """include/jscan_micro.h (the microbenchmarks) against libjscan_micro.so, and their argument
    checks, which return -1 before any launch."""
    from mamba_selective_scan_03_amd import micro

    text = open(os.path.join(ROOT, "include", "jscan_micro.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(jscan_micro_\w+)\s*\(", text, re.M)))
    assert names == ["jscan_micro_hbm", "jscan_micro_lds", "jscan_micro_mfma_rounding", "jscan_micro_mfma_valu",
                     "jscan_micro_valu"]
    lib = micro.library()
    for n in names:
        assert hasattr(lib, n), n
    ms = ctypes.c_float()
    assert lib.jscan_micro_valu(99, 10, 1, 64, P, None, ctypes.byref(ms)) == -1
    assert lib.jscan_micro_valu(0, 10, 1, 96, P, None, ctypes.byref(ms)) == -1
    assert lib.jscan_micro_mfma_valu(0, 10, 1, 1024, P, None, ctypes.byref(ms)) == -1
    assert lib.jscan_micro_mfma_rounding(2, P, P, P, P, P, None) == -1
    assert lib.jscan_micro_lds(10, 8, 1, 64, P, None, ctypes.byref(ms)) == -1
    assert lib.jscan_micro_hbm(0, 0, P, P, 1000, 1, 1, P, None, ctypes.byref(ms)) == -1
    assert lib.jscan_micro_hbm(1, 0, P, P + 4, 16384, 1, 1, P, None, ctypes.byref(ms)) == -1


def noalloc(**kw):
    a = dict(x=P, d=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, h0=None, y=P + 0x500000,
             h=P + 0x600000, batch=1, L=4096, D=64, N=16, chunk=256, dtype=BF16)
    a.update(kw)
    return jscan.library().jscan_prefill_chunked_noalloc(a["x"], a["d"], a["A"], a["B"], a["C"], a["h0"], a["y"],
                                                         a["h"], a["batch"], a["L"], a["D"], a["N"], a["chunk"],
                                                         a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), EDTYPE), (dict(N=8), ESHAPE), (dict(D=20), ESHAPE), (dict(chunk=-1), ESHAPE),
    (dict(x=None), ENULL), (dict(y=P + 0x100000), EALIAS), (dict(h=P + 0x200000), EALIAS),
    # 64 segments x 8192 channels x 68 bytes exceed the 24 MiB scratch: refused before any launch
    (dict(L=16384, D=8192, chunk=256, x=P, d=P + 0x10000000, A=P + 0x20000000, B=P + 0x20100000,
          C=P + 0x20200000, y=P + 0x20300000, h=P + 0x30300000), EWORKSPACE),
    (dict(batch=0), OK),
])
def test_chunked_noalloc_validation(kw, code):
    assert noalloc(**kw) == code


def test_status_strings_and_version():
    lib = jscan.library()
    for s in range(9):
        assert lib.jscan_status_string(s) and lib.jscan_status_string(s) != b"unknown status"
    assert lib.jscan_status_string(99) == b"unknown status"
    assert lib.jscan_version() == 109
    assert lib.jscan_last_hip_error() == 0


def prefill(x=P, d=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, y=P + 0x500000,
            h=P + 0x600000, batch=1, L=64, D=64, N=16, dtype=BF16):
    return jscan.library().jscan_prefill(x, d, A, B, C, y, h, batch, L, D, N, dtype, None)


def resume(h0, h=P + 0x600000, **kw):
    lib = jscan.library()
    return lib.jscan_prefill_resume(P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, h0,
                                    P + 0x500000, h, kw.get("batch", 1), kw.get("L", 64), kw.get("D", 64), 16,
                                    BF16, None)


def step(h=P, x=P + 0x100000, d=P + 0x200000, A=P + 0x300000, B=P + 0x400000, C=P + 0x500000,
         y=P + 0x600000, batch=2, D=64, N=16, ld_xd=64, ld_bc=16, ld_y=64, dtype=BF16):
    return jscan.library().jscan_step(h, x, d, A, B, C, y, batch, D, N, ld_xd, ld_bc, ld_y, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), EDTYPE), (dict(N=8), ESHAPE), (dict(D=60), ESHAPE), (dict(L=-1), ESHAPE),
    (dict(batch=-2), ESHAPE), (dict(x=None), ENULL), (dict(h=None), ENULL), (dict(A=None), ENULL),
    (dict(C=None), ENULL), (dict(y=P + 0x500008), EALIGN), (dict(B=P + 0x300002), EALIGN),
    (dict(y=P + 0x100000), EALIAS), (dict(h=P + 0x200000), EALIAS), (dict(h=P + 0x500000 + 64 * 64 * 2 - 16), EALIAS),
])
def test_prefill_validation(kw, code):
    assert prefill(**kw) == code


def test_prefill_zero_sized_is_a_no_op():
    assert prefill(batch=0, x=None, y=None, h=None, A=None) == OK
    assert prefill(D=0, x=None, y=None, h=None, A=None) == OK


def test_prefill_empty_sequence_needs_no_token_arrays():
    # L == 0 writes only h_final; the validation accepts NULL token arrays (the launch itself
    # would need a GPU, so only a failing variant is called here)
    assert prefill(L=0, x=None, d=None, B=None, C=None, y=None, A=None) == ENULL


def test_resume_aliasing_rules():
    assert resume(None) == ENULL
    assert resume(P + 0x600000 + 16) == EALIAS          # partial overlap with h_final
    assert resume(P + 0x500000) == EALIAS               # overlaps y


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), EDTYPE), (dict(N=17), ESHAPE), (dict(D=12), ESHAPE), (dict(ld_xd=32), ESHAPE),
    (dict(ld_bc=8), ESHAPE), (dict(ld_xd=68), ESHAPE), (dict(h=None), ENULL), (dict(B=None), ENULL),
    (dict(x=P + 0x100004), EALIGN), (dict(y=P + 0x100000), EALIAS), (dict(y=P + 64 * 16 * 4), EALIAS),
    (dict(h=P + 0x300000 - 64), EALIAS), (dict(ld_y=32), ESHAPE), (dict(ld_y=68), ESHAPE),
    (dict(y=P + 0x100000 - 8192, ld_y=4096), EALIAS),   # y's second row, 4096 elements on, is x
])
def test_step_validation(kw, code):
    assert step(**kw) == code


def prefill_sa(x=P, d=P + 0x100000, a=P + 0x200000, B=P + 0x300000, C=P + 0x400000, h0=None, y=P + 0x500000,
               h=P + 0x600000, batch=1, L=64, D=64, N=16, dtype=BF16):
    return jscan.library().jscan_prefill_scalar_a(x, d, a, B, C, h0, y, h, batch, L, D, N, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), EDTYPE), (dict(N=8), ESHAPE), (dict(D=60), ESHAPE), (dict(a=None), ENULL), (dict(x=None), ENULL),
    (dict(a=P + 0x200004), EALIGN), (dict(y=P + 0x200000), EALIAS),
    (dict(h=P + 0x200000 + 64 * 4 - 16), EALIAS),      # a is [D] fp32: its last 16 bytes
    (dict(h0=P + 0x500000), EALIAS), (dict(h0=P + 0x600000 + 16), EALIAS),
])
def test_prefill_scalar_a_validation(kw, code):
    assert prefill_sa(**kw) == code


def test_prefill_scalar_a_zero_sized_is_a_no_op():
    assert prefill_sa(batch=0, x=None, y=None, h=None, a=None) == OK


def step_sa(h=P, x=P + 0x100000, d=P + 0x200000, a=P + 0x300000, B=P + 0x400000, C=P + 0x500000,
            y=P + 0x600000, batch=2, D=64, N=16, ld_xd=64, ld_bc=16, ld_y=64, dtype=BF16):
    return jscan.library().jscan_step_scalar_a(h, x, d, a, B, C, y, batch, D, N, ld_xd, ld_bc, ld_y, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), EDTYPE), (dict(N=17), ESHAPE), (dict(D=12), ESHAPE), (dict(ld_xd=32), ESHAPE),
    (dict(a=None), ENULL), (dict(a=P + 0x300008), EALIGN), (dict(y=P + 0x300000), EALIAS),
    (dict(y=P + 0x300000 + 64 * 4 - 16 - 2 * 64 * 2), EALIAS),   # the second y row reaches into a
])
def test_step_scalar_a_validation(kw, code):
    assert step_sa(**kw) == code


WS = P + 0x700000  # fake workspace address


def chunked(x=P, d=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, h0=None, y=P + 0x500000,
            h=P + 0x600000, batch=1, L=4096, D=64, N=16, chunk=256, ws=WS, ws_bytes=1 << 20, dtype=BF16):
    return jscan.library().jscan_prefill_chunked(x, d, A, B, C, h0, y, h, batch, L, D, N, chunk, ws, ws_bytes, dtype,
                                                 None)


def test_chunked_workspace_sizes():
    ws = jscan.library().jscan_prefill_chunked_workspace
    # automatic chunking of one sequence of 1024 channels: 256 segments of 256 tokens give
    # 262144 segment-channel lanes, four waves per SIMD
    assert ws(1, 65536, 1024, 16, 0) == 256 * 1024 * 17 * 4
    assert ws(1, 4096, 64, 16, 256) == 16 * 64 * 17 * 4          # explicit 256-token segments
    assert ws(2, 4000, 64, 16, 1000) == 2 * 4 * 64 * 17 * 4       # 4 segments per sequence
    assert ws(1, 65536, 8192, 16, 0) == 0                         # enough channels: one segment
    assert ws(1, 65536, 8200, 16, 0) == 31 * 8200 * 17 * 4        # D not a multiple of 32: segments
    assert ws(1, 100, 64, 16, 0) == 0                             # too short to split
    assert ws(1, 4096, 64, 16, 4096) == 0 and ws(1, 4096, 64, 16, 10 ** 6) == 0
    assert ws(1, 0, 64, 16, 0) == 0
    assert ws(1, 4096, 64, 8, 0) == -1 and ws(1, 4096, 60, 16, 0) == -1 and ws(1, 4096, 64, 16, -1) == -1
    assert ws(1 << 20, 1 << 20, 64, 16, 1) == -1                  # too many segment rows


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), EDTYPE), (dict(N=4), ESHAPE), (dict(D=20), ESHAPE), (dict(chunk=-1), ESHAPE),
    (dict(ws=None), ENULL), (dict(ws_bytes=16 * 64 * 17 * 4 - 4), EWORKSPACE), (dict(ws=WS + 8), EALIGN),
    (dict(ws=P + 0x500000 + 1024), EALIAS), (dict(ws=P + 0x600000 - 64), EALIAS), (dict(h0=WS + 4096), EALIAS),
    (dict(x=None), ENULL), (dict(y=P + 0x100000), EALIAS), (dict(h0=P + 0x600000 + 16), EALIAS),
])
def test_chunked_validation(kw, code):
    assert chunked(**kw) == code


def ssm_inputs(x=P, wx=P + 0x100000, gd=P + 0x200000, gb=P + 0x210000, gc=P + 0x220000, wdt=P + 0x300000,
               bdt=P + 0x400000, dlow=P + 0x500000, delta=P + 0x600000, B=P + 0x700000, C=P + 0x710000,
               M=256, D=256, R=64, N=16, eps=1e-6, dtype=BF16):
    return jscan.library().jscan_ssm_inputs(x, wx, gd, gb, gc, wdt, bdt, dlow, delta, B, C, M, D, R, N, eps, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=F32), EDTYPE), (dict(dtype=9), EDTYPE), (dict(R=96), ESHAPE), (dict(N=8), ESHAPE),
    (dict(D=192), ESHAPE), (dict(M=-1), ESHAPE), (dict(M=(1 << 31) + 1), ESHAPE), (dict(eps=-1.0), ESHAPE),
    (dict(eps=float("nan")), ESHAPE),
    (dict(x=None), ENULL), (dict(C=None), ENULL), (dict(gb=P + 0x210004), EALIGN),
    (dict(delta=P + 0x100000), EALIAS), (dict(B=P + 0x500000 + 256 * 64 * 2 - 16), EALIAS),
    (dict(C=P + 0x700000 + 16), EALIAS),
])
def test_ssm_inputs_validation(kw, code):
    assert ssm_inputs(**kw) == code


def fused(x=P, dlow=P + 0x100000, wdt=P + 0x200000, bdt=P + 0x300000, A=P + 0x310000, B=P + 0x320000,
          C=P + 0x330000, h0=None, y=P + 0x400000, h=P + 0x500000, batch=1, L=64, D=64, N=16, R=256, dtype=BF16):
    return jscan.library().jscan_prefill_fused(x, dlow, wdt, bdt, A, B, C, h0, y, h, batch, L, D, N, R, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=F32), EDTYPE), (dict(R=128), ESHAPE), (dict(D=72), ESHAPE), (dict(D=40), ESHAPE),
    (dict(dlow=None), ENULL), (dict(wdt=None), ENULL), (dict(bdt=P + 0x300004), EALIGN),
    (dict(y=P + 0x100000), EALIAS), (dict(h=P + 0x200000 + 64), EALIAS), (dict(x=None), ENULL),
])
def test_prefill_fused_validation(kw, code):
    assert fused(**kw) == code


def test_ssm_inputs_without_delta_needs_no_second_weights():
    # delta == NULL: w_dt and b_dt may be NULL; a misaligned gain is still reported first
    assert ssm_inputs(delta=None, wdt=None, bdt=None, gb=P + 0x210004) == EALIGN
    assert ssm_inputs(wdt=None) == ENULL


def test_ssm_inputs_zero_tokens_is_a_no_op():
    assert ssm_inputs(M=0, x=None, delta=None) == OK


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        jscan.prefill(x, x, torch.zeros(32, 16), torch.zeros(1, 8, 16, dtype=torch.bfloat16),
                      torch.zeros(1, 8, 16, dtype=torch.bfloat16))


def test_binding_error_type():
    e = _binding.JScanError(2, "bad shape")
    assert e.status == 2 and "bad shape" in str(e)


def test_library_does_not_reference_the_oracle():
    lib_src = open(os.path.join(ROOT, "mamba_selective_scan_03_amd", "_binding.py")).read()
    assert "oracle" not in lib_src
    for f in os.listdir(os.path.join(ROOT, "mamba_selective_scan_03_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "mamba_selective_scan_03_amd", "csrc", f)).read().lower()
    syms = open(jscan.library_path(), "rb").read()
    assert b"oracle_prefill" not in syms


def test_last_hip_error_is_per_thread():
    """jscan_last_hip_error is thread-local: a thread that made no failing launch reads 0."""
    import threading

    lib = jscan.library()
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.jscan_last_hip_error()))
    t.start()
    t.join()
    assert seen == [0]


def test_complex_entry_points_validate_like_the_general_ones():
    lib = jscan.library()
    # A is [D][16] here (not [D]): a pointer 256 bytes past A's start still overlaps it
    assert lib.jscan_prefill_complex(P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, None,
                                     P + 0x500000, P + 0x200000 + 256, 1, 64, 64, 16, BF16, None) == EALIAS
    assert lib.jscan_prefill_complex(P, P + 0x100000, None, P + 0x300000, P + 0x400000, None, P + 0x500000,
                                     P + 0x600000, 1, 64, 64, 16, BF16, None) == ENULL
    assert lib.jscan_prefill_complex(P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, None,
                                     P + 0x500000, P + 0x600000, 1, 64, 60, 16, BF16, None) == ESHAPE
    assert lib.jscan_step_complex(P, P + 0x100000, P + 0x200000, P + 0x300000, P + 0x400000, P + 0x500000,
                                  P + 0x600000, 2, 64, 16, 64, 16, 64, 9, None) == EDTYPE
    assert lib.jscan_step_complex(P, P + 0x100000, P + 0x200000, None, P + 0x400000, P + 0x500000,
                                  P + 0x600000, 2, 64, 16, 64, 16, 64, BF16, None) == ENULL


def trap_prefill(x=P, d=P + 0x100000, lam=P + 0x700000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, h0=None,
                 xp=None, bp=None, y=P + 0x500000, h=P + 0x600000, batch=1, L=64, D=64, N=16, form=0, dtype=BF16):
    return jscan.library().jscan_prefill_trapezoid(x, d, lam, A, B, C, h0, xp, bp, y, h, batch, L, D, N, form, dtype,
                                                   None)


@pytest.mark.parametrize("kw,code", [
    (dict(form=3), EFORM), (dict(form=-1), EFORM), (dict(dtype=5), EDTYPE), (dict(D=60), ESHAPE),
    (dict(lam=None), ENULL), (dict(xp=P + 0x800000), ENULL), (dict(bp=P + 0x900000), ENULL), (dict(x=None), ENULL),
    (dict(lam=P + 0x700008), EALIGN), (dict(xp=P + 0x800008, bp=P + 0x900000), EALIGN),
    (dict(lam=P + 0x500000), EALIAS),                    # y overlaps lam
    (dict(xp=P + 0x600000, bp=P + 0x900000), EALIAS),    # h_final overlaps x_prev
    (dict(xp=P + 0x800000, bp=P + 0x500000 + 64), EALIAS),   # y overlaps B_prev
])
def test_prefill_trapezoid_validation(kw, code):
    assert trap_prefill(**kw) == code


def test_prefill_trapezoid_a_size_follows_the_form():
    # A is [D][16] (4 KiB at D = 64) in the diagonal form: h_final 256 bytes past its start overlaps it
    assert trap_prefill(A=P + 0x200000, h=P + 0x200000 + 256) == EALIAS
    assert trap_prefill(A=P + 0x200000, h=P + 0x200000 + 256, form=2) == EALIAS


def test_prefill_trapezoid_zero_sized_is_a_no_op():
    assert trap_prefill(batch=0, x=None, lam=None, y=None, h=None, A=None) == OK


def trap_step(h=P, xp=P + 0x700000, bp=P + 0x800000, x=P + 0x100000, d=P + 0x200000, lam=P + 0x900000,
              A=P + 0x300000, B=P + 0x400000, C=P + 0x500000, y=P + 0x600000, batch=2, D=64, N=16, ld_xd=64,
              ld_bc=16, ld_y=64, form=0, dtype=BF16):
    return jscan.library().jscan_step_trapezoid(h, xp, bp, x, d, lam, A, B, C, y, batch, D, N, ld_xd, ld_bc, ld_y,
                                                form, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(form=7), EFORM), (dict(xp=None), ENULL), (dict(bp=None), ENULL), (dict(lam=None), ENULL),
    (dict(lam=P + 0x900004), EALIGN), (dict(ld_xd=60), ESHAPE), (dict(y=P + 0x700000), EALIAS),
    (dict(h=P + 0x900000 - 64), EALIAS), (dict(dtype=3), EDTYPE), (dict(ld_y=60), ESHAPE),
])
def test_step_trapezoid_validation(kw, code):
    assert trap_step(**kw) == code


def test_trapezoid_binding_checks_shapes():
    x = torch.zeros(1, 8, 64)
    with pytest.raises(ValueError):
        jscan.prefill_trapezoid(x, x, x, torch.zeros(64, 16), torch.zeros(1, 8, 16), torch.zeros(1, 8, 16),
                                form="nope")


def mimo_prefill(x=P, d=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, h0=None, y=P + 0x500000,
                 h=P + 0x600000, batch=1, L=64, D=64, N=16, R=4, form=0, dtype=BF16):
    return jscan.library().jscan_prefill_mimo(x, d, A, B, C, h0, y, h, batch, L, D, N, R, form, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=3), ESHAPE), (dict(R=16), ESHAPE), (dict(R=0), ESHAPE), (dict(form=5), EFORM), (dict(dtype=2), EDTYPE),
    (dict(D=12), ESHAPE), (dict(x=None), ENULL), (dict(h=None), ENULL), (dict(B=P + 0x300008), EALIGN),
    (dict(y=P + 0x100000), EALIAS),                               # y overlaps delta
    (dict(h=P + 0x500000 + 64 * 64 * 4 * 2 - 16), EALIAS),        # h_final overlaps the end of y (R = 4)
])
def test_prefill_mimo_validation(kw, code):
    assert mimo_prefill(**kw) == code


def test_prefill_mimo_sizes_follow_the_rank():
    # y is batch * L * D * R elements: at R = 1 the same h_final offset no longer overlaps it,
    # so validation passes (and would launch); at R = 8 it overlaps
    assert mimo_prefill(R=8, h=P + 0x500000 + 64 * 64 * 4 * 2) == EALIAS
    assert mimo_prefill(batch=0, x=None, y=None, h=None, A=None) == OK


def mimo_step(h=P, x=P + 0x100000, d=P + 0x200000, A=P + 0x300000, B=P + 0x400000, C=P + 0x500000, y=P + 0x600000,
              batch=2, D=64, N=16, R=4, ld_x=256, ld_d=64, ld_bc=64, ld_y=256, form=0, dtype=BF16):
    return jscan.library().jscan_step_mimo(h, x, d, A, B, C, y, batch, D, N, R, ld_x, ld_d, ld_bc, ld_y, form, dtype,
                                           None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=5), ESHAPE), (dict(ld_x=128), ESHAPE), (dict(ld_bc=32), ESHAPE), (dict(ld_d=60), ESHAPE),
    (dict(form=9), EFORM), (dict(C=None), ENULL), (dict(y=P + 0x600004), EALIGN), (dict(y=P + 0x100000), EALIAS),
    (dict(ld_y=128), ESHAPE), (dict(ld_y=260), ESHAPE),
])
def test_step_mimo_validation(kw, code):
    assert mimo_step(**kw) == code


def mimo_trap_prefill(x=P, d=P + 0x100000, lam=P + 0x700000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, h0=None,
                      xp=None, bp=None, y=P + 0x500000, h=P + 0x600000, batch=1, L=64, D=64, N=16, R=4, form=0,
                      dtype=BF16):
    return jscan.library().jscan_prefill_mimo_trapezoid(x, d, lam, A, B, C, h0, xp, bp, y, h, batch, L, D, N, R, form,
                                                        dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=3), ESHAPE), (dict(form=4), EFORM), (dict(lam=None), ENULL), (dict(xp=P + 0x800000), ENULL),
    (dict(bp=P + 0x900000), ENULL), (dict(lam=P + 0x700004), EALIGN), (dict(lam=P + 0x500000 + 64), EALIAS),
    (dict(xp=P + 0x600000, bp=P + 0x900000), EALIAS),   # h_final overlaps x_prev
])
def test_prefill_mimo_trapezoid_validation(kw, code):
    assert mimo_trap_prefill(**kw) == code


def test_step_mimo_trapezoid_validation():
    lib = jscan.library()
    args = [P, P + 0x700000, P + 0x800000, P + 0x100000, P + 0x200000, P + 0x900000, P + 0x300000, P + 0x400000,
            P + 0x500000, P + 0x600000, 2, 64, 16, 4, 256, 64, 64, 256, 0, BF16, None]
    assert lib.jscan_step_mimo_trapezoid(*args[:1], None, *args[2:]) == ENULL          # x_prev
    assert lib.jscan_step_mimo_trapezoid(*args[:5], None, *args[6:]) == ENULL          # lam_t
    bad = list(args)
    bad[9] = P + 0x700000                                                               # y_t on x_prev
    assert lib.jscan_step_mimo_trapezoid(*bad) == EALIAS
    bad = list(args)
    bad[18] = 3
    assert lib.jscan_step_mimo_trapezoid(*bad) == EFORM
    bad = list(args)
    bad[17] = 200                                                                       # ld_y below D * R
    assert lib.jscan_step_mimo_trapezoid(*bad) == ESHAPE


def test_step_output_and_its_row_stride():
    """The decode steps' y_t: a new contiguous tensor (row stride D, or D * R for MIMO), or the
    caller's tensor with contiguous rows and a row stride of its own (passed on as ld_y)."""
    cpu = torch.device("cpu")
    y, ld = _binding._step_output(None, (3, 64), torch.bfloat16, cpu)
    assert y.shape == (3, 64) and y.is_contiguous() and ld == 64
    y, ld = _binding._step_output(None, (2, 64, 4), torch.float32, cpu)
    assert y.shape == (2, 64, 4) and y.is_contiguous() and ld == 256
    buf = torch.empty(3, 10, 64, dtype=torch.bfloat16)
    y, ld = _binding._step_output(buf[:, 7], (3, 64), torch.bfloat16, cpu)   # token view of [batch, L, D]
    assert ld == 640 and y.data_ptr() == buf[:, 7].data_ptr()
    wide = torch.empty(2, 64 * 4 + 64)
    _, ld = _binding._step_output(wide[:, :256].view(2, 64, 4), (2, 64, 4), torch.float32, cpu)
    assert ld == 320
    _, ld = _binding._step_output(buf[:1, 3], (1, 64), torch.bfloat16, cpu)    # one row: its length
    assert ld == 64
    with pytest.raises(ValueError):
        _binding._step_output(buf[:, :, 0], (3, 10), torch.bfloat16, cpu)       # strided row elements
    with pytest.raises(ValueError):
        _binding._step_output(torch.empty(3, 64), (3, 64), torch.bfloat16, cpu)  # wrong dtype
    with pytest.raises(ValueError):
        _binding._step_output(torch.empty(3, 32, dtype=torch.bfloat16), (3, 64), torch.bfloat16, cpu)
    with pytest.raises(ValueError):   # MIMO rows must be [D][R] with R contiguous
        _binding._step_output(torch.empty(2, 4, 64).transpose(1, 2), (2, 64, 4), torch.float32, cpu)


@pytest.mark.parametrize("fn", ["prefill", "step"])
def test_size_limits_are_where_the_header_puts_them(fn):
    """D up to 2^24 and batch up to 2^20 pass the shape checks (the call then stops at the
    missing x, before any launch); one step past either limit is a shape error."""
    call = prefill if fn == "prefill" else step
    extra = {} if fn == "prefill" else dict(ld_xd=1 << 24, ld_y=1 << 24)
    assert call(D=1 << 24, batch=1, x=None, **extra) == ENULL
    assert call(D=(1 << 24) + 8, batch=1, x=None, **{k: v + 8 for k, v in extra.items()}) == ESHAPE
    assert call(D=64, batch=1 << 20, x=None) == ENULL
    assert call(D=64, batch=(1 << 20) + 1, x=None) == ESHAPE
