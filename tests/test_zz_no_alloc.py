"""jscan_prefill_chunked_noalloc (the time-parallel prefill on the library's own scratch
array, for callers that cannot allocate) against jscan_prefill_chunked with a caller
workspace: both run the same kernels in the same order, so every output bit must agree.
The calls go straight through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import workloads
from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu

OK, EWORKSPACE = 0, 7
DT = {torch.float32: 0, torch.bfloat16: 1}


def p(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


def noalloc_call(d, h0, y, h, chunk):
    batch, L, D = d["x"].shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return jscan.library().jscan_prefill_chunked_noalloc(p(d["x"]), p(d["delta"]), p(d["A"]), p(d["B"]), p(d["C"]),
                                                         p(h0), p(y), p(h), batch, L, D, 16, chunk,
                                                         DT[d["x"].dtype], stream)


def workspace_call(d, h0, chunk):
    batch, L, D = d["x"].shape
    need = jscan.chunked_workspace_bytes(batch, L, D, chunk)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    return jscan.prefill_chunked(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0, chunk=chunk, workspace=ws)


@pytest.mark.parametrize("first,second", [
    # (batch, L, D, dtype, chunk, with h0): a large call, then a smaller one on the same scratch
    ((1, 65536, 1024, "bf16", 0, False), (2, 3000, 256, "f32", 500, True)),
    ((3, 2048, 96, "f32", 128, True), (1, 700, 64, "bf16", 100, False)),
])
def test_noalloc_matches_the_workspace_path_twice(first, second):
    for batch, L, D, dtype, chunk, with_h0 in (first, second):
        inp = workloads.small_prefill(batch, L, D, dtype, seed=L + D)
        d = to_dev(inp)
        h0 = None
        if with_h0:
            g = np.random.default_rng([L, D, 5])
            h0 = torch.from_numpy(g.normal(0.0, 0.1, size=(batch, D, 16)).astype(np.float32)).cuda()
        y_ref, h_ref = workspace_call(d, h0, chunk)
        y = torch.full_like(d["x"], float("nan"))
        h = torch.full((batch, D, 16), float("nan"), device="cuda")
        st = noalloc_call(d, h0, y, h, chunk)
        torch.cuda.synchronize()
        say(f"noalloc {batch}x{L}x{D} {dtype} chunk {chunk} h0={with_h0}: status {st}, "
            f"{jscan.chunked_workspace_bytes(batch, L, D, chunk)} scratch bytes")
        assert st == OK
        assert torch.equal(bits(y), bits(y_ref)), "y differs from the workspace path"
        assert torch.equal(bits(h), bits(h_ref)), "h_final differs from the workspace path"


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan needing more than 16 MiB of segment states returns JSCAN_ERR_WORKSPACE before any
    launch; the outputs stay untouched."""
    batch, L, D, chunk = 1, 16384, 8192, 256        # 64 segments x 8192 channels x 68 B = 34 MiB
    assert jscan.chunked_workspace_bytes(batch, L, D, chunk) > jscan._binding.NOALLOC_SCRATCH_BYTES
    inp = workloads.small_prefill(batch, L, D, "bf16", seed=3)
    d = to_dev(inp)
    y = torch.full_like(d["x"], float("nan"))
    h = torch.full((batch, D, 16), float("nan"), device="cuda")
    assert noalloc_call(d, None, y, h, chunk) == EWORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all() and torch.isnan(h).all()
