"""Failure behaviour on the GPU: a NaN in one channel's input stays in that channel, and a
launch on a stream handle that no longer exists returns JSCAN_ERR_HIP with the HIP error.

Channel isolation follows from the S6 recurrence itself (notes page "Jamba: A Hybrid
Transformer-Mamba Language Model", section "Mamba layer"; lesson page "Jamba - Hybrid
SSM-Transformer", section "the SSM on one page"): with a diagonal A, channel d's state and
output depend only on channel d's x and delta and on the shared B and C.  A NaN in x or delta
of one (token, channel) must therefore turn that channel's state and its outputs from that
token on into NaN, and leave every other output bit-identical.

With bf16 output the row-mapped prefill sums each channel's state partials over a 16-token
group on the matrix cores, as one product with a one-hot selection matrix: a NaN partial times
a zero selection weight is NaN, so the NaN also reaches the channel's outputs earlier in the
same 16-token group.  It still stays in its channel, and everything before that group is
unchanged."""
import json
import os
import subprocess
import sys

import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import workloads
from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def check_isolated(y0, h0, y1, h1, t_nan, ch, group=1):
    """y1/h1 (poisoned run) against y0/h0 (clean run): channel ch is NaN from token t_nan on
    and in its final state; every other element is bit-identical.  With group > 1 the channel's
    outputs from the start of t_nan's group of that many tokens up to t_nan are either unchanged
    or NaN."""
    D = y0.shape[2]
    others = torch.tensor([c for c in range(D) if c != ch], device=y0.device)
    assert torch.equal(bits(y1.index_select(2, others)), bits(y0.index_select(2, others))), "NaN leaked into y"
    assert torch.equal(bits(h1.index_select(1, others)), bits(h0.index_select(1, others))), "NaN leaked into h"
    t_safe = t_nan // group * group
    assert torch.equal(bits(y1[:, :t_safe, ch]), bits(y0[:, :t_safe, ch])), "outputs before the NaN changed"
    mid1, mid0 = y1[:, t_safe:t_nan, ch], y0[:, t_safe:t_nan, ch]
    assert (torch.isnan(mid1.float().cpu()) | (bits(mid1) == bits(mid0))).all(), "outputs before the NaN changed"
    assert torch.isnan(y1[:, t_nan:, ch].float()).all(), "channel's outputs after the NaN are not NaN"
    assert torch.isnan(h1[:, ch].float()).all(), "channel's final state is not NaN"


@pytest.mark.parametrize("batch,L,D,dtype,which", [
    (1, 1000, 512, "bf16", "x"),       # row-mapped kernel
    (1, 1000, 512, "bf16", "delta"),
    (2, 300, 64, "f32", "x"),          # row-mapped kernel, fp32, second sequence
    (1, 777, 40, "f32", "delta"),      # D not a multiple of 32: lane kernel
])
def test_nan_in_one_channel_stays_in_that_channel(batch, L, D, dtype, which):
    inp = workloads.small_prefill(batch, L, D, dtype, seed=L + D)
    d = to_dev(inp)
    y0, h0 = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    b, t_nan, ch = batch - 1, L // 3, D // 2 + 3
    poisoned = d[which].clone()
    poisoned[b, t_nan, ch] = float("nan")
    args = dict(d)
    args[which] = poisoned
    y1, h1 = jscan.prefill(args["x"], args["delta"], args["A"], args["B"], args["C"])
    torch.cuda.synchronize()
    say(f"NaN in {which}[{b}, {t_nan}, {ch}] of {batch}x{L}x{D} {dtype}")
    # the other sequences of the batch are untouched
    for bb in range(batch):
        if bb != b:
            assert torch.equal(bits(y1[bb]), bits(y0[bb])) and torch.equal(bits(h1[bb]), bits(h0[bb]))
    group = 16 if dtype == "bf16" and D % 32 == 0 else 1   # the row-mapped kernel's row sums
    check_isolated(y0[b:b + 1], h0[b:b + 1], y1[b:b + 1], h1[b:b + 1], t_nan, ch, group)


def test_nan_in_one_channel_of_a_decode_step():
    wl = workloads.get("decode_256x28")
    inp = workloads.decode_layer_inputs(wl, 0)
    d = to_dev(inp)
    h_clean, h_bad = d["h0"].clone(), d["h0"].clone()
    y0 = jscan.step(h_clean, d["x"], d["delta"], d["A"], d["B"], d["C"])
    x = d["x"].clone()
    x[17, 4000] = float("nan")
    y1 = jscan.step(h_bad, x, d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    mask = torch.ones_like(y0, dtype=torch.bool)
    mask[17, 4000] = False
    assert torch.equal(bits(y1.masked_select(mask)), bits(y0.masked_select(mask)))
    hm = mask[:, :, None].expand_as(h_clean)
    assert torch.equal(bits(h_bad.masked_select(hm)), bits(h_clean.masked_select(hm)))
    assert torch.isnan(y1[17, 4000].float()) and torch.isnan(h_bad[17, 4000]).all()


_CHILD = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
import torch
import mamba_selective_scan_03_amd as jscan
lib = jscan.library()
hip = ctypes.CDLL("libamdhip64.so")
D, L = 64, 128
x = torch.randn(1, L, D, device="cuda")
dl = torch.rand(1, L, D, device="cuda")
A = -torch.rand(D, 16, device="cuda")
B = torch.randn(1, L, 16, device="cuda")
C = torch.randn(1, L, 16, device="cuda")
y = torch.empty_like(x)
h = torch.empty(1, D, 16, device="cuda")
torch.cuda.synchronize()
s = ctypes.c_void_p()
assert hip.hipStreamCreate(ctypes.byref(s)) == 0
assert hip.hipStreamDestroy(s) == 0
p = lambda t: ctypes.c_void_p(t.data_ptr())
st = lib.jscan_prefill(p(x), p(dl), p(A), p(B), p(C), p(y), p(h), 1, L, D, 16, 0, s)
err = lib.jscan_last_hip_error()
ok = lib.jscan_prefill(p(x), p(dl), p(A), p(B), p(C), p(y), p(h), 1, L, D, 16, 0, None)
torch.cuda.synchronize()
print(json.dumps({"status": st, "hip_error": err, "after": ok}), flush=True)
"""


def test_destroyed_stream_returns_hip_error():
    """jscan_prefill on the handle of a destroyed stream: the HIP runtime refuses the launch,
    the library returns JSCAN_ERR_HIP and keeps the hipError_t, and the next call on a valid
    stream succeeds.  Run in a child process, so that the test reports a failure (not a crash
    of the test session) if the runtime were to mishandle the handle."""
    res = subprocess.run([sys.executable, "-c", _CHILD, ROOT], capture_output=True, text=True, timeout=120)
    say(f"child rc {res.returncode}: {res.stdout.strip()[-200:]} {res.stderr.strip()[-300:]}")
    assert res.returncode == 0, f"child process failed (rc {res.returncode})"
    out = json.loads(res.stdout.strip().splitlines()[-1])
    assert out["status"] == 6, out          # JSCAN_ERR_HIP
    assert out["hip_error"] != 0, out
    assert out["after"] == 0, out
