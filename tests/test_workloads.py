"""The seeded input generator: reproducible, order-independent, right distributions."""
import numpy as np
import torch

import workloads
from workloads import Workload

WL = Workload("gen_check", 77, 2, 9000, 64, 16, "bf16", True, extra_tokens=50)


def test_same_seed_same_bytes():
    a = workloads.prefill_inputs(WL, seed=0, threads=1)
    b = workloads.prefill_inputs(WL, seed=0, threads=4)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    c = workloads.prefill_inputs(WL, seed=1, threads=1)
    assert not torch.equal(a["x"], c["x"])


def test_token_ranges_are_independent_of_order():
    full = workloads.prefill_inputs(WL, seed=0, t0=0, t1=9050)
    tail = workloads.prefill_inputs(WL, seed=0, t0=5000, t1=9050)
    for k in ("x", "delta", "B", "C"):
        assert torch.equal(full[k][:, 5000:], tail[k]), k
    assert torch.equal(full["A"], tail["A"])


def test_distributions():
    inp = workloads.prefill_inputs(WL, seed=0)
    x = inp["x"].float().numpy()
    d = inp["delta"].float().numpy()
    A = inp["A"].numpy()
    assert inp["x"].dtype == torch.bfloat16 and inp["A"].dtype == torch.float32
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    assert d.min() > 0 and abs(d.mean() - 0.1826) < 0.01        # E[softplus(N(0,1) - 2)]
    n1 = np.arange(1, 17)
    ratio = -A / n1[None, :]
    assert ratio.min() >= 0.5 and ratio.max() <= 1.5 and abs(ratio.mean() - 1) < 0.05
    tiny = workloads.prefill_inputs("tiny_fp32")
    assert tiny["x"].dtype == torch.float32
    assert np.array_equal(tiny["A"].numpy(), -np.broadcast_to(n1, (64, 16)).astype(np.float32))


def test_named_workload_shapes():
    w = workloads.WORKLOADS
    assert (w["prefill_64k"].batch, w["prefill_64k"].L, w["prefill_64k"].D, w["prefill_64k"].N) == (1, 65536, 8192, 16)
    assert w["decode_256x28"].layers == 28 and w["decode_256x28"].batch == 256
    assert w["prefill_256k"].L == 262144 and w["prefill_256k"].extra_tokens == 64
    assert (w["prefill_64k_tp8"].batch, w["prefill_64k_tp8"].L, w["prefill_64k_tp8"].D) == (1, 65536, 1024)
    assert len({v.wid for v in w.values()}) == len(w)     # distinct seed streams


def test_decode_layer_inputs_small():
    wl = Workload("dec_check", 78, 4, 1, 32, 16, "bf16", True, layers=3)
    a = workloads.decode_layer_inputs(wl, layer=2)
    b = workloads.decode_layer_inputs(wl, layer=2)
    assert a["h0"].shape == (4, 32, 16) and a["x"].shape == (4, 32) and a["B"].shape == (4, 16)
    for k in a:
        assert torch.equal(a[k], b[k])
    c = workloads.decode_layer_inputs(wl, layer=1)
    assert not torch.equal(a["h0"], c["h0"])
    assert abs(a["h0"].std().item() - 0.1) < 0.02
