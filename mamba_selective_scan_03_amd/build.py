"""Build libjscan.so in place with hipcc for gfx950.

    python -m mamba_selective_scan_03_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "jscan.hip")
LIB = os.path.join(HERE, "libjscan.so")
# the microbenchmarks of the chip's ALU, matrix-core, LDS and HBM rates (measurement only)
MICRO_SRC = os.path.join(HERE, "csrc", "micro.hip")
MICRO_LIB = os.path.join(HERE, "libjscan_micro.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",          # every fused multiply-add in the kernels is written out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC",
    "-shared",
    "-Wall",
]


def _compile(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only target feature; that note is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the library and the microbenchmark library (always recompiles); returns the
    library's path."""
    _compile(MICRO_SRC, MICRO_LIB, verbose)
    return _compile(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
