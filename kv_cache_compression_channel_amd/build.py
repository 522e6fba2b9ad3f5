"""Build libkvq.so (all HIP sources, gfx950 only) in-tree.

    python -m kv_cache_compression_channel_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkvq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fp32 step is its own IEEE operation unless a kernel asks for fmaf explicitly
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the loop-carried sums of the attention
    # kernel are also rescaled by VALU code, and AGPR homes cost a copy each way per tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-I" + os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libkvq.so")
    # the host pass does not know the packed-fp32 feature name: that warning is expected
    noise = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32-ops" not in ln]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
