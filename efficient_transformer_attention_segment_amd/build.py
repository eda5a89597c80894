"""Build libnystrom.so (HIP, gfx950) in place, next to this file.

Usage: python -m efficient_transformer_attention_segment_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnystrom.so")
SRC = os.path.join(HERE, "csrc", "nystrom.hip")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs (no accvgpr copies before
    # the VALU work on them)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
    # the module's q/k/v projection is one library GEMM
    "-lhipblaslt",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnystrom.so)")


def build(verbose: bool = False) -> str:
    """Compile the library; always recompiles.  Returns the .so path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
