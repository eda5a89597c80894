"""Build libnystrom.so (HIP, gfx950) in place, next to this file.

The library is several translation units (csrc/*.hip): the host side and
C ABI, the forward pass per I/O type, the exact branch and the backward
pass.  They compile in parallel into objects under _build/ and are linked
into one shared library.

Usage: python -m efficient_transformer_attention_segment_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libnystrom.so")
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs (no accvgpr copies before
    # the VALU work on them)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]
LDFLAGS = [
    "-shared", f"--offload-arch={ARCH}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnystrom.so)")


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _jobs() -> int:
    n = os.cpu_count() or 4
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        if os.environ.get(var, "").isdigit():
            n = min(n, int(os.environ[var]))
    return max(1, min(n, 16))


def build(verbose: bool = False) -> str:
    """Compile every translation unit and link the library; always
    recompiles.  Returns the .so path."""
    cc = hipcc()
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(OBJ, os.path.splitext(os.path.basename(src))[0] + ".o")
        cmd = [cc, *CFLAGS, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        return obj, res

    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        results = list(ex.map(compile_one, srcs))
    failed = [(o, r) for o, r in results if r.returncode != 0]
    for o, r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError(f"hipcc failed for {[os.path.basename(o) for o, _ in failed]}")
    tmp = LIB + ".tmp"
    cmd = [cc, *LDFLAGS, "-o", tmp, *[o for o, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"link failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
