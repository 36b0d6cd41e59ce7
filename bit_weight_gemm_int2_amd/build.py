"""Build the gfx950 HIP library ``liblowbit.so`` in-tree with hipcc.

Usage: ``python -m bit_weight_gemm_int2_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblowbit.so")
SOURCES = ["api.hip", "pack.hip", "gemm.hip"]

# Packed FP32 VALU instructions are disabled for all device code; plain
# float code is scheduled as scalar v_fma_f32 / v_mul_f32 instead.
# MFMA accumulators are kept in VGPRs (the per-group rescale of the large-M
# kernel is VALU work on them; VALU instructions cannot read AGPRs), which
# leaves the AGPR file to the MFMA A operands.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def command(out: str = LIB, extra=()) -> list:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Wall", "-Wno-unused-function", *DEVICE_FLAGS, *extra, "-o", out, *srcs]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liblowbit.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
