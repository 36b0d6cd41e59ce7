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
SOURCES = ["api.hip", "pack.hip", "gemm.hip", "gemm_large.hip", "quant.hip"]

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


COMPILE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                 *DEVICE_FLAGS]


def compile_command(src: str, obj: str, extra=()) -> list:
    return [hipcc(), *COMPILE_FLAGS, *extra, "-c", src, "-o", obj]


def link_command(out: str, objs) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out, *objs]


def _errors(r) -> str:
    return "\n".join(l for l in (r.stderr or "").splitlines() if "not a recognized feature" not in l)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liblowbit.so (always recompiles): the
    sources compile in parallel, then one link."""
    import tempfile
    with tempfile.TemporaryDirectory(prefix="lowbit_build_") as tmpdir:
        cmds = [compile_command(os.path.join(CSRC, src), os.path.join(tmpdir, src + ".o")) for src in SOURCES]
        procs = []
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        failed = []
        for cmd, pr in zip(cmds, procs):
            out, err = pr.communicate()
            r = subprocess.CompletedProcess(cmd, pr.returncode, out, err)
            if r.returncode != 0:
                failed.append(f"{os.path.basename(cmd[-3])}:\n{_errors(r)}")
            elif verbose and _errors(r).strip():
                print(_errors(r), file=sys.stderr)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        tmp = LIB + ".tmp"
        cmd = link_command(tmp, [os.path.join(tmpdir, src + ".o") for src in SOURCES])
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{_errors(r)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
