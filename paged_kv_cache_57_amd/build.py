"""Builds libpa.so in-tree for gfx950 with hipcc.

The library is one shared object: the HIP kernels with their C-ABI launchers
and the host allocator.  Packed-FP32 instructions are disabled for device
code (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass of
hipcc warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
# measurement-only probes (not part of the attention path), a library of their own
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")
PROBE_SOURCES = [os.path.join("measure", "pa_probe.hip")]
SOURCES = ["pa_status.cpp", "pa_alloc.cpp", "pa_splitfuse.cpp", "pa_step.cpp", "pa_cache.hip", "pa_attention.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
# No packed FP32 instructions; and no atomic optimizer, which wraps each atomic in a
# branch on the first active lane (the kernels keep their work loops free of
# lane-dependent branches).
# -fno-honor-nans: maxima need no NaN quieting first (masked keys are removed by
# integer compares, selects and bit masks, never by float comparisons).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None", "-fno-honor-nans"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so (and the measurement library libpa_probe.so);
    returns libpa.so's path. Always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip", *DEVICE_FLAGS]
        else:
            # host code only: no device pass (the HIP runtime API header for the upload of a step)
            cmd[1:1] = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    pobjs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        _run([HIPCC, "-x", "hip", *DEVICE_FLAGS, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        pobjs.append(obj)
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *pobjs, "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
