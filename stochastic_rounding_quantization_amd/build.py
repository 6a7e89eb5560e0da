"""Build libs3r.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m stochastic_rounding_quantization_amd.build [--verbose]

The library lands next to this file.  hipcc cross-compiles for gfx950 on a
machine without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libs3r.so")
SOURCES = ["capi.hip", "quantize.hip", "gemm.hip", "swiglu.hip", "groups.hip", "mx.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # one IEEE rounding per fp32 operation: the quantizer's codes depend on it
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    # no packed-FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filter(stderr: str) -> str:
    noise = "not a recognized feature for this target"
    return "\n".join(l for l in stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object in parallel, then link libs3r.so."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(ROOT, "_build", "s3r")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *compile_flags, *extra, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for (obj, res), src in zip(results, SOURCES):
        err = _filter(res.stderr)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({res.returncode}):\n{err}")
        if verbose and err.strip():
            print(err)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{_filter(res.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
