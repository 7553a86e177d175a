"""Build libte_mi355x.so (gfx950 only) in-tree with hipcc.

Flags that matter for bit-exactness: correctly rounded fp32 division (the scale
fp8_max / amax and 1 / scale), no fast-math, no denormal flushing, and no contraction
of a multiply and an add into one fused operation (-ffp-contract=off), so every
operation the kernels write is rounded on its own, as the documented formulas state.
Packed fp32 instructions are disabled (-packed-fp32-ops) so plain float code is emitted.
Code object v5 keeps the library loadable by the HIP runtime PyTorch ships.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libte_mi355x.so")
SOURCES = ["api.cpp", "quant.hip", "gemm.hip"]
PEAK_LIB = os.path.join(PKG, "libte_peak.so")  # MFMA-only throughput probe (microbench tooling)
PEAK_SOURCES = ["peak.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = HIP_FLAGS + list(extra_flags or [])
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + flags + inc
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and (r.stderr.strip()):
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES) + len(PEAK_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PEAK_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PEAK_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + lib_objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
