"""Builds libffnwb.so (the HIP library behind include/ffnwb.h) for gfx950, in-tree.

Usage: ``python -m unpermute_ffnwb_batching_amd.build`` or ``build()`` from Python.
Compiles on a machine without a GPU (hipcc cross-compiles the device code).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libffnwb.so")
# a measurement probe for the benchmark, in a library of its own (not the product's interface)
PROBE_SOURCE = "probe_copy.hip"
PROBE_LIB = os.path.join(LIBDIR, "libffnwb_probe.so")
SOURCES = ["api.hip", "batching.hip", "unpermute.hip", "permute.hip", "context.hip", "update_expert.hip",
           "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # Products and sums are rounded separately, as the method's kernel does (no FMA contraction).
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    # Keep hipcc from emitting packed-FP32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wextra",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose=False):
    """Compile every source and link ``_lib/libffnwb.so``.  Always recompiles."""
    hipcc = _hipcc()
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs_all = list(ex.map(compile_one, SOURCES + [PROBE_SOURCE]))
    objs, probe_obj = objs_all[:-1], objs_all[-1]
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", PROBE_LIB + ".tmp", probe_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
