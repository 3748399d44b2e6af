"""Build libivftk.so (HIP kernels + C ABI runtime) for gfx950 with hipcc.

Run as `python -m ivf_top_key_amd.build` or call build().  Objects go to
ivf_top_key_amd/_build/, the library to ivf_top_key_amd/libivftk.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libivftk.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["score.hip", "rescore.hip", "rescore_f32.hip", "rescore_bf16.hip", "rescore_e4m3.hip", "route.hip", "seal.hip", "refit.hip", "encoder.hip", "runtime.cpp"]

# -ffp-contract=off: the clustering arithmetic is defined operation by operation
#   (no fused multiply-add); the score epilogue calls fmaf explicitly.
# correctly rounded fp32 divide/sqrt: centroid means and representative scales.
# packed fp32 ops are disabled for every kernel.
# MFMA accumulators in ordinary VGPRs: the score epilogue reads all of them, and
# the accumulation-register form would add one copy per accumulator.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _up_to_date(src: str, obj: str) -> bool:
    """True if obj is newer than src and every header it may include."""
    if not os.path.exists(obj):
        return False
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")] + \
        [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    t = os.path.getmtime(obj)
    return all(os.path.getmtime(dep) < t for dep in deps)


def _compile(src: str, verbose: bool, incremental: bool = False) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    if incremental and _up_to_date(src, obj):
        return obj
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int | None = None, incremental: bool = False) -> str:
    """Compile every source and link the library.  incremental=True skips sources
    whose object is newer than the source and every header."""
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
