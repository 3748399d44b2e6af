"""Build libivftk_asan.so: the library with its host runtime (runtime.cpp) compiled
under AddressSanitizer, for the CPU tests of the C ABI's argument and error paths.

Only the host side is instrumented (the sanitizer flags apply to the host
compilation only); the kernels are the objects of the normal build in _build/,
which must exist.  Run with the clang ASan runtime preloaded, e.g.
    LD_PRELOAD=<asan runtime> IVFTK_LIBRARY=ivf_top_key_amd/_build_asan/libivftk_asan.so
"""
from __future__ import annotations

import glob
import os
import subprocess

from .build import CSRC, FLAGS, OUT_DIR, SOURCES, _hipcc

ASAN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build_asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libivftk_asan.so")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime shipped with the ROCm compiler."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_asan() -> str:
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = [os.path.join(OUT_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "runtime.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first (missing {missing[0]})")
    rt_obj = os.path.join(ASAN_DIR, "runtime_asan.o")
    cmd = [_hipcc(), "-x", "hip", *FLAGS, *HOST_ASAN, "-c", os.path.join(CSRC, "runtime.cpp"), "-o", rt_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on runtime.cpp (ASan):\n{res.stderr}")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *HOST_ASAN, rt_obj, *objs,
           "-o", ASAN_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed (ASan):\n{res.stderr}")
    return ASAN_LIB


if __name__ == "__main__":
    print(build_asan())
