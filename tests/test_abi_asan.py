"""The host runtime of the C ABI under AddressSanitizer (CPU only).

The library is rebuilt with runtime.cpp compiled under AddressSanitizer on the
host side (ivf_top_key_amd/build_asan.py; the kernels are the normal objects), and
the CPU ABI tests (tests/test_abi.py: exported symbols, every argument and
configuration check, null handles, the create and cleanup paths) run against it
in a child process with the sanitizer runtime preloaded.  Any sanitizer report
fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_address_sanitizer():
    from ivf_top_key_amd import build_asan, _lib
    if not os.path.exists(os.path.join(ROOT, "ivf_top_key_amd", "_build", "runtime.o")):
        from ivf_top_key_amd.build import build
        build()
    rt = build_asan.asan_runtime()
    if rt is None:
        pytest.skip("the toolchain has no clang AddressSanitizer runtime")
    lib = build_asan.build_asan()
    env = dict(os.environ, LD_PRELOAD=rt, IVFTK_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:exitcode=99")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout
