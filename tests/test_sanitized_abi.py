"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Links the library with a host-sanitized nm_api.cpp (the device code is not
instrumented) and runs the CPU ABI tests (argument checks, error paths, size
queries, symbol exports) against it in a child process with the ASan runtime
preloaded; any sanitizer report fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_abi_under_asan_ubsan():
    from structured_sparse_gemm_nm_amd import build as B
    if not os.path.exists(B.SANITIZER_RUNTIME):
        pytest.skip(f"no ASan runtime at {B.SANITIZER_RUNTIME}")
    try:
        B.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_sanitized(verbose=False)
    env = dict(os.environ)
    env.update({"NMSPARSE_LIB": lib, "LD_PRELOAD": B.SANITIZER_RUNTIME,
                # the interpreter itself is not built for leak checking
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    code = ("import ctypes, sys, pytest, structured_sparse_gemm_nm_amd as nm\n"
            "ctypes.CDLL(None).__asan_init\n"                       # the runtime is live
            f"assert nm.lib_path() == {lib!r}\n"
            "sys.exit(pytest.main(['-x', '-q', '-m', 'not gpu', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
