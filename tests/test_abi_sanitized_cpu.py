"""The C ABI's CPU checks (tests/test_abi_cpu.py) again, against a build of
the library whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (sparse_query_gqa_amd.build.build_sanitized): any
out-of-bounds access, use of a bad pointer or undefined arithmetic in the
argument validation, size queries and status strings aborts that run.

The sanitized library is built on first use (about half a minute; it is kept
under sparse_query_gqa_amd/_build/san and rebuilt when a source is newer).
The child process preloads the sanitizer runtime, since the Python
interpreter itself is not instrumented. No GPU is touched: every call in
those tests fails validation or is an empty call.
"""
import glob
import os
import subprocess
import sys

import pytest

from sparse_query_gqa_amd import build as gqe_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(gqe_build.CSRC, "*")) + [os.path.join(ROOT, "include", "gqe.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


def test_abi_checks_under_host_sanitizers():
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm image")
    try:
        gqe_build._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    lib = gqe_build.SAN_LIB
    if _stale(lib):
        gqe_build.build_sanitized()
    env = dict(os.environ, GQE_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:])
    print(r.stderr[-3000:])
    assert r.returncode == 0, "ABI checks failed under the host sanitizers"
    assert " passed" in r.stdout
