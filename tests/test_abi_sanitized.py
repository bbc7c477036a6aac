"""The C-ABI checks of tests/test_abi.py run again against a host build of the
validation layer instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(build.build_sanitized_abi): every rejected call must also be free of memory
and undefined-behaviour errors.  CPU only; needs g++ and the kernel objects of
the last build."""

import os
import shutil
import subprocess
import sys

import pytest

from hybrid_sparse_linear_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_checks_under_asan_and_ubsan():
    objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o") for s in B.SOURCES if s != "sala_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run __graft_entry__.build())")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("ASan runtime not found")
    lib = B.build_sanitized_abi()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, SALA_LIB_PATH=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
    assert " passed" in out
