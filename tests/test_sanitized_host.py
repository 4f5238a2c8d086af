"""The planner and the C-ABI validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the host tests of the library (test_host_lib.py,
malformed offsets, record budgets and tail ranges included) run in a child
interpreter against libkvdec_san.so -- plan.cpp and api.cpp built with ASan
and UBSan on the host side, the ASan runtime preloaded -- and every report
aborts the run.  CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_tests_clean_under_asan_and_ubsan():
    from long_context_decode_kv_amd import build
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no shared AddressSanitizer runtime in this toolchain")
    assert os.path.exists(build.SAN_LIB)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "KVDEC_LIB_NAME": "libkvdec_san.so",
        # the interpreter and torch are not instrumented: their leaks are not
        # ours; huge allocations must fail as bad_alloc, not abort
        "ASAN_OPTIONS": "detect_leaks=0:allocator_may_return_null=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import ctypes\n"
             "from long_context_decode_kv_amd import kvdec\n"
             "assert kvdec.LIB_PATH.endswith('libkvdec_san.so'), kvdec.LIB_PATH\n"
             "ctypes.CDLL(None).__asan_init\n"
             "print('sanitized library loaded')\n")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_host_lib.py", "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
