"""The C ABI's host code (argument validation, workspace sizing and the planner's checks) under
AddressSanitizer and UndefinedBehaviorSanitizer: the host ABI tests run against a copy of the
library whose host code is built with both (device code uninstrumented), in a child process that
preloads the sanitizer runtime. Any report aborts the child, which fails this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_host_abi_tests_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from unified_transformer_recommender_amd import build

    lib = build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), ONETRANS_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import ctypes; from unified_transformer_recommender_amd import _lib as L; L.lib(); "
             "assert L.LIB_PATH == %r; ctypes.CDLL(None).__asan_init; print('sanitized library loaded')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "sanitized library loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
