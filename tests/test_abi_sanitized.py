"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with its host code (argument checks, error messages,
scratch bookkeeping) instrumented by ASan + UBSan and its device code as
usual, and the host-side ABI tests (``test_abi_host.py``: symbol exports,
every argument check, the no-op paths, the thread-local error message) run
against that build in a child process that preloads the sanitizer runtime.
Any sanitizer report fails the test.  No GPU is needed: none of these calls
reaches a kernel launch.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def test_abi_host_checks_are_clean_under_asan_and_ubsan(tmp_path):
    from vision_encoder_varlen_amd import build
    lib = build.build_host_sanitized(str(tmp_path / "libvit_host_sanitized.so"))
    env = dict(os.environ)
    env.update({
        "VIT_LIBRARY": lib,
        "LD_PRELOAD": build.sanitizer_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    # the child really runs the instrumented build with the sanitizer runtime
    probe = ("import ctypes, os; ctypes.CDLL(os.environ['VIT_LIBRARY']); "
             "maps = open('/proc/self/maps').read(); "
             "print('asan' if 'libclang_rt.asan' in maps else 'none', "
             "'lib' if os.environ['VIT_LIBRARY'] in maps else 'nolib')")
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.stdout.split() == ["asan", "lib"], r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
