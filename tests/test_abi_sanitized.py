"""The C ABI's host side (argument validation, overlap checks, workspace layout) built with
AddressSanitizer and UndefinedBehaviorSanitizer (host compiler, kernel launchers stubbed),
running every check of test_abi.py: no sanitizer report, and the same results."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    gxx = shutil.which("g++")
    if not gxx:
        return None
    path = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(asan_runtime() is None, reason="g++ with AddressSanitizer not available")
def test_abi_checks_under_address_and_undefined_behavior_sanitizers():
    sys.path.insert(0, ROOT)
    from kv_vector_index_amd import build_lib
    lib = build_lib.build_sanitized()
    env = dict(os.environ, WAVE_INDEX_LIB=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out.split("\n")[-2], out[-2000:]
