"""The CPU suite once more under AddressSanitizer and UndefinedBehaviorSanitizer
builds of the library's host code and of the oracle (tests/run_sanitized.py),
every report fatal.  Skipped inside that run itself, and where hipcc or the
sanitizer runtime is missing."""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_cpu_suite_under_host_sanitizers():
    if os.environ.get("VERIFY_ATTN_LIB") or os.environ.get("ORACLE_LIB"):
        pytest.skip("already running against other builds")
    if not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")):
        pytest.skip("hipcc not found")
    clang = "/opt/rocm/llvm/bin/clang"
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip() if os.path.exists(clang) else ""
    if not rt or not os.path.exists(rt):
        pytest.skip("the AddressSanitizer runtime was not found")
    r = subprocess.run([sys.executable, os.path.join(HERE, "run_sanitized.py"), "-k", "not sanitizers"],
                       capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
