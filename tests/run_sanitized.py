"""Host-side sanitizer run of the CPU test suite.

Builds, in a temporary directory,
  * libverify_attn.so with its host code (plan validation, workspace layout,
    launch set-up, the ctypes-facing entry points) under AddressSanitizer and
    UndefinedBehaviorSanitizer; the gfx950 device code is compiled as usual;
  * liboracle.so (oracle.c) under the same two sanitizers;
then runs `pytest -m "not gpu"` against both builds (VERIFY_ATTN_LIB,
ORACLE_LIB) with the sanitizer runtime preloaded, any error fatal.

    python tests/run_sanitized.py [extra pytest arguments]

Only host code is instrumented: GPU-side sanitizers are not used.  Leak
detection is off (the Python interpreter itself keeps allocations alive at
exit).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from speculative_decoding_verify_kv_amd import build as B  # noqa: E402

LLVM = "/opt/rocm/llvm/bin"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g", "-Xarch_host", "-O1"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def build_library(tmp: str) -> str:
    objs = []
    for src in B.SOURCES:
        obj = os.path.join(tmp, src + ".o")
        cmd = [B.hipcc(), *B._flags(), *B.PER_SOURCE_FLAGS.get(src, []), *HOST_SAN, "-c",
               os.path.join(B.CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, stderr=subprocess.DEVNULL)
        objs.append(obj)
    lib = os.path.join(tmp, "libverify_attn.so")
    subprocess.run([os.path.join(LLVM, "clang++"), "-shared", "-shared-libasan", *SAN, "-o", lib, *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return lib


def build_oracle(tmp: str) -> str:
    lib = os.path.join(tmp, "liboracle.so")
    subprocess.run([os.path.join(LLVM, "clang"), "-std=c11", "-fPIC", "-shared", "-shared-libasan", *SAN,
                    "-Wall", "-Wextra", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lpthread", "-lm"],
                   check=True)
    return lib


def main(argv) -> int:
    runtime = subprocess.run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.exists(runtime):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    tmp = tempfile.mkdtemp(prefix="va_san_")
    try:
        lib = build_library(tmp)
        olib = build_oracle(tmp)
        print(f"[sanitized] {lib}\n[sanitized] {olib}", flush=True)
        env = dict(os.environ)
        env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        env["VERIFY_ATTN_LIB"] = lib
        env["ORACLE_LIB"] = olib
        cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q",
               "-p", "no:cacheprovider", *argv]
        return subprocess.run(cmd, cwd=ROOT, env=env).returncode
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
