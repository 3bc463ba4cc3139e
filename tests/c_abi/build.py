"""Build tests/c_abi/verify_c_client, a plain-C caller of libverify_attn.so,
with gcc against include/verify_attn.h and the HIP runtime's C API.  The
binary finds the library through an rpath relative to its own directory."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "verify_c_client.c")
BIN = os.path.join(HERE, "verify_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    lib_dir = os.path.join(ROOT, "speculative_decoding_verify_kv_amd")
    rel = os.path.relpath(lib_dir, HERE)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", BIN + ".tmp",
           "-L", lib_dir, "-lverify_attn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/" + rel, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
