"""Build tests/_build/c_abi_caller, the plain C caller of include/fd.h.

Test infrastructure: gcc in C11 mode against the public header, libfd.so
and the HIP runtime (no hipcc, no C++), so the tests can show the boundary
working from C.  The binary finds libfd.so beside the package through its
run path.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_caller.c")
OUT = os.path.join(HERE, "_build", "c_abi_caller")
PKG = os.path.join(ROOT, "long_context_decode_fd_amd")


def build(out: str = OUT) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    rel = os.path.relpath(PKG, os.path.dirname(out))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), SRC, "-o", out + ".tmp",
           "-L", PKG, "-l:libfd.so", f"-Wl,-rpath,$ORIGIN/{rel}",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
