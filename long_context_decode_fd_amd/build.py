"""Build libfd.so (HIP for gfx950) in place.

    python -m long_context_decode_fd_amd.build [-D NAME=VALUE ...] [-o PATH]

The library lands next to this file unless -o says otherwise.  Extra -D
definitions override the planner's tunables (used for sweeps).
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfd.so")
SOURCES = ["fd_api.hip", "fd_kernels.hip", "fd_plan.cpp"]
# Exports of libfd.so: exactly the fd_* entry points of include/fd.h.
VERSION_SCRIPT = os.path.join(CSRC, "libfd.version")
# The benchmark's streaming-read helper (not part of the decode path).
PROBE_LIB = os.path.join(PKG, "libfdprobe.so")
PROBE_SOURCES = ["fd_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, defines=(), verbose: bool = False,
          sources=SOURCES) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Wall", "-I", INCLUDE, "-I", CSRC,
           # no packed-fp32 instructions anywhere in the device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument"]
    if sources == SOURCES:
        cmd += ["-fvisibility=hidden",
                f"-Wl,--version-script={VERSION_SCRIPT}"]
    cmd += [f"-D{d}" for d in defines]
    cmd += [os.path.join(CSRC, s) for s in sources]
    cmd += ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-D", action="append", default=[], dest="defines")
    ap.add_argument("-o", default=LIB)
    ap.add_argument("-q", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.o, a.defines, verbose=not a.q))
    if a.o == LIB:
        print(build(PROBE_LIB, verbose=not a.q, sources=PROBE_SOURCES))


if __name__ == "__main__":
    sys.exit(main())
