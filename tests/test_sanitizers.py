"""The fp64 oracle and the host planner under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Both are built here with gcc / g++ (no HIP) into a temporary folder and run
as child processes.  tests/sanitize_oracle_driver.c calls every oracle entry
point on seeded inputs -- NaN-padded rows, empty and clamped sequences,
pages in both layouts, several tokens -- and checks them against each other;
tests/sanitize_planner_driver.cpp plans some 42 thousand shapes, extremes
included, and checks every plan's invariants.  A sanitizer report aborts the
child (no recovery), which fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "long_context_decode_fd_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-static-libasan"]
# leak checks need ptrace, which containers may not allow; the runtime's
# link-order check is relaxed so that a preloaded library does not stop it
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _tool(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} is not installed")
    return path


def _run(exe):
    r = subprocess.run([str(exe)], capture_output=True, text=True,
                       timeout=300, env=ENV)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr, report
    assert "AddressSanitizer" not in r.stderr, report
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    subprocess.run([_tool("gcc"), "-std=c11", "-Wall", "-Wextra", "-fopenmp",
                    *SAN, os.path.join(HERE, "sanitize_oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "fd_oracle.c"), "-lm",
                    "-o", str(exe)], check=True)
    assert _run(exe).strip().endswith("ok")


def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "planner_driver"
    subprocess.run([_tool("g++"), "-std=c++17", "-Wall", "-Wextra", *SAN,
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(HERE, "sanitize_planner_driver.cpp"),
                    os.path.join(CSRC, "fd_plan.cpp"), "-o", str(exe)],
                   check=True)
    out = _run(exe)
    assert "failures 0" in out, out
