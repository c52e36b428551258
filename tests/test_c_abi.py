"""The C ABI driven from plain C (tests/c_abi_caller.c), not through Python.

Host mode (no GPU): the planner's choices for two workloads, the status
strings and the argument errors, answered before the library touches HIP.
GPU mode: a C program reads a seeded problem, runs fd_decode (library
workspace) and fd_decode_ex (its own workspace, forced split count), and the
results are compared with the fp64 oracle under the suite's rule (|out - ref|
<= 1e-2 or faithful bf16 rounding, |lse - ref| <= 1e-3).
"""
import os
import subprocess

import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from parity import check_lse, check_out

import c_abi_build

FD_OK, FD_ERR_WORKSPACE = 0, -3


def _binary(build_if_missing: bool) -> str:
    if not os.path.exists(c_abi_build.OUT):
        if not build_if_missing:
            pytest.fail("tests/_build/c_abi_caller is missing: run build()")
        c_abi_build.build()
    return c_abi_build.OUT


def test_host_mode_from_c():
    fd.load_library()  # the caller links the same in-tree libfd.so
    r = subprocess.run([_binary(True), "host"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    got = dict(line.split()[:2] for line in r.stdout.splitlines())
    # the C caller's plan is the binding's plan
    p = fd.fd_plan(1, 64, 8, 128, 65536, "bf16", num_cus=256)
    assert int(got["plan_splits"]) == p["num_splits"]
    assert int(got["plan_chunk"]) == p["chunk"]
    assert int(got["plan_grid"]) == p["grid"]
    assert int(got["plan_workspace"]) == p["workspace_bytes"]
    assert "MISMATCH" not in r.stdout


W = wl.Workload("c_abi", B=3, Hq=16, Hkv=2, D=128, Lmax=3000, dtype="bf16",
                seed=95)
SEQLENS = np.array([3000, 1234, 0], np.int32)
SPLITS = 7


@pytest.mark.gpu
def test_decode_from_c(oracle_mod, tmp_path):
    exe = _binary(False)
    w = W
    q = wl.gen_q(w)
    k = np.empty((w.B, w.Hkv, w.Lmax, w.D), w.np_dtype)
    v = np.empty_like(k)
    for b in range(w.B):
        for g in range(w.Hkv):
            wl.fill_slab(w, b, g, int(SEQLENS[b]), k[b, g], v[b, g])
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([w.B, w.Hq, w.Hkv, w.D, w.Lmax, SPLITS, 1],
                         np.int32).tobytes())
        f.write(np.float32(w.scale).tobytes())
        for a in (q, k, v, SEQLENS):
            f.write(np.ascontiguousarray(a).tobytes())
    print(f"[c abi] running {exe} on B={w.B} Hq={w.Hq} Hkv={w.Hkv} "
          f"Lmax={w.Lmax} splits={SPLITS}", flush=True)
    r = subprocess.run([exe, "run", str(inp), str(outp)], capture_output=True,
                       text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    raw = outp.read_bytes()
    status = np.frombuffer(raw[:16], np.int32)
    assert status[0] == FD_OK and status[1] == FD_OK, status
    assert status[2] == FD_ERR_WORKSPACE, status   # one byte too small
    assert status[3] == 1, status                  # plan and size agree
    nq, nl = w.B * w.Hq * w.D, w.B * w.Hq
    off = 16
    ref_o, ref_l = oracle_mod.decode(q, k, v, SEQLENS, w.scale)
    for call in ("fd_decode", "fd_decode_ex"):
        out = np.frombuffer(raw[off:off + 2 * nq], np.uint16).reshape(
            w.B, w.Hq, w.D)
        off += 2 * nq
        lse = np.frombuffer(raw[off:off + 4 * nl], np.float32).reshape(
            w.B, w.Hq)
        off += 4 * nl
        ok_o, rep_o = check_out(out, ref_o, "bf16")
        ok_l, rep_l = check_lse(lse, ref_l)
        print(f"[c abi] {call}: out {rep_o} lse {rep_l}", flush=True)
        assert ok_o, (call, rep_o)
        assert ok_l, (call, rep_l)
    assert off == len(raw)
