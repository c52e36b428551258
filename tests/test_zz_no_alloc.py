"""fd_decode_noalloc, the entry point that allocates nothing, through the C
ABI (the ctypes binding passes raw pointers to libfd.so).

Its partials live in the library's fixed per-device scratch array instead
of a workspace.  Two calls in a row, the second with a smaller input (the
array still holds the first call's partials), must each equal fd_decode_ex
with a caller workspace bit for bit (same plan, same kernels) and the fp64
oracle on every row; a plan too large for the array is refused before
anything is launched; the call replays from a HIP graph like an eager call.
"""
import ctypes

import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import out_to_host, upload_full
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


def _note(msg):
    print(f"[noalloc] {msg}", flush=True)


def _bits(torch, t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16,
                                              torch.float16) else t


def _check_case(torch, oracle_mod, w, seqlens, num_splits, tag):
    q, k, v, sl, seqlens, ref = upload_full(w, oracle_mod, seqlens=seqlens)
    plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                      varlen=sl is not None, num_splits=num_splits)
    _note(f"{tag}: B={w.B} Lmax={w.Lmax} plan {plan}")
    assert plan["workspace_bytes"] <= fd.NOALLOC_SCRATCH_BYTES
    out, lse = fd.fd_decode_noalloc(q, k, v, sl, w.scale,
                                    num_splits=num_splits)
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8,
                     device="cuda")
    out_e, lse_e = fd.fd_decode_ex(q, k, v, sl, w.scale,
                                   num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch, out), _bits(torch, out_e)), tag
    assert torch.equal(lse, lse_e), tag
    ok_o, rep_o = check_out(out_to_host(out), ref[0], w.dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref[1])
    _note(f"{tag}: out {rep_o} lse {rep_l}")
    assert ok_o, (tag, rep_o)
    assert ok_l, (tag, rep_l)
    return plan


def test_two_calls_in_a_row_second_smaller(torch, oracle_mod):
    big = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=8, Lmax=16384, varlen=(300, 16384))
    p1 = _check_case(torch, oracle_mod, big, None, 0, "first, larger")
    assert p1["combine"]
    small = wl.WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(Lmax=3000)
    p2 = _check_case(torch, oracle_mod, small, None, 5, "second, smaller")
    assert p2["combine"] and p2["workspace_bytes"] < p1["workspace_bytes"]
    # and once more with forced splits, fp32 and the vector-ALU kernel
    tiny = wl.WORKLOADS["tiny_mha_f32_b1_h8_d64_l1024"]
    _check_case(torch, oracle_mod, tiny, None, 3, "third, fp32")
    # fp32 on the matrix cores
    f32 = wl.ALL_WORKLOADS["f32_b1_gqa8_h64_d128_l65536"].with_(Lmax=2000)
    p4 = _check_case(torch, oracle_mod, f32, None, 0, "fourth, fp32 MFMA")
    assert p4["variant"] == fd.FD_VARIANT_MFMA
    # an fp16 cache
    f16 = wl.ALL_WORKLOADS["f16_b1_gqa8_h64_d128_l65536"].with_(Lmax=2500)
    _check_case(torch, oracle_mod, f16, None, 0, "fifth, fp16")


def test_single_pass_plan_uses_no_scratch(torch, oracle_mod):
    w = wl.WORKLOADS["b64_gqa4_h32_d128_l4096"].with_(Lmax=1000)
    plan = _check_case(torch, oracle_mod, w, None, 0, "single pass")
    assert not plan["combine"]


def test_plans_too_large_or_fused_are_refused(torch):
    """Host-side refusals: nothing is launched, so the pointers below (fake,
    aligned, never dereferenced) are never touched."""
    lib = fd.load_library()
    A = 1 << 20
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B, Hq, Hkv, D, L, S = 64, 32, 8, 128, 4096, 128
    plan = fd.fd_plan(B, Hq, Hkv, D, L, "bf16", num_splits=S)
    assert plan["workspace_bytes"] > fd.NOALLOC_SCRATCH_BYTES
    rc = lib.fd_decode_noalloc(A, A, A, None, B, Hq, Hkv, D, L, 0.1, 0, A, A,
                               S, 0, 0, st)
    assert rc == fd.FD_ERR_TOO_LARGE
    rc = lib.fd_decode_noalloc(A, A, A, None, 1, 8, 8, 128, 4096, 0.1, 0, A,
                               A, 0, 0, fd.FD_FLAG_FUSED_MERGE, st)
    assert rc == fd.FD_ERR_UNSUPPORTED
    rc = lib.fd_decode_noalloc(A, A, A, None, 1, 8, 8, 128, 4096, 0.1, 0, A,
                               A, 0, 0, fd.FD_FLAG_UNIFIED_MAX, st)
    assert rc == fd.FD_ERR_INVALID_ARG
    assert "64 MiB" in fd.fd_status_string(fd.FD_ERR_TOO_LARGE)


def test_captured_noalloc_replays_match_eager(torch):
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=3, Lmax=3000, varlen=(1, 3000))
    seqlens = np.array([3000, 1234, 17], np.int32)
    q, k, v, sl, _, _ = upload_full(w, None, seqlens=seqlens)
    out_g = torch.empty_like(q)
    lse_g = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    fd.fd_decode_noalloc(q, k, v, sl, w.scale, out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_decode_noalloc(q, k, v, sl, w.scale, out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    for rep in range(3):
        _note(f"graph replay {rep}")
        q.mul_(-1.0 if rep % 2 else 1.5)
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = fd.fd_decode_noalloc(q, k, v, sl, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16))
        assert torch.equal(lse_g, lse_e)
