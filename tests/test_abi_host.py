"""libfd.so on the host: it loads, exports what fd.h declares, validates
arguments before touching the device, and plans as documented.  No GPU is
needed (nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import _binding as bnd
from long_context_decode_fd_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bnd.LIB_PATH):
        pytest.fail("libfd.so is not built; run __graft_entry__.build()")
    return bnd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fd_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    assert names == sorted(["fd_decode", "fd_decode_ex", "fd_plan",
                            "fd_workspace_bytes", "fd_status_string",
                            "fd_version", "fd_decode_partials",
                            "fd_merge_partials", "fd_decode_paged",
                            "fd_decode_multiquery", "fd_plan_ex",
                            "fd_decode_unified_max"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in bnd.SIGNATURES


def test_status_strings_and_version(lib):
    for code in (fd.FD_OK, fd.FD_ERR_INVALID_ARG, fd.FD_ERR_UNSUPPORTED,
                 fd.FD_ERR_WORKSPACE, fd.FD_ERR_HIP):
        s = fd.fd_status_string(code)
        assert s and s != "unknown status"
    assert fd.fd_status_string(12345) == "unknown status"
    assert fd.fd_version() == 10000


# Fake, never dereferenced device addresses: every call below must be
# rejected by host-side checks before anything reaches HIP.
A = 1 << 20


def call_ex(lib, q=A, k=A, v=A, seqlens=None, B=1, Hq=8, Hkv=8, D=128,
            Lmax=64, scale=0.1, dtype=0, out=A, lse=A, num_splits=0,
            variant=0, flags=0, ws=None, ws_bytes=0):
    return lib.fd_decode_ex(q, k, v, seqlens, B, Hq, Hkv, D, Lmax, scale,
                            dtype, out, lse, num_splits, variant, flags, ws,
                            ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fd.FD_ERR_INVALID_ARG),
    (dict(k=None), fd.FD_ERR_INVALID_ARG),
    (dict(v=None), fd.FD_ERR_INVALID_ARG),
    (dict(out=None), fd.FD_ERR_INVALID_ARG),
    (dict(lse=None), fd.FD_ERR_INVALID_ARG),
    (dict(q=A + 8), fd.FD_ERR_INVALID_ARG),
    (dict(k=A + 2), fd.FD_ERR_INVALID_ARG),
    (dict(out=A + 4), fd.FD_ERR_INVALID_ARG),
    (dict(lse=A + 2), fd.FD_ERR_INVALID_ARG),
    (dict(seqlens=A + 1), fd.FD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fd.FD_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fd.FD_ERR_INVALID_ARG),
    (dict(B=0), fd.FD_ERR_INVALID_ARG),
    (dict(Hq=0), fd.FD_ERR_INVALID_ARG),
    (dict(Hkv=-1), fd.FD_ERR_INVALID_ARG),
    (dict(Lmax=0), fd.FD_ERR_INVALID_ARG),
    (dict(Hq=12, Hkv=8), fd.FD_ERR_INVALID_ARG),
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(D=256), fd.FD_ERR_UNSUPPORTED),
    (dict(dtype=7), fd.FD_ERR_UNSUPPORTED),
    (dict(Hq=64, Hkv=2), fd.FD_ERR_UNSUPPORTED),
    (dict(Lmax=(1 << 30) + 1), fd.FD_ERR_UNSUPPORTED),   # above 2^30 keys
    (dict(Lmax=2**31 - 1), fd.FD_ERR_UNSUPPORTED),
    (dict(num_splits=-1), fd.FD_ERR_INVALID_ARG),
    (dict(variant=3), fd.FD_ERR_INVALID_ARG),
    (dict(variant=-1), fd.FD_ERR_INVALID_ARG),
    (dict(flags=4), fd.FD_ERR_INVALID_ARG),     # unified max needs phi
    (dict(flags=8), fd.FD_ERR_INVALID_ARG),
    (dict(flags=-1), fd.FD_ERR_INVALID_ARG),
    (dict(ws=None, ws_bytes=64), fd.FD_ERR_INVALID_ARG),
    (dict(ws=A + 16, ws_bytes=1 << 20), fd.FD_ERR_INVALID_ARG),
])
def test_invalid_arguments_rejected_on_host(lib, kw, code):
    assert call_ex(lib, **kw) == code


def test_fd_decode_rejects_like_ex(lib):
    rc = lib.fd_decode(None, A, A, None, 1, 8, 8, 128, 64, 0.1, 0, A, A,
                       None)
    assert rc == fd.FD_ERR_INVALID_ARG
    rc = lib.fd_decode(A, A, A, None, 1, 8, 8, 80, 64, 0.1, 0, A, A, None)
    assert rc == fd.FD_ERR_UNSUPPORTED


def test_phase_calls_reject_on_host(lib):
    P = lib.fd_decode_partials
    M = lib.fd_merge_partials
    ok = dict(B=1, Hq=8, Hkv=8, D=128, Lmax=64)
    # chunk phase: needs q/k/v and a caller workspace, no fused merge
    assert P(None, A, A, None, 1, 8, 8, 128, 64, 0.1, 0, 0, 0, 0, A, 4096,
             None) == fd.FD_ERR_INVALID_ARG
    assert P(A, A, A, None, 1, 8, 8, 128, 64, 0.1, 0, 0, 0, 0, None, 0,
             None) == fd.FD_ERR_INVALID_ARG
    assert P(A, A, A, None, 1, 8, 8, 128, 64, float("nan"), 0, 0, 0, 0, A,
             4096, None) == fd.FD_ERR_INVALID_ARG
    assert P(A, A, A, None, 1, 8, 8, 96, 64, 0.1, 0, 0, 0, 0, A, 4096,
             None) == fd.FD_ERR_UNSUPPORTED
    # merge phase: needs out/lse and the workspace
    assert M(None, 1, 8, 8, 128, 64, 0, 0, 0, 0, A, 4096, None, A,
             None) == fd.FD_ERR_INVALID_ARG
    assert M(None, 1, 8, 8, 128, 64, 0, 0, 0, 0, None, 0, A, A,
             None) == fd.FD_ERR_INVALID_ARG
    assert M(None, 1, 8, 8, 128, 64, 0, 0, 0, 4, A, 4096, A, A,
             None) == fd.FD_ERR_INVALID_ARG
    assert ok


def test_partials_flag_plans_partials_for_one_chunk(lib):
    p = fd.fd_plan(64, 32, 8, 128, 4096, "bf16", num_cus=256)
    assert p["combine"] == 0 and p["workspace_bytes"] == 0
    p = fd.fd_plan(64, 32, 8, 128, 4096, "bf16", num_cus=256,
                   flags=fd.FD_FLAG_PARTIALS)
    assert p["combine"] == 1 and p["num_splits"] == 1
    rows = 64 * 32
    assert p["o_part_offset"] == 0
    assert p["lse_part_offset"] == rows * 128 * 4
    assert p["workspace_bytes"] == rows * 128 * 4 + rows * 4


def plan(w, varlen=None, **kw):
    return fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                      varlen=(w.varlen is not None) if varlen is None
                      else varlen, num_cus=256, **kw)


def test_plans_for_the_five_workloads_on_256_cus(lib):
    W = wl.WORKLOADS
    # batch 1, 64k, 8 KV heads: 8 units -> 32 chunks of 2048 keys, one
    # workgroup per CU
    p = plan(W["b1_gqa8_h64_d128_l65536"])
    assert (p["num_splits"], p["chunk"], p["grid"], p["combine"]) == \
        (32, 2048, 256, 1)
    assert p["variant"] == fd.FD_VARIANT_MFMA
    assert p["merge"] == fd.FD_MERGE_SEPARATE and p["ticket_bytes"] == 0
    assert p["workspace_bytes"] == 64 * 32 * 128 * 4 + 64 * 32 * 4
    p = plan(W["b1_gqa8_h64_d128_l65536"], flags=fd.FD_FLAG_FUSED_MERGE)
    assert p["merge"] == fd.FD_MERGE_FUSED
    assert p["ticket_bytes"] == 256          # 8 int32 tickets, aligned
    assert p["workspace_bytes"] == 256 + 64 * 32 * 128 * 4 + 64 * 32 * 4
    # 4 x 32 MHA heads at 32k: 128 units -> 2 chunks of 16384
    p = plan(W["b4_mha_h32_d128_l32768_peaked"])
    assert (p["num_splits"], p["chunk"], p["grid"]) == (2, 16384, 256)
    # 64 x 8 units already fill the chip: no split, no merge, no workspace
    p = plan(W["b64_gqa4_h32_d128_l4096"])
    assert (p["num_splits"], p["combine"], p["workspace_bytes"]) == (1, 0, 0)
    assert p["merge"] == fd.FD_MERGE_NONE
    assert p["grid"] == 512
    # var-len: balance-sized chunks over the padded length
    p = plan(W["varlen_b16_gqa8_h64_d128_lmax131072"])
    # (the work list's upper bound 16 * 8 * 64, halved: two chunks per
    # workgroup)
    assert (p["chunk"], p["num_splits"], p["grid"]) == (2048, 64, 16 * 8 * 32)
    # fp32 runs on the vector ALU
    p = plan(W["tiny_mha_f32_b1_h8_d64_l1024"])
    assert p["variant"] == fd.FD_VARIANT_VALU and p["chunk"] % 32 == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("varlen", [False, True])
def test_short_caches_take_one_launch(lib, dtype, varlen):
    # Up to 512 keys (twice the 256-key minimum chunk) the planner keeps one
    # chunk per sequence: no partials, no merge pass.  One key more and the
    # usual split applies.
    for L in (32, 300, 512):
        p = fd.fd_plan(1, 8, 8, 128, L, dtype, varlen=varlen, num_cus=256)
        assert (p["num_splits"], p["combine"], p["workspace_bytes"]) == \
            (1, 0, 0), (L, p)
    p = fd.fd_plan(1, 8, 8, 128, 513, dtype, varlen=varlen, num_cus=256)
    assert (p["num_splits"], p["chunk"], p["combine"]) == (3, 256, 1)
    # a paged table of that capacity plans the same way
    if dtype == "bf16":
        p = fd.fd_plan_ex(1, 1, 8, 8, 128, 512, "bf16", varlen=True,
                          paged=True, num_cus=256)
        assert p["num_splits"] == 1 and p["combine"] == 0


@pytest.mark.parametrize("L,S", [(1, 1), (31, 1), (33, 2), (1000, 7),
                                 (65536, 64), (65536, 5000), (100, 100)])
def test_forced_splits_cover_the_sequence(lib, L, S):
    p = fd.fd_plan(1, 8, 8, 128, L, "bf16", num_splits=S, num_cus=256)
    C, n = p["chunk"], p["num_splits"]
    assert C % 32 == 0 and C * n >= L and C * (n - 1) < L
    assert n <= max(1, -(-L // 32))
    assert p["combine"] == (n > 1)


def test_plan_rejections(lib):
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 8, 8, 128, 64, "f32", variant=fd.FD_VARIANT_MFMA,
                   num_cus=256)
    with pytest.raises(fd.FdError):        # bf16 vector path: G <= 4
        fd.fd_plan(1, 64, 8, 128, 64, "bf16", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 8, 8, 128, 64, "bf16", flags=8, num_cus=256)
    assert plan(wl.WORKLOADS["b1_gqa8_h64_d128_l65536"],
                num_splits=1)["workspace_bytes"] == 0


def test_plan_scales_with_cu_count(lib):
    w = wl.WORKLOADS["b1_gqa8_h64_d128_l65536"]
    p104 = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", num_cus=104)
    p256 = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", num_cus=256)
    assert p104["num_splits"] < p256["num_splits"]


def test_binding_marshals_nothing_but_pointers():
    # The binding's table must match the header one-to-one.
    assert set(bnd.SIGNATURES) == set(declared_functions())
    for name, (res, args) in bnd.SIGNATURES.items():
        for a in args:
            assert a in (ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                         ctypes.c_size_t) or hasattr(a, "_type_"), name


def test_binding_rejects_tensors_on_another_device():
    torch = pytest.importorskip("torch")
    here = torch.empty(2)
    bnd._same_device(here.device, a=here, b=None)
    with pytest.raises(ValueError, match="b is on meta"):
        bnd._same_device(here.device, a=here, b=torch.empty(2, device="meta"))


def test_binding_rejects_outputs_that_overlap():
    torch = pytest.importorskip("torch")
    buf = torch.zeros(64)
    q, out = buf[:32], buf[16:48]
    bnd._no_overlap(dict(out=buf[32:48], lse=buf[48:]), dict(q=q, s=None))
    with pytest.raises(ValueError, match="out overlaps q"):
        bnd._no_overlap(dict(out=out), dict(q=q))
    with pytest.raises(ValueError, match="out overlaps lse"):
        bnd._no_overlap(dict(out=buf[:8], lse=buf[7:9]), {})
    # touching ends do not overlap; empty tensors never do
    bnd._no_overlap(dict(out=buf[8:16], lse=buf[16:16]), dict(q=buf[:8]))


def call_paged(lib, q=A, k=A, v=A, bt=A, max_pages=4, page_size=32,
               num_pages=8, layout=0, seqlens=A, B=1, Tq=1, Hq=8, Hkv=8,
               D=128, scale=0.1, dtype=0, out=A, lse=A, num_splits=0,
               flags=0):
    return lib.fd_decode_paged(q, k, v, bt, max_pages, page_size, num_pages,
                               layout, seqlens, B, Tq, Hq, Hkv, D, scale,
                               dtype, out, lse, num_splits, flags, None)


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), fd.FD_ERR_INVALID_ARG),
    (dict(bt=A + 2), fd.FD_ERR_INVALID_ARG),
    (dict(seqlens=None), fd.FD_ERR_INVALID_ARG),   # required when paged
    (dict(max_pages=0), fd.FD_ERR_INVALID_ARG),
    (dict(page_size=0), fd.FD_ERR_INVALID_ARG),
    (dict(num_pages=-1), fd.FD_ERR_INVALID_ARG),
    (dict(page_size=24), fd.FD_ERR_UNSUPPORTED),   # not a multiple of 16
    (dict(page_size=8), fd.FD_ERR_UNSUPPORTED),
    (dict(max_pages=1 << 26, page_size=64), fd.FD_ERR_UNSUPPORTED),
    (dict(num_pages=1 << 26, page_size=64), fd.FD_ERR_UNSUPPORTED),
    (dict(num_pages=1 << 22, page_size=64, Hkv=8), fd.FD_ERR_UNSUPPORTED),
    (dict(layout=2), fd.FD_ERR_INVALID_ARG),
    (dict(layout=-1), fd.FD_ERR_INVALID_ARG),
    (dict(layout=1, page_size=8), fd.FD_ERR_UNSUPPORTED),
    (dict(Tq=0), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=3, Hq=48, Hkv=8), fd.FD_ERR_UNSUPPORTED),   # 6 x 3 = 18 rows
    (dict(Tq=17, Hq=8, Hkv=8), fd.FD_ERR_UNSUPPORTED),
    (dict(dtype=1), fd.FD_ERR_UNSUPPORTED),        # bf16 only
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(Hq=64, Hkv=2), fd.FD_ERR_UNSUPPORTED),
    (dict(q=None), fd.FD_ERR_INVALID_ARG),
    (dict(k=A + 8), fd.FD_ERR_INVALID_ARG),
    (dict(lse=None), fd.FD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fd.FD_ERR_INVALID_ARG),
    (dict(flags=4), fd.FD_ERR_INVALID_ARG),
    (dict(flags=8), fd.FD_ERR_INVALID_ARG),
    (dict(num_splits=-2), fd.FD_ERR_INVALID_ARG),
    (dict(B=0), fd.FD_ERR_INVALID_ARG),
])
def test_paged_arguments_rejected_on_host(lib, kw, code):
    assert call_paged(lib, **kw) == code


def call_mq(lib, q=A, k=A, v=A, seqlens=None, B=1, Tq=2, Hq=8, Hkv=8,
            D=128, Lmax=64, scale=0.1, dtype=0, out=A, lse=A, num_splits=0,
            flags=0):
    return lib.fd_decode_multiquery(q, k, v, seqlens, B, Tq, Hq, Hkv, D, Lmax,
                                    scale, dtype, out, lse, num_splits, flags,
                                    None)


@pytest.mark.parametrize("kw,code", [
    (dict(Tq=0), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=-3), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=17, Hq=8, Hkv=8), fd.FD_ERR_UNSUPPORTED),   # 17 columns
    (dict(Tq=5, Hq=32, Hkv=8), fd.FD_ERR_UNSUPPORTED),   # 4 x 5 = 20
    (dict(Tq=2, Hq=64, Hkv=4), fd.FD_ERR_UNSUPPORTED),   # G alone is 16
    (dict(dtype=1), fd.FD_ERR_UNSUPPORTED),
    (dict(Tq=1, dtype=1), fd.FD_ERR_UNSUPPORTED),
    (dict(B=1 << 20, Tq=16, Hq=128, Hkv=128), fd.FD_ERR_UNSUPPORTED),
    (dict(q=None), fd.FD_ERR_INVALID_ARG),
    (dict(seqlens=A + 1), fd.FD_ERR_INVALID_ARG),
    (dict(D=80), fd.FD_ERR_UNSUPPORTED),
    (dict(Lmax=0), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=1, flags=4), fd.FD_ERR_INVALID_ARG),   # unified max: own call
])
def test_multiquery_arguments_rejected_on_host(lib, kw, code):
    assert call_mq(lib, **kw) == code


def test_plan_ex_for_several_tokens_and_pages(lib):
    w = wl.WORKLOADS["b1_gqa8_h64_d128_l65536"]
    base = plan(w)
    # one token: identical to fd_plan
    p1 = fd.fd_plan_ex(w.B, 1, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", num_cus=256)
    assert p1 == base
    # Tq tokens: same chunks and grid, Tq times the partial rows
    p2 = fd.fd_plan_ex(w.B, 2, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", num_cus=256)
    assert (p2["num_splits"], p2["chunk"], p2["grid"]) == \
        (base["num_splits"], base["chunk"], base["grid"])
    rows = w.B * 2 * w.Hq * p2["num_splits"]
    assert p2["lse_part_offset"] == rows * w.D * 4
    assert p2["workspace_bytes"] == rows * w.D * 4 + rows * 4
    # paged: per-sequence lengths are implied; the even split (here 2048
    # keys, equal to the var-len cap) still applies when it is finer
    pp = fd.fd_plan_ex(w.B, 1, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", paged=True,
                       num_cus=256)
    assert (pp["chunk"], pp["num_splits"]) == (2048, 32)
    pp = fd.fd_plan_ex(w.B, 1, w.Hq, w.Hkv, w.D, 32768, "bf16", paged=True,
                       num_cus=256)
    assert (pp["chunk"], pp["num_splits"]) == (1024, 32)
    pv = fd.fd_plan_ex(16, 1, 64, 8, 128, 131072, "bf16", paged=True,
                       num_cus=256)
    assert pv["chunk"] == 2048
    for kw in (dict(Tq=3, Hq=64, Hkv=8), dict(Tq=2, dtype="f32"),
               dict(Tq=1, dtype="f32", paged=True),
               dict(Tq=2, variant=fd.FD_VARIANT_VALU), dict(Tq=0)):
        args = dict(B=1, Tq=1, Hq=8, Hkv=8, D=128, Lmax=4096, dtype="bf16",
                    num_cus=256)
        args.update(kw)
        with pytest.raises(fd.FdError):
            fd.fd_plan_ex(**args)


def call_uni(lib, q=A, k=A, v=A, seqlens=None, B=1, Hq=8, Hkv=8, D=128,
             Lmax=64, scale=0.1, dtype=0, out=A, lse=A, phi=0.0,
             num_splits=0, flags=0, ws=None, ws_bytes=0):
    return lib.fd_decode_unified_max(q, k, v, seqlens, B, Hq, Hkv, D, Lmax,
                                     scale, dtype, out, lse, phi, num_splits,
                                     flags, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(phi=float("nan")), fd.FD_ERR_INVALID_ARG),
    (dict(phi=float("inf")), fd.FD_ERR_INVALID_ARG),
    (dict(phi=-float("inf")), fd.FD_ERR_INVALID_ARG),
    (dict(dtype=1), fd.FD_ERR_UNSUPPORTED),          # bf16 only
    (dict(q=None), fd.FD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fd.FD_ERR_INVALID_ARG),
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(flags=2 | 8), fd.FD_ERR_INVALID_ARG),
    (dict(num_splits=-1), fd.FD_ERR_INVALID_ARG),
    (dict(ws=A + 8, ws_bytes=4096), fd.FD_ERR_INVALID_ARG),
])
def test_unified_max_arguments_rejected_on_host(lib, kw, code):
    assert call_uni(lib, **kw) == code


def test_unified_max_plans_like_the_exact_pass(lib):
    w = wl.WORKLOADS["b1_gqa8_h64_d128_l65536"]
    base = plan(w)
    uni = plan(w, flags=fd.FD_FLAG_UNIFIED_MAX)
    assert uni == base
    with pytest.raises(fd.FdError):
        plan(wl.WORKLOADS["tiny_mha_f32_b1_h8_d64_l1024"],
             flags=fd.FD_FLAG_UNIFIED_MAX)
    with pytest.raises(fd.FdError):
        fd.fd_plan_ex(1, 2, 8, 8, 128, 4096, "bf16",
                      flags=fd.FD_FLAG_UNIFIED_MAX, num_cus=256)
    with pytest.raises(fd.FdError):
        fd.fd_plan_ex(1, 1, 8, 8, 128, 4096, "bf16", paged=True,
                      flags=fd.FD_FLAG_UNIFIED_MAX, num_cus=256)
