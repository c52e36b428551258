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
                            "fd_decode_unified_max", "fd_decode_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in bnd.SIGNATURES


def test_library_exports_nothing_else(lib):
    """The dynamic symbol table holds the header's functions and nothing of
    the library's internals (planner, launch code, C++ helpers)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    res = subprocess.run([nm, "-D", "--defined-only", bnd.LIB_PATH],
                         check=True, capture_output=True, text=True)
    exported = sorted(line.split()[-1] for line in res.stdout.splitlines()
                      if line.strip())
    assert exported == declared_functions()


def test_status_strings_and_version(lib):
    for code in (fd.FD_OK, fd.FD_ERR_INVALID_ARG, fd.FD_ERR_UNSUPPORTED,
                 fd.FD_ERR_WORKSPACE, fd.FD_ERR_HIP, fd.FD_ERR_CAPTURE,
                 fd.FD_ERR_TOO_LARGE):
        s = fd.fd_status_string(code)
        assert s and s != "unknown status"
    assert fd.fd_status_string(12345) == "unknown status"
    assert fd.fd_version() == 20200


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
    (dict(D=512), fd.FD_ERR_UNSUPPORTED),
    (dict(dtype=7), fd.FD_ERR_UNSUPPORTED),
    (dict(Hq=258, Hkv=2), fd.FD_ERR_UNSUPPORTED),    # 129 heads per KV head
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
    # fp32 runs on the vector ALU: the tiny decode (8 units) splits 1024
    # keys into 32 one-tile chunks (measured 6.8 us against 7.0 in 16
    # chunks of 64 keys)
    p = plan(W["tiny_mha_f32_b1_h8_d64_l1024"])
    assert p["variant"] == fd.FD_VARIANT_VALU
    assert (p["chunk"], p["num_splits"], p["grid"]) == (32, 32, 256)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("varlen", [False, True])
def test_short_caches_take_one_launch(lib, dtype, varlen):
    # The planner splits only when a split takes more than 64 KB of K (256
    # bf16 rows of D = 128, 128 fp32 ones) off each workgroup's share.
    # With 8 units (batch 1, 8 KV heads) the matrix cores (bf16) take
    # one-tile chunks of 32 keys, so up to 288 keys stay in one chunk per
    # sequence, with no partials and no merge pass, and one key more is cut
    # into 32-key chunks; the vector ALU (fp32) decides on 64-key chunks,
    # so its bound is 192 keys, and then cuts one-tile chunks too.
    one = 288 if dtype == "bf16" else 192
    for L in (32, 150, one):
        p = fd.fd_plan(1, 8, 8, 128, L, dtype, varlen=varlen, num_cus=256)
        assert (p["num_splits"], p["combine"], p["workspace_bytes"]) == \
            (1, 0, 0), (L, p)
    p = fd.fd_plan(1, 8, 8, 128, one + 1, dtype, varlen=varlen, num_cus=256)
    assert (p["num_splits"], p["chunk"], p["combine"]) == \
        ((10, 32, 1) if dtype == "bf16" else (7, 32, 1))
    # a paged table of that capacity plans the same way
    if dtype == "bf16":
        p = fd.fd_plan_ex(1, 1, 8, 8, 128, 288, "bf16", varlen=True,
                          paged=True, num_cus=256)
        assert p["num_splits"] == 1 and p["combine"] == 0
        p = fd.fd_plan_ex(1, 1, 8, 8, 128, 289, "bf16", varlen=True,
                          paged=True, num_cus=256)
        assert (p["num_splits"], p["chunk"]) == (10, 32)


def test_head_dim_64_counts_the_split_gain_in_bytes(lib):
    # D = 64 rows are half as long: up to 512 keys (minus a chunk) stay in
    # one launch (measured, batch 1, 64 query / 8 KV heads, 384 keys: 5.8
    # us unsplit against 6.9 in six chunks); beyond, one-tile chunks.
    for L in (384, 544):
        p = fd.fd_plan(1, 64, 8, 64, L, "bf16", num_cus=256)
        assert p["num_splits"] == 1, (L, p)
    p = fd.fd_plan(1, 64, 8, 64, 640, "bf16", num_cus=256)
    assert (p["num_splits"], p["chunk"]) == (20, 32)


@pytest.mark.parametrize("B,Hq,Hkv,L,S", [
    # measured fastest or within 7% of it (device time, MI355X)
    (1, 64, 8, 1024, 32), (1, 64, 8, 4096, 32), (1, 64, 8, 65536, 32),
    (1, 64, 8, 512, 16), (2, 64, 8, 512, 16), (1, 64, 8, 1280, 20),
    (2, 64, 8, 640, 10), (1, 16, 2, 2048, 32),
    (2, 64, 8, 2048, 16), (4, 64, 8, 512, 8), (8, 32, 8, 512, 4),
    (16, 32, 8, 512, 1), (16, 32, 8, 768, 2), (4, 32, 32, 512, 1),
    (4, 32, 32, 32768, 2), (64, 32, 8, 4096, 1)])
def test_split_counts_follow_the_measured_rule(lib, B, Hq, Hkv, L, S):
    p = fd.fd_plan(B, Hq, Hkv, 128, L, "bf16", num_cus=256)
    assert p["num_splits"] == S, p


@pytest.mark.parametrize("B,L,S", [(1, 1024, 32), (1, 4096, 64),
                                   (4, 1024, 16), (4, 4096, 16),
                                   (1, 256, 1), (1, 320, 1), (1, 2048, 32),
                                   (1, 16384, 64)])
def test_fp32_plans_for_two_workgroups_per_cu(lib, B, L, S):
    # the vector-ALU kernel: two workgroups per CU; one-tile chunks up to 32
    # per sequence, 64-key ones beyond (measured fastest or within 5% of
    # it, 8 heads, D = 64)
    p = fd.fd_plan(B, 8, 8, 64, L, "f32", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_VALU
    assert p["num_splits"] == S, p


@pytest.mark.parametrize("Hq,Hkv,D,L,S", [(16, 1, 64, 256, 8),
                                          (16, 1, 64, 2048, 64),
                                          (16, 4, 128, 2048, 64),
                                          (8, 8, 128, 256, 8)])
def test_fp32_groups_split_sooner(lib, Hq, Hkv, D, L, S):
    # G dot products per key on the vector ALU: the split gain shrinks with
    # G and, from G = 4 on, one-tile chunks pay at any length that fits one
    # round (measured: 16 heads on one KV head, D = 64, 256 keys 53 us
    # unsplit against 17 in 8 chunks; 4 on each of 4, D = 128, 2048 keys
    # 12.6 in 32 chunks against 10.6 in 64)
    B = 2 if Hq == 8 else 1
    p = fd.fd_plan(B, Hq, Hkv, D, L, "f32", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_VALU
    assert (p["num_splits"], p["chunk"]) == (S, 32), p


@pytest.mark.parametrize("Hq,Hkv,D,L,S,C", [(8, 1, 128, 16384, 256, 64),
                                            (8, 1, 128, 65536, 512, 128),
                                            (16, 4, 128, 16384, 128, 128),
                                            (16, 1, 64, 65536, 256, 256)])
def test_fp32_long_caches_keep_chunks_of_64_keys_or_more(lib, Hq, Hkv, D, L,
                                                         S, C):
    # measured fastest (fp32, one sequence): past 64 tiles the split count
    # follows two workgroups per CU and chunks stay at 64 keys or more
    p = fd.fd_plan(1, Hq, Hkv, D, L, "f32", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    assert (p["num_splits"], p["chunk"]) == (S, C), p


def test_fp32_groups_past_8_heads_run_as_half_groups(lib):
    # 16 query heads on one KV head: two virtual groups of 8 on the same
    # slab, so the plan counts two units (grid = 2 * S)
    valu = fd.FD_VARIANT_VALU
    p = fd.fd_plan(1, 16, 1, 64, 65536, "f32", variant=valu, num_cus=256)
    assert p["grid"] == 2 * p["num_splits"]
    # odd groups past 8 keep one 16-row group
    p = fd.fd_plan(1, 9, 1, 64, 65536, "f32", variant=valu, num_cus=256)
    assert p["grid"] == p["num_splits"]


@pytest.mark.parametrize("L,S", [(1, 1), (31, 1), (33, 2), (1000, 7),
                                 (65536, 64), (65536, 5000), (100, 100)])
def test_forced_splits_cover_the_sequence(lib, L, S):
    p = fd.fd_plan(1, 8, 8, 128, L, "bf16", num_splits=S, num_cus=256)
    C, n = p["chunk"], p["num_splits"]
    assert C % 32 == 0 and C * n >= L and C * (n - 1) < L
    assert n <= max(1, -(-L // 32))
    assert p["combine"] == (n > 1)


def test_plan_rejections(lib):
    with pytest.raises(fd.FdError):  # paged / several tokens: matrix cores
        fd.fd_plan_ex(1, 1, 8, 8, 128, 64, "f32", paged=True,
                      variant=fd.FD_VARIANT_VALU, num_cus=256)
    with pytest.raises(fd.FdError):
        fd.fd_plan_ex(1, 2, 8, 8, 128, 64, "f32",
                      variant=fd.FD_VARIANT_VALU, num_cus=256)
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 8, 8, 128, 64, "f32", variant=fd.FD_VARIANT_MFMA,
                   flags=fd.FD_FLAG_UNIFIED_MAX, num_cus=256)
    with pytest.raises(fd.FdError):        # 16-bit vector path: G <= 4
        fd.fd_plan(1, 64, 8, 128, 64, "bf16", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 8, 8, 128, 64, "bf16", flags=8, num_cus=256)
    assert plan(wl.WORKLOADS["b1_gqa8_h64_d128_l65536"],
                num_splits=1)["workspace_bytes"] == 0


@pytest.mark.parametrize("B,Hq,Hkv,D,L", [
    (1, 64, 8, 128, 65536), (4, 32, 32, 128, 32768), (64, 32, 8, 128, 4096),
    (1, 8, 8, 64, 1024), (2, 16, 2, 256, 1700), (1, 64, 2, 128, 1500),
    (3, 8, 8, 128, 300)])
@pytest.mark.parametrize("varlen", [False, True])
def test_fp16_plans_like_bf16(lib, B, Hq, Hkv, D, L, varlen):
    # fp16 rows have the bf16 rows' size and run on the same matrix-core
    # pass, so every planner decision is the same.
    pb = fd.fd_plan(B, Hq, Hkv, D, L, "bf16", varlen=varlen, num_cus=256)
    ph = fd.fd_plan(B, Hq, Hkv, D, L, "f16", varlen=varlen, num_cus=256)
    assert ph == pb
    assert fd.fd_workspace_bytes(B, Hq, Hkv, D, L, "f16", varlen=varlen) == \
        fd.fd_workspace_bytes(B, Hq, Hkv, D, L, "bf16", varlen=varlen)


def test_fp16_entry_point_rules(lib):
    # unified maximum: bf16 and fp16, never fp32
    fd.fd_plan(1, 8, 8, 128, 4096, "f16", flags=fd.FD_FLAG_UNIFIED_MAX,
               num_cus=256)
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 8, 8, 128, 4096, "f32", flags=fd.FD_FLAG_UNIFIED_MAX,
                   num_cus=256)
    # the 16-bit vector-ALU pass takes groups of at most 4 query heads
    p = fd.fd_plan(1, 32, 8, 128, 4096, "f16", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_VALU
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 64, 8, 128, 64, "f16", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    # paged and several-token plans accept fp16
    p = fd.fd_plan_ex(1, 2, 8, 8, 128, 4096, "f16", paged=True, num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_MFMA


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
               flags=0, ws=None, ws_bytes=0):
    return lib.fd_decode_paged(q, k, v, bt, max_pages, page_size, num_pages,
                               layout, seqlens, B, Tq, Hq, Hkv, D, scale,
                               dtype, out, lse, num_splits, flags, ws,
                               ws_bytes, None)


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
    # products that would overflow a signed 64-bit long are refused too
    (dict(num_pages=(1 << 31) - 1, page_size=(1 << 30) + 16 * 4,
          Hkv=1 << 29, Hq=1 << 29), fd.FD_ERR_UNSUPPORTED),
    (dict(max_pages=(1 << 31) - 1, page_size=(1 << 31) - 16),
     fd.FD_ERR_UNSUPPORTED),
    (dict(Hkv=0), fd.FD_ERR_INVALID_ARG),
    (dict(Hkv=-8), fd.FD_ERR_INVALID_ARG),
    (dict(ws=None, ws_bytes=256), fd.FD_ERR_INVALID_ARG),
    (dict(ws=A + 16, ws_bytes=1 << 20), fd.FD_ERR_INVALID_ARG),  # alignment
    (dict(layout=2), fd.FD_ERR_INVALID_ARG),
    (dict(layout=-1), fd.FD_ERR_INVALID_ARG),
    (dict(layout=1, page_size=8), fd.FD_ERR_UNSUPPORTED),
    (dict(Tq=0), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=3, Hq=1032, Hkv=8), fd.FD_ERR_UNSUPPORTED),  # 129 per KV head
    (dict(Tq=17, Hq=8, Hkv=8), fd.FD_ERR_UNSUPPORTED),
    (dict(dtype=3), fd.FD_ERR_UNSUPPORTED),        # bf16, fp32 or fp16
    (dict(dtype=1, Tq=3, Hq=1032, Hkv=8), fd.FD_ERR_UNSUPPORTED),
    (dict(D=96), fd.FD_ERR_UNSUPPORTED),
    (dict(Hq=258, Hkv=2), fd.FD_ERR_UNSUPPORTED),    # 129 heads per KV head
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
            flags=0, ws=None, ws_bytes=0):
    return lib.fd_decode_multiquery(q, k, v, seqlens, B, Tq, Hq, Hkv, D, Lmax,
                                    scale, dtype, out, lse, num_splits, flags,
                                    ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Tq=0), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=-3), fd.FD_ERR_INVALID_ARG),
    (dict(Tq=17, Hq=8, Hkv=8), fd.FD_ERR_UNSUPPORTED),   # 17 columns
    (dict(Tq=17, Hq=16, Hkv=8), fd.FD_ERR_UNSUPPORTED),  # no split fits
    (dict(Tq=2, Hq=1032, Hkv=8), fd.FD_ERR_UNSUPPORTED),  # 129 per KV head
    (dict(dtype=3), fd.FD_ERR_UNSUPPORTED),
    (dict(Tq=1, dtype=-1), fd.FD_ERR_UNSUPPORTED),
    (dict(Tq=17, Hq=32, Hkv=8, dtype=1), fd.FD_ERR_UNSUPPORTED),
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
    for kw in (dict(Tq=17, Hq=64, Hkv=8), dict(Tq=17, Hq=64, Hkv=8, dtype="f32"),
               dict(Tq=2, Hq=1032, Hkv=8),
               dict(Tq=2, dtype="f32", variant=fd.FD_VARIANT_VALU),
               dict(Tq=1, dtype="f32", paged=True,
                    variant=fd.FD_VARIANT_VALU),
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
    (dict(dtype=1), fd.FD_ERR_UNSUPPORTED),          # 16-bit only
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


@pytest.mark.parametrize("name,layout", [
    ("b1_gqa8_h64_d128_l65536", fd.FD_PARTIALS_ROW_MAJOR),
    ("b4_mha_h32_d128_l32768_peaked", fd.FD_PARTIALS_ROW_MAJOR),
    ("varlen_b16_gqa8_h64_d128_lmax131072", fd.FD_PARTIALS_CHUNK_MAJOR),
])
def test_partial_layout_follows_the_rounds_of_workgroups(lib, name, layout):
    """Plans whose chunks run in several rounds of workgroups keep each
    chunk's partial rows together; one-round plans keep each query row's
    chunks together.  Same workspace size either way."""
    w = wl.WORKLOADS[name]
    p = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                   varlen=w.varlen is not None, num_cus=256)
    assert p["partial_layout"] == layout
    assert (p["grid"] > 256) == (layout == fd.FD_PARTIALS_CHUNK_MAJOR)
    rows = w.B * w.Hq * p["num_splits"]
    assert p["lse_part_offset"] - p["o_part_offset"] >= rows * w.D * 4
    # one chunk per sequence: no partials, and the layout field says row
    one = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype, num_splits=1,
                     num_cus=256)
    assert not one["combine"] and \
        one["partial_layout"] == fd.FD_PARTIALS_ROW_MAJOR


@pytest.mark.parametrize("G", [1, 5, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_fp32_matrix_core_plans(lib, G, D):
    # fp32 on the matrix cores: the whole group in one q-tile (no half
    # groups), four wavefronts, the matrix-core split rule
    p = fd.fd_plan(2, 2 * G, 2, D, 4096, "f32", variant=fd.FD_VARIANT_MFMA,
                   num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_MFMA
    assert p["waves_per_block"] == 4
    assert p["grid"] == 2 * 2 * p["num_splits"]
    if D == 64:
        # rows of 256 bytes, as bf16 at D = 128: the same chunks
        pb = fd.fd_plan(2, 2 * G, 2, 128, 4096, "bf16", num_cus=256)
        assert (p["num_splits"], p["chunk"]) == (pb["num_splits"],
                                                 pb["chunk"])


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 8, 9, 16])
@pytest.mark.parametrize("D,L", [(128, 1024), (128, 16384), (64, 1024),
                                 (64, 2048), (64, 4096), (64, 65536)])
def test_fp32_variant_follows_the_measured_rule(lib, G, D, L):
    # fp32 on the matrix cores from G = 3, and at D = 64 from 4096 keys at
    # any G; the vector ALU otherwise (measured, one sequence on 8 KV heads:
    # D = 128, 16k keys, G = 2 26.7 against 28.6 us, G = 3 30.5 against
    # 28.7; D = 64, G = 1, 1024 keys 6.6 against 7.2, 4096 keys 8.8 against
    # 8.7)
    p = fd.fd_plan(1, 8 * G, 8, D, L, "f32", num_cus=256)
    mfma = G >= 3 or (D == 64 and L >= 4096)
    assert p["variant"] == (fd.FD_VARIANT_MFMA if mfma
                            else fd.FD_VARIANT_VALU)
    if mfma:
        # the matrix-core rule: one workgroup per CU
        assert p["waves_per_block"] == 4 and p["grid"] <= 256


@pytest.mark.parametrize("Tq,paged", [(2, False), (1, True), (4, True)])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_fp32_paged_and_several_tokens_take_the_matrix_cores(lib, Tq, paged,
                                                             G):
    # the vector-ALU kernel serves neither, so fp32 takes the matrix cores
    # at any group size, like bf16
    p = fd.fd_plan_ex(2, Tq, 4 * G, 4, 128, 4096, "f32", paged=paged,
                      num_cus=256)
    pb = fd.fd_plan_ex(2, Tq, 4 * G, 4, 64, 4096, "bf16", paged=paged,
                       num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_MFMA
    # 512-byte rows count as bf16 rows of D = 256: at most the bf16 chunks
    assert p["chunk"] <= pb["chunk"] or p["num_splits"] >= pb["num_splits"]


@pytest.mark.parametrize("G,Tq,rep", [(17, 1, 17), (24, 1, 2), (32, 1, 2),
                                      (48, 1, 3), (64, 1, 4), (128, 1, 8),
                                      (8, 3, 2), (8, 4, 2), (6, 3, 2),
                                      (16, 2, 2), (4, 16, 4), (64, 2, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_groups_run_as_virtual_kv_heads(lib, G, Tq, rep, dtype):
    # more than 16 query rows per KV head (G * Tq): the fewest equal
    # virtual groups that fit the 16-column q-tile, each its own workgroup
    # on the same K/V slab, so the grid counts rep virtual heads per head
    Hkv, B = 2, 3
    p = fd.fd_plan_ex(B, Tq, G * Hkv, Hkv, 128, 4096, dtype,
                      num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_MFMA
    assert p["grid"] == B * Hkv * rep * p["num_splits"]
    assert (G // rep) * Tq <= 16 and G % rep == 0
    # the partials still hold one row per real query head and token
    if p["combine"]:
        rows = B * Tq * G * Hkv * p["num_splits"]
        assert p["lse_part_offset"] == p["o_part_offset"] + rows * 128 * 4


def test_groups_past_128_heads_are_refused(lib):
    with pytest.raises(fd.FdError):
        fd.fd_plan(1, 129, 1, 128, 4096, "bf16", num_cus=256)
    fd.fd_plan(1, 128, 1, 128, 4096, "bf16", num_cus=256)
    with pytest.raises(fd.FdError):   # the vector ALU takes up to 16
        fd.fd_plan(1, 32, 1, 128, 4096, "f32", variant=fd.FD_VARIANT_VALU,
                   num_cus=256)


@pytest.mark.parametrize("Hq,Hkv,dtype,variant,P", [
    (64, 8, "bf16", fd.FD_VARIANT_AUTO, 8),
    (64, 2, "bf16", fd.FD_VARIANT_AUTO, 16),      # 32 rows: two groups
    (48, 1, "f32", fd.FD_VARIANT_AUTO, 16),
    (16, 1, "f32", fd.FD_VARIANT_VALU, 8),        # vector-ALU halves
    (16, 1, "f32", fd.FD_VARIANT_MFMA, 16)])
def test_partial_group_names_the_chunk_major_rows(lib, Hq, Hkv, dtype,
                                                  variant, P):
    p = fd.fd_plan(4, Hq, Hkv, 128, 65536, dtype, varlen=True,
                   variant=variant, num_cus=256)
    assert p["partial_group"] == P


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 2, 8, 32])
def test_head_dim_256_runs_on_the_matrix_cores(lib, dtype, G):
    # D = 256: the matrix-core kernels only, planned like D = 128 with
    # rows twice as long (512 or 1024 bytes)
    p = fd.fd_plan(2, 4 * G, 4, 256, 8192, dtype, num_cus=256)
    assert p["variant"] == fd.FD_VARIANT_MFMA
    assert p["waves_per_block"] == 4
    with pytest.raises(fd.FdError):
        fd.fd_plan(2, 4 * G, 4, 256, 8192, dtype, variant=fd.FD_VARIANT_VALU,
                   num_cus=256)
    pp = fd.fd_plan_ex(2, 2, 4 * G, 4, 256, 8192, dtype, paged=True,
                       num_cus=256)
    assert pp["variant"] == fd.FD_VARIANT_MFMA
