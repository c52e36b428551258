"""GPU parity of the paged-cache and multi-token entry points.

fd_decode_paged is compared element by element with the oracle's
decode_paged on the same shuffled page pools (NaN in every row a sequence
does not own, spare pages included); fd_decode_multiquery with the oracle's
decode_multiquery.  Sizes span several 32-key tiles, several chunks and a
ragged tail; page sizes 16 .. 256; lengths include 0, 1, a page boundary,
lengths below Tq, and lengths beyond the table's capacity (clamped).  At
the 64k shape the paged call must reproduce the contiguous call bit for bit
(same plan, same rows), and every row is checked against the oracle; so
are the two multi-token workloads at full size.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import out_to_host, to_dev, upload_full
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
    print(f"[paged/mq] {msg}", flush=True)


def _bits(torch, t):
    """The raw bits of a bf16, fp16 or fp32 tensor, for bitwise
    comparisons."""
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def _assert_parity(out, lse, ref_o, ref_l, tag, dtype="bf16"):
    ok_o, rep_o = check_out(out_to_host(out), ref_o, dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref_l)
    _note(f"{tag}: out {rep_o} lse {rep_l}")
    assert ok_o, (tag, rep_o)
    assert ok_l, (tag, rep_l)


# ---------------------------------------------------------------------------
# Paged cache.

def paged_case(torch, w, seqlens, table_fill=None):
    """Host pools and table for workload w (page_size > 0), uploaded."""
    sl = wl.paged_seqlens(w, seqlens)
    q, k, v, _ = _gen_with(w, sl)
    bt = wl.gen_block_table(w)
    kp, vp = wl.scatter_pages(w, k, v, bt, sl)
    if table_fill is not None:
        # entries past each sequence's last page must never be read
        for b in range(w.B):
            used = -(-min(int(sl[b]), w.Lmax) // w.page_size)
            bt[b, used:] = table_fill
    dev = (to_dev(q), to_dev(kp), to_dev(vp),
           torch.from_numpy(bt).to("cuda"),
           torch.from_numpy(sl).to("cuda"))
    return (q, kp, vp, bt, sl), dev


def _gen_with(w, seqlens):
    """gen_all with explicit lengths (rows past them NaN)."""
    q = wl.gen_q(w)
    k = np.empty((w.B, w.Hkv, w.Lmax, w.D), w.np_dtype)
    v = np.empty_like(k)
    for b in range(w.B):
        for g in range(w.Hkv):
            wl.fill_slab(w, b, g, min(max(int(seqlens[b]), 0), w.Lmax),
                         k[b, g], v[b, g])
    return q, k, v, seqlens


PAGED_SHAPES = [
    # (B, Hq, Hkv, D, Lmax, page_size, seqlens)
    (3, 16, 2, 128, 1000, 32, [1000, 517, 33]),
    (3, 16, 2, 128, 1000, 16, [999, 1, 0]),
    (2, 8, 8, 64, 700, 64, [640, 641]),
    (2, 32, 2, 128, 2048, 256, [2048, 1500]),
    (4, 8, 1, 128, 600, 48, [600, 47, 48, 49]),
    (1, 4, 4, 64, 96, 16, [200]),                    # beyond capacity
    (1, 8, 1, 128, 9000, 16, [8999]),     # one chunk: > 32 tiles per wave
    (2, 64, 2, 128, 900, 32, [900, 450]),            # 32 per KV head
    (2, 16, 2, 256, 700, 16, [700, 301]),            # head dim 256
]


@pytest.mark.parametrize("hm", [False, True], ids=["token_major",
                                                   "head_major"])
@pytest.mark.parametrize("shape", PAGED_SHAPES,
                         ids=[f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_D{s[3]}_L{s[4]}"
                              f"_P{s[5]}" for s in PAGED_SHAPES])
@pytest.mark.parametrize("splits,flags", [(0, 0), (1, 0), (5, 0),
                                          (0, fd.FD_FLAG_FUSED_MERGE)])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_matches_oracle(torch, oracle_mod, shape, splits, flags, hm,
                              dtype):
    B, Hq, Hkv, D, L, P, sls = shape
    w = wl.Workload("paged_case", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=L,
                    dtype=dtype, seed=40 + P, page_size=P, head_major=hm)
    seqlens = np.array(sls, np.int32)
    (q, kp, vp, bt, sl), (qd, kd, vd, btd, sld) = paged_case(torch, w,
                                                             seqlens)
    _note(f"{shape} {dtype} hm={hm} splits={splits} flags={flags} "
          f"pages={w.num_pages}")
    out, lse = fd.fd_decode_paged(qd, kd, vd, btd, sld, w.scale,
                                  num_splits=splits, flags=flags,
                                  head_major=hm)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode_paged(q, kp, vp, bt, sl, w.scale,
                                           head_major=hm)
    _assert_parity(out, lse, ref_o, ref_l, f"paged {shape} hm={hm}", dtype)


@pytest.mark.parametrize("hm", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_table_entries_past_the_length_are_not_read(torch, hm, dtype):
    w = wl.Workload("paged_tail", B=3, Hq=16, Hkv=2, D=128, Lmax=1024,
                    dtype=dtype, seed=47, page_size=64, head_major=hm)
    seqlens = np.array([1024, 300, 0], np.int32)
    _, (qd, kd, vd, btd, sld) = paged_case(torch, w, seqlens)
    _, (_, _, _, btd2, _) = paged_case(torch, w, seqlens,
                                       table_fill=w.num_pages + 12345)
    _note("table entries past the length: out of range values")
    o1, l1 = fd.fd_decode_paged(qd, kd, vd, btd, sld, w.scale, head_major=hm)
    o2, l2 = fd.fd_decode_paged(qd, kd, vd, btd2, sld, w.scale,
                                head_major=hm)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch, o1), _bits(torch, o2))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("hm", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_equals_contiguous_bitwise(torch, hm, dtype):
    # Same lengths, so the same plan; the pool holds the same rows (G = 8:
    # fp32 runs on the matrix cores either way).
    w = wl.Workload("paged_vs_contig", B=4, Hq=32, Hkv=4, D=128, Lmax=3072,
                    dtype=dtype, seed=48, page_size=32, head_major=hm)
    seqlens = np.array([3072, 2048, 777, 5], np.int32)
    (q, k_unused, _, _, _), (qd, kd, vd, btd, sld) = paged_case(
        torch, w, seqlens)
    _, k, v, _ = _gen_with(w, seqlens)
    kc, vc = to_dev(k), to_dev(v)
    for splits in (0, 3):
        po, pl = fd.fd_decode_paged(qd, kd, vd, btd, sld, w.scale,
                                    num_splits=splits, head_major=hm)
        co, cl = fd.fd_decode_ex(qd, kc, vc, sld, w.scale,
                                 num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(_bits(torch, po), _bits(torch, co))
        assert torch.equal(pl, cl)


@pytest.mark.parametrize("name", ["paged_p64_b1_gqa8_h64_d128_l65536",
                                  "paged_hm_p64_b1_gqa8_h64_d128_l65536"])
def test_paged_full_size_64k(torch, oracle_mod, name):
    """The 64k batch-1 shape from 64-token pages, in the benchmark's launch
    configuration: bit-identical to the contiguous call, every row against
    the oracle."""
    w = wl.EXTRA_WORKLOADS[name]
    _note(f"{w.name}: generating inputs and the oracle's rows")
    seqlens = wl.paged_seqlens(w)
    q, k, v, sld, seqlens, ref = upload_full(w.with_(page_size=0),
                                             oracle_mod, seqlens=seqlens)
    kp, vp, btd, _ = wl.pages_from_contiguous(w, k, v)
    out, lse = fd.fd_decode_paged(q, kp, vp, btd, sld, w.scale,
                                  head_major=w.head_major)
    co, cl = fd.fd_decode(q, k, v, sld, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), co.view(torch.int16))
    assert torch.equal(lse, cl)
    assert out.shape == (1, 64, 128) and lse.shape == (1, 64)
    _assert_parity(out, lse, ref[0], ref[1], f"{w.name} every row")


PAGED_MQ_SHAPES = [
    # (B, Tq, Hq, Hkv, D, Lmax, page_size, seqlens)
    (3, 2, 16, 2, 128, 1000, 32, [1000, 517, 1]),
    (2, 4, 16, 4, 128, 700, 16, [700, 3]),
    (2, 3, 8, 8, 64, 640, 64, [641, 64]),
    (1, 16, 4, 4, 128, 9000, 48, [8999]),
    (2, 2, 64, 4, 128, 700, 32, [700, 33]),          # 16 x 2 rows
    (2, 3, 8, 2, 256, 500, 32, [500, 97]),           # head dim 256
]


@pytest.mark.parametrize("hm", [False, True], ids=["token_major",
                                                   "head_major"])
@pytest.mark.parametrize("shape", PAGED_MQ_SHAPES,
                         ids=[f"B{s[0]}_Tq{s[1]}_Hq{s[2]}_Hkv{s[3]}_D{s[4]}"
                              f"_L{s[5]}_P{s[6]}" for s in PAGED_MQ_SHAPES])
@pytest.mark.parametrize("splits,flags", [(0, 0), (1, 0), (7, 0),
                                          (0, fd.FD_FLAG_FUSED_MERGE)])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_multiquery_matches_oracle(torch, oracle_mod, shape, splits,
                                         flags, hm, dtype):
    B, Tq, Hq, Hkv, D, L, P, sls = shape
    w = wl.Workload("paged_mq_case", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=L,
                    dtype=dtype, seed=80 + Tq, page_size=P, head_major=hm,
                    Tq=Tq)
    seqlens = np.array(sls, np.int32)
    (q, kp, vp, bt, sl), (qd, kd, vd, btd, sld) = paged_case(torch, w,
                                                             seqlens)
    _note(f"paged mq {shape} {dtype} hm={hm} splits={splits} "
          f"flags={flags}")
    out, lse = fd.fd_decode_paged(qd, kd, vd, btd, sld, w.scale,
                                  num_splits=splits, flags=flags,
                                  head_major=hm)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode_paged(q, kp, vp, bt, sl, w.scale,
                                           head_major=hm)
    _assert_parity(out, lse, ref_o, ref_l, f"paged mq {shape} hm={hm}",
                   dtype)


def test_paged_multiquery_full_size_equals_contiguous(torch, oracle_mod):
    """Two new tokens over 64-token head-major pages at batch-1 64k: bit
    for bit the contiguous multi-token call on the same rows (same plan),
    every row against the oracle."""
    w = wl.EXTRA_WORKLOADS["paged_hm_p64_mq2_b1_gqa8_h64_d128_l65536"]
    _note(f"{w.name}: generating inputs and the oracle's rows")
    seqlens = wl.paged_seqlens(w)
    q, k, v, sld, seqlens, ref = upload_full(w.with_(page_size=0),
                                             oracle_mod, seqlens=seqlens)
    kp, vp, btd, _ = wl.pages_from_contiguous(w, k, v)
    out, lse = fd.fd_decode_paged(q, kp, vp, btd, sld, w.scale,
                                  head_major=True)
    co, cl = fd.fd_decode_multiquery(q, k, v, sld, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), co.view(torch.int16))
    assert torch.equal(lse, cl)
    _assert_parity(out, lse, ref[0], ref[1], f"{w.name} every row")


# ---------------------------------------------------------------------------
# Several causal new tokens.

MQ_SHAPES = [
    # (B, Tq, Hq, Hkv, D, Lmax, seqlens or None)
    (2, 2, 16, 2, 128, 1000, [1000, 517]),
    (3, 4, 16, 4, 128, 777, [777, 3, 0]),            # 3 < Tq: one sees none
    (2, 3, 8, 8, 64, 500, None),
    (2, 16, 4, 4, 128, 300, [300, 9]),                # 16 tokens, MHA
    (1, 1, 64, 4, 128, 400, [399]),                   # Tq = 1
    (2, 2, 8, 1, 128, 640, [641, 64]),                # clamped; G = 8
    (2, 4, 32, 4, 128, 600, [600, 5]),                # 8 x 4 = 32 rows
    (1, 3, 48, 1, 64, 500, [500]),                    # 48 x 3 = 144 rows
    (2, 2, 8, 2, 256, 400, [400, 37]),                # head dim 256
]


@pytest.mark.parametrize("shape", MQ_SHAPES,
                         ids=[f"B{s[0]}_Tq{s[1]}_Hq{s[2]}_Hkv{s[3]}_D{s[4]}"
                              f"_L{s[5]}" for s in MQ_SHAPES])
@pytest.mark.parametrize("splits,flags", [(0, 0), (1, 0), (9, 0),
                                          (0, fd.FD_FLAG_FUSED_MERGE)])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_multiquery_matches_oracle(torch, oracle_mod, shape, splits, flags,
                                   dtype):
    B, Tq, Hq, Hkv, D, L, sls = shape
    w = wl.Workload("mq_case", B=B, Hq=Hq, Hkv=Hkv, D=D, Lmax=L,
                    dtype=dtype, seed=60 + Tq, Tq=Tq)
    seqlens = None if sls is None else np.array(sls, np.int32)
    if seqlens is None:
        q, k, v, _ = wl.gen_all(w)
    else:
        q, k, v, _ = _gen_with(w, seqlens)
    q = q.reshape(B, Tq, Hq, D)          # Tq = 1 is drawn as [B, Hq, D]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sld = None if seqlens is None else torch.from_numpy(seqlens).to("cuda")
    _note(f"{shape} {dtype} splits={splits} flags={flags}")
    out, lse = fd.fd_decode_multiquery(qd, kd, vd, sld, w.scale,
                                       num_splits=splits, flags=flags)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode_multiquery(q, k, v, seqlens, w.scale)
    _assert_parity(out, lse, ref_o, ref_l, f"mq {shape}", dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_multiquery_causal_boundary_inside_every_chunk(torch, oracle_mod,
                                                       dtype):
    # 32-key chunks: the last Tq - 1 keys straddle a chunk edge for some
    # lengths and sit inside one for others (and, in the fp32 kernel's
    # 16-key halves, a half edge).
    w = wl.Workload("mq_edges", B=8, Hq=8, Hkv=2, D=128, Lmax=256,
                    dtype=dtype, seed=70, Tq=4)
    seqlens = np.array([256, 255, 226, 225, 224, 33, 32, 4] if dtype !=
                       "f32" else [256, 242, 241, 209, 18, 17, 16, 2],
                       np.int32)
    q, k, v, _ = _gen_with(w, seqlens)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sld = torch.from_numpy(seqlens).to("cuda")
    ref_o, ref_l = oracle_mod.decode_multiquery(q, k, v, seqlens, w.scale)
    for splits in (8, 3, 1):
        out, lse = fd.fd_decode_multiquery(qd, kd, vd, sld, w.scale,
                                           num_splits=splits)
        torch.cuda.synchronize()
        _assert_parity(out, lse, ref_o, ref_l, f"mq edges splits={splits}",
                       dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_multiquery_one_token_is_decode_bitwise(torch, dtype):
    w = wl.Workload("mq1", B=3, Hq=32, Hkv=4, D=128, Lmax=2000,
                    dtype=dtype, seed=71)
    seqlens = np.array([2000, 1000, 31], np.int32)
    q, k, v, _ = _gen_with(w, seqlens)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sld = torch.from_numpy(seqlens).to("cuda")
    mo, ml = fd.fd_decode_multiquery(qd[:, None].contiguous(), kd, vd, sld,
                                     w.scale)
    do, dl = fd.fd_decode(qd, kd, vd, sld, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch, mo[:, 0].contiguous()), _bits(torch, do))
    assert torch.equal(ml[:, 0].contiguous(), dl)


@pytest.mark.parametrize("name", ["mq2_b1_gqa8_h64_d128_l65536",
                                  "mq4_b64_gqa4_h32_d128_l4096"])
def test_multiquery_full_size(torch, oracle_mod, name):
    """The two multi-token workloads at full size, as the benchmark runs
    them: every (b, token, head) row against the oracle, bitwise
    repeatable, and every row inside its V column range."""
    w = wl.EXTRA_WORKLOADS[name]
    _note(f"{name}: generating inputs and the oracle's rows")
    q, k, v, sl, seqlens, ref = upload_full(w, oracle_mod)
    out, lse = fd.fd_decode_multiquery(q, k, v, sl, w.scale)
    out2, lse2 = fd.fd_decode_multiquery(q, k, v, sl, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    vmax = v.float().amax(2).repeat_interleave(w.G, dim=1)   # [B, Hq, D]
    vmin = v.float().amin(2).repeat_interleave(w.G, dim=1)
    of = out.float()
    slack = 1e-2 + 2 ** -7 * torch.maximum(vmax.abs(), vmin.abs())
    assert bool((of <= vmax[:, None] + slack[:, None]).all())
    assert bool((of >= vmin[:, None] - slack[:, None]).all())
    _assert_parity(out, lse, ref[0], ref[1], f"{name} every row")

