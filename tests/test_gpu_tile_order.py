"""GPU parity where a chunk's tiles are walked in rotated order.

When every KV slab starts at the same offset modulo 32 MB (Lmax * D * 2
bytes a multiple of 32 MB: 128k keys at D = 128, 256k at D = 64), the
matrix-core pass starts
each chunk's tiles at a point taken from its (b, g) and wraps around, keeping
the last two tiles last.  These cases put every kind of chunk on that path --
chunks of hundreds of tiles, of a dozen, of one to three (too short to
rotate), ragged last tiles, several new tokens with causal limits, paged pools
of that capacity, the unified maximum and its fallback -- and compare them
with the fp64 oracle under the suite's rule (|out - ref| <= 1e-2 or faithful
bf16 rounding, |lse - ref| <= 1e-3).  Entry points that visit a chunk's keys
in the same order must still agree bit for bit.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import out_to_host, to_dev
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu

LMAX = 131072          # 128k keys x 256 bytes: KV heads 32 MB apart
ROTATING_STRIDE = 32 << 20


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


def _note(msg):
    print(f"[tile order] {msg}", flush=True)


def _parity(out, lse, ref_o, ref_l, tag):
    ok_o, rep_o = check_out(out_to_host(out), ref_o, "bf16")
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref_l)
    _note(f"{tag}: out {rep_o} lse {rep_l}")
    assert ok_o, (tag, rep_o)
    assert ok_l, (tag, rep_l)


def _gen(w, seqlens):
    """Host q, K, V with explicit lengths (rows past them NaN)."""
    assert w.Lmax * w.D * 2 % ROTATING_STRIDE == 0
    q = wl.gen_q(w)
    k = np.empty((w.B, w.Hkv, w.Lmax, w.D), w.np_dtype)
    v = np.empty_like(k)
    for b in range(w.B):
        for g in range(w.Hkv):
            wl.fill_slab(w, b, g, int(seqlens[b]), k[b, g], v[b, g])
    return q, k, v


W_DEC = wl.Workload("rot_decode", B=3, Hq=16, Hkv=2, D=128, Lmax=LMAX,
                    dtype="bf16", seed=91)
# a near-full sequence with a ragged last tile, one of 2187 full tiles plus
# 25 keys, and one of three tiles (a chunk too short to rotate)
SL_DEC = np.array([LMAX - 5, 70001, 70], np.int32)


@pytest.fixture(scope="module")
def dec_case(torch, oracle_mod):
    q, k, v = _gen(W_DEC, SL_DEC)
    ref = oracle_mod.decode(q, k, v, SL_DEC, W_DEC.scale)
    dev = (to_dev(q), to_dev(k), to_dev(v),
           torch.from_numpy(SL_DEC).to("cuda"))
    return (q, k, v), dev, ref


@pytest.mark.parametrize("splits", [0, 7, 300, 4096])
def test_rotated_order_parity(torch, dec_case, splits):
    # 0: the planner's 2048-key chunks; 7: chunks of 586 tiles; 300: chunks
    # of 14 tiles; 4096: one-tile chunks (nothing to rotate).
    _, (qd, kd, vd, sld), (ref_o, ref_l) = dec_case
    plan = fd.fd_plan(W_DEC.B, W_DEC.Hq, W_DEC.Hkv, W_DEC.D, W_DEC.Lmax,
                      "bf16", varlen=True, num_splits=splits)
    for flags in (0, fd.FD_FLAG_FUSED_MERGE):
        out, lse = fd.fd_decode_ex(qd, kd, vd, sld, W_DEC.scale,
                                   num_splits=splits, flags=flags)
        torch.cuda.synchronize()
        _parity(out, lse, ref_o, ref_l,
                f"decode chunk={plan['chunk']} flags={flags}")


def test_rotated_order_is_repeatable_and_shared(torch, dec_case):
    # fd_decode (library workspace) and fd_decode_ex take the same plan and
    # the same tile order: identical bits, call after call.
    _, (qd, kd, vd, sld), _ = dec_case
    o1, l1 = fd.fd_decode(qd, kd, vd, sld, W_DEC.scale)
    o2, l2 = fd.fd_decode_ex(qd, kd, vd, sld, W_DEC.scale)
    o3, l3 = fd.fd_decode(qd, kd, vd, sld, W_DEC.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l1, l2) and torch.equal(l1, l3)


@pytest.mark.parametrize("phi", [0.0, 1000.0])
def test_rotated_order_unified_max(torch, dec_case, phi):
    # phi 0: the unified pass itself (scores of these inputs lie well inside
    # the range); phi 1000: every chunk falls back to the exact pass, whose
    # bits fd_decode_ex must reproduce.
    _, (qd, kd, vd, sld), (ref_o, ref_l) = dec_case
    for splits in (0, 5):
        uo, ul = fd.fd_decode_unified_max(qd, kd, vd, sld, W_DEC.scale, phi,
                                          num_splits=splits)
        torch.cuda.synchronize()
        _parity(uo, ul, ref_o, ref_l, f"unified phi={phi} splits={splits}")
        if phi == 1000.0:
            eo, el = fd.fd_decode_ex(qd, kd, vd, sld, W_DEC.scale,
                                     num_splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(uo.view(torch.int16), eo.view(torch.int16))
            assert torch.equal(ul, el)


def test_rotated_order_multiquery(torch, oracle_mod):
    # Three new tokens: the causal limits cut into each chunk's last two
    # tiles only, which the rotation leaves in place.
    w = wl.Workload("rot_mq", B=2, Hq=8, Hkv=2, D=128, Lmax=LMAX,
                    dtype="bf16", seed=92, Tq=3)
    sl = np.array([LMAX, 5000], np.int32)
    q, k, v = _gen(w, sl)
    ref_o, ref_l = oracle_mod.decode_multiquery(q, k, v, sl, w.scale)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sld = torch.from_numpy(sl).to("cuda")
    for splits in (0, 9, 200):
        out, lse = fd.fd_decode_multiquery(qd, kd, vd, sld, w.scale,
                                           num_splits=splits)
        torch.cuda.synchronize()
        _parity(out, lse, ref_o, ref_l, f"multiquery splits={splits}")
    # one token through the multi-token entry: the decode's bits
    w1 = w.with_(Tq=1)
    q1 = wl.gen_q(w1)
    q1d = to_dev(q1)
    mo, ml = fd.fd_decode_multiquery(q1d[:, None].contiguous(), kd, vd, sld,
                                     w.scale)
    do, dl = fd.fd_decode(q1d, kd, vd, sld, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(mo[:, 0].contiguous().view(torch.int16),
                       do.view(torch.int16))
    assert torch.equal(ml[:, 0].contiguous(), dl)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("hm", [False, True], ids=["token_major",
                                                   "head_major"])
def test_rotated_order_paged(torch, oracle_mod, hm, D):
    # A block table of 32 MB of keys per head (128k keys at D = 128, 256k at
    # D = 64; K goes through LDS only at D = 128) takes the same order as
    # the contiguous cache of that stride: the same bits, and the oracle's
    # values.
    lmax = LMAX * 128 // D
    w = wl.Workload("rot_paged", B=2, Hq=16, Hkv=2, D=D, Lmax=lmax,
                    dtype="bf16", seed=93, page_size=64, head_major=hm)
    sl = np.array([lmax - 100, 4000], np.int32)
    q, k, v = _gen(w, sl)
    ref_o, ref_l = oracle_mod.decode(q, k, v, sl, w.scale)
    bt = wl.gen_block_table(w)
    kp, vp = wl.scatter_pages(w, k, v, bt, sl)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kpd, vpd = to_dev(kp), to_dev(vp)
    btd = torch.from_numpy(bt).to("cuda")
    sld = torch.from_numpy(sl).to("cuda")
    for splits in (0, 5):
        po, pl = fd.fd_decode_paged(qd, kpd, vpd, btd, sld, w.scale,
                                    num_splits=splits, head_major=hm)
        co, cl = fd.fd_decode_ex(qd, kd, vd, sld, w.scale, num_splits=splits)
        torch.cuda.synchronize()
        _parity(po, pl, ref_o, ref_l, f"paged hm={hm} splits={splits}")
        assert torch.equal(po.view(torch.int16), co.view(torch.int16))
        assert torch.equal(pl, cl)


@pytest.mark.parametrize("splits", [0, 11])
def test_rotated_order_d64(torch, oracle_mod, splits):
    # D = 64 reaches the same stride at 256k keys (128-byte rows).
    w = wl.Workload("rot_d64", B=2, Hq=8, Hkv=2, D=64, Lmax=2 * LMAX,
                    dtype="bf16", seed=94)
    sl = np.array([2 * LMAX - 7, 1000], np.int32)
    q, k, v = _gen(w, sl)
    ref_o, ref_l = oracle_mod.decode(q, k, v, sl, w.scale)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sld = torch.from_numpy(sl).to("cuda")
    for flags in (0, fd.FD_FLAG_FUSED_MERGE):
        out, lse = fd.fd_decode_ex(qd, kd, vd, sld, w.scale,
                                   num_splits=splits, flags=flags)
        torch.cuda.synchronize()
        _parity(out, lse, ref_o, ref_l, f"D=64 splits={splits} flags={flags}")
