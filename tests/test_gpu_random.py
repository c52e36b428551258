"""Seeded random sweep of every decode entry point against the fp64 oracle.

Each case draws a shape (B, Hq, Hkv, D, lengths, token count, page size and
layout, split count, merge mode, dtype) from a fixed seed, so a failure
names a case that can be rerun alone.  Sizes stay small enough for the
oracle (at most a few hundred thousand key rows per case) while spanning
several tiles, chunks and ragged tails; some cases draw 60-80 short
sequences, whose work lists go past one round of workgroups, and the long
cases caches of up to 24k keys.  The rule is the suite's (tests/parity.py):
|out - ref| <= max(1e-2, half an ulp of ref in the output type),
|lse - ref| <= 1e-3.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import out_to_host, to_dev
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu

N_CASES = 64


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    kind = ["decode", "decode", "paged", "multiquery", "paged_mq",
            "unified"][i % 6]
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    Tq = 1
    if kind in ("multiquery", "paged_mq"):
        Tq = int(rng.integers(2, 16 // G + 1)) if G <= 8 else 1
        G = min(G, 16 // Tq)
    Hkv = int(rng.choice([1, 2, 3, 4]))
    B = int(rng.integers(1, 5))
    Lmax = int(rng.integers(1, 2500))
    if rng.random() < 0.15:
        # many short sequences: work lists past one round of workgroups,
        # more than 64 sequences in the length scans
        B = int(rng.integers(60, 80))
        Lmax = int(rng.integers(1, 600))
    dtype = "bf16"
    if kind == "decode" and rng.random() < 0.3:
        dtype = "f32"
    seqlens = rng.integers(0, Lmax + 3, size=B).astype(np.int32)
    if rng.random() < 0.3:
        seqlens[0] = Lmax
    if kind in ("paged", "paged_mq"):
        # past Lmax the last page holds NaN rows the sequence would own
        seqlens = np.minimum(seqlens, Lmax)
    splits = int(rng.choice([0, 0, 1, 2, 5, 33, 150]))
    flags = fd.FD_FLAG_FUSED_MERGE if rng.random() < 0.25 else 0
    page = int(rng.choice([16, 32, 48, 64, 128]))
    head_major = bool(rng.random() < 0.5)
    phi = float(rng.choice([0.0, 3.0, -50.0]))
    if kind in ("paged", "multiquery", "paged_mq") and (i // 6) % 3 == 2:
        dtype = "f32"        # without a draw: the other fields stay as they were
    if i % 17 == 5:
        G *= 4               # past 16 query rows per KV head, also without a draw
    if i % 13 == 7:
        D = 256              # head dimension 256, also without a draw
    if dtype == "bf16" and i % 5 == 3:
        dtype = "f16"        # fp16 caches, also without a draw
    return dict(kind=kind, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, Lmax=Lmax,
                dtype=dtype, seqlens=seqlens, Tq=Tq, splits=splits,
                flags=flags, page=page, head_major=head_major, phi=phi,
                seed=2000 + i)


N_LONG_CASES = 24


def draw_long_case(i):
    """A case of draw_case(i) with longer caches (up to 24k keys, up to 8
    sequences, often all full): plans of 2048-key var-len chunks, direct
    and listed chunk ids, and split counts up to 100."""
    c = draw_case(i)
    rng = np.random.default_rng(50000 + i)
    c["B"] = int(rng.integers(1, 9))
    c["Lmax"] = int(rng.integers(1, 24000))
    c["seqlens"] = rng.integers(0, c["Lmax"] + 3,
                                size=c["B"]).astype(np.int32)
    if rng.random() < 0.4:
        c["seqlens"][:] = c["Lmax"]
    if c["kind"] in ("paged", "paged_mq"):
        c["seqlens"] = np.minimum(c["seqlens"], c["Lmax"])
    c["splits"] = int(rng.choice([0, 0, 0, 3, 40, 100]))
    return c


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


def _host(w, seqlens):
    q = wl.gen_q(w)
    k = np.empty((w.B, w.Hkv, w.Lmax, w.D), w.np_dtype)
    v = np.empty_like(k)
    for b in range(w.B):
        for g in range(w.Hkv):
            wl.fill_slab(w, b, g, min(int(seqlens[b]), w.Lmax), k[b, g],
                         v[b, g])
    return q, k, v


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(torch, oracle_mod, i):
    _run_case(torch, oracle_mod, i, draw_case(i))


@pytest.mark.parametrize("i", range(N_LONG_CASES))
def test_random_long_case(torch, oracle_mod, i):
    _run_case(torch, oracle_mod, i, draw_long_case(i))


def _run_case(torch, oracle_mod, i, c):
    print(f"[random {i}] {dict((k, v) for k, v in c.items() if k != 'seqlens')}"
          f" seqlens={c['seqlens'].tolist()}", flush=True)
    kind = c["kind"]
    paged = kind in ("paged", "paged_mq")
    w = wl.Workload(f"random_{i}", B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"],
                    D=c["D"], Lmax=c["Lmax"], dtype=c["dtype"],
                    seed=c["seed"], Tq=c["Tq"],
                    page_size=c["page"] if paged else 0,
                    head_major=c["head_major"])
    sl = c["seqlens"]
    q, k, v = _host(w, sl)
    if kind == "multiquery":
        q = q.reshape(w.B, w.Tq, w.Hq, w.D)     # Tq = 1 is drawn 3-d
    sld = torch.from_numpy(sl).to("cuda")
    qd = to_dev(q)
    if paged:
        bt = wl.gen_block_table(w)
        kp, vp = wl.scatter_pages(w, k, v, bt, sl)
        out, lse = fd.fd_decode_paged(
            qd, to_dev(kp), to_dev(vp), torch.from_numpy(bt).to("cuda"), sld,
            w.scale, num_splits=c["splits"], flags=c["flags"],
            head_major=w.head_major)
        ref_o, ref_l = oracle_mod.decode_paged(q, kp, vp, bt, sl, w.scale,
                                               head_major=w.head_major)
    elif kind == "multiquery":
        out, lse = fd.fd_decode_multiquery(qd, to_dev(k), to_dev(v), sld,
                                           w.scale, num_splits=c["splits"],
                                           flags=c["flags"])
        ref_o, ref_l = oracle_mod.decode_multiquery(q, k, v, sl, w.scale)
    elif kind == "unified":
        out, lse = fd.fd_decode_unified_max(qd, to_dev(k), to_dev(v), sld,
                                            w.scale, c["phi"],
                                            num_splits=c["splits"],
                                            flags=c["flags"])
        ref_o, ref_l = oracle_mod.decode(q, k, v, sl, w.scale)
    else:
        # fp32 cases take the planner's kernel, the matrix cores or the
        # vector ALU in turn
        variant = ((fd.FD_VARIANT_AUTO, fd.FD_VARIANT_MFMA,
                    fd.FD_VARIANT_VALU)[(i // 6) % 3]
                   if w.dtype == "f32" and w.G <= 16 and w.D <= 128
                   else fd.FD_VARIANT_AUTO)
        print(f"[random {i}] variant {variant}", flush=True)
        out, lse = fd.fd_decode_ex(qd, to_dev(k), to_dev(v), sld, w.scale,
                                   num_splits=c["splits"], variant=variant,
                                   flags=c["flags"])
        ref_o, ref_l = oracle_mod.decode(q, k, v, sl, w.scale)
    torch.cuda.synchronize()
    ok_o, rep_o = check_out(out_to_host(out), ref_o, w.dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref_l)
    print(f"[random {i}] out {rep_o} lse {rep_l}", flush=True)
    assert ok_o, rep_o
    assert ok_l, rep_l
