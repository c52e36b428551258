"""GPU parity of the var-len work order and of workgroups that run two chunks.

With per-sequence lengths the per-chunk pass takes its work list in two
passes (every full chunk, then each sequence's short last chunk, longest
first; sequences past the 64th in their natural order), and launches as few
as half the list's upper bound of workgroups, workgroup i taking chunks i
and i + grid.  The cases below force each of those paths -- a work list
longer than the grid (plain, fused merge, paged), more than 64 sequences,
equal remainders, empty and exact-multiple lengths -- and compare every
output row with the fp64 oracle under the suite's rule (|out - ref| <= 1e-2
or faithful bf16 rounding, |lse - ref| <= 1e-3).
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import dev_inputs, out_to_host, to_dev
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


def work_items(seqlens, Hkv, chunk):
    """Chunks in the work list: max(1, ceil(L / C)) per sequence and head."""
    return int(sum(max(1, -(-int(L) // chunk)) for L in seqlens)) * Hkv


def _parity(w, out, lse, ref_o, ref_l, what):
    ok_o, rep_o = check_out(out_to_host(out), ref_o, w.dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref_l)
    print(f"[workorder] {what}: out {rep_o} lse {rep_l}", flush=True)
    assert ok_o, (what, rep_o)
    assert ok_l, (what, rep_l)


LONG = W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(B=4, Lmax=8192,
                                                      varlen=(1, 8192))
LONG_LENS = np.array([8192, 8000, 7777, 8190], np.int32)
SPLITS = 256  # 32-key chunks: a work list of ~8000 chunks


@pytest.mark.parametrize("flags", [0, fd.FD_FLAG_FUSED_MERGE])
def test_work_list_longer_than_grid(torch, oracle_mod, flags):
    w = LONG
    plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", varlen=True,
                      num_splits=SPLITS, flags=flags)
    items = work_items(LONG_LENS, w.Hkv, plan["chunk"])
    print(f"[workorder] plan {plan} items {items}", flush=True)
    assert plan["grid"] < items <= 2 * plan["grid"]
    q, k, v, sl, seqlens, host = dev_inputs(w, seqlens=LONG_LENS,
                                            keep_host=True)
    out, lse = fd.fd_decode_ex(q, k, v, sl, w.scale, num_splits=SPLITS,
                               flags=flags)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode(*host, seqlens, w.scale)
    _parity(w, out, lse, ref_o, ref_l, f"two chunks per workgroup, "
            f"flags={flags}")


@pytest.mark.parametrize("head_major", [False, True])
def test_paged_work_list_longer_than_grid(torch, oracle_mod, head_major):
    w = LONG.with_(page_size=64, head_major=head_major)
    sl = LONG_LENS
    plan = fd.fd_plan_ex(w.B, 1, w.Hq, w.Hkv, w.D, w.Lmax, "bf16",
                         varlen=True, paged=True, num_splits=SPLITS)
    items = work_items(sl, w.Hkv, plan["chunk"])
    assert plan["grid"] < items <= 2 * plan["grid"]
    q = wl.gen_q(w)
    k = np.empty((w.B, w.Hkv, w.Lmax, w.D), w.np_dtype)
    v = np.empty_like(k)
    for b in range(w.B):
        for g in range(w.Hkv):
            wl.fill_slab(w, b, g, int(sl[b]), k[b, g], v[b, g])
    bt = wl.gen_block_table(w)
    kp, vp = wl.scatter_pages(w, k, v, bt, sl)
    out, lse = fd.fd_decode_paged(
        to_dev(q), to_dev(kp), to_dev(vp), torch.from_numpy(bt).to("cuda"),
        torch.from_numpy(sl).to("cuda"), w.scale, num_splits=SPLITS,
        head_major=head_major)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode_paged(q, kp, vp, bt, sl, w.scale,
                                           head_major=head_major)
    _parity(w, out, lse, ref_o, ref_l, f"paged two chunks, "
            f"head_major={head_major}")


@pytest.mark.parametrize("splits", [0, 7])
def test_more_than_64_sequences(torch, oracle_mod, splits):
    # 130 sequences: the scans run over three 64-lane batches, and the last
    # chunks of sequences past the 64th keep their natural order.
    w = W["b64_gqa4_h32_d128_l4096"].with_(B=130, Hq=8, Hkv=2, D=64,
                                           Lmax=700, varlen=(1, 700))
    rng = np.random.default_rng(77)
    sl = rng.integers(0, 701, size=w.B).astype(np.int32)
    sl[[0, 5, 64, 129]] = 0
    sl[[1, 70, 128]] = 700
    q, k, v, sld, seqlens, host = dev_inputs(w, seqlens=sl, keep_host=True)
    out, lse = fd.fd_decode_ex(q, k, v, sld, w.scale, num_splits=splits)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode(*host, seqlens, w.scale)
    _parity(w, out, lse, ref_o, ref_l, f"B=130 splits={splits}")
    assert float(lse[0].max()) == float("-inf")


def test_equal_remainders_and_exact_multiples(torch, oracle_mod):
    # Several sequences whose last chunks have the same length (ranked by
    # sequence index), lengths that are exact multiples of the chunk (no
    # short last chunk) and a zero length (one empty chunk).
    w = LONG.with_(B=7, Lmax=3000, varlen=(1, 3000))
    C = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", varlen=True,
                   num_splits=9)["chunk"]
    sl = np.array([100, 100 + C, 100 + 2 * C, C, 2 * C, 0, 3000], np.int32)
    sl = np.minimum(sl, w.Lmax)
    q, k, v, sld, seqlens, host = dev_inputs(w, seqlens=sl, keep_host=True)
    for flags in (0, fd.FD_FLAG_FUSED_MERGE):
        out, lse = fd.fd_decode_ex(q, k, v, sld, w.scale, num_splits=9,
                                   flags=flags)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_mod.decode(*host, seqlens, w.scale)
        _parity(w, out, lse, ref_o, ref_l,
                f"equal remainders C={C} flags={flags}")
