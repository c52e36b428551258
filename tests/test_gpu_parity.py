"""GPU parity: libfd.so (through its C ABI) against the fp64 oracle.

Element-by-element comparison at sizes the oracle finishes in seconds that
still span several 32-key tiles, several chunks and a ragged tail, for all
five workload shapes, every kernel variant and forced split counts; plus
edge lengths, NaN padding, determinism, streams/workspaces and negative
controls that show the comparison can fail.  The rule (tests/parity.py):
|out - ref| <= 1e-2 or correct rounding to the output type,
|lse - ref| <= 1e-3.
"""
import math

import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import dev_inputs, out_to_host, to_dev
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
# Reduced copies of the five workloads (same heads, head dim, dtype and
# value recipe; shorter caches): several tiles, several chunks, ragged tails.
SMALL = {
    "tiny_mha_f32": W["tiny_mha_f32_b1_h8_d64_l1024"],
    "b1_gqa8": W["b1_gqa8_h64_d128_l65536"].with_(Lmax=4133),
    "b4_mha_peaked": W["b4_mha_h32_d128_l32768_peaked"].with_(
        B=2, Hq=8, Hkv=8, Lmax=3001),
    "b64_gqa4": W["b64_gqa4_h32_d128_l4096"].with_(B=8, Lmax=517),
    "varlen_gqa8": W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=6, Lmax=4096, varlen=(1, 4096)),
    "gqa8_d64": W["b1_gqa8_h64_d128_l65536"].with_(D=64, B=2, Hq=16, Hkv=2,
                                                   Lmax=1999),
    "gqa16_d128": W["b1_gqa8_h64_d128_l65536"].with_(B=1, Hq=32, Hkv=2,
                                                     Lmax=777),
    "gqa3_d128": W["b1_gqa8_h64_d128_l65536"].with_(B=2, Hq=6, Hkv=2,
                                                    Lmax=300),
    "f32_gqa4_d128": W["tiny_mha_f32_b1_h8_d64_l1024"].with_(
        D=128, B=2, Hq=16, Hkv=4, Lmax=450),
    "f32_gqa16_d64": W["tiny_mha_f32_b1_h8_d64_l1024"].with_(
        B=1, Hq=16, Hkv=1, Lmax=300),
    "f32_gqa5_d64": W["tiny_mha_f32_b1_h8_d64_l1024"].with_(
        B=3, Hq=10, Hkv=2, Lmax=700),
    "f32_varlen_gqa8_d128": W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=5, Hq=16, Hkv=2, Lmax=2100, varlen=(1, 2100), dtype="f32"),
    # more than 16 query heads per KV head: virtual KV heads
    "gqa32_d128": W["b1_gqa8_h64_d128_l65536"].with_(B=2, Hq=64, Hkv=2,
                                                     Lmax=1500),
    "mqa48_d64": W["b1_gqa8_h64_d128_l65536"].with_(B=1, Hq=48, Hkv=1, D=64,
                                                    Lmax=2100),
    "f32_mqa64_d128": W["tiny_mha_f32_b1_h8_d64_l1024"].with_(
        B=1, Hq=64, Hkv=1, D=128, Lmax=1000),
    "varlen_gqa24": W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=4, Hq=48, Hkv=2, Lmax=3000, varlen=(1, 3000)),
    # head dimension 256 (matrix cores only)
    "gqa8_d256": W["b1_gqa8_h64_d128_l65536"].with_(B=2, Hq=16, Hkv=2, D=256,
                                                    Lmax=1700),
    "mha_d256_varlen": W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=3, Hq=4, Hkv=4, D=256, Lmax=2500, varlen=(1, 2500)),
    "f32_gqa2_d256": W["tiny_mha_f32_b1_h8_d64_l1024"].with_(
        B=2, Hq=4, Hkv=2, D=256, Lmax=900),
    "gqa32_d256": W["b1_gqa8_h64_d128_l65536"].with_(B=1, Hq=32, Hkv=1, D=256,
                                                     Lmax=700),
    # fp16 caches (the same value recipe rounded to IEEE binary16)
    "f16_b1_gqa8": W["b1_gqa8_h64_d128_l65536"].with_(Lmax=4133,
                                                      dtype="f16"),
    "f16_mha_peaked": W["b4_mha_h32_d128_l32768_peaked"].with_(
        B=2, Hq=8, Hkv=8, Lmax=3001, dtype="f16"),
    "f16_varlen_gqa8": W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=6, Lmax=4096, varlen=(1, 4096), dtype="f16"),
    "f16_gqa4_d64": W["b64_gqa4_h32_d128_l4096"].with_(B=3, D=64, Lmax=517,
                                                       dtype="f16"),
    "f16_gqa8_d256": W["b1_gqa8_h64_d128_l65536"].with_(
        B=2, Hq=16, Hkv=2, D=256, Lmax=1700, dtype="f16"),
    "f16_gqa32_d128": W["b1_gqa8_h64_d128_l65536"].with_(
        B=2, Hq=64, Hkv=2, Lmax=1500, dtype="f16"),
}


@pytest.fixture(scope="module")
def cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return torch


_cache = {}


def inputs(name, w, seqlens=None):
    key = (name, None if seqlens is None else tuple(seqlens))
    if key not in _cache:
        _cache.clear()
        _cache[key] = dev_inputs(w, seqlens=seqlens, keep_host=True)
    return _cache[key]


def reference(oracle_mod, w, host, seqlens, scale=None):
    q, k, v = host
    return oracle_mod.decode(q, k, v, seqlens,
                             w.scale if scale is None else scale)


def assert_parity(w, out, lse, ref_out, ref_lse, what=""):
    ok_o, rep_o = check_out(out_to_host(out), ref_out, w.dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref_lse)
    print(f"{what}: out {rep_o} lse {rep_l}", flush=True)
    assert ok_o, f"{what} out mismatch {rep_o}"
    assert ok_l, f"{what} lse mismatch {rep_l}"
    return rep_o, rep_l


def variants_for(w):
    if w.G > 16 or w.D > 128:
        return [fd.FD_VARIANT_MFMA]      # matrix cores only
    if w.dtype == "f32":
        return [fd.FD_VARIANT_MFMA, fd.FD_VARIANT_VALU]
    if w.G <= 4:
        return [fd.FD_VARIANT_MFMA, fd.FD_VARIANT_VALU]
    return [fd.FD_VARIANT_MFMA]


MERGES = [0, fd.FD_FLAG_FUSED_MERGE]


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 7, 100000])
def test_small_workloads_match_oracle(cuda, oracle_mod, name, num_splits):
    w = SMALL[name]
    q, k, v, sl_dev, seqlens, host = inputs(name, w)
    ref_out, ref_lse = reference(oracle_mod, w, host, seqlens)
    for variant in variants_for(w):
        for flags in MERGES:
            out, lse = fd.fd_decode_ex(q, k, v, sl_dev, w.scale,
                                       num_splits=num_splits, variant=variant,
                                       flags=flags)
            cuda.cuda.synchronize()
            assert_parity(w, out, lse, ref_out, ref_lse,
                          f"{name} S={num_splits} variant={variant} "
                          f"flags={flags}")


@pytest.mark.parametrize("G,D,dtype", [(8, 128, "bf16"), (1, 128, "bf16"),
                                       (4, 64, "bf16"), (1, 64, "f32"),
                                       (2, 128, "f32"), (8, 128, "f16"),
                                       (2, 64, "f16")])
@pytest.mark.parametrize("num_splits", [0, 1, 4])
def test_edge_lengths_with_nan_padding(cuda, oracle_mod, G, D, dtype,
                                       num_splits):
    # lengths 0, 1, a tile boundary +-1, Lmax-1, Lmax; padding is NaN
    Hkv = 2
    w = W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=9, Hq=Hkv * G, Hkv=Hkv, D=D, Lmax=1000, dtype=dtype,
        varlen=(1, 1000))
    seqlens = np.array([0, 1, 31, 32, 33, 64, 999, 1000, 517], np.int32)
    q, k, v, sl_dev, seqlens, host = inputs(f"edge{G}{D}{dtype}", w, seqlens)
    ref_out, ref_lse = reference(oracle_mod, w, host, seqlens)
    assert ref_lse[0, 0] == -np.inf
    for variant in variants_for(w):
        for flags in MERGES:
            out, lse = fd.fd_decode_ex(q, k, v, sl_dev, w.scale,
                                       num_splits=num_splits, variant=variant,
                                       flags=flags)
            cuda.cuda.synchronize()
            assert_parity(w, out, lse, ref_out, ref_lse,
                          f"edge G={G} D={D} {dtype} S={num_splits} "
                          f"v={variant} f={flags}")
            o = out_to_host(out)
            assert np.all(o[0] == 0)
            assert np.all(lse.cpu().numpy()[0] == -np.inf)


def test_seqlens_out_of_range_are_clamped(cuda, oracle_mod):
    w = SMALL["b1_gqa8"].with_(B=3, Lmax=300, varlen=(1, 300))
    q, k, v, _, _, host = inputs("clamp", w, np.array([300] * 3, np.int32))
    sl = cuda.tensor([-7, 1 << 30, 150], dtype=cuda.int32, device="cuda")
    out, lse = fd.fd_decode(q, k, v, sl, w.scale)
    cuda.cuda.synchronize()
    ref_out, ref_lse = reference(oracle_mod, w, host,
                                 np.array([0, 300, 150], np.int32))
    assert_parity(w, out, lse, ref_out, ref_lse, "clamped seqlens")


@pytest.mark.parametrize("name", ["b1_gqa8", "varlen_gqa8", "tiny_mha_f32"])
def test_results_are_bitwise_deterministic(cuda, name):
    """Same plan, same bits -- in particular whichever workgroup of a group
    happens to finish last and run the fused merge."""
    w = SMALL[name]
    q, k, v, sl_dev, _, _ = inputs(name, w)
    for flags in MERGES:
        runs = []
        for _ in range(4):
            out, lse = fd.fd_decode_ex(q, k, v, sl_dev, w.scale,
                                       num_splits=7, flags=flags)
            cuda.cuda.synchronize()
            runs.append((out_to_host(out).copy(), lse.cpu().numpy().copy()))
        for o, l_ in runs[1:]:
            assert np.array_equal(o.view(np.uint16),
                                  runs[0][0].view(np.uint16))
            assert np.array_equal(l_.view(np.uint32),
                                  runs[0][1].view(np.uint32))


def test_negative_controls_fail_the_comparison(cuda, oracle_mod):
    """The comparison must reject plausible wrong answers: zeros, the GQA
    map h % Hkv, and a missing scale (mistakes planted in the oracle's
    inputs, on the CPU)."""
    w = SMALL["b1_gqa8"]
    q, k, v, sl_dev, seqlens, host = inputs("b1_gqa8", w)
    out, lse = fd.fd_decode(q, k, v, sl_dev, w.scale)
    cuda.cuda.synchronize()
    o_h, l_h = out_to_host(out), lse.cpu().numpy()
    ref_out, ref_lse = reference(oracle_mod, w, host, seqlens)
    assert check_out(o_h, ref_out, w.dtype)[0]
    # zeros
    zero = np.zeros_like(o_h)
    assert not check_out(zero, ref_out, w.dtype)[0]
    # h % Hkv instead of h // G: permute query heads accordingly
    qh, kh, vh = host
    perm = [(h % w.Hkv) * w.G + h // w.Hkv for h in range(w.Hq)]
    bad_o, bad_l = oracle_mod.decode(qh[:, perm].copy(), kh, vh, seqlens,
                                     w.scale)
    inv = np.argsort(perm)
    bad_o, bad_l = bad_o[:, inv], bad_l[:, inv]
    assert not (check_out(o_h, bad_o, w.dtype)[0]
                and check_lse(l_h, bad_l)[0])
    # scale dropped
    bad_o, bad_l = oracle_mod.decode(qh, kh, vh, seqlens, 1.0)
    assert not check_lse(l_h, bad_l)[0]


def test_caller_workspace_and_streams(cuda, oracle_mod):
    w = SMALL["b1_gqa8"]
    q, k, v, sl_dev, seqlens, host = inputs("b1_gqa8", w)
    F = fd.FD_FLAG_FUSED_MERGE
    need = fd.fd_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16",
                                 num_splits=7, flags=F)
    p = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", num_splits=7,
                   flags=F)
    assert need == p["workspace_bytes"] > 0 and p["ticket_bytes"] > 0
    ws = cuda.zeros(need, dtype=cuda.uint8, device="cuda")
    s = cuda.cuda.Stream()
    for flags in (0, F):
        # the workspace was filled on the default stream: order it first
        s.wait_stream(cuda.cuda.current_stream())
        with cuda.cuda.stream(s):
            out, lse = fd.fd_decode_ex(q, k, v, sl_dev, w.scale,
                                       num_splits=7, flags=flags,
                                       workspace=ws)
        s.synchronize()
        ref = fd.fd_decode_ex(q, k, v, sl_dev, w.scale, num_splits=7,
                              flags=flags)
        cuda.cuda.synchronize()
        assert np.array_equal(out_to_host(out), out_to_host(ref[0]))
        if flags == 0:
            # a separate-merge call keeps partials from byte 0 on: zero the
            # ticket region again before the fused call (fd.h's rule)
            ws[:p["ticket_bytes"]].zero_()
        else:
            # the fused merge leaves its tickets at zero for the next call
            assert int(ws[:p["ticket_bytes"]].count_nonzero()) == 0
    small = cuda.zeros(need - 256, dtype=cuda.uint8, device="cuda")
    with pytest.raises(fd.FdError) as e:
        fd.fd_decode_ex(q, k, v, sl_dev, w.scale, num_splits=7, flags=F,
                        workspace=small)
    assert e.value.code == fd.FD_ERR_WORKSPACE
    # no merge needed -> no workspace needed
    assert fd.fd_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16",
                                 num_splits=1) == 0


def test_scale_is_applied_as_given(cuda, oracle_mod):
    w = SMALL["b4_mha_peaked"]
    q, k, v, sl_dev, seqlens, host = inputs("b4_mha_peaked", w)
    for scale in (0.0, 0.3, -0.05):
        out, lse = fd.fd_decode(q, k, v, sl_dev, scale)
        cuda.cuda.synchronize()
        ref_out, ref_lse = reference(oracle_mod, w, host, seqlens, scale)
        assert_parity(w, out, lse, ref_out, ref_lse, f"scale={scale}")


def test_nan_in_valid_prefix_propagates(cuda):
    w = SMALL["b1_gqa8"].with_(Lmax=200)
    q, k, v, sl_dev, _, _ = inputs("nanprefix", w)
    k2 = k.clone()
    k2[0, 3, 17, 5] = float("nan")
    out, lse = fd.fd_decode(q, k2, v, None, w.scale)
    cuda.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.isnan(o[0, 3 * w.G:(3 + 1) * w.G]).all()
    assert np.isfinite(o[0, :3 * w.G]).all()


def test_owned_workspace_across_shapes(cuda, oracle_mod):
    """The library's own workspace is reused across shapes whose ticket
    regions grow and shrink, and by separate-merge calls whose partials
    land where the next fused call keeps its tickets (stale partials must
    never be read as tickets)."""
    seq = [("b1_gqa8", SMALL["b1_gqa8"]),
           ("b64_gqa4_split", SMALL["b64_gqa4"]),
           ("b1_gqa8", SMALL["b1_gqa8"]),
           ("varlen_gqa8", SMALL["varlen_gqa8"]),
           ("b64_gqa4_split", SMALL["b64_gqa4"])]
    for name, w in seq:
        q, k, v, sl_dev, seqlens, host = inputs(name, w)
        ref_out, ref_lse = reference(oracle_mod, w, host, seqlens)
        for flags in (fd.FD_FLAG_FUSED_MERGE, fd.FD_FLAG_FUSED_MERGE, 0,
                      fd.FD_FLAG_FUSED_MERGE):
            out, lse = fd.fd_decode_ex(q, k, v, sl_dev, w.scale,
                                       num_splits=5, flags=flags)
            cuda.cuda.synchronize()
            assert_parity(w, out, lse, ref_out, ref_lse,
                          f"reuse {name} flags {flags}")


@pytest.mark.parametrize("name,S", [("b1_gqa8_h64_d128_l65536", 64),
                                    ("b1_gqa8_h64_d128_l65536", 32),
                                    ("varlen_b16_gqa8_h64_d128_lmax131072",
                                     0)])
def test_fused_merge_never_reads_stale_partials(cuda, name, S):
    """Alternate two different inputs of the full size on the same
    workspace: a partial of the previous call read by the fused merge would
    move that row's lse by O(0.1).  Every fused result must agree with the
    separate-merge result up to rounding (different summation order)."""
    wa = W[name]
    wb = wa.with_(seed=wa.seed + 100)
    ins = []
    for w in (wa, wb):
        q, k, v, sl, _, _ = dev_inputs(w)
        ins.append((q, k, v, sl))
    refs = []
    for q, k, v, sl in ins:
        o, l_ = fd.fd_decode_ex(q, k, v, sl, wa.scale, num_splits=S)
        cuda.cuda.synchronize()
        refs.append((o.float().cpu().numpy(), l_.cpu().numpy()))
    assert np.abs(refs[0][1] - refs[1][1]).max() > 0.05
    out = cuda.empty_like(ins[0][0])
    lse = cuda.empty((wa.B, wa.Hq), dtype=cuda.float32, device="cuda")
    for it in range(40):
        i = it % 2
        q, k, v, sl = ins[i]
        fd.fd_decode_ex(q, k, v, sl, wa.scale, out=out, lse=lse,
                        num_splits=S, flags=fd.FD_FLAG_FUSED_MERGE)
        if it % 4 < 2:       # also back-to-back launches without a sync
            cuda.cuda.synchronize()
            dl = np.abs(lse.cpu().numpy() - refs[i][1]).max()
            do = np.abs(out.float().cpu().numpy() - refs[i][0]).max()
            assert dl < 1e-4 and do < 2e-3, (it, dl, do)
    cuda.cuda.synchronize()


@pytest.mark.parametrize("name,num_splits", [("b1_gqa8", 7), ("b1_gqa8", 1),
                                             ("b64_gqa4", 7),
                                             ("varlen_gqa8", 0),
                                             ("b4_mha_peaked", 3),
                                             ("tiny_mha_f32", 4),
                                             ("gqa8_d64", 5)])
def test_phase_calls_and_chunk_partials(cuda, oracle_mod, name, num_splits):
    """fd_decode_partials leaves, for every existing chunk, that chunk's own
    normalised attention output and log-sum-exp (checked against the
    oracle's split twin with the same chunk length); fd_merge_partials then
    gives the same bits as the one-call path with the same plan."""
    w = SMALL[name]
    q, k, v, sl_dev, seqlens, host = inputs(name, w)
    P = fd.FD_FLAG_PARTIALS
    plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                      varlen=sl_dev is not None, num_splits=num_splits,
                      flags=P)
    S, C = plan["num_splits"], plan["chunk"]
    ws = cuda.zeros(plan["workspace_bytes"], dtype=cuda.uint8,
                    device="cuda")
    fd.fd_decode_partials(q, k, v, sl_dev, w.scale, ws,
                          num_splits=num_splits)
    out = cuda.empty_like(q)
    lse = cuda.empty((w.B, w.Hq), dtype=cuda.float32, device="cuda")
    fd.fd_merge_partials(sl_dev, w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype, ws,
                         out, lse, num_splits=num_splits)
    one_out, one_lse = fd.fd_decode_ex(q, k, v, sl_dev, w.scale,
                                       num_splits=num_splits, flags=P)
    cuda.cuda.synchronize()
    assert np.array_equal(out_to_host(out).view(np.uint16),
                          out_to_host(one_out).view(np.uint16))
    assert np.array_equal(lse.cpu().numpy(), one_lse.cpu().numpy())
    ref_out, ref_lse = reference(oracle_mod, w, host, seqlens)
    assert_parity(w, out, lse, ref_out, ref_lse, f"phases {name}")

    o_off, l_off = plan["o_part_offset"], plan["lse_part_offset"]
    wsh = ws.cpu().numpy()
    n = w.B * w.Hq * S
    o_flat = wsh[o_off:o_off + n * w.D * 4].view(np.float32)
    l_flat = wsh[l_off:l_off + n * 4].view(np.float32)
    if plan["partial_layout"] == fd.FD_PARTIALS_CHUNK_MAJOR:
        # [B][Hq/P][S][P] rows -> [B][Hq][S]
        P = plan["partial_group"]
        o_part = o_flat.reshape(w.B, w.Hq // P, S, P, w.D).transpose(
            0, 1, 3, 2, 4).reshape(w.B, w.Hq, S, w.D)
        l_part = l_flat.reshape(w.B, w.Hq // P, S, P).transpose(
            0, 1, 3, 2).reshape(w.B, w.Hq, S)
    else:
        assert plan["partial_layout"] == fd.FD_PARTIALS_ROW_MAJOR
        o_part = o_flat.reshape(w.B, w.Hq, S, w.D)
        l_part = l_flat.reshape(w.B, w.Hq, S)
    # several rounds of workgroups: chunk-major; one round: row-major
    rounds = plan["grid"] > plan["num_cus"]
    assert plan["partial_layout"] == (fd.FD_PARTIALS_CHUNK_MAJOR if rounds
                                      else fd.FD_PARTIALS_ROW_MAJOR)
    qh, kh, vh = host
    for b in range(w.B):
        L = wl.seqlen_of(w, seqlens, b)
        nb = max(1, -(-L // C))
        for h in range(0, w.Hq, max(1, w.Hq // 4)):
            g = h // w.G
            _, _, po, pl = oracle_mod.attend_row_split(
                qh[b, h], kh[b, g], vh[b, g], L, w.scale, C, nb)
            np.testing.assert_allclose(o_part[b, h, :nb], po, rtol=0,
                                       atol=2e-3)
            fin = np.isfinite(pl)
            assert np.array_equal(fin, np.isfinite(l_part[b, h, :nb]))
            np.testing.assert_allclose(l_part[b, h, :nb][fin], pl[fin],
                                       rtol=0, atol=1e-3)
