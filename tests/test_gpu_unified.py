"""GPU parity of the unified-maximum softmax (fd_decode_unified_max).

The same attention as fd_decode_ex, computed per chunk against a fixed
estimate phi of the row maximum; a chunk whose scores leave phi +- 64 ln 2
is recomputed with the running maximum.  Checked element by element against
the fp64 oracle for the bf16 shapes at several split counts and phi values;
with phi far from every score each chunk takes the fallback, whose result
must then equal fd_decode_ex's bit for bit; rows with scores far above the
others force the fallback in some chunks only.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import dev_inputs, out_to_host, upload_full
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
SMALL = {
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
    "f16_b1_gqa8": W["b1_gqa8_h64_d128_l65536"].with_(Lmax=4133,
                                                      dtype="f16"),
    "f16_varlen_gqa8": W["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=6, Lmax=4096, varlen=(1, 4096), dtype="f16"),
}


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


_cache = {}


def inputs(name, w):
    if name not in _cache:
        _cache.clear()
        _cache[name] = dev_inputs(w, keep_host=True)
    return _cache[name]


def _parity(w, out, lse, ref_o, ref_l, what):
    ok_o, rep_o = check_out(out_to_host(out), ref_o, w.dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref_l)
    print(f"[unified] {what}: out {rep_o} lse {rep_l}", flush=True)
    assert ok_o, (what, rep_o)
    assert ok_l, (what, rep_l)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("splits,flags,phi", [
    (0, 0, 0.0), (1, 0, 0.0), (7, 0, 0.0), (0, 0, 5.0), (0, 0, -20.0),
    (0, fd.FD_FLAG_FUSED_MERGE, 0.0)])
def test_unified_matches_oracle(torch, oracle_mod, name, splits, flags, phi):
    w = SMALL[name]
    q, k, v, sl, seqlens, host = inputs(name, w)
    out, lse = fd.fd_decode_unified_max(q, k, v, sl, w.scale, phi,
                                        num_splits=splits, flags=flags)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode(*host, seqlens, w.scale)
    _parity(w, out, lse, ref_o, ref_l,
            f"{name} splits={splits} flags={flags} phi={phi}")


@pytest.mark.parametrize("phi", [1000.0, -1000.0, 60.0])
@pytest.mark.parametrize("splits", [0, 5])
def test_fallback_reproduces_the_exact_pass_bitwise(torch, phi, splits):
    # Every score is far from phi (beyond 64 ln 2 ~ 44.4), so every chunk
    # is recomputed with the running maximum: fd_decode_ex's bits.
    w = SMALL["varlen_gqa8"]
    q, k, v, sl, _, _ = inputs("varlen_gqa8", w)
    uo, ul = fd.fd_decode_unified_max(q, k, v, sl, w.scale, phi,
                                      num_splits=splits)
    eo, el = fd.fd_decode_ex(q, k, v, sl, w.scale, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(uo.view(torch.int16), eo.view(torch.int16))
    assert torch.equal(ul, el)


@pytest.mark.parametrize("phi,fallback", [(-20.0, True), (20.0, True),
                                          (-3.0, False), (-1.0, False)])
def test_fp16_window_is_narrower(torch, oracle_mod, phi, fallback):
    # fp16 P operands stop at 65504 and flush below 2^-24: a chunk row
    # whose largest score lies outside [phi, phi + 14 ln 2] (~9.7) is
    # recomputed with the running maximum (bitwise fd_decode_ex); within
    # it the unified pass stands and still meets the oracle.
    w = SMALL["f16_varlen_gqa8"]
    q, k, v, sl, seqlens, host = inputs("f16_varlen_gqa8", w)
    uo, ul = fd.fd_decode_unified_max(q, k, v, sl, w.scale, phi)
    eo, el = fd.fd_decode_ex(q, k, v, sl, w.scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode(*host, seqlens, w.scale)
    _parity(w, uo, ul, ref_o, ref_l, f"fp16 window phi={phi}")
    same = (torch.equal(uo.view(torch.int16), eo.view(torch.int16))
            and torch.equal(ul, el))
    if fallback:
        assert same
    else:
        assert not same


def test_fallback_in_some_chunks_only(torch, oracle_mod):
    # Sequence 0's first 100 keys of KV head 0 are pushed far above phi:
    # the chunk holding them falls back, every other chunk does not.
    w = SMALL["b1_gqa8"].with_(B=2)
    q, k, v, sl, seqlens, host = dev_inputs(w, keep_host=True)
    qh, kh, vh = host
    kh = kh.copy()
    qrow = wl.bf16_to_f32(qh[0, 0]).astype(np.float64)
    push = 80.0 / w.scale * qrow / np.dot(qrow, qrow)    # score + ~80
    kh[0, 0, :100] = wl.bf16_bits((wl.bf16_to_f32(kh[0, 0, :100])
                                   + push.astype(np.float32)))
    k = wl.to_device(kh)
    for splits in (0, 8):
        out, lse = fd.fd_decode_unified_max(q, k, v, sl, w.scale, 0.0,
                                            num_splits=splits)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_mod.decode(qh, kh, vh, seqlens, w.scale)
        _parity(w, out, lse, ref_o, ref_l, f"partial fallback S={splits}")
        assert ref_l[0, 0] > 40 and abs(ref_l[1, 0]) < 20


def test_edges_and_nan_padding(torch, oracle_mod):
    w = SMALL["varlen_gqa8"].with_(B=6, Lmax=700)
    seqlens = np.array([0, 1, 31, 32, 33, 700], np.int32)
    q, k, v, sl, _, host = dev_inputs(w, seqlens=seqlens, keep_host=True)
    out, lse = fd.fd_decode_unified_max(q, k, v, sl, w.scale, 0.0)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mod.decode(*host, seqlens, w.scale)
    _parity(w, out, lse, ref_o, ref_l, "edges")
    assert float(lse[0].max()) == float("-inf")
    assert torch.count_nonzero(out[0].float()) == 0


def test_full_size_headline_shape(torch, oracle_mod):
    """Batch-1 64k in the planner's configuration, phi = 0: every row
    against the oracle, every row close to the exact pass, repeatable."""
    w = W["b1_gqa8_h64_d128_l65536"]
    q, k, v, sl, seqlens, ref = upload_full(w, oracle_mod)
    uo, ul = fd.fd_decode_unified_max(q, k, v, sl, w.scale, 0.0)
    uo2, ul2 = fd.fd_decode_unified_max(q, k, v, sl, w.scale, 0.0)
    eo, el = fd.fd_decode(q, k, v, sl, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(uo.view(torch.int16), uo2.view(torch.int16))
    assert torch.equal(ul, ul2)
    d_out = (uo.float() - eo.float()).abs().max().item()
    d_lse = (ul - el).abs().max().item()
    print(f"[unified] 64k vs exact pass: out {d_out:.2e} lse {d_lse:.2e}",
          flush=True)
    assert d_out <= 2e-2 and d_lse <= 1e-3
    ok_o, rep_o = check_out(out_to_host(uo), ref[0], w.dtype)
    ok_l, rep_l = check_lse(ul.cpu().numpy(), ref[1])
    print(f"[unified] 64k every row: out {rep_o} lse {rep_l}", flush=True)
    assert ok_o and ok_l
