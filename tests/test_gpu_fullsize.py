"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark uses (fd_decode, planner's choices), on EVERY row.

The operation is the one of "Flash-Decoding for long-context inference"
(Stanford CRFM), section "Multi-head attention for decoding".  Each
workload is uploaded slab by slab; each batch entry's slabs stay on the
host just long enough for the fp64 oracle to attend all of its query rows
(gpu_util.upload_full), so every (b, head) row of out and lse is compared
element by element with the oracle under the suite's tolerance rule.  The
single-pass plan (num_splits = 1) is compared with the oracle the same way.
Extras that hold at any size: bitwise repeatability, the output inside the
per-column range of V (a convex combination), split and single pass
agreeing.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import out_to_host, upload_full
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return torch


def _compare_all_rows(name, label, out, lse, ref, dtype):
    ok_o, rep_o = check_out(out_to_host(out), ref[0], dtype)
    ok_l, rep_l = check_lse(lse.cpu().numpy(), ref[1])
    print(f"[fullsize] {name} {label}: every row against the oracle\n"
          f"  out {rep_o}\n  lse {rep_l}", flush=True)
    assert ok_o, rep_o
    assert ok_l, rep_l


@pytest.mark.parametrize("name", wl.WORKLOAD_ORDER +
                         ["f32_b1_gqa8_h64_d128_l65536",
                          "f16_b1_gqa8_h64_d128_l65536",
                          "f16_varlen_b16_gqa8_h64_d128_lmax131072"])
def test_full_size_workload(cuda, oracle_mod, name):
    torch = cuda
    w = wl.ALL_WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs and the oracle's rows",
          flush=True)
    q, k, v, sl, seqlens, ref = upload_full(w, oracle_mod)
    plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                      varlen=sl is not None)
    print(f"[fullsize] {name}: plan {plan}", flush=True)
    out, lse = fd.fd_decode(q, k, v, sl, w.scale)
    out2, lse2 = fd.fd_decode(q, k, v, sl, w.scale)
    one, lse1 = fd.fd_decode_ex(q, k, v, sl, w.scale, num_splits=1)
    torch.cuda.synchronize()

    _compare_all_rows(name, f"planner's plan (S = {plan['num_splits']})",
                      out, lse, ref, w.dtype)
    _compare_all_rows(name, "single pass (S = 1)", one, lse1, ref, w.dtype)

    # bitwise repeatable
    bits = (lambda t: t.view(torch.int16)) if w.dtype != "f32" else \
        (lambda t: t)
    assert torch.equal(bits(out), bits(out2))
    assert torch.equal(lse, lse2)

    # every row inside V's column range (a convex combination of V rows)
    L = (torch.full((w.B,), w.Lmax, device="cuda") if sl is None
         else sl.clamp(0, w.Lmax))
    live = (L > 0)[:, None].expand(w.B, w.Hq)
    of = out.float()
    assert torch.isfinite(of[live]).all() and torch.isfinite(lse[live]).all()
    vmax = torch.empty((w.B, w.Hkv, w.D), device="cuda")
    vmin = torch.empty((w.B, w.Hkv, w.D), device="cuda")
    for b in range(w.B):
        n = int(L[b])
        if n:
            vf = v[b, :, :n].float()
            vmax[b], vmin[b] = vf.amax(1), vf.amin(1)
        else:
            vmax[b], vmin[b] = 0.0, 0.0
    vmax = vmax.repeat_interleave(w.G, dim=1)
    vmin = vmin.repeat_interleave(w.G, dim=1)
    slack = 1e-2 + 2 ** -7 * torch.maximum(vmax.abs(), vmin.abs())
    assert bool((of <= vmax + slack).all() and (of >= vmin - slack).all())

    # the split plan and the single pass agree everywhere
    d_out = (of - one.float()).abs().max().item()
    d_lse = (lse - lse1).abs()[live].max().item()
    print(f"[fullsize] {name}: split vs single pass: out {d_out:.2e} "
          f"lse {d_lse:.2e}", flush=True)
    assert d_out <= 2e-2 and d_lse <= 1e-3
