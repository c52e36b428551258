"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark uses (fd_decode, planner's choices).

The oracle checks a sample of (b, head) rows one by one (the first and last
rows, the shortest and longest sequence, random others), regenerating only
the slabs they read.  Every row is checked against properties that hold at
any size: finite results, the output inside the per-column range of V (a
convex combination), the split plan agreeing with the unsplit single pass,
and bitwise repeatability.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import dev_inputs, oracle_rows, out_to_host, sample_rows
from parity import check_lse, check_out

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return torch


@pytest.mark.parametrize("name", wl.WORKLOAD_ORDER)
def test_full_size_workload(cuda, oracle_mod, name):
    torch = cuda
    w = wl.WORKLOADS[name]
    print(f"[fullsize] {name}: generating", flush=True)
    q, k, v, sl, seqlens, _ = dev_inputs(w)
    plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, w.dtype,
                      varlen=sl is not None)
    print(f"[fullsize] {name}: plan {plan}", flush=True)
    out, lse = fd.fd_decode(q, k, v, sl, w.scale)
    out2, lse2 = fd.fd_decode(q, k, v, sl, w.scale)
    one, lse1 = fd.fd_decode_ex(q, k, v, sl, w.scale, num_splits=1)
    torch.cuda.synchronize()

    # bitwise repeatable
    assert torch.equal(out.view(torch.int16) if w.dtype == "bf16" else out,
                       out2.view(torch.int16) if w.dtype == "bf16" else out2)
    assert torch.equal(lse, lse2)

    # every row: finite where the sequence is non-empty, inside V's range
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

    # sampled rows against the oracle
    rows = sample_rows(w, seqlens, n=10, seed=w.seed)
    ref = oracle_rows(oracle_mod, w, seqlens, rows)
    o_h = out_to_host(out)
    l_h = lse.cpu().numpy()
    got_o = np.stack([o_h[b, h] for b, h in rows])
    got_l = np.array([l_h[b, h] for b, h in rows])
    ref_o = np.stack([ref[r][0] for r in rows])
    ref_l = np.array([ref[r][1] for r in rows])
    ok_o, rep_o = check_out(got_o, ref_o, w.dtype)
    ok_l, rep_l = check_lse(got_l, ref_l)
    print(f"[fullsize] {name}: rows {rows}\n  out {rep_o}\n  lse {rep_l}",
          flush=True)
    assert ok_o, rep_o
    assert ok_l, rep_l
