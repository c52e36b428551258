"""The decode calls inside HIP graph capture (torch.cuda.graph).

fd_decode_ex with a caller workspace allocates nothing and queues only
kernels on the caller's stream, so it can be captured once and replayed.
Each replay here follows a change of the inputs in place and some eager
work with a synchronisation, and must equal an eager call on the same
inputs bit for bit (same plan, so same bits); the fused merge's tickets
must come back to zero after every replay.  The paged and multi-token
calls are captured with a caller workspace too.  A call that would use the
library-owned workspace is refused under capture (FD_ERR_CAPTURE), while a
plan that needs no workspace at all captures through fd_decode itself.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import dev_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


def _same(torch, a, b):
    """Bitwise equality of two bf16 or fp32 tensors."""
    it = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.view(it), b.view(it))


@pytest.mark.parametrize("flags", [0, fd.FD_FLAG_FUSED_MERGE])
def test_captured_decode_replays_match_eager(torch, flags):
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=3, Lmax=3000, varlen=(1, 3000))
    seqlens = np.array([3000, 1234, 17], np.int32)
    q, k, v, sl, _, _ = dev_inputs(w, seqlens=seqlens)
    nbytes = fd.fd_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16",
                                   varlen=True, flags=flags)
    plan = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", varlen=True,
                      flags=flags)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out_g = torch.empty_like(q)
    lse_g = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    # warm up once outside the capture
    fd.fd_decode_ex(q, k, v, sl, w.scale, out=out_g, lse=lse_g, flags=flags,
                    workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_decode_ex(q, k, v, sl, w.scale, out=out_g, lse=lse_g,
                        flags=flags, workspace=ws)
    torch.cuda.synchronize()
    ws_eager = torch.zeros_like(ws)
    for rep in range(4):
        print(f"[graph] flags={flags} replay {rep}", flush=True)
        q.mul_(-1.0 if rep % 2 else 1.5)       # new inputs, in place
        g.replay()
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work
        torch.cuda.synchronize()
        out_e, lse_e = fd.fd_decode_ex(q, k, v, sl, w.scale, flags=flags,
                                       workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert _same(torch, out_g, out_e), f"replay {rep} out differs"
        assert torch.equal(lse_g, lse_e), f"replay {rep} lse differs"
        if plan["ticket_bytes"]:
            tickets = ws[:plan["ticket_bytes"]].view(torch.int32)
            assert int(tickets.abs().sum()) == 0, "tickets not reset"


def _replays_match_eager(torch, g, q, outs_g, eager, reps, tag):
    for rep in range(reps):
        print(f"[graph] {tag} replay {rep}", flush=True)
        q.mul_(0.5 if rep % 2 else -2.0)       # new inputs, in place
        g.replay()
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work
        torch.cuda.synchronize()
        outs_e = eager()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert _same(torch, outs_g[0], outs_e[0]), f"replay {rep} out"
        assert torch.equal(outs_g[1], outs_e[1]), f"replay {rep} lse"


@pytest.mark.parametrize("flags", [0, fd.FD_FLAG_FUSED_MERGE])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_captured_paged_decode_with_caller_workspace(torch, flags, dtype):
    w = wl.EXTRA_WORKLOADS["paged_hm_p64_b1_gqa8_h64_d128_l65536"].with_(
        Lmax=4096, dtype=dtype)
    q, kp, vp, bt, sl, _, _ = wl.device_paged_inputs(w)
    plan = fd.fd_plan_ex(w.B, w.Tq, w.Hq, w.Hkv, w.D,
                         w.max_pages * w.page_size, dtype, paged=True,
                         flags=flags)
    assert plan["combine"]
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8,
                     device="cuda")
    out_g = torch.empty_like(q)
    lse_g = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_decode_paged(q, kp, vp, bt, sl, w.scale, out=out_g, lse=lse_g,
                           flags=flags, head_major=True, workspace=ws)
    torch.cuda.synchronize()
    _replays_match_eager(
        torch, g, q, (out_g, lse_g),
        lambda: fd.fd_decode_paged(q, kp, vp, bt, sl, w.scale, flags=flags,
                                   head_major=True), 3,
        f"paged {dtype} {flags}")
    if plan["ticket_bytes"]:
        assert int(ws[:plan["ticket_bytes"]].count_nonzero()) == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_captured_multiquery_decode_with_caller_workspace(torch, dtype):
    w = wl.EXTRA_WORKLOADS["mq2_b1_gqa8_h64_d128_l65536"].with_(Lmax=4096,
                                                                 dtype=dtype)
    q, k, v, sl, _, _ = dev_inputs(w)
    plan = fd.fd_plan_ex(w.B, w.Tq, w.Hq, w.Hkv, w.D, w.Lmax, dtype)
    assert plan["combine"]
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8,
                     device="cuda")
    out_g = torch.empty_like(q)
    lse_g = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_decode_multiquery(q, k, v, sl, w.scale, out=out_g, lse=lse_g,
                                workspace=ws)
    torch.cuda.synchronize()
    _replays_match_eager(
        torch, g, q, (out_g, lse_g),
        lambda: fd.fd_decode_multiquery(q, k, v, sl, w.scale), 3,
        f"mq {dtype}")


def test_owned_workspace_is_refused_under_capture(torch):
    """Capturing a split plan on the library's workspace fails with
    FD_ERR_CAPTURE and queues nothing; a single-pass plan (no workspace)
    captures through fd_decode and replays like an eager call."""
    w = wl.WORKLOADS["b64_gqa4_h32_d128_l4096"].with_(B=2, Lmax=2048)
    q, k, v, sl, _, _ = dev_inputs(w)
    out_g = torch.empty_like(q)
    lse_g = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    split = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16")
    assert split["combine"]
    marker = torch.zeros(1, device="cuda")
    errors = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        marker.add_(1.0)
        try:
            fd.fd_decode(q, k, v, sl, w.scale, out=out_g, lse=lse_g)
        except fd.FdError as e:
            errors.append(e.code)
    torch.cuda.synchronize()
    assert errors == [fd.FD_ERR_CAPTURE]
    g.replay()
    torch.cuda.synchronize()
    assert float(marker) == 1.0      # only the marker was captured
    # a plan that needs no workspace: captured through fd_decode itself
    wb = w.with_(B=64)
    qb, kb, vb, slb, _, _ = dev_inputs(wb)
    assert not fd.fd_plan(wb.B, wb.Hq, wb.Hkv, wb.D, wb.Lmax,
                          "bf16")["combine"]
    ob = torch.empty_like(qb)
    lb = torch.empty((wb.B, wb.Hq), dtype=torch.float32, device="cuda")
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        fd.fd_decode(qb, kb, vb, slb, wb.scale, out=ob, lse=lb)
    torch.cuda.synchronize()
    _replays_match_eager(
        torch, g2, qb, (ob, lb),
        lambda: fd.fd_decode(qb, kb, vb, slb, wb.scale), 2, "single pass")
