"""The decode calls inside HIP graph capture (torch.cuda.graph).

fd_decode_ex with a caller workspace allocates nothing and queues only
kernels on the caller's stream, so it can be captured once and replayed.
Each replay here follows a change of the inputs in place and some eager
work with a synchronisation, and must equal an eager call on the same
inputs bit for bit (same plan, so same bits); the fused merge's tickets
must come back to zero after every replay.  The paged call, which uses the
library's own workspace, is captured after a warm-up call has sized it.
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
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


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


def test_captured_paged_decode_after_warm_up(torch):
    w = wl.EXTRA_WORKLOADS["paged_hm_p64_b1_gqa8_h64_d128_l65536"].with_(
        Lmax=4096)
    q, kp, vp, bt, sl, _, _ = wl.device_paged_inputs(w)
    out_g, lse_g = fd.fd_decode_paged(q, kp, vp, bt, sl, w.scale,
                                      head_major=True)   # sizes the workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_decode_paged(q, kp, vp, bt, sl, w.scale, out=out_g, lse=lse_g,
                           head_major=True)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[graph] paged replay {rep}", flush=True)
        q.mul_(0.5 if rep % 2 else -2.0)
        g.replay()
        torch.cuda.synchronize()
        out_e, lse_e = fd.fd_decode_paged(q, kp, vp, bt, sl, w.scale,
                                          head_major=True)
        torch.cuda.synchronize()
        assert _same(torch, out_g, out_e), f"replay {rep} out differs"
        assert torch.equal(lse_g, lse_e), f"replay {rep} lse differs"
