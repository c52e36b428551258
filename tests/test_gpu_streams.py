"""Concurrent calls on two streams, each with its own workspace.

fd_decode_ex keeps no state of its own when the caller passes a workspace
(fd.h): launches interleaved on two streams -- one with the separate merge,
one with the fused merge whose tickets live in its workspace -- must each
give the same bits as the same calls made one after another.
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


def test_two_streams_with_their_own_workspaces(torch):
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=4, Lmax=6000, varlen=(1, 6000))
    sl = np.array([6000, 4097, 1, 2500], np.int32)
    q, k, v, sld, _, _ = dev_inputs(w, seqlens=sl)
    F = fd.FD_FLAG_FUSED_MERGE
    calls = {"separate": (0, 5), "fused": (F, 9)}
    ws, refs, outs = {}, {}, {}
    for name, (flags, splits) in calls.items():
        nb = fd.fd_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16",
                                   varlen=True, num_splits=splits,
                                   flags=flags)
        ws[name] = torch.zeros(max(nb, 256), dtype=torch.uint8,
                               device="cuda")
        refs[name] = fd.fd_decode_ex(q, k, v, sld, w.scale,
                                     num_splits=splits, flags=flags,
                                     workspace=ws[name])
        outs[name] = (torch.empty_like(q),
                      torch.empty(w.B, w.Hq, device="cuda"))
    torch.cuda.synchronize()
    streams = {name: torch.cuda.Stream() for name in calls}
    for s in streams.values():
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(6):
        for name, (flags, splits) in calls.items():
            s = streams[name]
            with torch.cuda.stream(s):
                fd.fd_decode_ex(q, k, v, sld, w.scale, out=outs[name][0],
                                lse=outs[name][1], num_splits=splits,
                                flags=flags, workspace=ws[name], stream=s)
    torch.cuda.synchronize()
    for name in calls:
        o, l = outs[name]
        ro, rl = refs[name]
        print(f"[streams] {name}: checked", flush=True)
        assert torch.equal(o.view(torch.int16), ro.view(torch.int16)), name
        assert torch.equal(l, rl), name
    # the fused call's tickets are back at zero after the interleaved calls
    p = fd.fd_plan(w.B, w.Hq, w.Hkv, w.D, w.Lmax, "bf16", varlen=True,
                   num_splits=9, flags=F)
    assert int(ws["fused"][:p["ticket_bytes"]].count_nonzero()) == 0
