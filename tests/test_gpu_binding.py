"""The Python binding's own checks, on the GPU.

The binding only marshals arguments, but it is the layer that knows which
device a tensor lives on: the library plans for, and keeps its own
workspace on, the current HIP device, so the binding makes the tensors'
device current for each call.  Before anything is launched it rejects
tensors, workspaces or streams on another device, and outputs that overlap
an input.
"""
import numpy as np
import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import workloads as wl
from gpu_util import dev_inputs

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
    B=3, Lmax=2500, varlen=(1, 2500))
SEQLENS = np.array([2500, 1, 1300], np.int32)


@pytest.fixture(scope="module")
def torch():
    t = pytest.importorskip("torch")
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    fd.load_library()
    return t


@pytest.fixture(scope="module")
def inputs(torch):
    return dev_inputs(W, seqlens=SEQLENS)


def test_host_tensors_are_rejected_before_any_launch(torch, inputs):
    q, k, v, sl, _, _ = inputs
    with pytest.raises(ValueError, match="seqlens"):
        fd.fd_decode(q, k, v, sl.cpu(), W.scale)
    with pytest.raises(ValueError, match="out"):
        fd.fd_decode(q, k, v, sl, W.scale, out=torch.empty_like(q.cpu()))
    nb = fd.fd_workspace_bytes(W.B, W.Hq, W.Hkv, W.D, W.Lmax, "bf16",
                               varlen=True)
    host_ws = torch.zeros(nb, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace"):
        fd.fd_decode_ex(q, k, v, sl, W.scale, workspace=host_ws)
    with pytest.raises(ValueError, match="workspace"):
        fd.fd_decode_partials(q, k, v, sl, W.scale, host_ws)
    out = torch.empty_like(q)
    lse = torch.empty(W.B, W.Hq, device="cuda")
    dev_ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="seqlens"):
        fd.fd_merge_partials(sl.long(), W.B, W.Hq, W.Hkv, W.D, W.Lmax,
                             "bf16", dev_ws, out, lse)


def test_outputs_that_overlap_inputs_are_rejected(torch, inputs):
    q, k, v, sl, _, _ = inputs
    with pytest.raises(ValueError, match="out overlaps q"):
        fd.fd_decode(q, k, v, sl, W.scale, out=q)
    nb = fd.fd_workspace_bytes(W.B, W.Hq, W.Hkv, W.D, W.Lmax, "bf16",
                               varlen=True)
    ws = torch.zeros(nb + 4 * W.B * W.Hq, dtype=torch.uint8, device="cuda")
    lse_in_ws = ws[nb:].view(torch.float32).view(W.B, W.Hq)
    with pytest.raises(ValueError, match="lse overlaps workspace"):
        fd.fd_decode_ex(q, k, v, sl, W.scale, lse=lse_in_ws, workspace=ws)


def test_explicit_stream_and_current_device(torch, inputs):
    q, k, v, sl, _, _ = inputs
    ref_o, ref_l = fd.fd_decode(q, k, v, sl, W.scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    before = torch.cuda.current_device()
    with torch.cuda.stream(s):
        o, l = fd.fd_decode(q, k, v, sl, W.scale, stream=s)
    assert torch.cuda.current_device() == before
    s.synchronize()
    assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(l, ref_l)
