"""The full-size parity helper on the CPU: upload_full's per-batch-entry
oracle rows equal the oracle run over the whole batch at once, and its
uploaded tensors equal gen_all's arrays (NaN past every length)."""
import numpy as np
import pytest

from long_context_decode_fd_amd import workloads as wl
from gpu_util import upload_full


@pytest.mark.parametrize("Tq", [1, 3])
def test_upload_full_rows_equal_the_whole_batch_oracle(oracle_mod, Tq):
    torch = pytest.importorskip("torch")
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=3, Hq=8, Hkv=2, Lmax=400, varlen=(1, 400), Tq=Tq)
    seqlens = np.array([400, 0, 129], np.int32)
    q, k, v, sl, _, ref = upload_full(w, oracle_mod, seqlens=seqlens,
                                      device="cpu")
    qh, kh, vh, _ = wl.gen_all(w, seqlens=seqlens)
    if Tq > 1:
        ro, rl = oracle_mod.decode_multiquery(qh, kh, vh, seqlens, w.scale)
    else:
        ro, rl = oracle_mod.decode(qh, kh, vh, seqlens, w.scale)
    np.testing.assert_array_equal(ref[0], ro)
    np.testing.assert_array_equal(ref[1], rl)
    assert ref[0].shape == qh.shape
    np.testing.assert_array_equal(
        k.view(torch.int16).numpy().view(np.uint16), kh)
    np.testing.assert_array_equal(
        v.view(torch.int16).numpy().view(np.uint16), vh)
    np.testing.assert_array_equal(sl.numpy(), seqlens)
