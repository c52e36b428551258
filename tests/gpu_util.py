"""Helpers for the GPU tests: put seeded workloads on the device, run the
library, compare with the oracle."""
from __future__ import annotations

import numpy as np

from long_context_decode_fd_amd import workloads as wl


to_dev = wl.to_device
dev_inputs = wl.device_inputs


def out_to_host(t) -> np.ndarray:
    """Device out tensor -> uint16 bf16 bits or float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def sample_rows(w: wl.Workload, seqlens, n: int, seed: int = 0):
    """(b, h) rows to check one by one: first, last, the shortest and the
    longest sequence, and n random others."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (w.B - 1, w.Hq - 1)}
    if seqlens is not None:
        rows.add((int(np.argmin(seqlens)), 0))
        rows.add((int(np.argmax(seqlens)), w.Hq // 2))
    target = min(len(rows) + n, w.B * w.Hq)
    while len(rows) < target:
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq))))
    return sorted(rows)


def oracle_rows(oracle_mod, w: wl.Workload, seqlens, rows):
    """Exact out/lse for the given (b, h) rows, regenerating only the
    slabs they read."""
    q = wl.gen_q(w)
    res = {}
    by_slab = {}
    for b, h in rows:
        by_slab.setdefault((b, h // w.G), []).append(h)
    for (b, g), hs in by_slab.items():
        L = wl.seqlen_of(w, seqlens, b)
        kr, vr = wl.gen_slab_rows(w, b, g, L)
        if L == 0:
            kr = np.zeros((1, w.D), w.np_dtype)
            vr = np.zeros((1, w.D), w.np_dtype)
        for h in hs:
            res[(b, h)] = oracle_mod.attend_row(q[b, h], kr, vr, L, w.scale)
    return res
