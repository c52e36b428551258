"""Helpers for the GPU tests: put seeded workloads on the device, run the
library, compare with the oracle."""
from __future__ import annotations

import numpy as np

from long_context_decode_fd_amd import workloads as wl


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def out_to_host(t) -> np.ndarray:
    """Device out tensor -> uint16 bf16 bits or float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dev_inputs(w: wl.Workload, seqlens=None, keep_host=False):
    """q, k, v (device), seqlens (device or None), seqlens (host), host
    arrays (if keep_host).  K/V are generated slab by slab; padding rows are
    filled with NaN on the device."""
    import torch
    if seqlens is None:
        seqlens = wl.gen_seqlens(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q_h = wl.gen_q(w)
    q = to_dev(q_h)
    shape = (w.B, w.Hkv, w.Lmax, w.D)
    k = torch.empty(shape, dtype=tdt, device="cuda")
    v = torch.empty(shape, dtype=tdt, device="cuda")
    if seqlens is not None:
        iv = torch.int16 if w.dtype == "bf16" else torch.int32
        k.view(iv).fill_(-1)       # all-ones bits: NaN poison
        v.view(iv).fill_(-1)
    host = None
    if keep_host:
        host = (q_h, np.empty(shape, w.np_dtype), np.empty(shape, w.np_dtype))
    for b in range(w.B):
        L = wl.seqlen_of(w, seqlens, b)
        for g in range(w.Hkv):
            kr, vr = wl.gen_slab_rows(w, b, g, L)
            if L:
                k[b, g, :L].copy_(to_dev(kr))
                v[b, g, :L].copy_(to_dev(vr))
            if keep_host:
                host[1][b, g, :L], host[2][b, g, :L] = kr, vr
                if L < w.Lmax:
                    host[1][b, g, L:].view(np.uint8)[:] = 0xFF
                    host[2][b, g, L:].view(np.uint8)[:] = 0xFF
    sl_dev = None
    if seqlens is not None:
        sl_dev = torch.from_numpy(np.asarray(seqlens, np.int32)).to("cuda")
    return q, k, v, sl_dev, seqlens, host


def sample_rows(w: wl.Workload, seqlens, n: int, seed: int = 0):
    """(b, h) rows to check one by one: first, last, the shortest and the
    longest sequence, and n random others."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0), (w.B - 1, w.Hq - 1)}
    if seqlens is not None:
        rows.add((int(np.argmin(seqlens)), 0))
        rows.add((int(np.argmax(seqlens)), w.Hq // 2))
    while len(rows) < n + 2:
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
