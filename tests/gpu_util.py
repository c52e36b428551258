"""Helpers for the GPU tests: put seeded workloads on the device, run the
library, compare with the oracle."""
from __future__ import annotations

import numpy as np

from long_context_decode_fd_amd import workloads as wl


to_dev = wl.to_device
dev_inputs = wl.device_inputs


def out_to_host(t) -> np.ndarray:
    """Device out tensor -> uint16 bf16 bits, float16 or float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def upload_full(w: wl.Workload, oracle_mod=None, seqlens=None,
                device: str = "cuda"):
    """Device inputs of workload w, built slab by slab as
    wl.device_inputs builds them, and, with oracle_mod, the oracle's
    out/lse for EVERY row: each batch entry's slabs are kept on the host
    just long enough for the fp64 oracle to attend all its query rows
    (all host threads), so no padded host copy of the cache is made.

    Returns (q, k, v, seqlens_dev, seqlens_host, ref) with ref =
    (out [B, Hq, D] or [B, Tq, Hq, D], lse [B, Hq] or [B, Tq, Hq]),
    float64, or None without oracle_mod."""
    import torch
    if seqlens is None:
        seqlens = wl.gen_seqlens(w)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16,
           "f32": torch.float32}[w.dtype]
    q_h = wl.gen_q(w)
    q = to_dev(q_h, device)
    shape = (w.B, w.Hkv, w.Lmax, w.D)
    k = torch.empty(shape, dtype=tdt, device=device)
    v = torch.empty(shape, dtype=tdt, device=device)
    if seqlens is not None:
        iv = torch.int32 if w.dtype == "f32" else torch.int16
        k.view(iv).fill_(-1)            # NaN past every length
        v.view(iv).fill_(-1)
    ref = None
    if oracle_mod is not None:
        ref = (np.empty(q_h.shape, np.float64),
               np.empty(q_h.shape[:-1], np.float64))
    slab = {}

    def attend(b):
        L = slab["L"]
        sl1 = np.array([L], np.int32)
        if w.Tq > 1:
            o, l = oracle_mod.decode_multiquery(q_h[b:b + 1], slab["k"],
                                                slab["v"], sl1, w.scale)
        else:
            o, l = oracle_mod.decode(q_h[b:b + 1], slab["k"], slab["v"],
                                     sl1, w.scale)
        ref[0][b], ref[1][b] = o[0], l[0]

    for b, g, L, kr, vr in wl.iter_slabs(w, seqlens):
        if L:
            k[b, g, :L].copy_(to_dev(kr, device))
            v[b, g, :L].copy_(to_dev(vr, device))
        if ref is None:
            continue
        if slab.get("b") != b:
            if "b" in slab:
                attend(slab["b"])
            n = max(L, 1)
            slab = {"b": b, "L": L,
                    "k": np.zeros((1, w.Hkv, n, w.D), w.np_dtype),
                    "v": np.zeros((1, w.Hkv, n, w.D), w.np_dtype)}
        slab["k"][0, g, :L], slab["v"][0, g, :L] = kr, vr
    if ref is not None and "b" in slab:
        attend(slab["b"])
    sl_dev = None
    if seqlens is not None:
        sl_dev = torch.from_numpy(np.asarray(seqlens, np.int32)).to(device)
    return q, k, v, sl_dev, seqlens, ref
