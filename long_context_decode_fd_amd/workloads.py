"""Seeded synthetic decode workloads (inputs only; no attention arithmetic).

This module is the one piece shared by the GPU tests, the benchmark and the
fp64 oracle's tests: it draws the inputs both sides receive.  It computes
nothing of the method itself.

The workloads mirror the long-context decode settings that "Flash-Decoding
for long-context inference" (Stanford CRFM) motivates in its "Motivation"
section (batch 1 at tens of thousands of tokens, small batches at long
context, large batches at short context) plus a variable-length batch as in
serving.  The pages name no dataset; everything is synthetic.

Recipe (every stream is an independent PCG64 seeded from
``SeedSequence(seed, spawn_key=...)`` so any one slab can be rebuilt alone):

* q           spawn_key (0,)        standard normal float32 -> dtype,
                                     [B, Hq, D] ([B, Tq, Hq, D] if Tq > 1)
* seqlens     spawn_key (4,)        u ~ U[0,1): floor(lo * (hi/lo)**u), <= hi
* pages       spawn_key (5,)        paged cache: the pool holds
                                     B * max_pages + spare pages; the block
                                     table is a random permutation's first
                                     B * max_pages entries
* K[b, g]     spawn_key (1, b, g)   standard normal float32 rows [0, L_b)
* V[b, g]     spawn_key (2, b, g)   standard normal float32 rows [0, L_b)
* peaks[b, g] spawn_key (3, b, g)   ceil(frac * L_b) distinct rows of K
                                     multiplied by ``peak_mult`` (exact)
* rows >= L_b of a padded slab hold NaN (bf16 and fp16 0xFFFF, fp32
  0xFFFFFFFF) so
  that a kernel reading past the valid prefix is caught; so do the unused
  rows of a sequence's last page and every spare page of a paged pool.

bf16 values are produced by rounding float32 to nearest-even on the bit
pattern and are handled as ``numpy.uint16`` arrays throughout; fp16 values
are numpy's own float32 -> float16 conversion (nearest-even) and are
handled as ``numpy.float16`` arrays.
"""
from __future__ import annotations

import math
import os
from collections import deque
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0xFFFF)
F32_NAN_BITS = np.uint32(0xFFFFFFFF)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    Lmax: int
    dtype: str            # "bf16", "f16" or "f32"
    seed: int
    peak_frac: float = 0.0
    peak_mult: float = 8.0
    varlen: tuple | None = None   # (lo, hi) for log-uniform seqlens
    Tq: int = 1                   # new query tokens per sequence
    page_size: int = 0            # > 0: K/V in a paged pool
    head_major: bool = False      # pages [Hkv][t][D], else [t][Hkv][D]
    note: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def np_dtype(self):
        return {"bf16": np.uint16, "f16": np.float16,
                "f32": np.float32}[self.dtype]

    @property
    def max_pages(self) -> int:
        return -(-self.Lmax // self.page_size)

    @property
    def num_pages(self) -> int:
        n = self.B * self.max_pages
        return n + 2 + n // 16          # a few spare pages stay unused

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five decode settings, by what they are.
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_mha_f32_b1_h8_d64_l1024", B=1, Hq=8, Hkv=8, D=64,
                 Lmax=1024, dtype="f32", seed=1,
                 note="tiny multi-head decode in fp32"),
        Workload("b1_gqa8_h64_d128_l65536", B=1, Hq=64, Hkv=8, D=128,
                 Lmax=65536, dtype="bf16", seed=2,
                 note="batch-1 long context, grouped-query (8 per KV head)"),
        Workload("b4_mha_h32_d128_l32768_peaked", B=4, Hq=32, Hkv=32, D=128,
                 Lmax=32768, dtype="bf16", seed=3, peak_frac=0.01,
                 peak_mult=8.0,
                 note="small batch, longer context, 1% of keys x8"),
        Workload("b64_gqa4_h32_d128_l4096", B=64, Hq=32, Hkv=8, D=128,
                 Lmax=4096, dtype="bf16", seed=4,
                 note="batch-dominated short context"),
        Workload("varlen_b16_gqa8_h64_d128_lmax131072", B=16, Hq=64, Hkv=8,
                 D=128, Lmax=131072, dtype="bf16", seed=5,
                 varlen=(1024, 131072),
                 note="variable-length batch, log-uniform seqlens"),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)
BENCH_WORKLOAD = "b1_gqa8_h64_d128_l65536"

# The same data behind the two cache layouts / query counts beyond plain
# decode: a vLLM-style paged pool, and several causal new tokens.
EXTRA_WORKLOADS = {
    w.name: w for w in [
        WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(
            name="paged_p64_b1_gqa8_h64_d128_l65536", page_size=64,
            note="batch-1 64k decode from 64-token pages"),
        WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(
            name="paged_hm_p64_b1_gqa8_h64_d128_l65536", page_size=64,
            head_major=True,
            note="batch-1 64k decode from 64-token head-major pages"),
        WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(
            name="paged_hm_p64_mq2_b1_gqa8_h64_d128_l65536", page_size=64,
            head_major=True, Tq=2,
            note="two causal new tokens over 64-token head-major pages"),
        WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
            name="paged_p16_varlen_b16_gqa8_h64_d128_lmax131072",
            page_size=16,
            note="variable-length batch from 16-token pages"),
        WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(
            name="mq2_b1_gqa8_h64_d128_l65536", Tq=2,
            note="two causal new tokens, batch-1 64k (16 q-tile columns)"),
        WORKLOADS["b64_gqa4_h32_d128_l4096"].with_(
            name="mq4_b64_gqa4_h32_d128_l4096", Tq=4,
            note="four causal new tokens, batch 64 at 4k"),
        WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(
            name="f32_b1_gqa8_h64_d128_l65536", dtype="f32",
            note="the batch-1 64k shape with an fp32 cache"),
        WORKLOADS["b1_gqa8_h64_d128_l65536"].with_(
            name="f16_b1_gqa8_h64_d128_l65536", dtype="f16",
            note="the batch-1 64k shape with an fp16 cache"),
        WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
            name="f16_varlen_b16_gqa8_h64_d128_lmax131072", dtype="f16",
            note="the variable-length batch with an fp16 cache"),
    ]
}
ALL_WORKLOADS = {**WORKLOADS, **EXTRA_WORKLOADS}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x0040).astype(np.uint16)
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32)


def _encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x32)
    return x32.astype(np.float16 if dtype == "f16" else np.float32)


def gen_seqlens(w: Workload) -> np.ndarray | None:
    """Per-sequence valid lengths (None: every sequence is Lmax long)."""
    if w.varlen is None:
        return None
    lo, hi = w.varlen
    u = _rng(w.seed, 4).random(w.B)
    s = np.floor(lo * np.power(hi / lo, u)).astype(np.int64)
    return np.minimum(s, hi).astype(np.int32)


def seqlen_of(w: Workload, seqlens, b: int) -> int:
    return w.Lmax if seqlens is None else int(seqlens[b])


def gen_q(w: Workload) -> np.ndarray:
    shape = ((w.B, w.Hq, w.D) if w.Tq == 1 else (w.B, w.Tq, w.Hq, w.D))
    x = _rng(w.seed, 0).standard_normal(shape, dtype=np.float32)
    return _encode(x, w.dtype)


def paged_seqlens(w: Workload, seqlens=None) -> np.ndarray:
    """A paged call always takes lengths: the workload's, else Lmax."""
    if seqlens is None:
        seqlens = gen_seqlens(w)
    if seqlens is None:
        seqlens = np.full(w.B, w.Lmax, np.int32)
    return np.asarray(seqlens, np.int32)


def gen_block_table(w: Workload) -> np.ndarray:
    """int32 [B, max_pages]: distinct pool pages in random order."""
    perm = _rng(w.seed, 5).permutation(w.num_pages)
    return perm[:w.B * w.max_pages].reshape(w.B, w.max_pages).astype(
        np.int32)


def scatter_pages(w: Workload, k: np.ndarray, v: np.ndarray,
                  block_table: np.ndarray, seqlens):
    """Host pools [num_pages, page_size, Hkv, D] ([num_pages, Hkv,
    page_size, D] when head_major) holding rows [0, L_b) of the contiguous
    k/v [B, Hkv, Lmax, D]; every other row is NaN."""
    P = w.page_size
    shape = ((w.num_pages, w.Hkv, P, w.D) if w.head_major
             else (w.num_pages, P, w.Hkv, w.D))
    kp = np.empty(shape, w.np_dtype)
    vp = np.empty(shape, w.np_dtype)
    kp.view(np.uint8)[:] = 0xFF
    vp.view(np.uint8)[:] = 0xFF
    for b in range(w.B):
        L = min(int(seqlens[b]), w.Lmax)
        for j in range(-(-L // P)):
            n = min(P, L - j * P)
            pg = block_table[b, j]
            if w.head_major:
                kp[pg, :, :n] = k[b, :, j * P:j * P + n]
                vp[pg, :, :n] = v[b, :, j * P:j * P + n]
            else:
                kp[pg, :n] = k[b, :, j * P:j * P + n].transpose(1, 0, 2)
                vp[pg, :n] = v[b, :, j * P:j * P + n].transpose(1, 0, 2)
    return kp, vp


def peak_rows(w: Workload, b: int, g: int, L: int) -> np.ndarray:
    """Rows of K[b, g] that are multiplied by peak_mult (sorted)."""
    if w.peak_frac <= 0.0 or L <= 0:
        return np.zeros(0, dtype=np.int64)
    n = min(L, int(math.ceil(w.peak_frac * L)))
    return np.sort(_rng(w.seed, 3, b, g).choice(L, size=n, replace=False))


def gen_slab_rows(w: Workload, b: int, g: int, L: int):
    """The L valid rows of K[b, g] and V[b, g] ([L, D], storage dtype)."""
    D = w.D
    kx = _rng(w.seed, 1, b, g).standard_normal((L, D), dtype=np.float32)
    pr = peak_rows(w, b, g, L)
    if pr.size:
        kx[pr] *= np.float32(w.peak_mult)
    vx = _rng(w.seed, 2, b, g).standard_normal((L, D), dtype=np.float32)
    return _encode(kx, w.dtype), _encode(vx, w.dtype)


def fill_slab(w: Workload, b: int, g: int, L: int, k_out: np.ndarray,
              v_out: np.ndarray) -> None:
    """Write K[b, g] and V[b, g] ([Lmax, D], storage dtype) in place; rows
    at or beyond L get the NaN poison."""
    assert k_out.shape == (w.Lmax, w.D) and v_out.shape == (w.Lmax, w.D)
    k_out[:L], v_out[:L] = gen_slab_rows(w, b, g, L)
    if L < w.Lmax:
        if w.dtype != "f32":
            k_out[L:].view(np.uint16)[:] = BF16_NAN   # NaN in fp16 too
            v_out[L:].view(np.uint16)[:] = BF16_NAN
        else:
            k_out[L:].view(np.uint32)[:] = F32_NAN_BITS
            v_out[L:].view(np.uint32)[:] = F32_NAN_BITS


def gen_slab(w: Workload, b: int, g: int, seqlens=None):
    """K[b, g], V[b, g] as fresh [Lmax, D] arrays."""
    L = seqlen_of(w, seqlens, b)
    k = np.empty((w.Lmax, w.D), dtype=w.np_dtype)
    v = np.empty((w.Lmax, w.D), dtype=w.np_dtype)
    fill_slab(w, b, g, L, k, v)
    return k, v


def gen_threads() -> int:
    """Host threads for slab generation: the cores this process may use,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def iter_slabs(w: Workload, seqlens=None, threads: int | None = None):
    """Yields (b, g, L, k_rows, v_rows) for every slab in b-major order,
    KV head fastest: the rows gen_slab_rows gives, drawn on a thread pool
    (every slab has its own generator stream, so the values do not depend
    on the thread count).  L is the length clamped to [0, Lmax].  At most
    2 * threads slabs are held at once."""
    jobs = [(b, g, min(max(seqlen_of(w, seqlens, b), 0), w.Lmax))
            for b in range(w.B) for g in range(w.Hkv)]
    n = threads or gen_threads()
    if n <= 1:
        for b, g, L in jobs:
            yield (b, g, L) + gen_slab_rows(w, b, g, L)
        return
    with ThreadPoolExecutor(n) as ex:
        pending = deque()
        it = iter(jobs)
        for job in it:
            pending.append((job, ex.submit(gen_slab_rows, w, *job)))
            if len(pending) >= 2 * n:
                break
        while pending:
            (b, g, L), fut = pending.popleft()
            job = next(it, None)
            if job is not None:
                pending.append((job, ex.submit(gen_slab_rows, w, *job)))
            yield (b, g, L) + fut.result()


def _poison(a: np.ndarray) -> None:
    a.view(np.uint8)[:] = 0xFF          # all-ones bit patterns are NaN


def gen_all(w: Workload, seqlens=None, threads: int | None = None):
    """q, k, v, seqlens as host arrays (only for workloads that fit easily);
    rows at or beyond a sequence's length hold NaN."""
    if seqlens is None:
        seqlens = gen_seqlens(w)
    q = gen_q(w)
    k = np.empty((w.B, w.Hkv, w.Lmax, w.D), dtype=w.np_dtype)
    v = np.empty_like(k)
    for b, g, L, kr, vr in iter_slabs(w, seqlens, threads):
        k[b, g, :L], v[b, g, :L] = kr[:L], vr[:L]
        if L < w.Lmax:
            _poison(k[b, g, L:])
            _poison(v[b, g, L:])
    return q, k, v, seqlens


def to_device(a: np.ndarray, device: str = "cuda"):
    """Host array (uint16 bf16 bits, float16 or float32) -> torch device
    tensor."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def device_inputs(w: Workload, seqlens=None, keep_host: bool = False,
                  device: str = "cuda"):
    """Upload a workload: (q, k, v, seqlens_dev, seqlens_host, host).

    K/V are generated slab by slab on the host and copied into place; rows
    at or beyond a sequence's length are filled with NaN bits on the
    device.  ``host`` is (q, k, v) as host arrays when keep_host, else None.
    """
    import torch
    if seqlens is None:
        seqlens = gen_seqlens(w)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16,
           "f32": torch.float32}[w.dtype]
    q_h = gen_q(w)
    q = to_device(q_h, device)
    shape = (w.B, w.Hkv, w.Lmax, w.D)
    k = torch.empty(shape, dtype=tdt, device=device)
    v = torch.empty(shape, dtype=tdt, device=device)
    if seqlens is not None:
        iv = torch.int32 if w.dtype == "f32" else torch.int16
        k.view(iv).fill_(-1)       # all-ones bit patterns are NaN
        v.view(iv).fill_(-1)
    host = None
    if keep_host:
        host = (q_h, np.empty(shape, w.np_dtype), np.empty(shape, w.np_dtype))
    for b, g, L, kr, vr in iter_slabs(w, seqlens):
        if L:
            k[b, g, :L].copy_(to_device(kr, device))
            v[b, g, :L].copy_(to_device(vr, device))
        if keep_host:
            host[1][b, g, :L], host[2][b, g, :L] = kr, vr
            if L < w.Lmax:
                _poison(host[1][b, g, L:])
                _poison(host[2][b, g, L:])
    sl_dev = None
    if seqlens is not None:
        sl_dev = torch.from_numpy(np.asarray(seqlens, np.int32)).to(device)
    return q, k, v, sl_dev, seqlens, host


def device_paged_inputs(w: Workload, seqlens=None, device: str = "cuda"):
    """Upload a paged workload: (q, k_pages, v_pages, block_table_dev,
    seqlens_dev, seqlens_host, block_table_host).

    The contiguous cache of ``device_inputs`` is scattered into the pool on
    the device (rows past a length and spare pages hold NaN bits), then
    released.
    """
    seqlens = paged_seqlens(w, seqlens)
    q, k, v, sl_dev, _, _ = device_inputs(w, seqlens=seqlens, device=device)
    kp, vp, bt_dev, bt = pages_from_contiguous(w, k, v, device)
    del k, v
    return q, kp, vp, bt_dev, sl_dev, seqlens, bt


def pages_from_contiguous(w: Workload, k, v, device: str = "cuda"):
    """Page pools holding the rows of the contiguous device cache k, v
    [B, Hkv, Lmax, D] (whose rows past each length must already be NaN):
    (k_pages, v_pages, block_table_dev, block_table_host).  Page j of
    sequence b is pool page block_table[b, j]; spare pages are NaN."""
    import torch
    bt = gen_block_table(w)
    P, mp = w.page_size, w.max_pages
    iv = torch.int32 if w.dtype == "f32" else torch.int16
    pools = []
    for src in (k, v):
        shape = ((w.num_pages, w.Hkv, P, w.D) if w.head_major
                 else (w.num_pages, P, w.Hkv, w.D))
        pool = torch.empty(shape, dtype=src.dtype, device=device)
        pool.view(iv).fill_(-1)
        pad = mp * P - w.Lmax
        if pad:
            src = torch.nn.functional.pad(src.view(iv), (0, 0, 0, pad),
                                          value=-1).view(src.dtype)
        # [B, Hkv, mp, P, D] -> [B * mp, P, Hkv, D] (or [B * mp, Hkv, P,
        # D]), page j of sequence b
        pages = src.view(w.B, w.Hkv, mp, P, w.D).permute(
            (0, 2, 1, 3, 4) if w.head_major else (0, 2, 3, 1, 4))
        idx = torch.from_numpy(bt.reshape(-1).astype(np.int64)).to(device)
        pool.view(iv).index_copy_(0, idx, pages.reshape(
            (w.B * mp,) + shape[1:]).view(iv))
        pools.append(pool)
    bt_dev = torch.from_numpy(bt).to(device)
    return pools[0], pools[1], bt_dev, bt


def algorithmic_bytes(w: Workload, seqlens=None) -> int:
    """Bytes one decode step must move at minimum: every valid K and V row
    once, q, out, and the fp32 lse (Tq rows of each per sequence and head),
    plus, for a paged cache, the block-table entries of the valid pages."""
    eb = w.elem_bytes
    Ls = (np.full(w.B, w.Lmax) if seqlens is None
          else np.clip(np.asarray(seqlens, np.int64), 0, w.Lmax))
    rows = int(np.sum(Ls))
    kv = 2 * rows * w.Hkv * w.D * eb
    qo = w.Tq * (2 * w.B * w.Hq * w.D * eb + 4 * w.B * w.Hq)
    table = 0
    if w.page_size:
        table = 4 * int(np.sum(-(-Ls // w.page_size)))
    return kv + qo + table


def flops(w: Workload, seqlens=None) -> int:
    rows = (w.Lmax * w.B if seqlens is None
            else int(np.sum(np.clip(seqlens, 0, w.Lmax))))
    return 4 * rows * w.Hq * w.D * w.Tq
