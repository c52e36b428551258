"""fp64 CPU oracle for single-query decode attention (ctypes over fd_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
smoke check and the benchmark's CPU-baseline leg may import this module.
It never imports the GPU package and the GPU package never imports it.

It computes exact softmax attention of one query per head against the KV
cache, as described in "Flash-Decoding for long-context inference"
(Stanford CRFM), section "Multi-head attention for decoding"; the twin
``*_split`` functions follow that page's section "A faster attention for
decoding: Flash-Decoding" (chunk the keys/values, attend per chunk with one
log-sum-exp per row and chunk, merge the chunks by their log-sum-exp).
``decode_paged`` reads the same rows through a page table and
``decode_multiquery`` attends several newest tokens per sequence causally
(the Flash-Decoding search-result page notes both cache layouts that differ
between frameworks and decoding several query tokens at once).

Arrays: bf16 tensors are passed as ``numpy.uint16`` bit patterns, fp16 as
``numpy.float16``, fp32 as ``numpy.float32``.  Shapes: q [B, Hq, D], k/v [B, Hkv, Lmax, D], seqlens
int32 [B] or None.  Results are float64: out [B, Hq, D], lse [B, Hq].
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfdoracle.so")

_BF16 = 0
_F32 = 1
_F16 = 2


def _bind(path: str):
    lib = ctypes.CDLL(path)
    vp, i32p, dp = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    ci, cd = ctypes.c_int, ctypes.c_double
    lib.fdo_decode.argtypes = [vp, vp, vp, i32p, ci, ci, ci, ci, ci, cd, ci,
                               ci, dp, dp]
    lib.fdo_decode.restype = ci
    lib.fdo_decode_split.argtypes = [vp, vp, vp, i32p, ci, ci, ci, ci, ci,
                                     cd, ci, ci, ci, dp, dp]
    lib.fdo_decode_split.restype = ci
    lib.fdo_attend_row.argtypes = [vp, vp, vp, ci, ci, cd, ci, dp, dp]
    lib.fdo_attend_row.restype = ci
    lib.fdo_attend_row_split.argtypes = [vp, vp, vp, ci, ci, cd, ci, ci, ci,
                                         dp, dp, dp, dp]
    lib.fdo_attend_row_split.restype = ci
    lib.fdo_decode_paged.argtypes = [vp, vp, vp, i32p, ci, ci, ci, ci, i32p,
                                     ci, ci, ci, ci, ci, cd, ci, ci, dp, dp]
    lib.fdo_decode_paged.restype = ci
    lib.fdo_decode_multiquery.argtypes = [vp, vp, vp, i32p, ci, ci, ci, ci,
                                          ci, ci, cd, ci, ci, dp, dp]
    lib.fdo_decode_multiquery.restype = ci
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with `python oracle/build.py`")
        _lib = _bind(LIB_PATH)
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return _BF16
    if a.dtype == np.float32:
        return _F32
    if a.dtype == np.float16:
        return _F16
    raise TypeError(
        f"oracle takes uint16 (bf16 bits), float16 or float32, not {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a):
    return np.ascontiguousarray(a)


def _scale(scale) -> float:
    # The GPU library receives the scale as a C float; use that same value.
    return float(np.float32(scale))


def decode(q, k, v, seqlens, scale, nthreads: int = 0, _lib_override=None):
    """Exact attention for a whole batch. Returns (out[B,Hq,D], lse[B,Hq])."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    assert k.dtype == q.dtype and v.dtype == q.dtype
    B, Hq, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    assert Bk == B and Dk == D and v.shape == k.shape
    sl = None if seqlens is None else _c(np.asarray(seqlens, dtype=np.int32))
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.fdo_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), B, Hq, Hkv, D,
                        Lmax, _scale(scale), dt, int(nthreads), _ptr(out),
                        _ptr(lse))
    if rc != 0:
        raise ValueError(f"fdo_decode failed with {rc}")
    return out, lse


def decode_split(q, k, v, seqlens, scale, chunk: int, nthreads: int = 0,
                 _lib_override=None):
    """The split/merge twin for a whole batch, chunk keys per split."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    sl = None if seqlens is None else _c(np.asarray(seqlens, dtype=np.int32))
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.fdo_decode_split(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), B, Hq, Hkv,
                              D, Lmax, _scale(scale), dt, int(chunk),
                              int(nthreads), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"fdo_decode_split failed with {rc}")
    return out, lse


def attend_row(q_row, k_slab, v_slab, L: int, scale, _lib_override=None):
    """One query row [D] against rows [0, L) of one slab [>=L, D]."""
    q_row, k_slab, v_slab = _c(q_row), _c(k_slab), _c(v_slab)
    dt = _dtype_code(q_row)
    D = q_row.shape[-1]
    assert k_slab.shape[-1] == D and k_slab.shape[0] >= L
    out = np.empty(D, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.fdo_attend_row(_ptr(q_row), _ptr(k_slab), _ptr(v_slab), int(L),
                            D, _scale(scale), dt, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"fdo_attend_row failed with {rc}")
    return out, float(lse[0])


def attend_row_split(q_row, k_slab, v_slab, L: int, scale, chunk: int,
                     nchunks: int | None = None, _lib_override=None):
    """Split/merge twin for one row; also returns the per-chunk partials."""
    q_row, k_slab, v_slab = _c(q_row), _c(k_slab), _c(v_slab)
    dt = _dtype_code(q_row)
    D = q_row.shape[-1]
    if nchunks is None:
        nchunks = max(1, -(-L // chunk))
    out = np.empty(D, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    po = np.empty((nchunks, D), dtype=np.float64)
    pl = np.empty(nchunks, dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.fdo_attend_row_split(_ptr(q_row), _ptr(k_slab), _ptr(v_slab),
                                  int(L), D, _scale(scale), dt, int(chunk),
                                  int(nchunks), _ptr(out), _ptr(lse),
                                  _ptr(po), _ptr(pl))
    if rc != 0:
        raise ValueError(f"fdo_attend_row_split failed with {rc}")
    return out, float(lse[0]), po, pl


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale,
                 head_major: bool = False, nthreads: int = 0,
                 _lib_override=None):
    """Exact attention over a paged cache.  k_pages/v_pages
    [num_pages, page_size, Hkv, D] (token-major) or [num_pages, Hkv,
    page_size, D] (head_major); block_table int32 [B, max_pages]; seqlens
    int32 [B] (required).  q [B, Hq, D], or [B, Tq, Hq, D] for Tq causal
    new tokens (out and lse then carry the Tq axis too)."""
    q, k_pages, v_pages = _c(q), _c(k_pages), _c(v_pages)
    dt = _dtype_code(q)
    if q.ndim == 4:
        B, Tq, Hq, D = q.shape
    else:
        (B, Hq, D), Tq = q.shape, 1
    if head_major:
        num_pages, Hkv, page_size, Dk = k_pages.shape
    else:
        num_pages, page_size, Hkv, Dk = k_pages.shape
    assert Dk == D and v_pages.shape == k_pages.shape
    bt = _c(np.asarray(block_table, dtype=np.int32))
    assert bt.shape[0] == B
    sl = _c(np.asarray(seqlens, dtype=np.int32))
    out = np.empty(q.shape, dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.fdo_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages),
                              _ptr(bt), bt.shape[1], page_size, num_pages,
                              int(bool(head_major)), _ptr(sl), B, Tq, Hq, Hkv,
                              D, _scale(scale), dt,
                              int(nthreads), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"fdo_decode_paged failed with {rc}")
    return out, lse


def decode_multiquery(q, k, v, seqlens, scale, nthreads: int = 0,
                      _lib_override=None):
    """Exact causal attention of Tq new query tokens per sequence.
    q [B, Tq, Hq, D]; k/v [B, Hkv, Lmax, D]; returns out [B, Tq, Hq, D],
    lse [B, Tq, Hq]."""
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, Tq, Hq, D = q.shape
    _, Hkv, Lmax, _ = k.shape
    sl = None if seqlens is None else _c(np.asarray(seqlens, dtype=np.int32))
    out = np.empty((B, Tq, Hq, D), dtype=np.float64)
    lse = np.empty((B, Tq, Hq), dtype=np.float64)
    lib = _lib_override or _load()
    rc = lib.fdo_decode_multiquery(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), B,
                                   Tq, Hq, Hkv, D, Lmax, _scale(scale), dt,
                                   int(nthreads), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"fdo_decode_multiquery failed with {rc}")
    return out, lse


class Variant:
    """The same API bound to another build of fd_oracle.c (used by the
    mutation tests, which compile deliberately broken copies)."""

    def __init__(self, path: str):
        self._l = _bind(path)

    def decode(self, *a, **kw):
        return decode(*a, _lib_override=self._l, **kw)

    def decode_split(self, *a, **kw):
        return decode_split(*a, _lib_override=self._l, **kw)

    def attend_row(self, *a, **kw):
        return attend_row(*a, _lib_override=self._l, **kw)

    def attend_row_split(self, *a, **kw):
        return attend_row_split(*a, _lib_override=self._l, **kw)

    def decode_paged(self, *a, **kw):
        return decode_paged(*a, _lib_override=self._l, **kw)

    def decode_multiquery(self, *a, **kw):
        return decode_multiquery(*a, _lib_override=self._l, **kw)
