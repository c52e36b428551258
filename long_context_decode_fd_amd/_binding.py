"""ctypes binding over libfd.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this
module checks tensor shapes/dtypes/devices, passes raw device pointers and
the current HIP stream, and turns status codes into exceptions.  PyTorch is
used for device memory and streams.  When libfd.so has not been built the
calls raise; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FD_LIBRARY") or os.path.join(_PKG, "libfd.so")

FD_BF16 = 0
FD_F32 = 1
FD_F16 = 2
FD_OK = 0
FD_ERR_INVALID_ARG = -1
FD_ERR_UNSUPPORTED = -2
FD_ERR_WORKSPACE = -3
FD_ERR_HIP = -4
FD_ERR_CAPTURE = -5
FD_ERR_TOO_LARGE = -6
NOALLOC_SCRATCH_BYTES = 64 << 20
FD_VARIANT_AUTO = 0
FD_VARIANT_MFMA = 1
FD_VARIANT_VALU = 2
FD_FLAG_FUSED_MERGE = 1
FD_FLAG_PARTIALS = 2
FD_FLAG_UNIFIED_MAX = 4
FD_MERGE_NONE = 0
FD_MERGE_FUSED = 1
FD_MERGE_SEPARATE = 2
FD_PAGES_TOKEN_MAJOR = 0
FD_PAGES_HEAD_MAJOR = 1
FD_PARTIALS_ROW_MAJOR = 0
FD_PARTIALS_CHUNK_MAJOR = 1

# Every function the C header declares, with its ctypes signature.
_vp, _i32p = ctypes.c_void_p, ctypes.c_void_p
_ci, _cf, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class FdPlanStruct(ctypes.Structure):
    _fields_ = [("num_splits", _ci), ("chunk", _ci), ("variant", _ci),
                ("waves_per_block", _ci), ("grid", _ci), ("combine", _ci),
                ("merge", _ci), ("num_cus", _ci), ("workspace_bytes", _sz),
                ("ticket_bytes", _sz), ("o_part_offset", _sz),
                ("lse_part_offset", _sz), ("partial_layout", _ci),
                ("partial_group", _ci)]


SIGNATURES = {
    "fd_decode": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci, _ci, _ci, _cf,
                        _ci, _vp, _vp, _vp]),
    "fd_decode_ex": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci, _ci, _ci,
                           _cf, _ci, _vp, _vp, _ci, _ci, _ci, _vp, _sz,
                           _vp]),
    "fd_decode_noalloc": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci, _ci,
                                _ci, _cf, _ci, _vp, _vp, _ci, _ci, _ci,
                                _vp]),
    "fd_decode_partials": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci, _ci,
                                 _ci, _cf, _ci, _ci, _ci, _ci, _vp, _sz,
                                 _vp]),
    "fd_merge_partials": (_ci, [_i32p, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                                _ci, _ci, _vp, _sz, _vp, _vp, _vp]),
    "fd_decode_paged": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci, _ci,
                              _i32p, _ci, _ci, _ci, _ci, _ci, _cf, _ci, _vp,
                              _vp, _ci, _ci, _vp, _sz, _vp]),
    "fd_decode_multiquery": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci, _ci,
                                   _ci, _ci, _cf, _ci, _vp, _vp, _ci, _ci,
                                   _vp, _sz, _vp]),
    "fd_decode_unified_max": (_ci, [_vp, _vp, _vp, _i32p, _ci, _ci, _ci,
                                    _ci, _ci, _cf, _ci, _vp, _vp, _cf, _ci,
                                    _ci, _vp, _sz, _vp]),
    "fd_plan": (_ci, [_ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                      ctypes.POINTER(FdPlanStruct)]),
    "fd_plan_ex": (_ci, [_ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                         _ci, _ci, _ci, ctypes.POINTER(FdPlanStruct)]),
    "fd_workspace_bytes": (_sz, [_ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                                 _ci, _ci]),
    "fd_status_string": (ctypes.c_char_p, [_ci]),
    "fd_version": (_ci, []),
}

_lib = None


class FdError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({fd_status_string(code)})")


def load_library(path: str | None = None):
    """Load libfd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} not found: build it with "
            "`python -m long_context_decode_fd_amd.build` (needs hipcc)")
    # Streams and memory pass between torch and the library, so both must
    # use one HIP runtime.  torch ships its own: load it first, so that the
    # library's HIP dependency resolves to it.  Loading the library first
    # would put the system runtime under torch instead.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def fd_status_string(code: int) -> str:
    return load_library().fd_status_string(int(code)).decode()


def fd_version() -> int:
    return load_library().fd_version()


def _dtype_code(dtype) -> int:
    if dtype in (FD_BF16, "bf16", "bfloat16"):
        return FD_BF16
    if dtype in (FD_F32, "f32", "fp32", "float32"):
        return FD_F32
    if dtype in (FD_F16, "f16", "fp16", "float16"):
        return FD_F16
    import torch
    if dtype == torch.bfloat16:
        return FD_BF16
    if dtype == torch.float32:
        return FD_F32
    if dtype == torch.float16:
        return FD_F16
    raise ValueError(f"unsupported dtype {dtype!r}")


def fd_plan(B, Hq, Hkv, D, Lmax, dtype, varlen=False, num_splits=0,
            variant=FD_VARIANT_AUTO, flags=0, num_cus=0) -> dict:
    """The planner's decision (see fd.h); num_cus 0 = query the device."""
    p = FdPlanStruct()
    rc = load_library().fd_plan(B, Hq, Hkv, D, Lmax, _dtype_code(dtype),
                                int(bool(varlen)), num_splits, variant, flags,
                                num_cus, ctypes.byref(p))
    if rc != FD_OK:
        raise FdError("fd_plan", rc)
    return {f: getattr(p, f) for f, _ in FdPlanStruct._fields_}


def fd_plan_ex(B, Tq, Hq, Hkv, D, Lmax, dtype, varlen=False, paged=False,
               num_splits=0, variant=FD_VARIANT_AUTO, flags=0,
               num_cus=0) -> dict:
    """The plan of fd_decode_multiquery (Tq tokens) / fd_decode_paged."""
    p = FdPlanStruct()
    rc = load_library().fd_plan_ex(B, Tq, Hq, Hkv, D, Lmax, _dtype_code(dtype),
                                   int(bool(varlen)), int(bool(paged)),
                                   num_splits, variant, flags, num_cus,
                                   ctypes.byref(p))
    if rc != FD_OK:
        raise FdError("fd_plan_ex", rc)
    return {f: getattr(p, f) for f, _ in FdPlanStruct._fields_}


def fd_workspace_bytes(B, Hq, Hkv, D, Lmax, dtype, varlen=False,
                       num_splits=0, variant=FD_VARIANT_AUTO,
                       flags=0) -> int:
    return int(load_library().fd_workspace_bytes(
        B, Hq, Hkv, D, Lmax, _dtype_code(dtype), int(bool(varlen)),
        num_splits, variant, flags))


def _check(q, k_cache, v_cache, seqlens, out, lse, need_out=True):
    import torch
    if q.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise TypeError("q/k/v must be bfloat16, float16 or float32 tensors")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,Hq,D], k/v [B,Hkv,Lmax,D]")
    B, Hq, D = q.shape
    Bk, Hkv, Lmax, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} "
                         f"k {tuple(k_cache.shape)}")
    if seqlens is not None:
        if (seqlens.dtype != torch.int32 or not seqlens.is_cuda
                or seqlens.shape != (B,) or not seqlens.is_contiguous()):
            raise ValueError("seqlens must be a contiguous int32 [B] "
                             "device tensor")
    _same_device(q.device, k_cache=k_cache, v_cache=v_cache, seqlens=seqlens)
    if not need_out:
        return (B, Hq, Hkv, D, Lmax), None, None
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda
            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    if (lse.shape != (B, Hq) or lse.dtype != torch.float32 or not lse.is_cuda
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B,Hq] tensor")
    _same_device(q.device, out=out, lse=lse)
    _no_overlap(dict(out=out, lse=lse), dict(q=q, k_cache=k_cache,
                                             v_cache=v_cache, seqlens=seqlens))
    return (B, Hq, Hkv, D, Lmax), out, lse


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _spans(tensors):
    """(name, first byte, end) of the non-empty tensors of a name -> tensor
    mapping."""
    res = []
    for k, t in tensors.items():
        if t is not None:
            n = t.nbytes
            if n:
                p = t.data_ptr()
                res.append((k, p, p + n))
    return res


def _no_overlap(outs, ins):
    """Outputs must not share memory with each other or with an input."""
    o = _spans(outs)
    others = o + _spans(ins)
    for i, (a, a0, a1) in enumerate(o):
        for b, b0, b1 in others[i + 1:]:
            if a0 < b1 and b0 < a1:
                raise ValueError(f"{a} overlaps {b}")


_raw_stream = None


def _current_stream_ptr(device):
    """hipStream_t of `device`'s current stream, as an int: torch's raw
    getter where it has one (no Stream object is built), else the public
    API."""
    global _raw_stream
    import torch
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _invoke(name, device, stream, *args):
    """Call libfd's `name` on `stream` (default: the current stream of
    `device`) with `device` current for the call: the library plans for,
    and keeps its own workspace on, the current device."""
    import torch
    if stream is None:
        sp = _current_stream_ptr(device)
    elif stream.device != device:
        raise ValueError(f"stream is on {stream.device}, expected {device}")
    else:
        sp = stream.cuda_stream
    fn = getattr(load_library(), name)
    if torch.cuda.current_device() == device.index:
        rc = fn(*args, sp)
    else:
        with torch.cuda.device(device):
            rc = fn(*args, sp)
    if rc != FD_OK:
        raise FdError(name, rc)


def _opt_ws(workspace, device, out, lse):
    """(pointer, bytes) of an optional caller workspace tensor, checked to
    be on `device` and apart from the outputs; (None, 0) for none."""
    if workspace is None:
        return None, 0
    _same_device(device, workspace=workspace)
    _no_overlap(dict(out=out, lse=lse), dict(workspace=workspace))
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fd_decode_ex(q, k_cache, v_cache, seqlens, scale, out=None, lse=None,
                 num_splits=0, variant=FD_VARIANT_AUTO, flags=0,
                 workspace=None, stream=None):
    """out, lse = attention(q, k_cache, v_cache) -- see fd.h.

    q [B,Hq,D], k_cache/v_cache [B,Hkv,Lmax,D] (bf16, fp16 or fp32, on the GPU),
    seqlens int32 [B] on the GPU or None, scale a float.  Returns (out, lse);
    out/lse are allocated if not given.  workspace: a zero-filled uint8
    device tensor of at least fd_workspace_bytes(...) bytes (see fd.h for
    the ticket rule), or None for the library's.
    """
    dims, out, lse = _check(q, k_cache, v_cache, seqlens, out, lse)
    B, Hq, Hkv, D, Lmax = dims
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    ws_ptr, ws_bytes = _opt_ws(workspace, q.device, out, lse)
    _invoke("fd_decode_ex", q.device, stream,
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if seqlens is None else seqlens.data_ptr(),
        B, Hq, Hkv, D, Lmax, float(scale), _dtype_code(q.dtype),
        out.data_ptr(), lse.data_ptr(), int(num_splits), int(variant),
        int(flags), ws_ptr, ws_bytes)
    return out, lse


def fd_decode_unified_max(q, k_cache, v_cache, seqlens, scale, phi,
                          out=None, lse=None, num_splits=0, flags=0,
                          workspace=None, stream=None):
    """fd_decode_ex with the unified-maximum softmax against phi (natural
    log units of the scaled score) -- see fd.h."""
    dims, out, lse = _check(q, k_cache, v_cache, seqlens, out, lse)
    B, Hq, Hkv, D, Lmax = dims
    if not math.isfinite(float(scale)) or not math.isfinite(float(phi)):
        raise ValueError("scale and phi must be finite")
    ws_ptr, ws_bytes = _opt_ws(workspace, q.device, out, lse)
    _invoke("fd_decode_unified_max", q.device, stream,
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if seqlens is None else seqlens.data_ptr(),
        B, Hq, Hkv, D, Lmax, float(scale), _dtype_code(q.dtype),
        out.data_ptr(), lse.data_ptr(), float(phi), int(num_splits),
        int(flags), ws_ptr, ws_bytes)
    return out, lse


def fd_decode(q, k_cache, v_cache, seqlens, scale, out=None, lse=None,
              stream=None):
    """Same as the C fd_decode: planner's choices, library workspace."""
    dims, out, lse = _check(q, k_cache, v_cache, seqlens, out, lse)
    B, Hq, Hkv, D, Lmax = dims
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    _invoke("fd_decode", q.device, stream,
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if seqlens is None else seqlens.data_ptr(),
        B, Hq, Hkv, D, Lmax, float(scale), _dtype_code(q.dtype),
        out.data_ptr(), lse.data_ptr())
    return out, lse


def fd_decode_noalloc(q, k_cache, v_cache, seqlens, scale, out=None,
                      lse=None, num_splits=0, variant=FD_VARIANT_AUTO,
                      flags=0, stream=None):
    """fd_decode_ex with the partials in the library's fixed per-device
    scratch array: allocates nothing (see fd.h for the size limit and the
    rule that calls overlapping on one device race)."""
    dims, out, lse = _check(q, k_cache, v_cache, seqlens, out, lse)
    B, Hq, Hkv, D, Lmax = dims
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    _invoke("fd_decode_noalloc", q.device, stream,
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if seqlens is None else seqlens.data_ptr(),
        B, Hq, Hkv, D, Lmax, float(scale), _dtype_code(q.dtype),
        out.data_ptr(), lse.data_ptr(), int(num_splits), int(variant),
        int(flags))
    return out, lse


def _ws(workspace, device):
    if workspace is None:
        raise ValueError("the phase calls need a caller workspace tensor")
    _same_device(device, workspace=workspace)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def fd_decode_partials(q, k_cache, v_cache, seqlens, scale, workspace,
                       num_splits=0, variant=FD_VARIANT_AUTO, flags=0,
                       stream=None):
    """Chunk phase only: partials into `workspace` (see fd.h)."""
    dims, _, _ = _check(q, k_cache, v_cache, seqlens, None, None,
                        need_out=False)
    B, Hq, Hkv, D, Lmax = dims
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    ws_ptr, ws_bytes = _ws(workspace, q.device)
    _no_overlap(dict(workspace=workspace), dict(q=q, k_cache=k_cache,
                                                v_cache=v_cache,
                                                seqlens=seqlens))
    _invoke("fd_decode_partials", q.device, stream,
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if seqlens is None else seqlens.data_ptr(),
        B, Hq, Hkv, D, Lmax, float(scale), _dtype_code(q.dtype),
        int(num_splits), int(variant), int(flags), ws_ptr, ws_bytes)


def fd_merge_partials(seqlens, B, Hq, Hkv, D, Lmax, dtype, workspace, out,
                      lse, num_splits=0, variant=FD_VARIANT_AUTO, flags=0,
                      stream=None):
    """Merge phase only: out/lse from the partials in `workspace`."""
    import torch
    tdt = {FD_BF16: torch.bfloat16, FD_F16: torch.float16,
           FD_F32: torch.float32}[_dtype_code(dtype)]
    if (out.shape != (B, Hq, D) or out.dtype != tdt or not out.is_cuda
            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [B,Hq,D] device tensor")
    if (lse.shape != (B, Hq) or lse.dtype != torch.float32 or not lse.is_cuda
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B,Hq] tensor")
    if seqlens is not None:
        _device_tensor("seqlens", seqlens, torch.int32, (B,))
    _same_device(out.device, lse=lse, seqlens=seqlens)
    ws_ptr, ws_bytes = _ws(workspace, out.device)
    _no_overlap(dict(out=out, lse=lse), dict(workspace=workspace,
                                             seqlens=seqlens))
    _invoke("fd_merge_partials", out.device, stream,
        None if seqlens is None else seqlens.data_ptr(), B, Hq, Hkv, D, Lmax,
        _dtype_code(dtype), int(num_splits), int(variant), int(flags),
        ws_ptr, ws_bytes, out.data_ptr(), lse.data_ptr())


def _device_tensor(name, t, dtype, shape=None):
    import torch
    if (not isinstance(t, torch.Tensor) or not t.is_cuda
            or not t.is_contiguous() or t.dtype != dtype
            or (shape is not None and tuple(t.shape) != tuple(shape))):
        want = "" if shape is None else f" {list(shape)}"
        raise ValueError(f"{name} must be a contiguous {dtype}{want} "
                         "device tensor")


def _out_lse(out, lse, shape, lse_shape, dtype, device):
    import torch
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=device)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=device)
    _device_tensor("out", out, dtype, shape)
    _device_tensor("lse", lse, torch.float32, lse_shape)
    return out, lse


def fd_decode_paged(q, k_pages, v_pages, block_table, seqlens, scale,
                    out=None, lse=None, num_splits=0, flags=0,
                    head_major=False, workspace=None, stream=None):
    """Decode attention over a paged KV cache -- see fd.h.

    q [B,Hq,D] bf16, fp16 or fp32, or [B,Tq,Hq,D] for Tq causal new tokens;
    k_pages/v_pages [num_pages,page_size,Hkv,D] of q's dtype (token-major) or
    [num_pages,Hkv,page_size,D] (head_major); block_table int32
    [B,max_pages]; seqlens int32 [B] (required); all on the GPU.  Returns
    (out, lse) shaped like q and q without its last axis.  workspace: a
    uint8 device tensor of fd_plan_ex(..., paged=True)'s workspace_bytes
    (zero-filled for the fused merge), or None for the library's.
    """
    import torch
    if q.dim() not in (3, 4) or k_pages.dim() != 4:
        raise ValueError("expected q [B,Hq,D] or [B,Tq,Hq,D], 4-d page "
                         "pools")
    if q.dim() == 4:
        B, Tq, Hq, D = q.shape
    else:
        (B, Hq, D), Tq = q.shape, 1
    if head_major:
        num_pages, Hkv, page_size, Dk = k_pages.shape
    else:
        num_pages, page_size, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError(f"head dim mismatch q {D} vs pages {Dk}")
    _device_tensor("q", q, q.dtype)
    _device_tensor("k_pages", k_pages, q.dtype)
    _device_tensor("v_pages", v_pages, q.dtype, k_pages.shape)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    _device_tensor("block_table", block_table, torch.int32)
    _device_tensor("seqlens", seqlens, torch.int32, (B,))
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    out, lse = _out_lse(out, lse, tuple(q.shape), tuple(q.shape[:-1]),
                        q.dtype, q.device)
    _same_device(q.device, k_pages=k_pages, v_pages=v_pages,
                 block_table=block_table, seqlens=seqlens, out=out, lse=lse)
    _no_overlap(dict(out=out, lse=lse),
                dict(q=q, k_pages=k_pages, v_pages=v_pages,
                     block_table=block_table, seqlens=seqlens))
    ws_ptr, ws_bytes = _opt_ws(workspace, q.device, out, lse)
    _invoke("fd_decode_paged", q.device, stream,
        q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
        block_table.data_ptr(), block_table.shape[1], page_size, num_pages,
        FD_PAGES_HEAD_MAJOR if head_major else FD_PAGES_TOKEN_MAJOR,
        seqlens.data_ptr(), B, Tq, Hq, Hkv, D, float(scale),
        _dtype_code(q.dtype), out.data_ptr(), lse.data_ptr(),
        int(num_splits), int(flags), ws_ptr, ws_bytes)
    return out, lse


def fd_decode_multiquery(q, k_cache, v_cache, seqlens, scale, out=None,
                         lse=None, num_splits=0, flags=0, workspace=None,
                         stream=None):
    """Tq causal query tokens per sequence -- see fd.h.

    q [B,Tq,Hq,D] bf16, fp16 or fp32; k_cache/v_cache [B,Hkv,Lmax,D] of q's
    dtype; seqlens int32 [B]
    on the GPU or None.  Returns (out [B,Tq,Hq,D], lse [B,Tq,Hq]).
    workspace: a uint8 device tensor of fd_plan_ex(B, Tq, ...)'s
    workspace_bytes (zero-filled for the fused merge), or None for the
    library's.
    """
    import torch
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("expected q [B,Tq,Hq,D], k/v [B,Hkv,Lmax,D]")
    B, Tq, Hq, D = q.shape
    Bk, Hkv, Lmax, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} "
                         f"k {tuple(k_cache.shape)}")
    _device_tensor("q", q, q.dtype)
    _device_tensor("k_cache", k_cache, q.dtype)
    _device_tensor("v_cache", v_cache, q.dtype, k_cache.shape)
    if seqlens is not None:
        _device_tensor("seqlens", seqlens, torch.int32, (B,))
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    out, lse = _out_lse(out, lse, (B, Tq, Hq, D), (B, Tq, Hq), q.dtype,
                        q.device)
    _same_device(q.device, k_cache=k_cache, v_cache=v_cache, seqlens=seqlens,
                 out=out, lse=lse)
    _no_overlap(dict(out=out, lse=lse), dict(q=q, k_cache=k_cache,
                                             v_cache=v_cache, seqlens=seqlens))
    ws_ptr, ws_bytes = _opt_ws(workspace, q.device, out, lse)
    _invoke("fd_decode_multiquery", q.device, stream,
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if seqlens is None else seqlens.data_ptr(), B, Tq, Hq, Hkv, D,
        Lmax, float(scale), _dtype_code(q.dtype), out.data_ptr(),
        lse.data_ptr(), int(num_splits), int(flags), ws_ptr, ws_bytes)
    return out, lse
