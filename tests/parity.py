"""Comparison rule between a GPU result and the fp64 oracle (test helper).

Output (bf16, fp16 or fp32 ``out``): an element passes when
|gpu - ref| <= max(1e-2, (1 + 2^-10) * ulp(ref) / 2) for the 16-bit types
(ulp of bf16 or of fp16), and |gpu - ref| <= 1e-2 for fp32.  The second
bound is correct rounding to the nearest value of the output type, the
best any such output can do; it exceeds 1e-2 only once |ref| >= 4 in bf16
(ulp 2^-5 there) or |ref| >= 32 in fp16, so below that the bound is the
plain 1e-2.  The factor 1 + 2^-10 leaves room for the fp32 accumulation's
own error when ref lies next to a rounding midpoint.
LSE (fp32): |gpu - ref| <= 1e-3.  NaN must meet NaN, -inf must meet -inf.

Besides pass/fail, ``report`` carries diagnostics that are not part of the
contract: max |err|, max error in bf16 ulps of ref, relative L2 error.
"""
from __future__ import annotations

import numpy as np

OUT_ATOL = 1e-2
LSE_ATOL = 1e-3
# Slack on half a bf16 ulp for the fp32 result's own error near a midpoint.
HALF_ULP_SLACK = 1.0 + 2.0 ** -10


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(ref, dtype=np.float64))
    a = np.maximum(a, np.finfo(np.float32).tiny)
    e = np.floor(np.log2(a))
    return np.power(2.0, e - 7)


def f16_ulp(ref: np.ndarray) -> np.ndarray:
    """Spacing of IEEE binary16 values at |ref| (2^-24 below 2^-14)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    a = np.maximum(a, 2.0 ** -14)
    e = np.floor(np.log2(a))
    return np.power(2.0, e - 10)


def _special_match(gpu, ref):
    both_nan = np.isnan(gpu) & np.isnan(ref)
    same_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    return both_nan | same_inf


def check_out(gpu, ref, dtype: str):
    """gpu: uint16 bf16 bits, float16 or float32 array; ref: float64 of the
    same shape; dtype "bf16", "f16" or "f32"."""
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "f16":
        assert np.asarray(gpu).dtype == np.float16
    g = bf16_to_f64(gpu) if dtype == "bf16" else np.asarray(
        gpu, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - ref)
        ok = err <= OUT_ATOL
        if dtype == "bf16":
            ok |= err <= 0.5 * bf16_ulp(ref) * HALF_ULP_SLACK
        elif dtype == "f16":
            ok |= err <= 0.5 * f16_ulp(ref) * HALF_ULP_SLACK
        ok |= _special_match(g, ref)
        finite = np.isfinite(ref) & np.isfinite(g)
        ferr = np.where(finite, err, 0.0)
        ulps = np.where(finite, ferr / bf16_ulp(ref), 0.0)
        nref = np.linalg.norm(np.where(finite, ref, 0.0))
        rel_l2 = (np.linalg.norm(ferr) / nref) if nref > 0 else 0.0
    rep = {
        "n": int(ok.size),
        "n_bad": int((~ok).sum()),
        "max_abs_err": float(ferr.max()) if ferr.size else 0.0,
        "max_ulp_bf16": float(ulps.max()) if ulps.size else 0.0,
        "rel_l2": float(rel_l2),
        "max_abs_ref": float(np.abs(np.where(finite, ref, 0)).max())
        if ref.size else 0.0,
    }
    if rep["n_bad"]:
        idx = np.argwhere(~ok)[:5]
        rep["first_bad"] = [(tuple(int(i) for i in ix), float(g[tuple(ix)]),
                             float(ref[tuple(ix)])) for ix in idx]
    return bool(ok.all()), rep


def check_lse(gpu, ref):
    ref = np.asarray(ref, dtype=np.float64)
    g = np.asarray(gpu, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - ref)
        ok = (err <= LSE_ATOL) | _special_match(g, ref)
        finite = np.isfinite(ref) & np.isfinite(g)
    rep = {
        "n": int(ok.size),
        "n_bad": int((~ok).sum()),
        "max_abs_err": float(np.where(finite, err, 0).max()) if ok.size else 0,
    }
    if rep["n_bad"]:
        idx = np.argwhere(~ok)[:5]
        rep["first_bad"] = [(tuple(int(i) for i in ix), float(g[tuple(ix)]),
                             float(ref[tuple(ix)])) for ix in idx]
    return bool(ok.all()), rep
