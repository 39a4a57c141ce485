"""Test infrastructure: the acceptance rule for GPU results against the oracle.

The contract ("tensor programs, part 1", section "One Program and One Numerical
Contract") lets the summation order vary, so for random data more than one FP16
projection is correct.  The oracle supplies one legal result (sequential FP32
order) plus FP64 band data S = sum x*w and A = sum |x*w|.  A GPU result is
accepted when it is within

    proj:  |p_gpu - p_ref| <= ulp16(p_ref) + ORDER_ALLOWANCE * u32 * A
    y:     |y_gpu - y_ref| <= ulp16(y_ref) + ulp16(p_ref) + ORDER_ALLOWANCE * u32 * A

(u32 = 2^-24), and it must always lie inside the rigorous outer band
[RNE16(S - gamma*A), RNE16(S + gamma*A)], gamma = (K-1)u32 / (1 - (K-1)u32),
the forward-error bound of recursive FP32 summation in any order; rounding to
FP16 is monotone, so a result outside it is a bug, not a legal reordering.
Integer-exact cases are compared bit for bit instead.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
ORDER_ALLOWANCE = 16.0


def words_to_f64(h) -> np.ndarray:
    h = np.asarray(h)
    if h.dtype == np.float16:
        return h.astype(np.float64)
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp16(h) -> np.ndarray:
    """Gap from |v| to the next larger binary16 value (v itself binary16 words).

    2^-24 throughout the subnormal range; 32 at 65504 (the gap to where 65536
    would be); inf for inf; nan for nan."""
    h = np.asarray(h, dtype=np.uint16) & np.uint16(0x7FFF)
    v = h.view(np.float16).astype(np.float64)
    nxt = (h.astype(np.uint32) + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    gap = nxt - v
    gap = np.where(h == 0x7BFF, 32.0, gap)
    gap = np.where(h == 0x7C00, np.inf, gap)
    gap = np.where(h > 0x7C00, np.nan, gap)
    return gap


def rne16_from_f64(v) -> np.ndarray:
    """Round FP64 values to binary16 words (numpy's correctly rounded conversion)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _same_special(a64, b64):
    both_nan = np.isnan(a64) & np.isnan(b64)
    same_inf = np.isinf(a64) & np.isinf(b64) & (np.sign(a64) == np.sign(b64))
    return both_nan | same_inf


def check_proj(p_gpu, p_ref, A, allowance: float = ORDER_ALLOWANCE):
    """Return (ok_mask, report) for projections (bias-less outputs)."""
    g = words_to_f64(p_gpu)
    r = words_to_f64(p_ref)
    A = np.asarray(A, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        diff = np.abs(g - r)
        tol = ulp16(p_ref) + allowance * U32 * A
        ok = (diff <= tol) | _same_special(g, r)
        strict = diff > ulp16(p_ref)
        ulps = np.where(np.isfinite(diff), diff / ulp16(p_ref), 0.0)
    return ok, _report(ok, strict & ~_same_special(g, r), ulps, r)


def check_y(y_gpu, y_ref, p_ref, A, allowance: float = ORDER_ALLOWANCE):
    """Return (ok_mask, report) for outputs of the bias call."""
    g = words_to_f64(y_gpu)
    r = words_to_f64(y_ref)
    A = np.asarray(A, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        diff = np.abs(g - r)
        tol = ulp16(y_ref) + ulp16(p_ref) + allowance * U32 * A
        ok = (diff <= tol) | _same_special(g, r)
        strict = diff > ulp16(y_ref)
        ulps = np.where(np.isfinite(diff), diff / ulp16(y_ref), 0.0)
    return ok, _report(ok, strict & ~_same_special(g, r), ulps, words_to_f64(p_ref))


def outer_band(S, A, K: int):
    """Return (lo, hi) binary16 words bounding every legal FP32-order projection."""
    S = np.asarray(S, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    km1 = max(int(K) - 1, 0)
    gamma = km1 * U32 / (1.0 - km1 * U32)
    # widen by a hair for the FP64 rounding of S, A and of the bound itself
    slack = gamma * A + 2.0 ** -50 * (np.abs(S) + A)
    return rne16_from_f64(S - slack), rne16_from_f64(S + slack)


def in_outer_band(p_gpu, S, A, K: int) -> np.ndarray:
    lo, hi = outer_band(S, A, K)
    g = words_to_f64(p_gpu)
    with np.errstate(invalid="ignore"):
        return (g >= words_to_f64(lo)) & (g <= words_to_f64(hi))


def _report(ok, strict, ulps, pvals):
    bad = ~ok
    rep = {
        "n": int(ok.size),
        "n_fail": int(bad.sum()),
        "strict_over_1ulp": int(strict.sum()),
        "max_ulp": float(np.nanmax(ulps)) if ulps.size else 0.0,
    }
    if strict.any():
        rep["strict_abs_proj_max"] = float(np.nanmax(np.abs(pvals[strict])))
    return rep
