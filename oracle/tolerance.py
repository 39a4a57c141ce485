"""Test infrastructure: the acceptance rule for GPU results against the oracle.

The contract ("tensor programs, part 1", section "One Program and One Numerical
Contract") lets the summation order vary, so for random data more than one
projection is correct.  The oracle supplies one legal result (sequential FP32
order) plus FP64 band data S = sum x*w and A = sum |x*w|.  A GPU result is
accepted when it is within

    proj:  |p_gpu - p_ref| <= ulp(p_ref) + ORDER_ALLOWANCE * u32 * A
    y:     |y_gpu - y_ref| <= ulp(y_ref) + ulp(p_ref) + ORDER_ALLOWANCE * u32 * A

(u32 = 2^-24; ulp of binary16 or bfloat16 as the element type says), and it
must always lie inside the rigorous outer band [RNE(S - G*A), RNE(S + G*A)].
Rounding to FP16 / BF16 is monotone, so a result outside it is a bug, not a
legal reordering.  Integer-exact cases are compared bit for bit instead.

G is the forward-error bound of FP32 accumulation as the matrix unit performs
it.  A matrix-core step adds n products (n = 16 or 32) to the FP32 accumulator
as one operation: every term is aligned to the largest one, bits below
2^(e-24) (e the largest term's exponent, one guard bit past FP32's last place)
are dropped toward zero, and the exact sum of what is left is rounded to FP32,
nearest even.  That is FP32 accumulation in the contract's sense, but not a
sequence of IEEE additions: one step errs by less than (n+1)*u32*max|t| +
u32*|sum| <= (n+2)*u32*sum|t|, against u32 per IEEE addition.  Over a chain of
ceil(K/n) steps and at most 8 IEEE additions of partial sums that gives

    G(K) = max over n in {16, 32} of ((n+2)*ceil(K/n) + 8) * u32, over (1 - that)

which also covers every IEEE summation order (their bound is (K-1)*u32 / (1-(K-1)*u32)).
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
ORDER_ALLOWANCE = 16.0


F16 = 0
BF16 = 1


def words_to_f64(h, elem: int = F16) -> np.ndarray:
    h = np.asarray(h)
    if elem == BF16:
        with np.errstate(invalid="ignore"):
            return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if h.dtype == np.float16:
        return h.astype(np.float64)
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp_bf16(h) -> np.ndarray:
    """Gap from |v| to the next larger bfloat16 value (v bfloat16 words)."""
    h = np.asarray(h, dtype=np.uint16) & np.uint16(0x7FFF)
    v = words_to_f64(h, BF16)
    nxt = words_to_f64((h.astype(np.uint32) + 1).astype(np.uint16), BF16)
    gap = nxt - v
    gap = np.where(h == 0x7F7F, 2.0 ** 120, gap)
    gap = np.where(h == 0x7F80, np.inf, gap)
    gap = np.where(h > 0x7F80, np.nan, gap)
    return gap


def ulp(h, elem: int = F16) -> np.ndarray:
    return ulp_bf16(h) if elem == BF16 else ulp16(h)


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


def rne_bf16_from_f64(v) -> np.ndarray:
    """Round FP64 values to bfloat16 words, ties to even (frexp / rint; normal range)."""
    v = np.asarray(v, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(v)
        r = np.ldexp(np.rint(m * 256.0), e - 8)
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rne_from_f64(v, elem: int = F16) -> np.ndarray:
    return rne_bf16_from_f64(v) if elem == BF16 else rne16_from_f64(v)


def _same_special(a64, b64):
    both_nan = np.isnan(a64) & np.isnan(b64)
    same_inf = np.isinf(a64) & np.isinf(b64) & (np.sign(a64) == np.sign(b64))
    return both_nan | same_inf


def check_proj(p_gpu, p_ref, A, allowance: float = ORDER_ALLOWANCE, elem: int = F16):
    """Return (ok_mask, report) for projections (bias-less outputs)."""
    g = words_to_f64(p_gpu, elem)
    r = words_to_f64(p_ref, elem)
    A = np.asarray(A, dtype=np.float64)
    u = ulp(p_ref, elem)
    with np.errstate(invalid="ignore"):
        diff = np.abs(g - r)
        tol = u + allowance * U32 * A
        ok = (diff <= tol) | _same_special(g, r)
        strict = diff > u
        ulps = np.where(np.isfinite(diff), diff / u, 0.0)
    return ok, _report(ok, strict & ~_same_special(g, r), ulps, r)


def check_y(y_gpu, y_ref, p_ref, A, allowance: float = ORDER_ALLOWANCE, elem: int = F16):
    """Return (ok_mask, report) for outputs of the bias call."""
    g = words_to_f64(y_gpu, elem)
    r = words_to_f64(y_ref, elem)
    A = np.asarray(A, dtype=np.float64)
    uy = ulp(y_ref, elem)
    with np.errstate(invalid="ignore"):
        diff = np.abs(g - r)
        tol = uy + ulp(p_ref, elem) + allowance * U32 * A
        ok = (diff <= tol) | _same_special(g, r)
        strict = diff > uy
        ulps = np.where(np.isfinite(diff), diff / uy, 0.0)
    return ok, _report(ok, strict & ~_same_special(g, r), ulps, words_to_f64(p_ref, elem))


def gamma_accumulation(K: int) -> float:
    """G(K) of the module docstring: relative bound (times A) of FP32 accumulation."""
    K = max(int(K), 0)
    if K == 0:
        return 0.0
    steps = max((n + 2) * (-(-K // n)) + 8 for n in (16, 32))
    return steps * U32 / (1.0 - steps * U32)


def check_sums(s_gpu, S, A, K: int):
    """FP32 sums against the FP64 sum: within G(K) * A (plus FP64 rounding slack)."""
    s_gpu = np.asarray(s_gpu, np.float64)
    gamma = gamma_accumulation(K)
    with np.errstate(invalid="ignore"):
        ok = np.abs(s_gpu - S) <= gamma * A + 2.0 ** -50 * (np.abs(S) + A)
    return ok, {"n": int(ok.size), "n_fail": int((~ok).sum())}


def outer_band(S, A, K: int, elem: int = F16):
    """Return (lo, hi) words bounding every legal FP32-order projection."""
    S = np.asarray(S, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    gamma = gamma_accumulation(K)
    # widen by a hair for the FP64 rounding of S, A and of the bound itself
    slack = gamma * A + 2.0 ** -50 * (np.abs(S) + A)
    return rne_from_f64(S - slack, elem), rne_from_f64(S + slack, elem)


def in_outer_band(p_gpu, S, A, K: int, elem: int = F16) -> np.ndarray:
    lo, hi = outer_band(S, A, K, elem)
    g = words_to_f64(p_gpu, elem)
    with np.errstate(invalid="ignore"):
        return (g >= words_to_f64(lo, elem)) & (g <= words_to_f64(hi, elem))


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
