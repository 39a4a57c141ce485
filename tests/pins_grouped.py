"""Pins of the oracle's grouped and indexed contractions ("The Graph IR", op
table: GroupedDenseContraction, a [G*N, K] weight read as G blocks of N rows
against a [G, M, K] activation; IndexedMatMul, x [M, K] against W [E, K, N] with
each row m taken against expert idx[m]).

The checks are independent of the oracle's loops: integer data against numpy
int64 contractions (exact), random data against numpy float64 sums through the
rigorous band, layout invariants (row permutations), and rows whose index has
no expert left untouched.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import tolerance

ELEMS = (tolerance.F16, tolerance.BF16)
DT = {tolerance.F16: torch.float16, tolerance.BF16: torch.bfloat16}


def _ints(shape, lo, hi, seed, elem):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g).to(DT[elem])


def _as_i64(t):
    return t.to(torch.float64).numpy().astype(np.int64)


def _rne(v, elem):
    return tolerance.rne_from_f64(np.asarray(v, np.float64), elem)


def pin_grouped_integers(orc):
    """Integer activations and weights (sums exact in FP32): the projection and the
    bias epilogue equal numpy int64 per-group products rounded once."""
    for elem in ELEMS:
        G, M, N, K = 3, 9, 11, 37
        r = 40 if elem == tolerance.F16 else 6        # sums past the type's exact integers
        x = _ints((G, M, K), -r, r, 1, elem)
        w = _ints((G * N, K), -r, r, 2, elem)
        b = _ints((G * N,), -40, 40, 3, elem)
        y, p, s = orc.grouped(x, w, b, elem=elem)
        exact = np.einsum("gmk,gnk->gmn", _as_i64(x), _as_i64(w).reshape(G, N, K))
        assert np.array_equal(s.astype(np.float64), exact.astype(np.float64))
        assert np.array_equal(p, _rne(exact, elem))
        yb = exact + _as_i64(b).reshape(G, 1, N)
        # one rounding of exact + b differs from the round-then-add definition only
        # when the projection rounded: compare against the definition's two roundings
        want = _rne(tolerance.words_to_f64(_rne(exact, elem), elem) + _as_i64(b).reshape(G, 1, N), elem)
        assert np.array_equal(y, want)
        assert (np.abs(exact) > (2048 if elem == tolerance.F16 else 256)).any(), "some sums must round"
        assert yb.shape == y.shape


def pin_grouped_random_band(orc, seed: int = 4):
    """Random data: every projection inside the rigorous band of the float64 sum."""
    for elem in ELEMS:
        G, M, N, K = 4, 17, 23, 300
        g = torch.Generator().manual_seed(seed)
        x = torch.randn(G, M, K, generator=g).to(DT[elem])
        w = (torch.rand(G * N, K, generator=g) * 2 - 1).mul(0.06).to(DT[elem])
        _, p, s = orc.grouped(x, w, None, elem=elem)
        xf = x.to(torch.float64).numpy()
        wf = w.to(torch.float64).numpy().reshape(G, N, K)
        S = np.einsum("gmk,gnk->gmn", xf, wf)
        A = np.einsum("gmk,gnk->gmn", np.abs(xf), np.abs(wf))
        assert tolerance.in_outer_band(p, S, A, K, elem=elem).all()
        ok, rep = tolerance.check_sums(s, S, A, K)
        assert ok.all(), rep


def pin_indexed_integers(orc):
    """Integer data: y[m] = x[m] @ W[idx[m]] exactly, each expert [K, N] read with k
    first; rows with an index outside [0, E) keep their previous contents."""
    for elem in ELEMS:
        M, E, K, N = 13, 5, 29, 19
        x = _ints((M, K), -5, 5, 5, elem)
        W = _ints((E, K, N), -5, 5, 6, elem)
        idx = np.array([0, 4, 4, 2, 1, 1, 0, 3, 7, -1, 2, 4, 5], np.int32)
        sentinel = np.full((M, N), 0x1234, np.uint16)
        y, s = orc.indexed(x, W, idx, elem=elem, y_init=sentinel)
        xi, Wi = _as_i64(x), _as_i64(W)
        for m in range(M):
            if 0 <= idx[m] < E:
                exact = xi[m] @ Wi[idx[m]]
                assert np.array_equal(s[m].astype(np.float64), exact.astype(np.float64)), m
                assert np.array_equal(y[m], _rne(exact, elem)), m
            else:
                assert (y[m] == 0x1234).all(), "a row without an expert was written"


def pin_indexed_random_band_and_permutation(orc, seed: int = 7):
    """Random data inside the band of the float64 sums; permuting the rows of x and
    idx together permutes y the same way; a single expert equals the dense
    contraction with that expert's [K, N] table."""
    for elem in ELEMS:
        M, E, K, N = 40, 6, 260, 33
        g = torch.Generator().manual_seed(seed)
        x = torch.randn(M, K, generator=g).to(DT[elem])
        W = (torch.rand(E, K, N, generator=g) * 2 - 1).mul(0.06).to(DT[elem])
        idx = torch.randint(0, E, (M,), generator=g).numpy().astype(np.int32)
        y, s = orc.indexed(x, W, idx, elem=elem)
        xf, Wf = x.to(torch.float64).numpy(), W.to(torch.float64).numpy()
        S = np.stack([xf[m] @ Wf[idx[m]] for m in range(M)])
        A = np.stack([np.abs(xf[m]) @ np.abs(Wf[idx[m]]) for m in range(M)])
        assert tolerance.in_outer_band(y, S, A, K, elem=elem).all()
        S2, A2 = orc.indexed_band(x, W, idx, elem=elem)
        assert np.allclose(S2, S, rtol=0, atol=1e-12 * (1 + np.abs(A))) and np.allclose(A2, A, rtol=1e-12)
        perm = np.random.default_rng(seed).permutation(M)
        yp, _ = orc.indexed(x[torch.from_numpy(perm)], W, idx[perm], elem=elem)
        assert np.array_equal(yp, y[perm])
        one = np.full(M, 2, np.int32)
        y1, _ = orc.indexed(x, W, one, elem=elem)
        _, p1 = orc.linear(x, W[2].t().contiguous(), None, elem=elem)
        assert np.array_equal(y1, p1)


def pin_indexed_k0_and_empty(orc):
    for elem in ELEMS:
        x = torch.zeros(4, 0, dtype=DT[elem])
        W = torch.zeros(3, 0, 5, dtype=DT[elem])
        y, s = orc.indexed(x, W, np.array([0, 1, 2, 0], np.int32), elem=elem)
        assert (y == 0).all() and (s == 0).all()


GROUPED_PINS = [
    pin_grouped_integers,
    pin_grouped_random_band,
    pin_indexed_integers,
    pin_indexed_random_band_and_permutation,
    pin_indexed_k0_and_empty,
]
