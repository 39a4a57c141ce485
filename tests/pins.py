"""Pins of the CPU oracle against facts fixed outside it.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  The references are independent of oracle.c: numpy's and torch's
binary16 conversions, FP64 exact arithmetic, integer arithmetic, closed forms
of structured inputs, brute force over summation trees, hand-derived fixtures
under tests/golden/.  The same functions run against deliberately broken
builds of the oracle (test_oracle_mutants.py), so every plausible mistake must
make at least one of them fail.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import torch

from linear_amd import workloads
from oracle import tolerance

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f16(vals) -> np.ndarray:
    return np.asarray(vals, dtype=np.float64).astype(np.float16)


def _words(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        return a.contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.astype(np.uint16)


def _eq_words(got, want):
    """Bitwise equality, except that any NaN matches any NaN and +0 matches -0."""
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    g = got.view(np.float16)
    w = want.view(np.float16)
    nan_ok = np.isnan(g) & np.isnan(w)
    zero_ok = (g == 0) & (w == 0)
    return (got == want) | nan_ok | zero_ok


def _assert_words(got, want, what):
    ok = _eq_words(got, want)
    if not ok.all():
        i = np.flatnonzero(~ok.ravel())[:5]
        raise AssertionError("%s: %d mismatches, first at %s: got %s want %s" % (
            what, (~ok).sum(), i.tolist(), np.asarray(got).ravel()[i].tolist(),
            np.asarray(want).ravel()[i].tolist()))


# --------------------------------------------------------------------------- conversions

def pin_decode_exhaustive(orc):
    """binary16 -> binary32 for all 65,536 words vs numpy's conversion."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN pattern differs"
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)), "decode differs"


def pin_rne_spot_values(orc):
    """Hand-derived binary16 rounding cases (tests/golden/binary16_spot.txt)."""
    rows = []
    for line in open(os.path.join(GOLDEN, "binary16_spot.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f_hex, h_hex = line.split()[:2]
        rows.append((int(f_hex, 16), int(h_hex, 16)))
    f = np.array([r[0] for r in rows], np.uint32).view(np.float32)
    want = np.array([r[1] for r in rows], np.uint16)
    got = orc.f32_to_f16(f)
    assert np.array_equal(got, want), list(zip(got.tolist(), want.tolist()))


def pin_rne_sampled(orc, count: int = 1 << 22, seed: int = 1):
    """binary32 -> binary16 on random words plus every binary32 exponent with the
    rounding-sensitive low fraction bits enumerated, vs torch's conversion."""
    g = np.random.default_rng(seed)
    rnd = g.integers(0, 1 << 32, count, dtype=np.uint64).astype(np.uint32)
    exps = np.arange(256, dtype=np.uint32) << 23
    low = np.arange(1 << 14, dtype=np.uint32)
    highs = np.array([0, 1 << 14, 0x155555 & ~0x3FFF, 0x7FC000], np.uint32)
    grid = (exps[:, None, None] | highs[None, :, None] | low[None, None, :]).ravel()
    words = np.concatenate([rnd, grid, grid | np.uint32(0x80000000)])
    check_rne_words(orc, words)


def check_rne_words(orc, words: np.ndarray):
    f = words.view(np.float32)
    got = orc.f32_to_f16(f)
    want = torch.from_numpy(f.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    _assert_words(got, want, "f32->f16")


# --------------------------------------------------------------------------- epilogue

def pin_bias_epilogue_vs_exact(orc, count: int = 1 << 21, seed: int = 2):
    """RNE16(f32(p) + f32(b)) equals the correctly rounded exact sum (FP64 holds any
    binary16 + binary16 sum exactly; numpy rounds FP64 to binary16 directly).
    Random finite pairs, plus every finite p against a set of b values that make
    ties and cancellations."""
    g = np.random.default_rng(seed)
    p = g.integers(0, 1 << 16, count, dtype=np.int64).astype(np.uint16)
    b = g.integers(0, 1 << 16, count, dtype=np.int64).astype(np.uint16)
    allp = np.arange(1 << 16, dtype=np.int64).astype(np.uint16)
    special_b = _words(_f16([0.0, -0.0, 1.0, -1.0, 0.5, 2.0 ** -24, -(2.0 ** -24), 2.0 ** -14,
                             1024.0, -2048.0, 65504.0, -65504.0, 3.0, 0.000123]))
    p = np.concatenate([p, np.repeat(allp, special_b.size)])
    b = np.concatenate([b, np.tile(special_b, allp.size)])
    fin = np.isfinite(p.view(np.float16)) & np.isfinite(b.view(np.float16))
    p, b = p[fin], b[fin]
    got = orc.bias_epilogue(p, b)
    exact = p.view(np.float16).astype(np.float64) + b.view(np.float16).astype(np.float64)
    want = exact.astype(np.float16).view(np.uint16)
    _assert_words(got, want, "bias epilogue")


# --------------------------------------------------------------------------- closed forms

def pin_k1_closed_form(orc, count: int = 1 << 16, seed: int = 3):
    """K = 1: proj = RNE16(x * w), the product exact in FP64; y = RNE16(proj + b)."""
    x = _words(workloads.random_words((count, 1), seed=seed))
    w = _words(workloads.random_words((count, 1), seed=seed + 1))
    b = _words(workloads.random_words((count,), seed=seed + 2))
    # evaluate as `count` independent 1x1 problems through the points interface
    # (row i of x against row i of w) and as one [count, count] product's diagonal
    ms = np.arange(count)
    r = orc.points(x, w, b, ms, ms)
    exact = x[:, 0].view(np.float16).astype(np.float64) * w[:, 0].view(np.float16).astype(np.float64)
    want_p = exact.astype(np.float16).view(np.uint16)
    _assert_words(r["proj"], want_p, "K=1 proj (points)")
    want_y = (want_p.view(np.float16).astype(np.float64)
              + b.view(np.float16).astype(np.float64)).astype(np.float16).view(np.uint16)
    _assert_words(r["y"], want_y, "K=1 y (points)")
    # full path: 256 x 256 outer product, every pair
    xs, ws = x[:256], w[:256]
    y, p = orc.linear(xs, ws, b[:256])
    ex = xs.view(np.float16).astype(np.float64) @ ws.view(np.float16).astype(np.float64).T
    wp = ex.astype(np.float16).view(np.uint16)
    _assert_words(p, wp, "K=1 proj (full)")
    wy = (wp.view(np.float16).astype(np.float64)
          + b[:256].view(np.float16).astype(np.float64)[None, :]).astype(np.float16).view(np.uint16)
    _assert_words(y, wy, "K=1 y (full)")


def pin_k2_unique(orc, count: int = 1 << 15, seed: int = 4):
    """K = 2: one commutative FP32 add of two exact products -- a unique result,
    computed here with numpy float32 arithmetic."""
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(count, 2, generator=g) * 4).to(torch.float16)
    w = (torch.randn(count, 2, generator=g) * 4).to(torch.float16)
    xn, wn = _words(x), _words(w)
    ms = np.arange(count)
    r = orc.points(xn, wn, None, ms, ms)
    xf = xn.view(np.float16).astype(np.float32)
    wf = wn.view(np.float16).astype(np.float32)
    s = (xf[:, 0] * wf[:, 0]) + (xf[:, 1] * wf[:, 1])  # float32 products exact, one rounded add
    want = torch.from_numpy(s).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    _assert_words(r["proj"], want, "K=2")


def _all_trees(vals):
    """Every FP32 value reachable by summing vals pairwise in any order and association."""
    vals = tuple(np.float32(v) for v in vals)
    if len(vals) == 1:
        return {vals[0].view(np.uint32).item()}
    out = set()
    for i, j in itertools.combinations(range(len(vals)), 2):
        rest = [vals[k] for k in range(len(vals)) if k not in (i, j)]
        out |= _all_trees(rest + [np.float32(vals[i] + vals[j])])
    return out


def pin_small_k_trees(orc, cases: int = 60, seed: int = 5):
    """K = 3, 4, 5: the oracle's projection is RNE16 of the left-to-right FP32 sum,
    which is one member of the set of all summation trees (brute force)."""
    g = torch.Generator().manual_seed(seed)
    for K in (3, 4, 5):
        # wide dynamic range so that different trees really give different sums
        x = (torch.randn(cases, K, generator=g) * torch.exp2(torch.randint(-6, 7, (cases, K), generator=g))).to(torch.float16)
        w = (torch.randn(cases, K, generator=g) * torch.exp2(torch.randint(-6, 7, (cases, K), generator=g))).to(torch.float16)
        xn, wn = _words(x), _words(w)
        ms = np.arange(cases)
        r = orc.points(xn, wn, None, ms, ms)
        y, p = orc.linear(xn, wn, None)
        xf = xn.view(np.float16).astype(np.float32)
        wf = wn.view(np.float16).astype(np.float32)
        for i in range(cases):
            prods = [np.float32(xf[i, k] * wf[i, k]) for k in range(K)]
            acc = np.float32(0.0)
            for v in prods:
                acc = np.float32(acc + v)
            seq = torch.tensor([float(acc)], dtype=torch.float32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)[0]
            trees = _all_trees(prods)
            tree16 = {torch.tensor([np.uint32(t).view(np.float32).item()], dtype=torch.float32)
                      .to(torch.float16).view(torch.int16).numpy().view(np.uint16)[0] for t in trees}
            got = r["proj"][i]
            assert _eq_words(np.array([got]), np.array([seq]))[0], (K, i, got, seq)
            assert got in tree16 or (got & 0x7FFF) == 0, (K, i, got, tree16)
            assert _eq_words(np.array([p[i, i]]), np.array([got]))[0], (K, i, "full vs points")


def pin_identity(orc, seed: int = 6):
    """W = I (N = K): proj = x exactly (a -0 input gives +0); y = RNE16(x + b)."""
    K = 96
    x = _words(workloads.random_words((40, K), seed=seed))
    w = _words(np.eye(K, dtype=np.float16))
    b = _words(workloads.random_words((K,), seed=seed + 1))
    y, p = orc.linear(x, w, b)
    _assert_words(p, x, "identity proj")
    want_y = (x.view(np.float16).astype(np.float64) + b.view(np.float16).astype(np.float64)[None, :]
              ).astype(np.float16).view(np.uint16)
    _assert_words(y, want_y, "identity y")


def pin_one_hot(orc, seed: int = 7):
    """W[n, k] = 2^e_n * delta(k, pi(n)): proj[m, n] = RNE16(2^e_n * x[m, pi(n)])."""
    g = np.random.default_rng(seed)
    M, N, K = 33, 70, 50
    x = _words(workloads.random_words((M, K), seed=seed))
    pi = g.integers(0, K, N)
    e = g.integers(-4, 5, N)
    w = np.zeros((N, K), np.float64)
    w[np.arange(N), pi] = 2.0 ** e
    w16 = _words(_f16(w))
    y, p = orc.linear(x, w16, None)
    want = (x.view(np.float16).astype(np.float64)[:, pi] * (2.0 ** e)[None, :]).astype(np.float16).view(np.uint16)
    _assert_words(p, want, "one-hot")


def pin_small_integers(orc, seed: int = 8):
    """Integer inputs with sum |x*w| < 2^24: every order is exact, so proj is the
    integer sum rounded once; compared with int64 arithmetic."""
    for (M, N, K) in ((17, 23, 300), (5, 9, 1), (64, 3, 1000)):
        x, w, b = workloads.small_integers(M, N, K, seed=seed + K)
        xi = x.to(torch.int64).numpy()
        wi = w.to(torch.int64).numpy()
        s = xi @ wi.T
        want_p = s.astype(np.float64).astype(np.float16).view(np.uint16)
        want_y = (want_p.view(np.float16).astype(np.float64) + b.to(torch.float64).numpy()[None, :]
                  ).astype(np.float16).view(np.uint16)
        y, p = orc.linear(x, w, b)
        _assert_words(p, want_p, "int proj %s" % ((M, N, K),))
        _assert_words(y, want_y, "int y %s" % ((M, N, K),))


def pin_golden_round_before_bias(orc):
    """The hand-derived cases of tests/golden/round_before_bias.txt."""
    for line in open(os.path.join(GOLDEN, "round_before_bias.txt")):
        if line.startswith("#") or not line.strip():
            continue
        xs, ws, b, p, y, _ = [s.strip() for s in line.split(";")]
        x = _words(_f16([[float(v) for v in xs.split(",")]]))
        w = _words(_f16([[float(v) for v in ws.split(",")]]))
        bb = _words(_f16([float(b)]))
        for v, raw in ((x, xs), (w, ws), (bb, b)):
            assert v.view(np.float16).astype(np.float64).ravel().tolist() == \
                [float(t) for t in raw.split(",")], "fixture input not a binary16 value: " + raw
        yy, pp = orc.linear(x, w, bb)
        assert float(pp.view(np.float16)[0, 0]) == float(p), (line, pp.view(np.float16))
        assert float(yy.view(np.float16)[0, 0]) == float(y), (line, yy.view(np.float16))


def pin_k0_empty_sum(orc):
    """K = 0: the empty sum is +0, so proj = +0 and y = RNE16(0 + b) = b (a -0 bias gives +0)."""
    b = _words(workloads.random_words((37,), seed=9))
    x = np.zeros((5, 0), np.uint16)
    w = np.zeros((37, 0), np.uint16)
    y, p = orc.linear(x, w, b)
    assert (p == 0).all()
    _assert_words(y, np.broadcast_to(b, (5, 37)), "K=0 y")


# --------------------------------------------------------------------------- invariants

def pin_scale_invariance(orc, seed: int = 10):
    """proj(2^j x) = 2^j proj(x) bit for bit, when nothing under- or overflows."""
    x, w, _ = workloads.make_inputs(24, 40, 200, 1.0 / 16, seed=seed)
    x = x.clamp(-8, 8)
    _, p0 = orc.linear(x, w, None)
    for j in (1, 3, -2):
        xs = (x.to(torch.float32) * 2.0 ** j).to(torch.float16)
        _, pj = orc.linear(xs, w, None)
        ref = p0.view(np.float16).astype(np.float64) * 2.0 ** j
        small = np.abs(p0.view(np.float16).astype(np.float64)) < 2.0 ** -10  # subnormal-prone
        want = ref.astype(np.float16).view(np.uint16)
        ok = _eq_words(pj, want) | small
        assert ok.all(), ("scale", j, int((~ok).sum()))


def pin_permutations(orc, seed: int = 11):
    """Permuting rows of W permutes columns of y; permuting rows of x permutes rows of y."""
    x, w, b = workloads.make_inputs(30, 50, 128, 0.1, seed=seed)
    y, p = orc.linear(x, w, b)
    g = torch.Generator().manual_seed(seed)
    pn = torch.randperm(50, generator=g).numpy()
    pm = torch.randperm(30, generator=g).numpy()
    y2, _ = orc.linear(x, w[torch.from_numpy(pn)], b[torch.from_numpy(pn)])
    _assert_words(y2, y[:, pn], "W-row permutation")
    y3, _ = orc.linear(x[torch.from_numpy(pm)], w, b)
    _assert_words(y3, y[pm, :], "x-row permutation")


def pin_thread_determinism(orc, seed: int = 12):
    """Bit-identical results with 1 thread and with every thread."""
    x, w, b = workloads.make_inputs(64, 96, 512, 1 / 16, seed=seed)
    y1, p1 = orc.linear(x, w, b, nthreads=1)
    yn, pn = orc.linear(x, w, b, nthreads=max(2, orc.max_threads()))
    assert np.array_equal(y1, yn) and np.array_equal(p1, pn)


def pin_random_band(orc, M: int = 96, N: int = 160, K: int = 768, seed: int = 13):
    """Random data with the toy's law: S and A agree with numpy FP64 matmuls; the
    oracle's projection lies in the rigorous outer band around S, is within the
    acceptance rule of RNE16(S), and the points interface reproduces the full one."""
    x, w, b = workloads.make_inputs(M, N, K, 1.0 / np.sqrt(768.0), seed=seed)
    xd = x.to(torch.float64).numpy()
    wd = w.to(torch.float64).numpy()
    S_np = xd @ wd.T
    A_np = np.abs(xd) @ np.abs(wd).T
    S, A = orc.band(x, w)
    assert np.allclose(S, S_np, rtol=1e-12, atol=1e-12), "S differs from numpy"
    assert np.allclose(A, A_np, rtol=1e-12, atol=1e-12), "A differs from numpy"
    y, p = orc.linear(x, w, b)
    assert tolerance.in_outer_band(p, S_np, A_np, K).all(), "outside the outer band"
    exact16 = tolerance.rne16_from_f64(S_np)
    ok, rep = tolerance.check_proj(p, exact16, A_np)
    assert ok.all(), rep
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    r = orc.points(x, w, b, ms.ravel(), ns.ravel())
    _assert_words(r["proj"], p.ravel(), "points vs full proj")
    _assert_words(r["y"], y.ravel(), "points vs full y")
    assert np.allclose(r["S"], S_np.ravel(), rtol=1e-12, atol=1e-12)
    # bias: y is the oracle's epilogue of its own projection
    _assert_words(y, orc.bias_epilogue(p, np.broadcast_to(_words(b), (M, N)).copy()), "y from proj")


def pin_strided_layout(orc, seed: int = 14):
    """Row strides larger than K read the same logical matrices (the points
    interface takes raw strided storage)."""
    x, w, b = workloads.make_inputs(9, 13, 40, 0.2, seed=seed)
    y, p = orc.linear(x, w, b)
    xpad = torch.zeros(9, 48, dtype=torch.float16)
    xpad[:, :40] = x
    xpad[:, 40:] = float("nan")
    import ctypes
    xw = _words(xpad)
    ww = _words(w)
    bw = _words(b)
    ms, ns = np.meshgrid(np.arange(9), np.arange(13), indexing="ij")
    ms = np.ascontiguousarray(ms.ravel(), np.int64)
    ns = np.ascontiguousarray(ns.ravel(), np.int64)
    out = np.zeros(ms.size, np.uint16)
    u16 = ctypes.POINTER(ctypes.c_uint16)
    i64 = ctypes.POINTER(ctypes.c_int64)
    orc.lib.oracle_linear_f16_points(xw.ctypes.data_as(u16), 48, ww.ctypes.data_as(u16), 40,
                                     bw.ctypes.data_as(u16), 40, ms.ctypes.data_as(i64),
                                     ns.ctypes.data_as(i64), ms.size, out.ctypes.data_as(u16),
                                     None, None, None, 0)
    _assert_words(out, y.ravel(), "strided x")


def pin_toy_shapes():
    """The toy workload has the shapes the pages give (tests/golden/toy_workload.json)."""
    spec = json.load(open(os.path.join(GOLDEN, "toy_workload.json")))
    wl = workloads.WORKLOADS["toy"]
    assert [wl.M, wl.K] == spec["x"]
    assert [wl.N, wl.K] == spec["weight"]
    assert [wl.N] == spec["b"]
    assert [wl.M, wl.N] == spec["y"]
    assert wl.K == spec["contraction_K"]


# --------------------------------------------------------------------------- bfloat16

def rne_bf16_ref(d) -> np.ndarray:
    """Round FP64 values to bfloat16 (8 significant bits), ties to even, via frexp/rint;
    returns the bfloat16 words.  Valid for results in the normal range."""
    d = np.asarray(d, np.float64)
    m, e = np.frexp(d)
    r = np.ldexp(np.rint(m * 256.0), e - 8)        # numpy rint rounds half to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_words_to_f64(h) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16(vals) -> np.ndarray:
    return rne_bf16_ref(np.asarray(vals, np.float64))


def pin_bf16_decode_exhaustive(orc):
    """bfloat16 -> binary32 for all 65,536 words vs torch's conversion."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    want = torch.from_numpy(h.astype(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def check_bf16_rne_words(orc, words: np.ndarray):
    f = words.view(np.float32)
    got = orc.f32_to_bf16(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gf = got.view(np.uint16)
    nan_g = (gf & 0x7F80) == 0x7F80
    nan_g &= (gf & 0x007F) != 0
    nan_w = ((want & 0x7F80) == 0x7F80) & ((want & 0x007F) != 0)
    ok = (got == want) | (nan_g & nan_w)
    if not ok.all():
        i = np.flatnonzero(~ok)[:5]
        raise AssertionError("f32->bf16: %d mismatches, e.g. %s -> %s want %s" % (
            (~ok).sum(), words[i].tolist(), got[i].tolist(), want[i].tolist()))


def pin_bf16_rne_sampled(orc, count: int = 1 << 22, seed: int = 21):
    """binary32 -> bfloat16 on random words plus every exponent with the low 17 bits
    enumerated (tie, carry and overflow patterns), vs torch's conversion."""
    g = np.random.default_rng(seed)
    rnd = g.integers(0, 1 << 32, count, dtype=np.uint64).astype(np.uint32)
    exps = np.arange(256, dtype=np.uint32) << 23
    low = np.arange(1 << 17, dtype=np.uint32)
    highs = np.array([0, 0x7E0000, 0x520000], np.uint32)
    grid = (exps[:, None, None] | highs[None, :, None] | low[None, None, :]).ravel()
    check_bf16_rne_words(orc, np.concatenate([rnd, grid, grid | np.uint32(0x80000000)]))


def _random_bf16(shape, seed, lo=-20, hi=20):
    """Random finite bfloat16 words with exponents in [lo, hi] (results stay normal)."""
    g = np.random.default_rng(seed)
    e = g.integers(lo, hi + 1, shape)
    m = g.integers(0, 128, shape)
    sgn = g.integers(0, 2, shape)
    v = np.ldexp(1.0 + m / 128.0, e) * np.where(sgn == 1, -1.0, 1.0)
    return rne_bf16_ref(v)


def pin_bf16_epilogue_vs_exact(orc, count: int = 1 << 20, seed: int = 22):
    """RNE_bf16(f32(p) + f32(b)) equals the FP64 sum rounded once to bfloat16."""
    p = _random_bf16(count, seed)
    b = _random_bf16(count, seed + 1)
    got = orc.bias_epilogue(p, b, elem=1)
    exact = bf16_words_to_f64(p) + bf16_words_to_f64(b)
    want = rne_bf16_ref(exact)
    zero = exact == 0
    want[zero] = 0
    ok = (got == want) | (zero & ((got & 0x7FFF) == 0))
    assert ok.all(), int((~ok).sum())


def pin_bf16_k1_closed_form(orc, count: int = 1 << 15, seed: int = 23):
    """K = 1 in bfloat16: proj = RNE_bf16(x * w), the product exact in FP64."""
    x = _random_bf16((count, 1), seed)
    w = _random_bf16((count, 1), seed + 1)
    ms = np.arange(count)
    r = orc.points(x, w, None, ms, ms, elem=1)
    want = rne_bf16_ref(bf16_words_to_f64(x[:, 0]) * bf16_words_to_f64(w[:, 0]))
    assert np.array_equal(r["proj"], want)


def pin_bf16_small_integers(orc, seed: int = 24):
    """Integer bfloat16 inputs: every order is exact; proj is the integer sum rounded once."""
    for (M, N, K) in ((17, 23, 300), (5, 9, 1), (40, 3, 700)):
        x, w, b = workloads.small_integers(M, N, K, seed=seed + K)
        xb, wb, bb = x.to(torch.bfloat16), w.to(torch.bfloat16), b.to(torch.bfloat16)
        s = x.to(torch.int64).numpy() @ w.to(torch.int64).numpy().T
        want_p = rne_bf16_ref(s.astype(np.float64))
        want_y = rne_bf16_ref(bf16_words_to_f64(want_p) + b.to(torch.float64).numpy()[None, :])
        z = (want_p & 0x7FFF) == 0
        y, p = orc.linear(xb, wb, bb, elem=1)
        assert np.array_equal(p[~z], want_p[~z]) and ((p[z] & 0x7FFF) == 0).all(), "bf16 int proj"
        zy = (want_y & 0x7FFF) == 0
        assert np.array_equal(y[~zy], want_y[~zy]) and ((y[zy] & 0x7FFF) == 0).all(), "bf16 int y"


def pin_bf16_golden_round_before_bias(orc):
    """The hand-derived cases of tests/golden/round_before_bias_bf16.txt."""
    for line in open(os.path.join(GOLDEN, "round_before_bias_bf16.txt")):
        if line.startswith("#") or not line.strip():
            continue
        xs, ws, b, p, y, _ = [t.strip() for t in line.split(";")]
        x = _bf16([[float(v) for v in xs.split(",")]])
        w = _bf16([[float(v) for v in ws.split(",")]])
        bb = _bf16([float(b)])
        assert bf16_words_to_f64(x).ravel().tolist() == [float(t) for t in xs.split(",")], xs
        yy, pp = orc.linear(x, w, bb, elem=1)
        assert bf16_words_to_f64(pp)[0, 0] == float(p), (line, bf16_words_to_f64(pp))
        assert bf16_words_to_f64(yy)[0, 0] == float(y), (line, bf16_words_to_f64(yy))


def pin_f32_sums(orc, seed: int = 25):
    """The unrounded sums: equal to a numpy float32 left-to-right accumulation, and
    within the recursive-summation bound of the FP64 sum."""
    for elem, dt in ((0, torch.float16), (1, torch.bfloat16)):
        x, w, _ = workloads.make_inputs(7, 11, 37, 0.2, seed=seed + elem)
        x, w = x.to(dt), w.to(dt)
        _, _, y32 = orc.linear(x, w, None, elem=elem, sums=True)
        xf, wf = x.to(torch.float32).numpy(), w.to(torch.float32).numpy()
        acc = np.zeros((7, 11), np.float32)
        for k in range(37):
            acc = (acc + xf[:, k:k + 1] * wf[None, :, k].reshape(1, 11)).astype(np.float32)
        assert np.array_equal(y32, acc), "FP32 sums differ from the left-to-right float32 loop"
        S = x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
        A = np.abs(x.to(torch.float64).numpy()) @ np.abs(w.to(torch.float64).numpy()).T
        gamma = 36 * 2.0 ** -24 / (1 - 36 * 2.0 ** -24)
        assert (np.abs(y32 - S) <= gamma * A + 1e-30).all()


FAST_PINS = [
    pin_decode_exhaustive, pin_rne_spot_values, pin_rne_sampled, pin_bias_epilogue_vs_exact,
    pin_k1_closed_form, pin_k2_unique, pin_small_k_trees, pin_identity, pin_one_hot,
    pin_small_integers, pin_golden_round_before_bias, pin_k0_empty_sum, pin_scale_invariance,
    pin_permutations, pin_thread_determinism, pin_random_band, pin_strided_layout,
    pin_bf16_decode_exhaustive, pin_bf16_rne_sampled, pin_bf16_epilogue_vs_exact, pin_bf16_k1_closed_form,
    pin_bf16_small_integers, pin_bf16_golden_round_before_bias, pin_f32_sums,
]
